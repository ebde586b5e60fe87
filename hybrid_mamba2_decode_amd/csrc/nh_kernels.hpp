// nh_kernels.hpp -- host-side launchers of the libnhmamba kernels (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nh {

// Profiling hook: start/stop events for the next kernel launch of this thread.  When set, the
// start event is recorded on the stream just before the launch (it completes once the
// preceding work has finished) and the launch goes through hipExtLaunchKernelGGL with the
// stop event, which is stamped at the kernel's own end; the slot is then cleared.
struct ProfEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents &prof_next();

template <typename... P, typename... Args>
inline void launch_k(void (*k)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args)
{
    ProfEvents &p = prof_next();
    if (p.start) {
        // a failure here is the runtime's last error, which every launcher returns after launching
        (void)hipEventRecord(p.start, st);
        hipExtLaunchKernelGGL(k, grid, block, lds, st, nullptr, p.stop, 0, static_cast<P>(args)...);
        p = ProfEvents{};
    } else {
        hipLaunchKernelGGL(k, grid, block, lds, st, static_cast<P>(args)...);
    }
}

enum DT { BF16 = 0, F32 = 1 };

struct W4 {
    const uint32_t *q;
    const uint16_t *s;
    const uint16_t *b;
    int n, k;
};

// ---- step mode (step.hip)
// Device address and size of this device's allocation-free scratch array (looked up once per
// device with hipGetSymbolAddress; the current device is the caller's).
hipError_t noalloc_scratch(void **ptr, size_t *bytes);
// y = W x (+ res): x [batch][W.k] bf16 or fp32 (x_t; fp32 values are rounded to bf16).
hipError_t launch_gemv(const W4 &W, const void *x, int x_t, int batch, const void *res, int res_t,
                       void *y, int y_t, hipStream_t st);
// Fused: RMSNorm(x) -> in_proj GEMV -> split; xBC rows go through the conv step (state
// updated in place), z and dt_raw rows are stored.  Also zeroes `nzero` words at zero_ptr.
hipError_t launch_inproj_step(const W4 &W, const void *x, int x_t, const uint16_t *norm_w,
                              float eps, int batch, uint16_t *z, uint16_t *xc, uint16_t *dtr,
                              uint16_t *conv_state, const uint16_t *conv_w,
                              const uint16_t *conv_b, uint32_t *zero_ptr, int nzero,
                              hipStream_t st);
// Pre-norm + MLP up projection (k = HIDDEN) + squared ReLU into h (bf16 [batch][W.n]).
hipError_t launch_mlp_up_step(const W4 &W, const void *x, int x_t, const uint16_t *norm_w, float eps, int batch,
                              uint16_t *h, hipStream_t st);
// The language model's input row: E[text_id] + audio + wf E[function_id] (fp32 out).
hipError_t launch_fused_embed(const W4 &E, const int *text_ids, const int *function_ids, const void *audio,
                              int audio_t, float wf, int batch, float *out, hipStream_t st);
// Final norm + one W4 head (k = HIDDEN) + greedy id per batch row; logits optional.  Two
// kernels; ws holds head_ws_bytes(batch) bytes of per-work-group partial results.
size_t head_ws_bytes(int batch);
hipError_t launch_head(const W4 &W, const void *x, int x_t, const uint16_t *norm_w, float eps, int batch,
                       float *logits, int *ids, void *ws, hipStream_t st);
hipError_t launch_ssm_step(const uint16_t *xc, const uint16_t *dtr, long ld_dt,
                           const float *dt_bias, const float *A_log, const float *D, float *S,
                           void *y, int y_t, int batch, hipStream_t st);
// SSM step that stores g w, the gate product g = bf16(y) * silu(z) times the gated-norm
// weight (fp32, [batch][d_inner]), and, per (sequence, head, half head), the sum of squares of
// g for the gated RMSNorm.
hipError_t launch_ssm_step_part(const uint16_t *xc, const uint16_t *dtr, long ld_dt,
                                const float *dt_bias, const float *A_log, const float *D,
                                float *S, float *gate, const uint16_t *z, const uint16_t *gw, float *part, int batch,
                                hipStream_t st);
// Gated RMSNorm (from g w and the SSM step's partial sums of g) fused into out_proj + residual.
// Above batch 1 it runs split over the gated-norm groups: partial receives the groups' sums
// (outproj_partial_floats(batch) floats; unused at batch 1).
size_t outproj_partial_floats(int batch);
hipError_t launch_outproj_step(const W4 &W, const float *gate, const float *part,
                               float eps, int batch, const void *res, int res_t, void *out, int out_t,
                               float *partial, hipStream_t st);
hipError_t launch_conv_step(const uint16_t *xbc, long ld, uint16_t *state, const uint16_t *w,
                            const uint16_t *b, uint16_t *out, int batch, int channels,
                            hipStream_t st);

// ---- attention layers (gemv.hip, attn.hip)
// Pre-norm + q/k/v projections: q into q ([batch][5120] bf16), k and v appended to the
// caches ([batch][8][max_len][128] bf16) at pos[b] (device int32 [batch]).
hipError_t launch_attn_qkv(const W4 &Wq, const W4 &Wk, const W4 &Wv, const void *x, int x_t, const uint16_t *norm_w,
                           float eps, int batch, uint16_t *q, uint16_t *kc, uint16_t *vc, const int *pos, int max_len,
                           hipStream_t st);
// Attention of each sequence's new position over its cache positions 0 .. pos[b] (the new k, v
// already appended): o ([batch][5120] bf16); part holds attn_part_bytes(batch) bytes.
size_t attn_part_bytes(int batch);
hipError_t launch_attn_decode(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, const int *pos, int max_len,
                              int batch, float *part, uint16_t *o, hipStream_t st);

// ---- row kernels (rows.hip)
// u = bf16(RMSNorm(x) * w); out_kind 0: bf16 bits, 1: fp16 bits of the same value (the
// matrix-core operand format); su (nullable): per-64-group sums of u, [d/64][rows].
hipError_t launch_rmsnorm(const void *x, int x_t, const uint16_t *w, uint16_t *u, int out_kind,
                          float *su, int rows, int d, float eps, hipStream_t st);
hipError_t launch_rmsnorm_gated(const void *y, int y_t, const uint16_t *z, long ld_z,
                                const uint16_t *w, uint16_t *out, int out_kind, float *su,
                                int rows, int d, int group, float eps, hipStream_t st);
hipError_t launch_conv_seq(const uint16_t *xbc, long ld, int T, const uint16_t *state_in,
                           uint16_t *state_out, const uint16_t *w, const uint16_t *b,
                           uint16_t *out, int batch, int channels, hipStream_t st);
// bf16 [M][K] -> fp16 bits [M][K] plus per-64-group sums [K/64][M].
hipError_t launch_to_f16(const uint16_t *x, uint16_t *xh, float *su, int M, int K,
                         hipStream_t st);

// ---- seq mode (gemm.hip, scan.hip)
// Y = Xh W^T (+ res); Xh holds fp16 bits, su the per-group row sums of Xh as [K/64][M].
hipError_t launch_w4_gemm(const W4 &W, const uint16_t *Xh, const float *su, int M,
                          const void *res, int res_t, void *Y, int y_t, hipStream_t st);
// Workspace of the scan: the fp16 C.B^T tiles of every (sequence, chunk, group).
size_t ssd_scan_ws_bytes(int batch, int T, int Q);
hipError_t launch_ssd_scan(const uint16_t *xc, const uint16_t *dtr, long ld_dt, int T, int Q,
                           const float *dt_bias, const float *A_log, const float *D,
                           const float *h0, float *hT, void *y, int y_t, int batch, uint16_t *Gws,
                           hipStream_t st);

}  // namespace nh
