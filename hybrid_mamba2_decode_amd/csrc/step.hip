// step.hip -- per-position (decode) kernels of the Mamba2 mixer block on gfx950.
//
// The per-position block is bound by HBM: the two W4 projections stream 82.9 MB of packed
// weights and the SSM step streams the 5.2 MB fp32 state twice, while the arithmetic is a few
// hundred MFLOP.  The kernels therefore aim at coalesced 128-bit loads of every weight byte
// exactly once, with the dequantisation folded into a packed bf16 dot product and all other
// work (pre-norm, conv, discretisation, gated norm, residual) fused into the streaming kernels.
#include <mutex>

#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

// ============================================================ allocation-free scratch
//
// The block step's workspace (z, xc, dt_raw, g w and the gated-norm partial sums) for callers
// that cannot allocate: one file-scope device array, which every GPU the library runs on holds
// until the process ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = 1u << 20;  // >= the batch-4 step workspace (about 0.9 MiB)
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void **ptr, size_t *bytes)
{
    constexpr int MAXDEV = 64;
    static std::mutex mu;
    static void *addr[MAXDEV] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

// ============================================================================ SSM step
//
// One work-group per (sequence, head, half of the head's 80 rows): 40 rows of 128 fp32 state
// values.  32 lanes cover a row with float4 accesses, so every state byte is read and written
// exactly once with 128-bit transactions; the readout C.S is a 32-lane reduction.
// S[p][:] = exp(dt A) S[p][:] + dt x[p] B[:],  y[p] = C . S[p][:] + D x[p].

constexpr int SSM_ROWS = HDIM / 2;        // rows per work-group
constexpr int SSM_IT = SSM_ROWS / 8;      // 8 rows per pass of 256 threads

template <bool GN, int YT>
__global__ __launch_bounds__(256) void k_ssm_step(const uint16_t *__restrict__ xc,
                                                  const uint16_t *__restrict__ dtr, long ld_dt,
                                                  const float *__restrict__ dt_bias,
                                                  const float *__restrict__ A_log,
                                                  const float *__restrict__ Dp,
                                                  float *__restrict__ S, void *__restrict__ y,
                                                  const uint16_t *__restrict__ z,
                                                  const uint16_t *__restrict__ gw,
                                                  float *__restrict__ part)
{
    const int half = blockIdx.x & 1;
    const int h = (blockIdx.x >> 1) % NHEADS;
    const int b = (blockIdx.x >> 1) / NHEADS;
    const int g = h / HPG;
    const int nl = threadIdx.x & 31, slot = threadIdx.x >> 5;

    // Every load is issued before any arithmetic: the small parameter loads first, then the
    // state rows.  A wave's loads complete in issue order, so the discretisation (which needs
    // dt) then waits only for the parameters while the 20 KB of state are still in flight.
    const uint16_t *xb = xc + (size_t)b * CONVDIM;
    const uint16_t dtb = dtr[(size_t)b * ld_dt + h];
    const uint2 bw = *reinterpret_cast<const uint2 *>(xb + OFF_B + g * DSTATE + 4 * nl);
    const uint2 cw = *reinterpret_cast<const uint2 *>(xb + OFF_C + g * DSTATE + 4 * nl);
    uint16_t xr[SSM_IT], zr[SSM_IT], wr[SSM_IT];
#pragma unroll
    for (int it = 0; it < SSM_IT; ++it) xr[it] = xb[h * HDIM + half * SSM_ROWS + slot + 8 * it];
    // the gate's z and the gated-norm weight, loaded with the rest (every lane of a row loads
    // the same value): the epilogue then makes no round trip to memory
    if constexpr (GN) {
#pragma unroll
        for (int it = 0; it < SSM_IT; ++it) {
            const int p = half * SSM_ROWS + slot + 8 * it;
            zr[it] = z[(size_t)b * DINNER + h * HDIM + p];
            wr[it] = gw[h * HDIM + p];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float4 *Sh = reinterpret_cast<float4 *>(S + ((size_t)b * NHEADS + h) * HDIM * DSTATE);
    float4 s[SSM_IT];
#pragma unroll
    for (int it = 0; it < SSM_IT; ++it) {
        const int p = half * SSM_ROWS + slot + 8 * it;
        s[it] = ld_nt(Sh + p * (DSTATE / 4) + nl);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float dt = softplus(bf16_to_f32(dtb) + dt_bias[h]);
    const float A = -expf(A_log[h]);
    const float dA = expf(dt * A);
    const float Dh = Dp[h];
    const float B0 = bf16lo(bw.x), B1 = bf16hi(bw.x), B2 = bf16lo(bw.y), B3 = bf16hi(bw.y);
    const float C0 = bf16lo(cw.x), C1 = bf16hi(cw.x), C2 = bf16lo(cw.y), C3 = bf16hi(cw.y);
    float xp[SSM_IT];
#pragma unroll
    for (int it = 0; it < SSM_IT; ++it) xp[it] = bf16_to_f32(xr[it]);
    float yv[SSM_IT];
#pragma unroll
    for (int it = 0; it < SSM_IT; ++it) {
        const int p = half * SSM_ROWS + slot + 8 * it;
        const float u = dt * xp[it];
        float4 v = s[it];
        v.x = fmaf(dA, v.x, u * B0);
        v.y = fmaf(dA, v.y, u * B1);
        v.z = fmaf(dA, v.z, u * B2);
        v.w = fmaf(dA, v.w, u * B3);
        st_nt(v, Sh + p * (DSTATE / 4) + nl);
        float part_c = (C0 * v.x + C1 * v.y) + (C2 * v.z + C3 * v.w);
        yv[it] = half_wave_sum(part_c) + Dh * xp[it];
    }

    if (!GN) {
        if (nl == 0)
#pragma unroll
            for (int it = 0; it < SSM_IT; ++it) {
                const int p = half * SSM_ROWS + slot + 8 * it;
                const size_t i = (size_t)b * DINNER + h * HDIM + p;
                if (YT == BF16)
                    reinterpret_cast<uint16_t *>(y)[i] = f32_to_bf16(yv[it]);
                else
                    reinterpret_cast<float *>(y)[i] = yv[it];
            }
        return;
    }

    // ---- the gate product g = bf16(y) * silu(z) (fp32; y is rounded to bf16 first, its
    // storage point) times the gated-norm weight, and this work-group's sum of squares of g,
    // both consumed by the gated RMSNorm in the out_proj kernel, which so needs neither y, z
    // nor the norm weight: o = bf16((g w) / rms(g)).
    __shared__ float red[8];
    float ss = 0.f;
    if (nl == 0)
#pragma unroll
        for (int it = 0; it < SSM_IT; ++it) {
            const int p = half * SSM_ROWS + slot + 8 * it;
            const size_t i = (size_t)b * DINNER + h * HDIM + p;
            const float gm = round_bf16(yv[it]) * silu(bf16_to_f32(zr[it]));
            reinterpret_cast<float *>(y)[i] = gm * bf16_to_f32(wr[it]);
            ss += gm * gm;
        }
    if (nl == 0) red[slot] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) t += red[i];
        part[((size_t)b * NHEADS + h) * 2 + half] = t;
    }
}

hipError_t launch_ssm_step(const uint16_t *xc, const uint16_t *dtr, long ld_dt,
                           const float *dt_bias, const float *A_log, const float *D, float *S,
                           void *y, int y_t, int batch, hipStream_t st)
{
    dim3 grid(batch * NHEADS * 2), block(256);
    if (y_t == BF16)
        k_ssm_step<false, BF16><<<grid, block, 0, st>>>(xc, dtr, ld_dt, dt_bias, A_log, D, S, y,
                                                        nullptr, nullptr, nullptr);
    else
        k_ssm_step<false, F32><<<grid, block, 0, st>>>(xc, dtr, ld_dt, dt_bias, A_log, D, S, y,
                                                       nullptr, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_ssm_step_part(const uint16_t *xc, const uint16_t *dtr, long ld_dt,
                                const float *dt_bias, const float *A_log, const float *D,
                                float *S, float *gate, const uint16_t *z, const uint16_t *gw, float *part,
                                int batch, hipStream_t st)
{
    dim3 grid(batch * NHEADS * 2), block(256);
    launch_k(k_ssm_step<true, F32>, grid, block, 0, st, xc, dtr, ld_dt, dt_bias, A_log, D, S, gate, z, gw, part);
    return hipGetLastError();
}

// ============================================================================ conv step

__global__ __launch_bounds__(256) void k_conv_step(const uint16_t *__restrict__ xbc, long ld,
                                                   uint16_t *__restrict__ state,
                                                   const uint16_t *__restrict__ w,
                                                   const uint16_t *__restrict__ bias,
                                                   uint16_t *__restrict__ out, int channels)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int b = blockIdx.y;
    if (c >= channels) return;
    uint16_t *st = state + (size_t)b * (CONVK - 1) * channels + c;
    const uint16_t s0 = st[0], s1 = st[channels], s2 = st[2 * (size_t)channels];
    const uint16_t v = xbc[(size_t)b * ld + c];
    const uint2 wv = *reinterpret_cast<const uint2 *>(w + 4 * (size_t)c);
    float a = bf16_to_f32(bias[c]);
    a = fmaf(bf16lo(wv.x), bf16_to_f32(s0), a);
    a = fmaf(bf16hi(wv.x), bf16_to_f32(s1), a);
    a = fmaf(bf16lo(wv.y), bf16_to_f32(s2), a);
    a = fmaf(bf16hi(wv.y), bf16_to_f32(v), a);
    out[(size_t)b * channels + c] = f32_to_bf16(silu(a));
    st[0] = s1;
    st[channels] = s2;
    st[2 * (size_t)channels] = v;
}

hipError_t launch_conv_step(const uint16_t *xbc, long ld, uint16_t *state, const uint16_t *w,
                            const uint16_t *b, uint16_t *out, int batch, int channels,
                            hipStream_t st)
{
    dim3 grid((channels + 255) / 256, batch), block(256);
    k_conv_step<<<grid, block, 0, st>>>(xbc, ld, state, w, b, out, channels);
    return hipGetLastError();
}

// ====================================================================== fused input row
//
// out[b] = E[text_ids[b]] + audio[b] + wf E[function_ids[b]], E the W4 embedding table.  One
// thread per packed word (8 values) of a row: the two rows' words, their group scales and
// biases, 8 audio values, and 32 bytes of fp32 output.  E rows are dequantised as
// fmaf(s, q, b) (s q is exact; one rounding), then (e_t + a) and fmaf(wf, e_f, .) in that
// order.  An id outside the table writes NaN and reads row 0 instead.
template <int AT>
__global__ __launch_bounds__(64) void k_fused_embed(W4 E, const int *__restrict__ tid,
                                                    const int *__restrict__ fid,
                                                    const void *__restrict__ audio, float wf,
                                                    float *__restrict__ out)
{
    const int b = blockIdx.y, nw = E.k >> 3;
    const int w = blockIdx.x * 64 + threadIdx.x;
    if (w >= nw) return;
    const int t = tid[b], f = fid[b];
    const bool ok = t >= 0 && t < E.n && f >= 0 && f < E.n;
    const size_t rt = ok ? (size_t)t : 0, rf = ok ? (size_t)f : 0;
    const int kg = E.k >> 6;
    const uint32_t qt = E.q[rt * nw + w], qf = E.q[rf * nw + w];
    const float st = bf16_to_f32(E.s[rt * kg + (w >> 3)]), bt = bf16_to_f32(E.b[rt * kg + (w >> 3)]);
    const float sf = bf16_to_f32(E.s[rf * kg + (w >> 3)]), bf = bf16_to_f32(E.b[rf * kg + (w >> 3)]);
    float a[8];
    if (AT == BF16) {
        const uint4 v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(audio) + (size_t)b * E.k + 8 * w);
        a[0] = bf16lo(v.x); a[1] = bf16hi(v.x); a[2] = bf16lo(v.y); a[3] = bf16hi(v.y);
        a[4] = bf16lo(v.z); a[5] = bf16hi(v.z); a[6] = bf16lo(v.w); a[7] = bf16hi(v.w);
    } else {
        const float4 *src = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(audio) + (size_t)b * E.k + 8 * w);
        const float4 v0 = src[0], v1 = src[1];
        a[0] = v0.x; a[1] = v0.y; a[2] = v0.z; a[3] = v0.w;
        a[4] = v1.x; a[5] = v1.y; a[6] = v1.z; a[7] = v1.w;
    }
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float et = fmaf(st, (float)((qt >> (4 * j)) & 15u), bt);
        const float ef = fmaf(sf, (float)((qf >> (4 * j)) & 15u), bf);
        o[j] = ok ? fmaf(wf, ef, et + a[j]) : __builtin_nanf("");
    }
    float4 *dst = reinterpret_cast<float4 *>(out + (size_t)b * E.k + 8 * w);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_fused_embed(const W4 &E, const int *text_ids, const int *function_ids, const void *audio,
                              int audio_t, float wf, int batch, float *out, hipStream_t st)
{
    dim3 grid(((E.k >> 3) + 63) / 64, batch), block(64);
    if (audio_t == BF16)
        k_fused_embed<BF16><<<grid, block, 0, st>>>(E, text_ids, function_ids, audio, wf, out);
    else
        k_fused_embed<F32><<<grid, block, 0, st>>>(E, text_ids, function_ids, audio, wf, out);
    return hipGetLastError();
}

}  // namespace nh
