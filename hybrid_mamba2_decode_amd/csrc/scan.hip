// scan.hip -- chunked SSD scan of the Mamba2 selective SSM on gfx950 matrix cores.
//
// The recurrence  S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t,  y_t = C_t . S_t + D x_t
// is evaluated chunk by chunk (state-space duality, Dao & Gu 2024).  For a chunk of length L
// and cum_t = sum_{s<=t} dt_s A inside the chunk:
//   Y_off[i]  = exp(cum_i) C_i . S_in                                   (state -> output)
//   Y_diag[i] = sum_{j<=i} (C_i . B_j) exp(cum_i - cum_j) dt_j x_j       (intra-chunk)
//   S_out     = exp(cum_{L-1}) S_in + sum_j exp(cum_{L-1} - cum_j) dt_j x_j (outer) B_j
//   y         = Y_off + Y_diag + D x
//
// Work decomposition: one work-group (4 waves) per (sequence, head) walks the chunks in order,
// keeping the head's 80 x 128 fp32 state in registers as the accumulator of the state MFMA.
// Work-groups are numbered so that the 16 heads sharing a B/C group land on the same XCD
// (work-group i runs on XCD i mod 8) and read B and C through one L2.  Per chunk:
//   1. dt = softplus(dt_raw + dt_bias), the log2-scaled cumulative sum of dt*A (block scan);
//   2. B (L x 128) and x (as x^T, 80 x L) staged in LDS as fp16, S_in as fp16;
//   3. each wave takes 16-row blocks {w, 7-w, 8+w, 15-w} (balanced causal work): C rows are
//      loaded once into registers and serve both as the A operand of C S_in^T and as the B
//      operand of B C^T, whose D layout is exactly the A-operand layout that
//      (G o decay) X needs, so the intra-chunk product never leaves registers;
//   4. each wave updates its two 16-column slices of the state.
// Operands are fp16 (B, C, x are bf16-exact; the scaled operands round once, relative error
// 2^-11); all accumulation is fp32.  Chunks shorter than 16/32 rows are zero-padded in LDS.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

constexpr int BS_LD = DSTATE + 8;  // Bs row (fp16): 272 B
constexpr int XT_LD = QMAX + 8;    // Xt row (fp16): 528 B
constexpr int SI_LD = DSTATE + 8;  // Si row (fp16): 272 B

struct ScanSmem {
    uint16_t Bs[QMAX * BS_LD];  // B of the chunk, [j][n]
    uint16_t Xt[HDIM * XT_LD];  // x of the chunk transposed, [p][j]
    uint16_t Si[HDIM * SI_LD];  // state at chunk start, [p][n]
    float cum[QMAX];            // log2-scaled cumulative dt*A
    float dtv[QMAX];            // dt
    float wsum[4];
};

__device__ __forceinline__ half8 ld_half8(const uint16_t *p)
{
    return __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ uint32_t pack_rne(float a, float b)
{
    half2v v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

template <int YT>
__global__ __launch_bounds__(256) void k_ssd_scan(const uint16_t *__restrict__ xc,
                                                  const uint16_t *__restrict__ dtr, long ld_dt,
                                                  int T, int Q, const float *__restrict__ dt_bias,
                                                  const float *__restrict__ A_log,
                                                  const float *__restrict__ Dp,
                                                  const float *h0, float *hT,
                                                  void *__restrict__ y)
{
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    ScanSmem &sm = *reinterpret_cast<ScanSmem *>(smem_raw);

    const int g = blockIdx.x % NGROUPS;
    const int rr = blockIdx.x / NGROUPS;
    const int h = g * HPG + rr % HPG;
    const int b = rr / HPG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;

    const float LOG2E = 1.4426950408889634f;
    const float A2 = -expf(A_log[h]) * LOG2E;  // dt*A in log2 units
    const float dtb = dt_bias[h];
    const float Dh = Dp[h];

    const uint16_t *xcb = xc + (size_t)b * T * CONVDIM;
    const uint16_t *dtb_ptr = dtr + (size_t)b * T * ld_dt + h;

    // State registers: st[pb][nb] holds S[16pb + 4q4 + r][16(2 wave + nb) + l16], r = 0..3.
    floatx4 st[5][2];
    float *Sg = hT ? hT + ((size_t)b * NHEADS + h) * HDIM * DSTATE : nullptr;
    const float *S0 = h0 ? h0 + ((size_t)b * NHEADS + h) * HDIM * DSTATE : nullptr;
#pragma unroll
    for (int pb = 0; pb < 5; ++pb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = 16 * pb + 4 * q4 + r, n = 16 * (2 * wave + nb) + l16;
                st[pb][nb][r] = S0 ? S0[p * DSTATE + n] : 0.f;
            }

    for (int t0 = 0; t0 < T; t0 += Q) {
        const int L = min(Q, T - t0);
        const int LR = (L + 31) & ~31;

        // ---- 1. discretisation and cumulative sum (inclusive, 256-wide block scan)
        float dtt = 0.f, a = 0.f;
        if (tid < L) {
            dtt = softplus(bf16_to_f32(dtb_ptr[(size_t)(t0 + tid) * ld_dt]) + dtb);
            a = dtt * A2;
        }
        float v = a;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float nbv = __shfl_up(v, o, 64);
            if (lane >= o) v += nbv;
        }
        if (lane == 63) sm.wsum[wave] = v;
        __syncthreads();
        for (int w = 0; w < wave; ++w) v += sm.wsum[w];
        sm.cum[tid] = v;
        sm.dtv[tid] = dtt;

        // ---- 2. stage B [j][n], x^T [p][j] and S_in [p][n] as fp16
        for (int vi = tid; vi < LR * (DSTATE / 8); vi += 256) {
            const int j = vi >> 4, nv = vi & 15;
            uint4 o = make_uint4(0u, 0u, 0u, 0u);
            if (j < L) {
                const uint4 w = *reinterpret_cast<const uint4 *>(
                    xcb + (size_t)(t0 + j) * CONVDIM + OFF_B + g * DSTATE + 8 * nv);
                o.x = bf16x2_to_f16x2(w.x);
                o.y = bf16x2_to_f16x2(w.y);
                o.z = bf16x2_to_f16x2(w.z);
                o.w = bf16x2_to_f16x2(w.w);
            }
            *reinterpret_cast<uint4 *>(&sm.Bs[j * BS_LD + 8 * nv]) = o;
        }
        for (int vi = tid; vi < LR * (HDIM / 8); vi += 256) {
            const int j = vi / (HDIM / 8), pv = vi % (HDIM / 8);
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (j < L)
                w = *reinterpret_cast<const uint4 *>(xcb + (size_t)(t0 + j) * CONVDIM + h * HDIM + 8 * pv);
            const uint32_t wa[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t f = bf16x2_to_f16x2(wa[e]);
                sm.Xt[(8 * pv + 2 * e) * XT_LD + j] = (uint16_t)(f & 0xFFFFu);
                sm.Xt[(8 * pv + 2 * e + 1) * XT_LD + j] = (uint16_t)(f >> 16);
            }
        }
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = 16 * pb + 4 * q4 + r, n = 16 * (2 * wave + nb) + l16;
                    sm.Si[p * SI_LD + n] = __builtin_bit_cast(uint16_t, (_Float16)st[pb][nb][r]);
                }
        __syncthreads();

        // ---- 3. outputs, 16-row blocks per wave
        const int nblk = (L + 15) >> 4;
        const int blocks[4] = {wave, 7 - wave, 8 + wave, 15 - wave};
        for (int bi = 0; bi < 4; ++bi) {
            const int I = blocks[bi];
            if (I >= nblk) continue;
            const int ia = 16 * I + l16;  // row of this lane in A/B operand layouts
            half8 cf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint4 w = make_uint4(0u, 0u, 0u, 0u);
                if (ia < L)
                    w = *reinterpret_cast<const uint4 *>(xcb + (size_t)(t0 + ia) * CONVDIM + OFF_C +
                                                         g * DSTATE + 32 * ks + 8 * q4);
                uint4 f;
                f.x = bf16x2_to_f16x2(w.x);
                f.y = bf16x2_to_f16x2(w.y);
                f.z = bf16x2_to_f16x2(w.z);
                f.w = bf16x2_to_f16x2(w.w);
                cf[ks] = __builtin_bit_cast(half8, f);
            }
            // Y_off = C S_in^T, then rows scaled by exp(cum_i)
            floatx4 acc[5];
#pragma unroll
            for (int pb = 0; pb < 5; ++pb) {
                acc[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        cf[ks], ld_half8(&sm.Si[(16 * pb + l16) * SI_LD + 32 * ks + 8 * q4]), acc[pb], 0, 0, 0);
            }
            float ei[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ei[r] = __builtin_amdgcn_exp2f(sm.cum[16 * I + 4 * q4 + r]);
#pragma unroll
            for (int pb = 0; pb < 5; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pb][r] *= ei[r];

            // Y_diag: pairs of 16-column blocks (32 keys per MFMA)
            const float ci = sm.cum[ia];
            for (int jp = 0; 2 * jp <= I; ++jp) {
                float m[8];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int J = 2 * jp + hb;
                    if (J <= I) {
                        floatx4 gt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks)
                            gt = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                ld_half8(&sm.Bs[(16 * J + l16) * BS_LD + 32 * ks + 8 * q4]), cf[ks], gt, 0, 0, 0);
                        // gt[r] = G[i = ia][j = 16J + 4q4 + r]
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = 16 * J + 4 * q4 + r;
                            const bool ok = (j <= ia) && (j < L);
                            m[4 * hb + r] = ok ? gt[r] * __builtin_amdgcn_exp2f(ci - sm.cum[j]) * sm.dtv[j] : 0.f;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) m[4 * hb + r] = 0.f;
                    }
                }
                uint4 mp;
                mp.x = pack_rne(m[0], m[1]);
                mp.y = pack_rne(m[2], m[3]);
                mp.z = pack_rne(m[4], m[5]);
                mp.w = pack_rne(m[6], m[7]);
                const half8 mf = __builtin_bit_cast(half8, mp);
#pragma unroll
                for (int pb = 0; pb < 5; ++pb) {
                    const uint16_t *xr = &sm.Xt[(16 * pb + l16) * XT_LD + 32 * jp + 4 * q4];
                    const uint2 lo = *reinterpret_cast<const uint2 *>(xr);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(xr + 16);
                    const half8 xf = __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(mf, xf, acc[pb], 0, 0, 0);
                }
            }
            // y = Y_off + Y_diag + D x
#pragma unroll
            for (int pb = 0; pb < 5; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * q4 + r, p = 16 * pb + l16;
                    if (i < L) {
                        const float xv = f16_to_f32(sm.Xt[p * XT_LD + i]);
                        const float yv = fmaf(Dh, xv, acc[pb][r]);
                        const size_t o = ((size_t)b * T + t0 + i) * DINNER + h * HDIM + p;
                        if (YT == BF16)
                            reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16(yv);
                        else
                            reinterpret_cast<float *>(y)[o] = yv;
                    }
                }
        }

        // ---- 4. state update: S = exp(cum_last) S + (w x)^T B, w_j = exp(cum_last - cum_j) dt_j
        const float cl = sm.cum[L - 1];
        const float dec = __builtin_amdgcn_exp2f(cl);
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[pb][nb][r] *= dec;
        for (int ks = 0; ks < (LR >> 5); ++ks) {
            const int jb = 32 * ks + 8 * q4;
            float wj[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wj[e] = __builtin_amdgcn_exp2f(cl - sm.cum[jb + e]) * sm.dtv[jb + e];
            half8 bfr[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int n = 16 * (2 * wave + nb) + l16;
                uint16_t t8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) t8[e] = sm.Bs[(jb + e) * BS_LD + n];
                uint4 pk;
                pk.x = (uint32_t)t8[0] | ((uint32_t)t8[1] << 16);
                pk.y = (uint32_t)t8[2] | ((uint32_t)t8[3] << 16);
                pk.z = (uint32_t)t8[4] | ((uint32_t)t8[5] << 16);
                pk.w = (uint32_t)t8[6] | ((uint32_t)t8[7] << 16);
                bfr[nb] = __builtin_bit_cast(half8, pk);
            }
#pragma unroll
            for (int pb = 0; pb < 5; ++pb) {
                const uint4 xw = *reinterpret_cast<const uint4 *>(&sm.Xt[(16 * pb + l16) * XT_LD + jb]);
                const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w};
                uint4 ap;
                uint32_t *apw = &ap.x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const half2v hv = __builtin_bit_cast(half2v, xa[e]);
                    apw[e] = pack_rne((float)hv[0] * wj[2 * e], (float)hv[1] * wj[2 * e + 1]);
                }
                const half8 af = __builtin_bit_cast(half8, ap);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    st[pb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bfr[nb], st[pb][nb], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    if (Sg)
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = 16 * pb + 4 * q4 + r, n = 16 * (2 * wave + nb) + l16;
                    Sg[p * DSTATE + n] = st[pb][nb][r];
                }
}

hipError_t launch_ssd_scan(const uint16_t *xc, const uint16_t *dtr, long ld_dt, int T, int Q,
                           const float *dt_bias, const float *A_log, const float *D,
                           const float *h0, float *hT, void *y, int y_t, int batch,
                           hipStream_t st)
{
    const size_t smem = sizeof(ScanSmem);
    static bool attr_set[2] = {false, false};
    dim3 grid(batch * NHEADS), block(256);
    if (y_t == BF16) {
        if (!attr_set[0]) {
            hipError_t e = hipFuncSetAttribute((const void *)k_ssd_scan<BF16>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
            if (e != hipSuccess) return e;
            attr_set[0] = true;
        }
        k_ssd_scan<BF16><<<grid, block, smem, st>>>(xc, dtr, ld_dt, T, Q, dt_bias, A_log, D, h0, hT, y);
    } else {
        if (!attr_set[1]) {
            hipError_t e = hipFuncSetAttribute((const void *)k_ssd_scan<F32>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
            if (e != hipSuccess) return e;
            attr_set[1] = true;
        }
        k_ssd_scan<F32><<<grid, block, smem, st>>>(xc, dtr, ld_dt, T, Q, dt_bias, A_log, D, h0, hT, y);
    }
    return hipGetLastError();
}

}  // namespace nh
