// step.hip -- per-position (decode) kernels of the Mamba2 mixer block on gfx950.
//
// The per-position block is bound by HBM: the two W4 projections stream 82.9 MB of packed
// weights and the SSM step streams the 5.2 MB fp32 state twice, while the arithmetic is a few
// hundred MFLOP.  The kernels therefore aim at coalesced 128-bit loads of every weight byte
// exactly once, with the dequantisation folded into a packed bf16 dot product and all other
// work (pre-norm, conv, discretisation, gated norm, residual) fused into the streaming kernels.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

// ============================================================================ W4 GEMV
//
// Lane-over-K mapping: each wave owns whole output rows.  A row of k nibbles is k/32 chunks
// of 16 bytes (32 nibbles, half a quantisation group); lane l handles chunks l, l+64, ...
// (CPL of them), so one wave-wide 128-bit load reads 1 KB of contiguous weights and the
// lane's activations are the same for every row: they live in registers for the whole
// kernel.  A packed word of 8 nibbles turns into four bf16 pairs (128 + q_e, 128 + q_{e+4})
// with one and-or each (0x4300 is bf16 128.0, whose unit in the last place is 1), and a
// v_dot2_f32_bf16 multiplies such a pair with the matching activation pair.  Per chunk
//     sum_k W x = s * (dot - 128 * sum_k x) + beta * sum_k x
// with dot = sum_k (128 + q_k) x_k, which is the affine dequantisation W = s q + beta.

template <int CPL, int NB>
struct XFrag {
    uint32_t pr[NB][CPL][16];  // activation pairs (k, k+4) in nibble-extraction order
    float cs[NB][CPL];         // chunk sums of the activations
};

// 8 consecutive bf16 (four u32 words) -> pairs (0,4) (1,5) (2,6) (3,7).
__device__ __forceinline__ void pair_order(uint4 v, uint32_t *o)
{
    o[0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
}

template <int CPL, int NB>
__device__ __forceinline__ void load_x_plain(XFrag<CPL, NB> &f, const uint16_t *__restrict__ x,
                                             int k, int lane)
{
    const int nch = k >> 5;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < nch) {
                const uint4 *p = reinterpret_cast<const uint4 *>(x + (size_t)b * k + 32 * c);
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint4 v = p[j];
                    s += sum_bf16x8(v);
                    pair_order(v, &f.pr[b][i][4 * j]);
                }
                f.cs[b][i] = s;
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) f.pr[b][i][j] = 0u;
                f.cs[b][i] = 0.f;
            }
        }
}

// Eight input values of row b starting at element e (bf16 or f32 input).
template <int XT>
__device__ __forceinline__ void load8(const void *x, size_t e, float *v)
{
    if (XT == BF16) {
        uint4 w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + e);
        v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
        v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + e);
        float4 a = p[0], c = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    }
}

// Pre-norm prologue: u = bf16(x / rms(x) * w) for the lane's chunks.  The wave covers all
// chunks of the row, so the RMS is a wave reduction (no LDS, no barrier).
template <int CPL, int NB, int XT>
__device__ __forceinline__ void load_x_prenorm(XFrag<CPL, NB> &f, const void *__restrict__ x,
                                               const uint16_t *__restrict__ nw, float eps,
                                               int k, int lane)
{
    const int nch = k >> 5;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < nch)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[8];
                    load8<XT>(x, (size_t)b * k + 32 * c + 8 * j, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
                }
        }
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)k + eps);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            float s = 0.f;
            if (c < nch) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[8];
                    load8<XT>(x, (size_t)b * k + 32 * c + 8 * j, v);
                    uint4 wv = *reinterpret_cast<const uint4 *>(nw + 32 * c + 8 * j);
                    float w8[8] = {bf16lo(wv.x), bf16hi(wv.x), bf16lo(wv.y), bf16hi(wv.y),
                                   bf16lo(wv.z), bf16hi(wv.z), bf16lo(wv.w), bf16hi(wv.w)};
                    uint16_t u[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        u[e] = f32_to_bf16(v[e] * r * w8[e]);
                        s += bf16_to_f32(u[e]);
                    }
                    uint32_t *o = &f.pr[b][i][4 * j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (uint32_t)u[e] | ((uint32_t)u[e + 4] << 16);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) f.pr[b][i][j] = 0u;
            }
            f.cs[b][i] = s;
        }
    }
}

__device__ __forceinline__ float dot_chunk(uint4 w, const uint32_t *a, float acc)
{
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t q = ((ww[j] >> (4 * e)) & 0x000F000Fu) | 0x43004300u;
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q),
                                                  __builtin_bit_cast(bf16x2, a[4 * j + e]), acc,
                                                  false);
        }
    }
    return acc;
}

constexpr int GEMV_ROWS = 4;  // rows per wave per iteration (loads in flight before compute)

template <int CPL, int NB, class Epi>
__device__ __forceinline__ void gemv_rows(const W4 &W, const XFrag<CPL, NB> &f, const Epi &epi,
                                          int lane, int gwave, int nwaves)
{
    const int nch = W.k >> 5, kw = W.k >> 3, kg = W.k >> 6;
    for (int n0 = gwave * GEMV_ROWS; n0 < W.n; n0 += nwaves * GEMV_ROWS) {
        uint4 wq[GEMV_ROWS][CPL];
        float sc[GEMV_ROWS][CPL], bi[GEMV_ROWS][CPL];
#pragma unroll
        for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int n = n0 + r, c = lane + 64 * i;
                if (n < W.n && c < nch) {
                    wq[r][i] = ld_nt(reinterpret_cast<const uint4 *>(W.q + (size_t)n * kw) + c);
                    sc[r][i] = bf16_to_f32(W.s[(size_t)n * kg + (c >> 1)]);
                    bi[r][i] = bf16_to_f32(W.b[(size_t)n * kg + (c >> 1)]);
                } else {
                    wq[r][i] = make_uint4(0u, 0u, 0u, 0u);
                    sc[r][i] = 0.f;
                    bi[r][i] = 0.f;
                }
            }
        float acc[GEMV_ROWS][NB];
#pragma unroll
        for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const float d = dot_chunk(wq[r][i], f.pr[b][i], 0.f);
                    const float t = fmaf(-128.f, f.cs[b][i], d);
                    a = fmaf(sc[r][i], t, fmaf(bi[r][i], f.cs[b][i], a));
                }
                acc[r][b] = wave_sum(a);
            }
        if (lane == 0)
#pragma unroll
            for (int r = 0; r < GEMV_ROWS; ++r)
                if (n0 + r < W.n)
#pragma unroll
                    for (int b = 0; b < NB; ++b) epi(n0 + r, b, acc[r][b]);
    }
}

// y[b][n] = acc + res[b][n]
struct EpiStore {
    void *y;
    const void *res;
    int y_t, res_t, n;
    __device__ __forceinline__ void operator()(int row, int b, float v) const
    {
        const size_t i = (size_t)b * n + row;
        if (res) v += res_t == BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(res)[i])
                                    : reinterpret_cast<const float *>(res)[i];
        if (y_t == BF16)
            reinterpret_cast<uint16_t *>(y)[i] = f32_to_bf16(v);
        else
            reinterpret_cast<float *>(y)[i] = v;
    }
};

// in_proj rows of the per-position block: z | xBC | dt_raw.  The in_proj output is a bf16
// storage point; xBC channels immediately run the causal conv step (state row 0 oldest,
// tap 3 newest) and SiLU, and the conv state shifts by one position.
struct EpiInProjStep {
    uint16_t *z, *xc, *dtr, *cs;
    const uint16_t *cw, *cb;
    __device__ __forceinline__ void operator()(int n, int b, float acc) const
    {
        const uint16_t vb = f32_to_bf16(acc);
        if (n < DINNER) {
            z[(size_t)b * DINNER + n] = vb;
        } else if (n < DINNER + CONVDIM) {
            const int c = n - DINNER;
            uint16_t *st = cs + (size_t)b * (CONVK - 1) * CONVDIM + c;
            const uint16_t s0 = st[0], s1 = st[CONVDIM], s2 = st[2 * CONVDIM];
            const uint2 w = *reinterpret_cast<const uint2 *>(cw + 4 * (size_t)c);
            float a = bf16_to_f32(cb[c]);
            a = fmaf(bf16lo(w.x), bf16_to_f32(s0), a);
            a = fmaf(bf16hi(w.x), bf16_to_f32(s1), a);
            a = fmaf(bf16lo(w.y), bf16_to_f32(s2), a);
            a = fmaf(bf16hi(w.y), bf16_to_f32(vb), a);
            xc[(size_t)b * CONVDIM + c] = f32_to_bf16(silu(a));
            st[0] = s1;
            st[CONVDIM] = s2;
            st[2 * CONVDIM] = vb;
        } else {
            dtr[(size_t)b * NHEADS + (n - DINNER - CONVDIM)] = vb;
        }
    }
};

template <int CPL, int NB>
__global__ __launch_bounds__(256) void k_gemv(W4 W, const uint16_t *__restrict__ x, EpiStore epi)
{
    const int lane = threadIdx.x & 63;
    XFrag<CPL, NB> f;
    load_x_plain<CPL, NB>(f, x, W.k, lane);
    gemv_rows<CPL, NB>(W, f, epi, lane, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
}

template <int NB, int XT>
__global__ __launch_bounds__(256) void k_inproj_step(W4 W, const void *__restrict__ x,
                                                     const uint16_t *__restrict__ nw, float eps,
                                                     EpiInProjStep epi, uint32_t *zero_ptr,
                                                     int nzero)
{
    constexpr int CPL = (HIDDEN / 32 + 63) / 64;  // 3
    if (blockIdx.x == 0 && (int)threadIdx.x < nzero) zero_ptr[threadIdx.x] = 0u;
    const int lane = threadIdx.x & 63;
    XFrag<CPL, NB> f;
    load_x_prenorm<CPL, NB, XT>(f, x, nw, eps, W.k, lane);
    gemv_rows<CPL, NB>(W, f, epi, lane, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
}

static int gemv_grid(int n)
{
    const int groups = (n + GEMV_ROWS - 1) / GEMV_ROWS;  // one per wave
    int g = (groups + 3) / 4;
    return g < 1024 ? g : 1024;
}

template <int CPL>
static hipError_t gemv_cpl(const W4 &W, const uint16_t *x, int batch, EpiStore e, hipStream_t st)
{
    dim3 grid(gemv_grid(W.n)), block(256);
    switch (batch) {
    case 1: k_gemv<CPL, 1><<<grid, block, 0, st>>>(W, x, e); break;
    case 2: k_gemv<CPL, 2><<<grid, block, 0, st>>>(W, x, e); break;
    case 3: k_gemv<CPL, 3><<<grid, block, 0, st>>>(W, x, e); break;
    default: k_gemv<CPL, 4><<<grid, block, 0, st>>>(W, x, e); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv(const W4 &W, const uint16_t *x, int batch, const void *res, int res_t,
                       void *y, int y_t, hipStream_t st)
{
    EpiStore e{y, res, y_t, res_t, W.n};
    const int cpl = ((W.k >> 5) + 63) / 64;
    switch (cpl) {
    case 1: return gemv_cpl<1>(W, x, batch, e, st);
    case 2: return gemv_cpl<2>(W, x, batch, e, st);
    case 3: return gemv_cpl<3>(W, x, batch, e, st);
    case 4: return gemv_cpl<4>(W, x, batch, e, st);
    case 5: return gemv_cpl<5>(W, x, batch, e, st);
    case 6: return gemv_cpl<6>(W, x, batch, e, st);
    case 7: return gemv_cpl<7>(W, x, batch, e, st);
    default: return gemv_cpl<8>(W, x, batch, e, st);
    }
}

hipError_t launch_inproj_step(const W4 &W, const void *x, int x_t, const uint16_t *norm_w,
                              float eps, int batch, uint16_t *z, uint16_t *xc, uint16_t *dtr,
                              uint16_t *conv_state, const uint16_t *conv_w,
                              const uint16_t *conv_b, uint32_t *zero_ptr, int nzero,
                              hipStream_t st)
{
    EpiInProjStep e{z, xc, dtr, conv_state, conv_w, conv_b};
    dim3 grid(gemv_grid(W.n)), block(256);
#define NH_LAUNCH(NB)                                                                          \
    if (x_t == BF16)                                                                           \
        k_inproj_step<NB, BF16><<<grid, block, 0, st>>>(W, x, norm_w, eps, e, zero_ptr, nzero); \
    else                                                                                       \
        k_inproj_step<NB, F32><<<grid, block, 0, st>>>(W, x, norm_w, eps, e, zero_ptr, nzero);
    switch (batch) {
    case 1: NH_LAUNCH(1); break;
    case 2: NH_LAUNCH(2); break;
    case 3: NH_LAUNCH(3); break;
    default: NH_LAUNCH(4); break;
    }
#undef NH_LAUNCH
    return hipGetLastError();
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
                                                  const uint16_t *__restrict__ gw, float eps,
                                                  float *part, uint32_t *cnt,
                                                  uint16_t *__restrict__ o)
{
    const int half = blockIdx.x & 1;
    const int h = (blockIdx.x >> 1) % NHEADS;
    const int b = (blockIdx.x >> 1) / NHEADS;
    const int g = h / HPG;
    const int nl = threadIdx.x & 31, slot = threadIdx.x >> 5;

    const float dt = softplus(bf16_to_f32(dtr[(size_t)b * ld_dt + h]) + dt_bias[h]);
    const float A = -expf(A_log[h]);
    const float dA = expf(dt * A);
    const float Dh = Dp[h];

    const uint16_t *xb = xc + (size_t)b * CONVDIM;
    const uint2 bw = *reinterpret_cast<const uint2 *>(xb + OFF_B + g * DSTATE + 4 * nl);
    const uint2 cw = *reinterpret_cast<const uint2 *>(xb + OFF_C + g * DSTATE + 4 * nl);
    const float B0 = bf16lo(bw.x), B1 = bf16hi(bw.x), B2 = bf16lo(bw.y), B3 = bf16hi(bw.y);
    const float C0 = bf16lo(cw.x), C1 = bf16hi(cw.x), C2 = bf16lo(cw.y), C3 = bf16hi(cw.y);

    float4 *Sh = reinterpret_cast<float4 *>(S + ((size_t)b * NHEADS + h) * HDIM * DSTATE);
    float4 s[SSM_IT];
    float xp[SSM_IT];
#pragma unroll
    for (int it = 0; it < SSM_IT; ++it) {
        const int p = half * SSM_ROWS + slot + 8 * it;
        s[it] = ld_nt(Sh + p * (DSTATE / 4) + nl);
        xp[it] = bf16_to_f32(xb[h * HDIM + p]);
    }
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

    // ---- gated RMSNorm fused through a last-work-group-per-group hand-off.
    __shared__ uint16_t ys[SSM_ROWS];
    __shared__ float red[8];
    __shared__ int last;
    float ss = 0.f;
    if (nl == 0)
#pragma unroll
        for (int it = 0; it < SSM_IT; ++it) {
            const int pl = slot + 8 * it;
            const uint16_t yb = f32_to_bf16(yv[it]);
            ys[pl] = yb;
            const float gm = bf16_to_f32(yb) *
                             silu(bf16_to_f32(z[(size_t)b * DINNER + h * HDIM + half * SSM_ROWS + pl]));
            ss += gm * gm;
        }
    if (nl == 0) red[slot] = ss;
    __syncthreads();
    // y of this work-group: 40 bf16 = 20 words, published with device-scope atomic stores.
    uint32_t *yw = reinterpret_cast<uint32_t *>(y) + ((size_t)b * DINNER + h * HDIM + half * SSM_ROWS) / 2;
    if (threadIdx.x < SSM_ROWS / 2)
        __hip_atomic_store(yw + threadIdx.x,
                           (uint32_t)ys[2 * threadIdx.x] | ((uint32_t)ys[2 * threadIdx.x + 1] << 16),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) t += red[i];
        __hip_atomic_store(part + ((size_t)b * NHEADS + h) * 2 + half, t, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(cnt + b * NGROUPS + g, 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last = (old == 2 * HPG - 1);
    }
    __syncthreads();
    if (!last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    float tot = 0.f;
    const float *pg = part + ((size_t)b * NHEADS + g * HPG) * 2;
    for (int i = 0; i < 2 * HPG; ++i)
        tot += __hip_atomic_load(pg + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float r = 1.0f / sqrtf(tot / (float)GNORM + eps);
    const uint32_t *ygw = reinterpret_cast<const uint32_t *>(y) + ((size_t)b * DINNER + g * GNORM) / 2;
    for (int i = threadIdx.x; i < GNORM / 2; i += 256) {
        const uint32_t w2 = __hip_atomic_load(ygw + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const size_t ch = (size_t)g * GNORM + 2 * i;
        const uint32_t zz = *reinterpret_cast<const uint32_t *>(z + (size_t)b * DINNER + ch);
        const uint32_t ww = *reinterpret_cast<const uint32_t *>(gw + ch);
        const float g0 = bf16lo(w2) * silu(bf16lo(zz)), g1 = bf16hi(w2) * silu(bf16hi(zz));
        const uint32_t ov = (uint32_t)f32_to_bf16(g0 * r * bf16lo(ww)) |
                            ((uint32_t)f32_to_bf16(g1 * r * bf16hi(ww)) << 16);
        *reinterpret_cast<uint32_t *>(o + (size_t)b * DINNER + ch) = ov;
    }
}

hipError_t launch_ssm_step(const uint16_t *xc, const uint16_t *dtr, long ld_dt,
                           const float *dt_bias, const float *A_log, const float *D, float *S,
                           void *y, int y_t, int batch, hipStream_t st)
{
    dim3 grid(batch * NHEADS * 2), block(256);
    if (y_t == BF16)
        k_ssm_step<false, BF16><<<grid, block, 0, st>>>(xc, dtr, ld_dt, dt_bias, A_log, D, S, y,
                                                        nullptr, nullptr, 0.f, nullptr, nullptr,
                                                        nullptr);
    else
        k_ssm_step<false, F32><<<grid, block, 0, st>>>(xc, dtr, ld_dt, dt_bias, A_log, D, S, y,
                                                       nullptr, nullptr, 0.f, nullptr, nullptr,
                                                       nullptr);
    return hipGetLastError();
}

hipError_t launch_ssm_step_gnorm(const uint16_t *xc, const uint16_t *dtr, long ld_dt,
                                 const float *dt_bias, const float *A_log, const float *D,
                                 float *S, uint16_t *y_ws, const uint16_t *z, const uint16_t *gw,
                                 float eps, float *part, uint32_t *cnt, uint16_t *o, int batch,
                                 hipStream_t st)
{
    dim3 grid(batch * NHEADS * 2), block(256);
    k_ssm_step<true, BF16><<<grid, block, 0, st>>>(xc, dtr, ld_dt, dt_bias, A_log, D, S, y_ws, z,
                                                   gw, eps, part, cnt, o);
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

}  // namespace nh
