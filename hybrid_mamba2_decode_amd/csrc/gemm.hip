// gemm.hip -- W4 matrix product Y = X W^T (+ residual) on gfx950 matrix cores.
//
// Dequantisation is exact: with bf16 scales s, the value s*(q-8) has at most 11 significant
// bits (|q-8| <= 8 and s carries 8 bits), so it is an fp16 number.  The B operand is built as
// fp16 s*(q-8) straight from the packed word: (word & 0x000F000F) | 0x64006400 gives the fp16
// pair (1024+q_e, 1024+q_{e+4}) (1024's unit in the last place is 1), a packed subtract of 1032
// and a packed multiply by s finish it.  The rest of the affine map,
//     W = s*(q-8) + (beta + 8 s),
// is zero for symmetric groups (beta = -8 s); otherwise its contribution
// (beta + 8s) * sum_{k in group} X[m][k] is added in fp32 from precomputed group sums.
// Activations arrive as fp16 bits (bf16-exact values), so every product is exact and the
// accumulation is fp32 inside v_mfma_f32_32x32x16_f16.
//
// Tiling: 128 x 128 output tile per work-group of 4 waves (2 x 2), each wave 64 x 64 as
// 2 x 2 MFMA 32x32 tiles, K advanced two 64-wide quantisation groups per pipeline step.  The X
// tile is staged through LDS (double-buffered, padded rows); each wave reads its W rows straight
// from global memory into registers, one step ahead.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GKS = 2;                  // quantisation groups per pipeline step
constexpr int GALD = GKS * GBK + 8;     // LDS row of the X tile, in fp16 elements (272 B)

// Eight fp16 values in pair order (0,4) (1,5) (2,6) (3,7), matching the nibble extraction.
__device__ __forceinline__ uint4 pair_order16(uint4 v)
{
    uint4 o;
    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    return o;
}

// One packed word of 8 nibbles -> 8 fp16 values s*(q-8) in pair order.
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v s2)
{
    const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    half8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t m = ((w >> (4 * e)) & 0x000F000Fu) | 0x64006400u;
        half2v v = __builtin_bit_cast(half2v, m);
        v = (v - off) * s2;
        r[2 * e] = v[0];
        r[2 * e + 1] = v[1];
    }
    return r;
}

struct GemmEpi {
    void *y;
    const void *res;
    int y_t, res_t;
};

// One pipeline step covers GKS quantisation groups (K = 128): the X tile of the step is in
// LDS (double-buffered), the W words and scales of the step are in registers (double-buffered),
// and the next step's loads are in flight while this step's 32 MFMAs per wave run.  The W words
// are dequantised just before their MFMA step.
__global__ __launch_bounds__(256, 2) void k_w4_gemm(W4 W, const uint16_t *__restrict__ Xh,
                                                    const float *__restrict__ su, int M, GemmEpi ep)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM * GALD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int mtiles = (M + GBM - 1) / GBM;
    const int mt = blockIdx.x % mtiles, nt = blockIdx.x / mtiles;
    const int m0 = mt * GBM, n0 = nt * GBN;
    const int K = W.k, kw = K >> 3, kg = K >> 6;
    const int nsteps = (kg + GKS - 1) / GKS;
    const int l32 = lane & 31, kh = lane >> 5;

    // X tile staging: thread -> (row tid/2, 64 values at column 64*(tid&1) of the step)
    const int srow = tid >> 1, scol = 64 * (tid & 1);
    const bool srow_ok = (m0 + srow) < M;
    const uint16_t *xsrc = Xh + (size_t)(srow_ok ? m0 + srow : 0) * K + scol;

    // W rows of this lane: one per 32-column MFMA tile.
    int nrow[2];
    bool nok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        nrow[j] = n0 + 64 * wn + 32 * j + l32;
        nok[j] = nrow[j] < W.n;
    }

    // the step's X columns: group 2*st + (tid & 1); a missing second group (odd kg) reads zero.
    // Staged in two halves of 32 columns (h = 0, 1) to keep fewer values in flight in registers.
    auto load_x = [&](int st, int h, uint4 *v) {
        const bool ok = srow_ok && (GKS * st + (tid & 1)) < kg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = ok ? *reinterpret_cast<const uint4 *>(xsrc + (size_t)st * GKS * GBK + 32 * h + 8 * i)
                      : make_uint4(0u, 0u, 0u, 0u);
    };
    auto store_x = [&](int buf, int h, const uint4 *v) {
        uint16_t *dst = &As[buf][srow * GALD + scol + 32 * h];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(dst + 8 * i) = pair_order16(v[i]);
    };
    auto load_w = [&](int st, uint4 (*wq)[GKS], float (*sc)[GKS], float (*bb)[GKS]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int gg = 0; gg < GKS; ++gg) {
                const int g = GKS * st + gg;
                if (nok[j] && g < kg) {
                    // cached load: the 128-byte line serves the next groups and every row tile
                    wq[j][gg] = *(reinterpret_cast<const uint4 *>(W.q + (size_t)nrow[j] * kw + 8 * g) + kh);
                    sc[j][gg] = bf16_to_f32(W.s[(size_t)nrow[j] * kg + g]);
                    bb[j][gg] = bf16_to_f32(W.b[(size_t)nrow[j] * kg + g]);
                } else {
                    wq[j][gg] = make_uint4(0u, 0u, 0u, 0u);
                    sc[j][gg] = 0.f;
                    bb[j][gg] = 0.f;
                }
            }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 xv[4];
    uint4 wq[2][GKS], wq_n[2][GKS];
    float sc[2][GKS], bb[2][GKS], sc_n[2][GKS], bb_n[2][GKS];
    load_w(0, wq, sc, bb);
    load_x(0, 0, xv);
    store_x(0, 0, xv);
    load_x(0, 1, xv);
    store_x(0, 1, xv);
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int cur = st & 1;
        const bool more = st + 1 < nsteps;
        if (more) {
            load_x(st + 1, 0, xv);
            load_w(st + 1, wq_n, sc_n, bb_n);
        }
#pragma unroll
        for (int gg = 0; gg < GKS; ++gg) {
            const int g = GKS * st + gg;
            if (gg == 1 && more) {
                // first half of the next step's X to the other buffer, then the second half in flight
                store_x(cur ^ 1, 0, xv);
                load_x(st + 1, 1, xv);
            }
            half2v s2[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) s2[j] = half2v{(_Float16)sc[j][gg], (_Float16)sc[j][gg]};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                half8 bf[2], af[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t ww[4] = {wq[j][gg].x, wq[j][gg].y, wq[j][gg].z, wq[j][gg].w};
                    bf[j] = dequant_word(ww[ks], s2[j]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint16_t *src = &As[cur][(64 * wm + 32 * i + l32) * GALD + GBK * gg + 8 * (4 * kh + ks)];
                    af[i] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(src));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Asymmetric groups: add (beta + 8 s) * (group sum of the X row).
            float bpp[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) bpp[j] = fmaf(8.f, sc[j][gg], bb[j][gg]);
            if (g < kg && __builtin_amdgcn_ballot_w64(bpp[0] != 0.f || bpp[1] != 0.f) != 0ull) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
                        const float s = m < M ? su[(size_t)m * kg + g] : 0.f;
#pragma unroll
                        for (int j = 0; j < 2; ++j) acc[i][j][r] = fmaf(bpp[j], s, acc[i][j][r]);
                    }
            }
        }
        if (more) {
            store_x(cur ^ 1, 1, xv);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int gg = 0; gg < GKS; ++gg) {
                    wq[j][gg] = wq_n[j][gg];
                    sc[j][gg] = sc_n[j][gg];
                    bb[j][gg] = bb_n[j][gg];
                }
        }
        __syncthreads();
    }

    // Epilogue: D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
    // column l%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = nrow[j];
            if (!nok[j]) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
                if (m >= M) continue;
                const size_t o = (size_t)m * W.n + n;
                float v = acc[i][j][r];
                if (ep.res)
                    v += ep.res_t == BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(ep.res)[o])
                                          : reinterpret_cast<const float *>(ep.res)[o];
                if (ep.y_t == BF16)
                    reinterpret_cast<uint16_t *>(ep.y)[o] = f32_to_bf16(v);
                else
                    reinterpret_cast<float *>(ep.y)[o] = v;
            }
        }
}

hipError_t launch_w4_gemm(const W4 &W, const uint16_t *Xh, const float *su, int M,
                          const void *res, int res_t, void *Y, int y_t, hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    const int mtiles = (M + GBM - 1) / GBM, ntiles = (W.n + GBN - 1) / GBN;
    GemmEpi ep{Y, res, y_t, res_t};
    k_w4_gemm<<<dim3(mtiles * ntiles), dim3(256), 0, st>>>(W, Xh, su, M, ep);
    return hipGetLastError();
}

}  // namespace nh
