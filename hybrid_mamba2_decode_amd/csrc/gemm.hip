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
// 2 x 2 MFMA 32x32 tiles, K advanced one 64-wide quantisation group at a time.  The X tile is
// staged through LDS (double-buffered, padded rows); each wave reads its W rows straight from
// global memory into registers, one group ahead.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GALD = GBK + 8;  // LDS row of the X tile, in fp16 elements (144 B: conflict-free)

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

__global__ __launch_bounds__(256) void k_w4_gemm(W4 W, const uint16_t *__restrict__ Xh,
                                                 const float *__restrict__ su, int M, GemmEpi ep)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM * GALD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int mtiles = (M + GBM - 1) / GBM;
    const int mt = blockIdx.x % mtiles, nt = blockIdx.x / mtiles;
    const int m0 = mt * GBM, n0 = nt * GBN;
    const int K = W.k, kw = K >> 3, kg = K >> 6;
    const int l32 = lane & 31, kh = lane >> 5;

    // X tile staging: thread -> (row tid/2, 32 values at column 32*(tid&1)).
    const int srow = tid >> 1, scol = 32 * (tid & 1);
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

    auto load_x = [&](int g, uint4 *v) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = srow_ok ? *reinterpret_cast<const uint4 *>(xsrc + (size_t)g * GBK + 8 * i)
                           : make_uint4(0u, 0u, 0u, 0u);
    };
    auto store_x = [&](int buf, const uint4 *v) {
        uint16_t *dst = &As[buf][srow * GALD + scol];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(dst + 8 * i) = pair_order16(v[i]);
    };
    auto load_w = [&](int g, uint4 *wq, float *sc, float *bb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (nok[j]) {
                // cached load: the 128-byte line serves the next three groups and every row tile
                wq[j] = *(reinterpret_cast<const uint4 *>(W.q + (size_t)nrow[j] * kw + 8 * g) + kh);
                sc[j] = bf16_to_f32(W.s[(size_t)nrow[j] * kg + g]);
                bb[j] = bf16_to_f32(W.b[(size_t)nrow[j] * kg + g]);
            } else {
                wq[j] = make_uint4(0u, 0u, 0u, 0u);
                sc[j] = 0.f;
                bb[j] = 0.f;
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
    uint4 wq[2], wq_n[2];
    float sc[2], bb[2], sc_n[2], bb_n[2];
    load_x(0, xv);
    load_w(0, wq, sc, bb);
    store_x(0, xv);
    __syncthreads();

    for (int g = 0; g < kg; ++g) {
        const int cur = g & 1;
        const bool more = g + 1 < kg;
        if (more) {
            load_x(g + 1, xv);
            load_w(g + 1, wq_n, sc_n, bb_n);
        }
        // B fragments: word ks of this lane's 4-word slice <-> MFMA step ks.
        half8 bf[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const half2v s2 = {(_Float16)sc[j], (_Float16)sc[j]};
            const uint32_t ww[4] = {wq[j].x, wq[j].y, wq[j].z, wq[j].w};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) bf[j][ks] = dequant_word(ww[ks], s2);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            half8 af[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint16_t *src = &As[cur][(64 * wm + 32 * i + l32) * GALD + 8 * (4 * kh + ks)];
                af[i] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(src));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j][ks], acc[i][j], 0, 0, 0);
        }
        // Asymmetric groups: add (beta + 8 s) * (group sum of the X row).
        float bpp[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bpp[j] = fmaf(8.f, sc[j], bb[j]);
        if (__builtin_amdgcn_ballot_w64(bpp[0] != 0.f || bpp[1] != 0.f) != 0ull) {
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
        if (more) {
            store_x(cur ^ 1, xv);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                wq[j] = wq_n[j];
                sc[j] = sc_n[j];
                bb[j] = bb_n[j];
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
