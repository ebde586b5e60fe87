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
// Tiling: a 256 x 128 output tile per work-group of 8 waves with split roles.  Waves 4-7 load:
// one quantisation group (K = 64) of the X tile and of the W tile per step, from global memory
// into registers four steps ahead of use; they dequantise W to fp16 and write both tiles into
// a ring of three LDS slots.  Waves 0-3 compute: each owns a 128 x 64 block of the tile (4 x 2
// MFMA 32x32 tiles) and only reads LDS and issues MFMAs.  One barrier per step: at step k the
// compute waves read slot k mod 3 while the loaders fill slot (k + 2) mod 3, which the compute
// waves left at step k - 1.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

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

constexpr int WS_BM = 256, WS_BN = 128, WS_SLOTS = 3, WS_THREADS = 512;

// One LDS slot: the operands of one step (one quantisation group of the tile).
struct WsSlot {
    uint4 x[WS_BM * 8];  // fp16 X tile, [row][chunk], pair order inside a chunk
    uint4 w[WS_BN * 8];  // fp16 s (q - 8) tile, [column][chunk], pair order inside a chunk
    float bpp[WS_BN];    // beta + 8 s per column (zero for symmetric groups)
    float su[WS_BM];     // group sum of each X row
};

// An LDS tile row is 8 chunks of 16 bytes; chunk c of row r sits at position
// c ^ (r mod 8) ^ (r / 8 mod 2), so 16-byte accesses by 16 lanes to one chunk of 16 consecutive
// rows, or to all chunks of 2 rows, touch each of the 64 banks once.
__device__ __forceinline__ int ws_sw(int row, int c) { return row * 8 + (c ^ (row & 7) ^ ((row >> 3) & 1)); }

// A loader lane's global loads for one step: 8 x 16 bytes of X (rows 32 i + lane / 8, chunk
// lane mod 8), 16 bytes of packed W (column lane / 2, half lane mod 2), the column's scale and
// bias, and the group sum of X row lane.
struct WsRegs {
    uint4 x[8];
    uint4 w;
    uint16_t s, b;
    float su;
};

// Work-group i runs on XCD i mod 8; each XCD takes a contiguous range of tiles in row-major
// tile order, so the work-groups resident on one XCD share the X rows of their tiles in its L2.
__global__ __launch_bounds__(WS_THREADS, 1) void k_w4_gemm(W4 W, const uint16_t *__restrict__ Xh,
                                                           const float *__restrict__ su, int M, GemmEpi ep)
{
    extern __shared__ __attribute__((aligned(16))) char ws_smem[];
    WsSlot *slots = reinterpret_cast<WsSlot *>(ws_smem);

    const int K = W.k, kw = K >> 3, kg = K >> 6;
    const int ntiles = (W.n + WS_BN - 1) / WS_BN, mtiles = (M + WS_BM - 1) / WS_BM;
    const int tiles = ntiles * mtiles, per = (tiles + 7) / 8;
    const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (tile >= tiles) return;
    const int m0 = (tile / ntiles) * WS_BM, n0 = (tile % ntiles) * WS_BN;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nsteps = kg, nloop = (nsteps + 11) / 12 * 12;

    if (wave >= 4) {
        // ------------------------------------------------------------ loaders
        const int lid = tid - 256;
        const int xc = lid & 7, n = lid >> 1, h = lid & 1;
        // Buffer resources based at the tile's first row and covering only the tile's rows, so
        // rows past the end of X or W read 0 (every offset is in the per-lane operand, the scalar
        // offset operand stays 0, so the range check covers the whole offset).
        auto rsrc = [](const void *p, uint32_t bytes) {
            return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, (int)bytes, 0x00020000);
        };
        const uint32_t mrows = (uint32_t)min(M - m0, WS_BM), nrows = (uint32_t)min(W.n - n0, WS_BN);
        const __amdgpu_buffer_rsrc_t rx = rsrc(Xh + (size_t)m0 * K, mrows * (uint32_t)K * 2);
        const __amdgpu_buffer_rsrc_t rw = rsrc(W.q + (size_t)n0 * kw, nrows * (uint32_t)kw * 4);
        const __amdgpu_buffer_rsrc_t rs = rsrc(W.s + (size_t)n0 * kg, nrows * (uint32_t)kg * 2);
        const __amdgpu_buffer_rsrc_t rb = rsrc(W.b + (size_t)n0 * kg, nrows * (uint32_t)kg * 2);
        const uint32_t vx = ((uint32_t)(lid >> 3) * K + 8 * xc) * 2, vw = ((uint32_t)n * kw + 4 * h) * 4;
        const uint32_t vs = (uint32_t)n * kg * 2, vu = (uint32_t)lid * 4;
        auto issue = [&](WsRegs &R, int st) {
            const int g = min(st, kg - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                R.x[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, vx + (uint32_t)(32 * i * K * 2 + 128 * g), 0, 0));
            R.w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw + (uint32_t)(32 * g), 0, 0));
            R.s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs + (uint32_t)(2 * g), 0, 0);
            R.b = __builtin_amdgcn_raw_buffer_load_b16(rb, vs + (uint32_t)(2 * g), 0, 0);
            // group g's sums of the tile's rows (su is [group][row])
            const __amdgpu_buffer_rsrc_t ru = rsrc(su + (size_t)g * M + m0, mrows * 4);
            R.su = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ru, vu, 0, 0));
        };
        auto store = [&](const WsRegs &R, int slot) {
            WsSlot &sl = slots[slot];
#pragma unroll
            for (int i = 0; i < 8; ++i) sl.x[ws_sw(32 * i + (lid >> 3), xc)] = pair_order16(R.x[i]);
            const float sc = bf16_to_f32(R.s);
            const half2v s2 = {(_Float16)sc, (_Float16)sc};
            const uint32_t ww[4] = {R.w.x, R.w.y, R.w.z, R.w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)  // the two lanes of a column write in different bank orders
                sl.w[ws_sw(n, 4 * h + (j ^ h))] = __builtin_bit_cast(uint4, dequant_word(ww[j ^ h], s2));
            if (h == 0) sl.bpp[n] = fmaf(8.f, sc, bf16_to_f32(R.b));
            sl.su[lid] = R.su;
        };
        // stage s: register set s mod 4, LDS slot s mod 3; loaded at step s - 6, stored at step
        // s - 2.  Loads past the last group re-read it (no branch around a load) and the slots
        // they fill are never read.
        WsRegs rr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) issue(rr[j], j);
        store(rr[0], 0);
        issue(rr[0], 4);
        store(rr[1], 1);
        issue(rr[1], 5);
        for (int k = 0; k < nloop; k += 12) {
#pragma unroll
            for (int j = 0; j < 12; ++j) {
                __syncthreads();
                store(rr[(j + 2) & 3], (j + 2) % 3);
                issue(rr[(j + 2) & 3], k + j + 6);
            }
        }
        return;
    }

    // ---------------------------------------------------------------- compute
    const int lane = tid & 63, l32 = lane & 31, kh = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;  // rows 128 wm .. +127, columns 64 wn .. +63
    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto step = [&](int k, int slot) {
        __syncthreads();
        if (k >= nsteps) return;
        const WsSlot &sl = slots[slot];
        // operands of k-step ks + 1 are read while the MFMAs of k-step ks run
        half8 af[2][4], bf[2][2];
        auto rd = [&](int ks, half8 (&a)[4], half8 (&b)[2]) {
            const int c = 2 * ks + kh;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(half8, sl.x[ws_sw(128 * wm + 32 * i + l32, c)]);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = __builtin_bit_cast(half8, sl.w[ws_sw(64 * wn + 32 * j + l32, c)]);
        };
        rd(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) rd(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // asymmetric groups: add (beta + 8 s) * (group sum of the X row) as a rank-1 fp32
        // matrix-core update (K = 2 with the second k zero)
        float bq[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bq[j] = sl.bpp[64 * wn + 32 * j + l32];
        if (__builtin_amdgcn_ballot_w64(bq[0] != 0.f || bq[1] != 0.f) != 0ull) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = kh ? 0.f : sl.su[128 * wm + 32 * i + l32];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, kh ? 0.f : bq[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    for (int k = 0; k < nloop; k += 3) {
        step(k, 0);
        step(k + 1, 1);
        step(k + 2, 2);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + l32;
            if (n >= W.n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
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
    static bool attr = false;
    const size_t smem = WS_SLOTS * sizeof(WsSlot);
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)k_w4_gemm,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int tiles = ((M + WS_BM - 1) / WS_BM) * ((W.n + WS_BN - 1) / WS_BN);
    GemmEpi ep{Y, res, y_t, res_t};
    k_w4_gemm<<<dim3(8 * ((tiles + 7) / 8)), dim3(WS_THREADS), smem, st>>>(W, Xh, su, M, ep);
    return hipGetLastError();
}

}  // namespace nh
