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
// Tiling: a 256 x 128 output tile per work-group of 8 waves with split roles, one quantisation
// group (K = 64) per step, through a ring of four LDS slots.  Waves 4-7 load: X reaches its slot
// by DMA (buffer loads that write LDS directly, issued three steps ahead of use, so X spends no
// registers or instructions of theirs), and the packed W of the group, its scale, the offset
// term and the rows' group sums go through registers four steps ahead and are written to the
// slot as they are stored (W stays packed).  Waves 0-3 compute: each owns a 128 x 64 block of
// the tile (4 x 2 MFMA 32x32 tiles), reads its operands from LDS, dequantises its W columns in
// registers, between its MFMAs, and issues the MFMAs.  With W packed in LDS a step moves 100 KB
// through LDS instead of 144 KB (fp16 W written once and read by two waves each).  One barrier
// per step: at step k the compute waves read slot k mod 4 and the packed W and scales of slot
// (k + 1) mod 4 (dequantising that step's first k-step under their last MFMAs), the DMA fills
// slot (k + 3) mod 4 and the loaders store the register part of slot (k + 2) mod 4.
//
// X comes in the operand format of the producing kernels: fp16 bits, each 8-value chunk in pair
// order (0,4) (1,5) (2,6) (3,7), the order in which a packed word dequantises.  K order inside
// a step: lane half kh of an MFMA 32x32x16 supplies k-values 8 kh .. 8 kh + 7 of the MFMA's 16;
// for k-step ks (0..3) of the group those are the group's chunk 4 kh + ks, on both operands.
// So a compute lane's W values for the whole group are the 16 packed bytes kh of its column,
// one LDS read per column block and step.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

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

constexpr int WS_BM = 256, WS_BN = 128, WS_SLOTS = 4, WS_THREADS = 512;

// The register-loaded part of an LDS slot (one quantisation group of the tile).
struct WsSlotW {
    uint4 wq[2 * WS_BN];  // packed W, [half][column]: half h holds the group's nibbles 32 h .. 32 h + 31
    uint32_t s2[WS_BN];   // the group's scale s per column, as an fp16 pair (s, s)
    float bv[WS_BN];      // the group's offset beta per column
};

// An LDS tile row of X is 8 chunks of 16 bytes; chunk c of row r sits at position
// c ^ (r mod 8) ^ (r / 8 mod 2), so 16-byte accesses by 16 lanes to one chunk of 16 consecutive
// rows, or to all chunks of 2 rows, touch each of the 64 banks once.
__device__ __forceinline__ int ws_sw(int row, int c) { return row * 8 + (c ^ (row & 7) ^ ((row >> 3) & 1)); }

// A loader lane's register loads for one step: 16 bytes of packed W (column lane / 2, half
// lane mod 2) and the groups' scales or offsets: with an even group count, one 4-byte load
// per lane every other step carries two groups of one column's scales (loader waves 0 and 1)
// or offsets (waves 2 and 3); otherwise each step loads its group's scale and offset of
// column lane / 2 (2 bytes each).
struct WsRegs {
    uint4 w;
    uint32_t p;
    uint16_t s, b;
};

// Vector-memory loads a loader wave issues in the step that is j mod 4 of the unrolled loop:
// the DMA of X (8), of the row sums (loader wave 0), packed W (1), scales and offsets.
__host__ __device__ constexpr int ws_nonx(bool pairs, int j) { return 1 + (pairs ? ((j & 1) == 0) : 2); }
__host__ __device__ constexpr int ws_total(bool pairs, bool su, int j) { return 8 + (su ? 1 : 0) + ws_nonx(pairs, j); }
// loads that follow, by the end of the step, the X DMA issued two steps earlier
__host__ __device__ constexpr int ws_after(bool pairs, bool su, int j)
{
    return ws_nonx(pairs, j) + ws_total(pairs, su, j + 1) + ws_total(pairs, su, j);
}

typedef __attribute__((address_space(3))) void ws_lds_void;

// s_waitcnt with only the vector-memory counter limited (expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void ws_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Work-group barrier for LDS data: this wave's LDS operations complete, then s_barrier.
// __syncthreads() would also wait for every load in flight, the DMA of later steps and the
// register loads four steps ahead included.  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void ws_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Work-group i runs on XCD i mod 8; each XCD takes a contiguous range of tiles in row-major
// tile order, so the work-groups resident on one XCD share the X rows of their tiles in its L2.
template <bool PAIRS>
__global__ __launch_bounds__(WS_THREADS, 1) void k_w4_gemm(W4 W, const uint16_t *__restrict__ Xh,
                                                           const float *__restrict__ su, int M, GemmEpi ep)
{
    // separate static arrays, indexed by constants after unrolling, so that the compiler can
    // tell the DMA targets (X, row sums) from the loaders' LDS stores and does not wait for the
    // DMA before them
    __shared__ uint4 ws_x[WS_SLOTS][WS_BM * 8];  // fp16 X tiles, swizzled rows
    __shared__ float ws_su[WS_SLOTS][WS_BM];     // group sum of each X row
    __shared__ WsSlotW ws_w[WS_SLOTS];

    const int K = W.k, kw = K >> 3, kg = K >> 6;
    const int ntiles = (W.n + WS_BN - 1) / WS_BN, mtiles = (M + WS_BM - 1) / WS_BM;
    const int tiles = ntiles * mtiles, per = (tiles + 7) / 8;
    const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (tile >= tiles) return;
    const int m0 = (tile / ntiles) * WS_BM, n0 = (tile % ntiles) * WS_BN;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nsteps = kg, nloop = (nsteps + 3) / 4 * 4;

    if (wave >= 4) {
        // ------------------------------------------------------------ loaders
        const int lid = tid - 256, lw = wave - 4, lane = tid & 63;
        const int n = lid >> 1, h = lid & 1;
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
        const uint32_t vw = ((uint32_t)n * kw + 4 * h) * 4, vs = (uint32_t)n * kg * 2;
        // scale / offset pairs (even group count): column 64 (lw mod 2) + lane
        const int pc = 64 * (lw & 1) + lane;
        const __amdgpu_buffer_rsrc_t rsb = lw < 2 ? rs : rb;
        const uint32_t vp = (uint32_t)pc * kg * 2;
        // X DMA: load i (0..7) of loader wave lw fills slot positions 64 q + lane, q = 8 lw + i,
        // i.e. row r = 8 q + lane / 8 at stored chunk position lane mod 8, which holds chunk
        // (lane mod 8) ^ (lane / 8) ^ (q mod 2) of the row (the swizzle, with r mod 8 = lane / 8
        // and r / 8 mod 2 = i mod 2)
        const int r0 = 64 * lw + (lane >> 3), c0 = (lane & 7) ^ (lane >> 3);
        const uint32_t vx0 = (uint32_t)r0 * K * 2 + 16 * c0, vx1 = (uint32_t)r0 * K * 2 + 16 * (c0 ^ 1);
        const size_t su_n = (size_t)M * kg;
        // Loader wave 0 also moves the rows' group sums (1 KB per step, su is [group][row]) into
        // the slot by DMA; the loop is compiled once for it and once for the other waves, so
        // that no load sits behind a branch.
        auto run = [&](auto su_tag) {
            constexpr bool SU = decltype(su_tag)::value;
            auto dma = [&](int st, uint4 *xs, float *sus) {
                const int g = min(st, kg - 1);
                if constexpr (SU) {
                    // rows past the tile read the next rows of su (or zero past its end): unused
                    const size_t o = (size_t)g * M + m0;
                    const __amdgpu_buffer_rsrc_t ru = rsrc(su + o, (uint32_t)((su_n - o) * 4));
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (ws_lds_void *)sus, 16, (uint32_t)lane * 16, 0, 0, 0);
                }
                const uint32_t go = 128u * (uint32_t)g;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (ws_lds_void *)&xs[64 * (8 * lw + i)], 16,
                                                             ((i & 1) ? vx1 : vx0) + (uint32_t)(8 * i * K * 2) + go, 0, 0, 0);
            };
            // even: the step is even (with PAIRS its load carries this step's and the next one's
            // scales or offsets)
            auto issue = [&](WsRegs &R, int st, bool even) {
                const int g = min(st, kg - 1);
                R.w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw + (uint32_t)(32 * g), 0, 0));
                if (PAIRS) {
                    if (even) R.p = __builtin_amdgcn_raw_buffer_load_b32(rsb, vp + (uint32_t)(2 * min(st, kg - 2)), 0, 0);
                } else {
                    R.s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs + (uint32_t)(2 * g), 0, 0);
                    R.b = __builtin_amdgcn_raw_buffer_load_b16(rb, vs + (uint32_t)(2 * g), 0, 0);
                }
            };
            auto half_pair = [](uint16_t v) {
                const float sc = bf16_to_f32(v);
                const half2v s2 = {(_Float16)sc, (_Float16)sc};
                return __builtin_bit_cast(uint32_t, s2);
            };
            // sl: the step's slot; sn: the next step's (PAIRS, even steps only)
            auto store = [&](const WsRegs &R, WsSlotW &sl, WsSlotW &sn, bool even) {
                sl.wq[h * WS_BN + n] = R.w;
                if (PAIRS) {
                    if (even) {
                        const uint16_t lo = (uint16_t)(R.p & 0xffffu), hi = (uint16_t)(R.p >> 16);
                        if (lw < 2) {
                            sl.s2[pc] = half_pair(lo);
                            sn.s2[pc] = half_pair(hi);
                        } else {
                            sl.bv[pc] = bf16_to_f32(lo);
                            sn.bv[pc] = bf16_to_f32(hi);
                        }
                    }
                } else if (h == 0) {
                    sl.s2[n] = half_pair(R.s);
                    sl.bv[n] = bf16_to_f32(R.b);
                }
            };
            // step s: X and row sums by DMA at step s - 3; registers (set s mod 4) loaded at step
            // s - 6 and stored at step s - 2.  Loads past the last group re-read it (no branch
            // around a load) and the slots they fill are never read.
            WsRegs rr[4];
            dma(0, ws_x[0], ws_su[0]);
            dma(1, ws_x[1], ws_su[1]);
            dma(2, ws_x[2], ws_su[2]);
#pragma unroll
            for (int j = 0; j < 4; ++j) issue(rr[j], j, (j & 1) == 0);
            store(rr[0], ws_w[0], ws_w[1], true);
            issue(rr[0], 4, true);
            store(rr[1], ws_w[1], ws_w[2], false);
            issue(rr[1], 5, false);
            ws_wait_vm<ws_after(PAIRS, SU, 1)>();  // the DMA of step 0 (more loads follow it)
            auto block = [&](int k) {  // steps k .. k + 3
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ws_barrier();  // step k + j: its slot is complete
                    dma(k + j + 3, ws_x[(j + 3) & 3], ws_su[(j + 3) & 3]);
                    asm volatile("" ::: "memory");  // the DMA goes out before this step's other loads
                    store(rr[(j + 2) & 3], ws_w[(j + 2) & 3], ws_w[(j + 3) & 3], (j & 1) == 0);
                    issue(rr[(j + 2) & 3], k + j + 6, (j & 1) == 0);
                    // the DMA of step k + j + 1 (in the first two steps more loads follow it)
                    if ((j & 1) == 0)  // j is a constant once unrolled
                        ws_wait_vm<ws_after(PAIRS, SU, 0)>();
                    else
                        ws_wait_vm<ws_after(PAIRS, SU, 1)>();
                }
            };
            // the first block outside the loop, so that the loop is entered with the loads in
            // flight that its back edge has (the compiler's own waits before the stores are
            // then no stricter than in the steady state)
            block(0);
            for (int k = 4; k < nloop; k += 4) block(k);
            ws_wait_vm<0>();  // no DMA into LDS outlives the work-group
        };
        if (lw == 0)
            run(std::true_type{});
        else
            run(std::false_type{});
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

    // the packed W of the wave's two column blocks for the current step (lane: column l32,
    // nibbles 32 kh ..), their scales, and k-step 0 dequantised
    uint4 wr[2];
    half2v s2[2];
    half8 b0[2];
    auto wload = [&](const WsSlotW &sl) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            wr[j] = sl.wq[kh * WS_BN + 64 * wn + 32 * j + l32];
            s2[j] = __builtin_bit_cast(half2v, sl.s2[64 * wn + 32 * j + l32]);
            b0[j] = dequant_word(wr[j].x, s2[j]);
        }
    };
    auto step = [&](int k, const uint4 *xs, const float *sus, const WsSlotW &sl, const WsSlotW &sl_next) {
        ws_barrier();
        if (k >= nsteps) return;
        if (k == 0) wload(sl);
        // operands of k-step ks + 1 are read and dequantised while the MFMAs of k-step ks run;
        // during the last k-step, the next step's packed W (the register part of its slot is
        // complete since this step's barrier)
        half8 af[2][4], bf[2][2];
        auto rd = [&](int ks, half8 (&a)[4], half8 (&b)[2]) {
            const int c = 4 * kh + ks;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(half8, xs[ws_sw(128 * wm + 32 * i + l32, c)]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (ks == 0) {
                    b[j] = b0[j];
                } else {
                    const uint32_t w = ks == 1 ? wr[j].y : ks == 2 ? wr[j].z : wr[j].w;
                    b[j] = dequant_word(w, s2[j]);
                }
            }
        };
        rd(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4)
                rd(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
            else
                wload(sl_next);  // after the last step: stale values, never used
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
            {
                // the LDS reads first, then the dequantisation spread between the MFMAs: one
                // MFMA, four VALU instructions, eight times
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // asymmetric groups: add (beta + 8 s) * (group sum of the X row) as a rank-1 fp32
        // matrix-core update (K = 2 with the second k zero)
        float bq[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = 64 * wn + 32 * j + l32;
            bq[j] = fmaf(8.f, (float)__builtin_bit_cast(half2v, sl.s2[c])[0], sl.bv[c]);  // beta + 8 s
        }
        if (__builtin_amdgcn_ballot_w64(bq[0] != 0.f || bq[1] != 0.f) != 0ull) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = kh ? 0.f : sus[128 * wm + 32 * i + l32];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, kh ? 0.f : bq[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    for (int k = 0; k < nloop; k += 4) {
        step(k, ws_x[0], ws_su[0], ws_w[0], ws_w[1]);
        step(k + 1, ws_x[1], ws_su[1], ws_w[1], ws_w[2]);
        step(k + 2, ws_x[2], ws_su[2], ws_w[2], ws_w[3]);
        step(k + 3, ws_x[3], ws_su[3], ws_w[3], ws_w[0]);
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
    const int tiles = ((M + WS_BM - 1) / WS_BM) * ((W.n + WS_BN - 1) / WS_BN);
    GemmEpi ep{Y, res, y_t, res_t};
    const dim3 grid(8 * ((tiles + 7) / 8)), block(WS_THREADS);
    if ((W.k >> 6) % 2 == 0)
        k_w4_gemm<true><<<grid, block, 0, st>>>(W, Xh, su, M, ep);
    else
        k_w4_gemm<false><<<grid, block, 0, st>>>(W, Xh, su, M, ep);
    return hipGetLastError();
}

}  // namespace nh
