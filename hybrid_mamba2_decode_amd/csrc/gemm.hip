// gemm.hip -- W4 matrix product Y = X W^T (+ residual) on gfx950 matrix cores.
//
// Dequantisation is exact: with bf16 scales s, the value s*(q-8) has at most 11 significant
// bits (|q-8| <= 8 and s carries 8 bits), so it is an fp16 number.  The B operand is built as
// fp16 s*(q-8) straight from the packed word: the fp16 pair (1024+q_e, 1024+q_{e+4}) is the
// nibbles under a 0x64 exponent byte (1024's unit in the last place is 1), a packed subtract of
// 1032 and a packed multiply by s finish it.  The rest of the affine map,
//     W = s*(q-8) + (beta + 8 s),
// is zero for symmetric groups (beta = -8 s); otherwise its contribution
// (beta + 8s) * sum_{k in group} X[m][k] is added in fp32 from precomputed group sums.
// Activations arrive as fp16 bits (bf16-exact values), so every product is exact and the
// accumulation is fp32 inside v_mfma_f32_32x32x16_f16.
//
// Two kernels.  With an even number of quantisation groups (K a multiple of 128, as in_proj and
// out_proj) and enough rows to fill the chip, k_w4_gemm_wide: 256 x 256 tiles, all 8 waves
// compute, every operand reaches LDS by DMA (described with the kernel).  Otherwise
// k_w4_gemm: a 256 x 128 output tile per
// work-group of 8 waves with split roles, one quantisation group (K = 64) per step, through a
// ring of four LDS slots.  Waves 4-7 load: X (and, from loader wave 0, the rows' group sums)
// reaches its slot by DMA (buffer loads that write LDS directly, issued three steps ahead of use,
// so X spends no registers or instructions of theirs), and the packed W of the group, its scale
// and offset go through registers four steps ahead and are written to the slot as they are
// stored (W stays packed).  Waves 0-3 compute: each owns a 128 x 64 block of the tile (4 x 2
// MFMA 32x32 tiles), reads its operands from LDS, dequantises its W columns in registers,
// between its MFMAs, and issues the MFMAs.  With W packed in LDS a step moves 100 KB through LDS
// instead of 144 KB (fp16 W written once and read by two waves each).  One barrier per step: at
// step k the compute waves read slot k mod 4 and the packed W and scales of slot (k + 1) mod 4
// (dequantising that step's first k-step under their last MFMAs), the DMA fills slot
// (k + 3) mod 4 and the loaders store the register part of slot (k + 2) mod 4.
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

// One packed word of 8 nibbles -> 8 fp16 values s*(q-8) in pair order.  The low and high
// nibbles of each byte are split into bytes (lo: nibbles 0 2 4 6, hi: 1 3 5 7), and one byte
// permute per pair places two of them under a 0x64 exponent byte: the fp16 pair
// (1024 + q_e, 1024 + q_{e+4}) in 7 ALU instructions per word instead of 11.
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v s2)
{
    const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu, ex = 0x64646464u;
    // v_perm_b32: selector bytes 0-3 pick the second operand's bytes, 4-7 the first's
    const uint32_t m[4] = {__builtin_amdgcn_perm(ex, lo, 0x04020400u), __builtin_amdgcn_perm(ex, hi, 0x04020400u),
                           __builtin_amdgcn_perm(ex, lo, 0x04030401u), __builtin_amdgcn_perm(ex, hi, 0x04030401u)};
    half8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        half2v v = __builtin_bit_cast(half2v, m[e]);
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

// Epilogue of one 32x32 MFMA tile: rows mb + 8 (r / 4) + 4 kh + (r mod 4) of column n (the
// lane's), plus the residual, stored in the output type.  The residual loads of the tile go out
// together (addresses clamped into the matrix, values past the end unused), then one wait.
__device__ __forceinline__ void gemm_store_block(const floatx16 &acc, int mb, int n, int kh, int M, int N,
                                                 const GemmEpi &ep)
{
    const int nc = min(n, N - 1);
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = acc[r];
    auto at = [&](int r) { return (size_t)min(mb + 8 * (r >> 2) + 4 * kh + (r & 3), M - 1) * N + nc; };
    if (ep.res && ep.res_t == BF16) {
        uint16_t rv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) rv[r] = reinterpret_cast<const uint16_t *>(ep.res)[at(r)];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += bf16_to_f32(rv[r]);
    } else if (ep.res) {
        float rv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) rv[r] = reinterpret_cast<const float *>(ep.res)[at(r)];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += rv[r];
    }
    if (n >= N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (m >= M) continue;
        const size_t o = (size_t)m * N + n;
        if (ep.y_t == BF16)
            reinterpret_cast<uint16_t *>(ep.y)[o] = f32_to_bf16(v[r]);
        else
            reinterpret_cast<float *>(ep.y)[o] = v[r];
    }
}

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
// lane mod 2) and the group's scale and offset of that column (2 bytes each).
struct WsRegs {
    uint4 w;
    uint16_t s, b;
};

// Vector-memory loads a loader wave issues per step: the DMA of X (8) and of the row sums
// (loader wave 0), packed W, scale and offset (3); by the end of a step, the X DMA issued two
// steps earlier is followed by 3 + 2 (11 + su) loads.
__host__ __device__ constexpr int ws_after(bool su) { return 3 + 2 * (11 + (su ? 1 : 0)); }

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
                    const __amdgpu_buffer_rsrc_t ru = rsrc(su + o, (uint32_t)min((su_n - o) * 4, (size_t)0xFFFFFFF0u));
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (ws_lds_void *)sus, 16, (uint32_t)lane * 16, 0, 0, 0);
                }
                const uint32_t go = 128u * (uint32_t)g;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (ws_lds_void *)&xs[64 * (8 * lw + i)], 16,
                                                             ((i & 1) ? vx1 : vx0) + (uint32_t)(8 * i * K * 2) + go, 0, 0, 0);
            };
            auto issue = [&](WsRegs &R, int st) {
                const int g = min(st, kg - 1);
                R.w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw + (uint32_t)(32 * g), 0, 0));
                R.s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs + (uint32_t)(2 * g), 0, 0);
                R.b = __builtin_amdgcn_raw_buffer_load_b16(rb, vs + (uint32_t)(2 * g), 0, 0);
            };
            auto half_pair = [](uint16_t v) {
                const float sc = bf16_to_f32(v);
                const half2v s2 = {(_Float16)sc, (_Float16)sc};
                return __builtin_bit_cast(uint32_t, s2);
            };
            auto store = [&](const WsRegs &R, WsSlotW &sl) {
                sl.wq[h * WS_BN + n] = R.w;
                if (h == 0) {
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
            for (int j = 0; j < 4; ++j) issue(rr[j], j);
            store(rr[0], ws_w[0]);
            issue(rr[0], 4);
            store(rr[1], ws_w[1]);
            issue(rr[1], 5);
            ws_wait_vm<ws_after(SU)>();  // the DMA of step 0 (more loads follow it)
            auto block = [&](int k) {  // steps k .. k + 3
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ws_barrier();  // step k + j: its slot is complete
                    dma(k + j + 3, ws_x[(j + 3) & 3], ws_su[(j + 3) & 3]);
                    asm volatile("" ::: "memory");  // the DMA goes out before this step's other loads
                    store(rr[(j + 2) & 3], ws_w[(j + 2) & 3]);
                    issue(rr[(j + 2) & 3], k + j + 6);
                    // the DMA of step k + j + 1 (in the first two steps more loads follow it)
                    ws_wait_vm<ws_after(SU)>();
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
    // Asymmetric groups: (beta + 8 s) * (group sum of the X row) as a rank-1 fp32 matrix-core
    // update.  Its MFMA takes K = 2, so it carries two groups: an even step k ends by reading its
    // group's row sums and offset terms from its slot (su_e, bq_e: registers held only across
    // the barrier), and step k + 1 starts with the update of both, k = 0 the even group (lanes
    // 0-31), k = 1 its own (lanes 32-63).  A last even step (odd group count) adds its group
    // alone, the second k zero.
    float su_e[4], bq_e[2];
    auto offset_term = [&](const WsSlotW &sl, int j) __attribute__((always_inline)) {
        const int c = 64 * wn + 32 * j + l32;
        return fmaf(8.f, (float)__builtin_bit_cast(half2v, sl.s2[c])[0], sl.bv[c]);  // beta + 8 s
    };
    auto asym_update = [&](const float *sus, const WsSlotW &sl, bool pair) __attribute__((always_inline)) {
        float bq[2];
        bool asym = false;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bq[j] = kh ? (pair ? offset_term(sl, j) : 0.f) : bq_e[j];
            asym = asym || bq[j] != 0.f;
        }
        if (__builtin_amdgcn_ballot_w64(asym) != 0ull) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = kh ? (pair ? sus[128 * wm + 32 * i + l32] : 0.f) : su_e[i];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bq[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    auto step = [&](int k, const uint4 *xs, const float *sus, const WsSlotW &sl, const WsSlotW &sl_next) {
        ws_barrier();
        if (k >= nsteps) return;
        if (k & 1) asym_update(sus, sl, true);
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
        // an even step hands its group's row sums and offset terms to the next step (or, as the
        // last step, adds them alone)
        if ((k & 1) == 0) {
            bool asym = false;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bq_e[j] = offset_term(sl, j);
                asym = asym || bq_e[j] != 0.f;
            }
            // the row sums only for an asymmetric group (zero otherwise: the pair's update may
            // still run for the odd group, and multiplies them by a zero offset term)
            const bool any = __builtin_amdgcn_ballot_w64(asym) != 0ull;
#pragma unroll
            for (int i = 0; i < 4; ++i) su_e[i] = any ? sus[128 * wm + 32 * i + l32] : 0.f;
            if (k + 1 >= nsteps) asym_update(sus, sl, false);
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
        for (int j = 0; j < 2; ++j)
            gemm_store_block(acc[i][j], m0 + 128 * wm + 32 * i, n0 + 64 * wn + 32 * j + l32, kh, M, W.n, ep);
}

// ------------------------------------------------------------------ wide tiles
// With an even number of quantisation groups: 256 x 256 output tiles, all 8 waves compute
// (wave w owns rows 128 (w / 4) .. + 127 and columns 64 (w mod 4) .. + 63, 4 x 2 MFMA 32x32
// tiles) and every operand reaches LDS by DMA, so no wave spends registers or instructions on
// staging.  The X tile of a step (32 KB) is the same as for a 256 x 128 tile and now feeds
// twice the matrix-core work; with 256 x 128 tiles the X fetch (about 22 B per clock per CU)
// set the pace.  Per step each wave issues 6 loads into the slot of the step two ahead:
//   X: 4 x 1 KB (rows 32 w .. 32 w + 31, swizzled as in the split-role kernel);
//   W: 1 KB of packed nibbles (half w / 4, columns 64 (w mod 4) + lane);
//   the scales (waves 0-3) or offsets (waves 4-7) of 64 columns, 4 bytes per column holding
//   the group pair (g & ~1, g | 1) (aligned because the group count is even);
// and wave 0 the rows' group sums (1 KB).  Three slots, one barrier per step: at step k the
// waves read slot k mod 3 and fill slot (k + 2) mod 3, which everyone left at step k - 1.
constexpr int WG_BM = 256, WG_BN = 256, WG_THREADS = 512;

struct WgSlot {
    uint4 x[WG_BM * 8];   // fp16 X tile, [row][chunk] swizzled (ws_sw), pair order inside a chunk
    uint4 wq[2 * WG_BN];  // packed W, [half][column]
    uint32_t sp[WG_BN];   // bf16 scale pair (group g & ~1 low, g | 1 high) per column
    uint32_t bp[WG_BN];   // bf16 offset pair, the same groups
    float su[WG_BM];      // group sum of each X row
};

template <int WI>
__global__ __launch_bounds__(WG_THREADS, 1) void k_w4_gemm_wide(W4 W, const uint16_t *__restrict__ Xh,
                                                                const float *__restrict__ su, int M, GemmEpi ep)
{
    // three separate objects, so that the compiler can tell the slot being read from the ones
    // the DMA is filling and does not wait for the DMA before the reads
    __shared__ WgSlot sa, sb, sc;

    const int K = W.k, kw = K >> 3, kg = K >> 6;
    const int ntiles = (W.n + WG_BN - 1) / WG_BN, mtiles = (M + WG_BM - 1) / WG_BM;
    const int tiles = ntiles * mtiles, per = (tiles + 7) / 8;
    const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (tile >= tiles) return;
    const int m0 = (tile / ntiles) * WG_BM, n0 = (tile % ntiles) * WG_BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nsteps = kg;

    // ---- DMA sources (buffer resources cover only the tile's rows: rows past the end read 0)
    auto rsrc = [](const void *p, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, (int)bytes, 0x00020000);
    };
    const uint32_t mrows = (uint32_t)min(M - m0, WG_BM), nrows = (uint32_t)min(W.n - n0, WG_BN);
    const __amdgpu_buffer_rsrc_t rx = rsrc(Xh + (size_t)m0 * K, mrows * (uint32_t)K * 2);
    const __amdgpu_buffer_rsrc_t rw = rsrc(W.q + (size_t)n0 * kw, nrows * (uint32_t)kw * 4);
    const __amdgpu_buffer_rsrc_t rsb = wave < 4 ? rsrc(W.s + (size_t)n0 * kg, nrows * (uint32_t)kg * 2)
                                                : rsrc(W.b + (size_t)n0 * kg, nrows * (uint32_t)kg * 2);
    const size_t su_n = (size_t)M * kg;
    // X: load i (0..3) fills slot positions 64 q + lane, q = 4 w + i: row 8 q + lane / 8 at
    // stored chunk position lane mod 8, i.e. chunk (lane mod 8) ^ (lane / 8) ^ (q mod 2)
    const int r0 = 32 * wave + (lane >> 3), c0 = (lane & 7) ^ (lane >> 3);
    const uint32_t vx0 = (uint32_t)r0 * K * 2 + 16 * c0, vx1 = (uint32_t)r0 * K * 2 + 16 * (c0 ^ 1);
    // W: position 64 w + lane = half h, column n
    const int wp = 64 * wave + lane, wh = wp >> 8, wcol = wp & 255;
    const uint32_t vw = (uint32_t)wcol * kw * 4 + 16 * wh;
    const int sbcol = 64 * (wave & 3) + lane;
    const uint32_t vsb = (uint32_t)sbcol * kg * 2;
    // the loads of step st into slot sl, in three parts (issued between the k-steps of the
    // current step, so that a wave waiting for room in the memory queue still has MFMAs in flight)
    auto dma = [&](int part, int st, WgSlot &sl) __attribute__((always_inline)) {
        const int g = min(st, kg - 1);
        const uint32_t go = 128u * (uint32_t)g;
        if (part == 0) {
            if (wave == 0) {
                // rows past the tile read the next rows of su (or zero past its end): unused
                const size_t o = (size_t)g * M + m0;
                const __amdgpu_buffer_rsrc_t ru = rsrc(su + o, (uint32_t)min((su_n - o) * 4, (size_t)0xFFFFFFF0u));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (ws_lds_void *)sl.su, 16, (uint32_t)lane * 16, 0, 0, 0);
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (ws_lds_void *)&sl.wq[64 * wave], 16, vw + 32u * (uint32_t)g, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (ws_lds_void *)&sl.sp[64 * wave], 4,
                                                     vsb + 2u * (uint32_t)(g & ~1), 0, 0, 0);
        } else {
            const int i0 = 2 * (part - 1);
#pragma unroll
            for (int i = i0; i < i0 + 2; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (ws_lds_void *)&sl.x[64 * (4 * wave + i)], 16,
                                                         ((i & 1) ? vx1 : vx0) + (uint32_t)(8 * i * K * 2) + go, 0, 0, 0);
        }
    };

    // ---- compute
    const int l32 = lane & 31, kh = lane >> 5;
    // wave w: WI x WJ MFMA tiles, rows 32 WI wm .., columns 32 WJ wn ..  WI = 4 (128 x 64 per
    // wave); 64 x 128 (WI = 2) reads less of X from LDS but dequantises twice the W per wave,
    // and measured 10% slower
    constexpr int WJ = 8 / WI, NWN = 8 / (8 / WI);
    const int wm = wave / NWN, wn = wave % NWN;
    floatx16 acc[WI][WJ];
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Asymmetric groups: (beta + 8 s) * (group sum of the X row) as a rank-1 fp32 matrix-core
    // update.  Its MFMA takes K = 2, so it carries two groups (the group count is even): an even
    // step k ends by reading its group's row sums and offset terms from its own slot (su_e,
    // bq_e: registers held only across the barrier), and step k + 1 starts with the update of
    // both groups, k = 0 the even one (lanes 0-31), k = 1 its own (lanes 32-63).  The slot of
    // step k is not read after its barrier: the loads of step k + 3 go into it.  The even
    // slot's scale and offset pairs also hold the odd group's (high halves), so the even step
    // decides for both whether the update runs (pair_asym, wave-uniform); for symmetric groups
    // the odd step does nothing.
    float su_e[WI], bq_e[WJ];
    bool pair_asym = false;
    auto offset_term = [&](const WgSlot &sl, int hi, int j) __attribute__((always_inline)) {
        const int c = 32 * WJ * wn + 32 * j + l32;
        const uint32_t spv = sl.sp[c], bpv = sl.bp[c];
        const float sv = bf16_to_f32((uint16_t)(hi ? spv >> 16 : spv & 0xffffu));
        const float bv = bf16_to_f32((uint16_t)(hi ? bpv >> 16 : bpv & 0xffffu));
        return fmaf(8.f, sv, bv);  // beta + 8 s
    };
    auto asym_pair = [&](const WgSlot &cu) __attribute__((always_inline)) {
        float bq[WJ];
#pragma unroll
        for (int j = 0; j < WJ; ++j) bq[j] = kh ? offset_term(cu, 1, j) : bq_e[j];
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const float a = kh ? cu.su[32 * WI * wm + 32 * i + l32] : su_e[i];
#pragma unroll
            for (int j = 0; j < WJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bq[j], acc[i][j], 0, 0, 0);
        }
    };
    auto step = [&](int k, const WgSlot &sl, WgSlot &fill) __attribute__((always_inline)) {
        uint4 wr[WJ];
        half2v s2[WJ];
        const int hi = k & 1;
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int c = 32 * WJ * wn + 32 * j + l32;
            wr[j] = sl.wq[kh * WG_BN + c];
            const uint32_t spv = sl.sp[c];
            const float sv = bf16_to_f32((uint16_t)(hi ? spv >> 16 : spv & 0xffffu));
            s2[j] = half2v{(_Float16)sv, (_Float16)sv};
        }
        half8 af[2][WI], bf[2][WJ];
        auto rd = [&](int ks, half8 (&a)[WI], half8 (&b)[WJ]) {
            const int c = 4 * kh + ks;
#pragma unroll
            for (int i = 0; i < WI; ++i) a[i] = __builtin_bit_cast(half8, sl.x[ws_sw(32 * WI * wm + 32 * i + l32, c)]);
#pragma unroll
            for (int j = 0; j < WJ; ++j) {
                const uint32_t w = ks == 0 ? wr[j].x : ks == 1 ? wr[j].y : ks == 2 ? wr[j].z : wr[j].w;
                b[j] = dequant_word(w, s2[j]);
            }
        };
        rd(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) rd(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < WI; ++i)
#pragma unroll
                for (int j = 0; j < WJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
            if (ks + 1 < 4) {
                // the next k-step's LDS reads first, then its dequantisation spread between the
                // eight MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, WI, 0);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2 * WJ, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks < 3) {
                asm volatile("" ::: "memory");
                dma(ks, k + 2, fill);  // part ks of the loads of step k + 2
                asm volatile("" ::: "memory");
            }
        }
        if ((k & 1) == 0) {
            bool asym = false;
#pragma unroll
            for (int j = 0; j < WJ; ++j) {
                bq_e[j] = offset_term(sl, 0, j);
                asym = asym || bq_e[j] != 0.f || offset_term(sl, 1, j) != 0.f;
            }
            pair_asym = __builtin_amdgcn_ballot_w64(asym) != 0ull;
            if (pair_asym) {
#pragma unroll
                for (int i = 0; i < WI; ++i) su_e[i] = sl.su[32 * WI * wm + 32 * i + l32];
            }
        }
    };

    // step k: DMA at step k - 2 (wave 0 issues 7 loads a step, the others 6; each wave waits
    // for its own loads of the next step, which 6 or 7 loads follow, before the barrier)
    for (int p = 0; p < 3; ++p) dma(p, 0, sa);
    for (int p = 0; p < 3; ++p) dma(p, 1, sb);
    ws_wait_vm<6>();
    // fill: the slot of step k - 1, which takes the loads of step k + 2
    auto one = [&](int k, const WgSlot &cur, WgSlot &fill) __attribute__((always_inline)) {
        ws_barrier();  // step k: its slot is complete, the slot of step k - 1 is free
        if ((k & 1) && pair_asym) asym_pair(cur);
        step(k, cur, fill);
        ws_wait_vm<6>();  // this wave's loads of step k + 1
    };
    // every step computes: the loop leaves after the last one (the loads of the two steps past
    // the end re-read the last group into slots nobody reads)
    for (int k = 0;; k += 3) {
        one(k, sa, sc);
        if (k + 1 >= nsteps) break;
        one(k + 1, sb, sa);
        if (k + 2 >= nsteps) break;
        one(k + 2, sc, sb);
        if (k + 3 >= nsteps) break;
    }
    ws_wait_vm<0>();  // no DMA into LDS outlives the work-group

#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j)
            gemm_store_block(acc[i][j], m0 + 32 * WI * wm + 32 * i, n0 + 32 * WJ * wn + 32 * j + l32, kh, M, W.n, ep);
}

static int gemm_cu_count()
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

hipError_t launch_w4_gemm(const W4 &W, const uint16_t *Xh, const float *su, int M,
                          const void *res, int res_t, void *Y, int y_t, hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    GemmEpi ep{Y, res, y_t, res_t};
    const int tiles = ((M + WS_BM - 1) / WS_BM) * ((W.n + WS_BN - 1) / WS_BN);
    if ((W.k >> 6) % 2 == 0) {
        // A wide tile takes about 1.88 times as long as a split-role tile (measured at the
        // in_proj and out_proj shapes), so the wide kernel is taken when its rounds of one
        // work-group per CU, times 1.88, are fewer than the split kernel's: e.g. in_proj at
        // 7500 rows (11 rounds against 21), but not out_proj (3 against 5).
        const int wtiles = ((M + WG_BM - 1) / WG_BM) * ((W.n + WG_BN - 1) / WG_BN);
        const int cus = gemm_cu_count(), rw = (wtiles + cus - 1) / cus, rs = (tiles + cus - 1) / cus;
        if (47 * rw < 25 * rs) {
            k_w4_gemm_wide<4><<<dim3(8 * ((wtiles + 7) / 8)), dim3(WG_THREADS), 0, st>>>(W, Xh, su, M, ep);
            return hipGetLastError();
        }
    }
    k_w4_gemm<<<dim3(8 * ((tiles + 7) / 8)), dim3(WS_THREADS), 0, st>>>(W, Xh, su, M, ep);
    return hipGetLastError();
}

}  // namespace nh
