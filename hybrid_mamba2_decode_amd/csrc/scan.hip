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
// C.B^T depends on the group only, so a pre-pass (k_ssd_cb) computes it once per (sequence,
// chunk, group): bf16 matrix-core products of the bf16 inputs (exact products, fp32 sums),
// stored as fp16 16 x 16 tiles of the causal lower triangle in the lane order the scan reads
// them in (lane l = 16 q + i holds G[16I + i][16J + 4q + r], r = 0..3).  Tiles 2jp and 2jp + 1
// of row block I form a pair stored lane-interleaved (lane l's 4 values of one, then its 4 of
// the other), so a wave loads a pair with one 16-byte load per lane; row block I holds
// ceil((I + 1) / 2) pairs (the last one half used when I is even).
// Workspace layout: chunk-major, then (sequence, group); a chunk of L rows holds
// cb_pairs(L) pairs per (sequence, group), at most 8 KiB per position (chunks under 17 rows).
//
// Decomposition.  One work-group of 8 waves per (sequence, head) walks the chunks in order and
// keeps the head's 80 x 128 fp32 state in registers as the accumulator of the state MFMA (wave
// w owns state columns 16w .. 16w+15).  Work-group i runs on XCD i mod 8, so the 16 heads that
// share a B/C group are numbered to land on one XCD and read B and C through one L2.
//
// Per chunk:
//   1. the chunk's B and x (prefetched into registers during the previous chunk) go to LDS as
//      row-major fp16 tiles; dt = softplus(dt_raw + dt_bias) and the log2-scaled cumulative
//      sum of dt A (256-wide block scan); S_in as fp16;
//   2. (after step 3) the next chunk's B, x, dt_raw and C rows are issued to registers;
//   3. wave w takes 16-row output blocks {w, 15-w} (equal causal work) and computes them
//      transposed, Y^T = S_in C^T + X^T (G o decay)^T: its C rows, already in registers, are the
//      B operand of S_in C^T, and the block's G tiles come from the pre-pass in the B-operand
//      layout, so the scaled tile never leaves registers; each lane ends with 4 consecutive
//      columns of one output row, and the block goes through the wave's LDS rows so that each
//      16-byte store covers 8 consecutive columns of one row;
//   4. each wave adds x^T (w B) to its state columns, w_j = exp(cum_{L-1} - cum_j) dt_j taken
//      from an fp16 table and multiplied into the B fragment in registers (steps 3 and 4 only
//      read LDS, so no barrier separates them).
// Operands with k = chunk position (x, w x, B in the state update) are read with
// ds_read_b64_tr_b16, which transposes 4 x 16-bit elements across each group of 16 lanes, so
// both tiles stay row-major in LDS.  Matrix-core operands are fp16 (B, C, x are bf16-exact;
// computed operands round once, 2^-11 relative); accumulation is fp32.  Chunks shorter than
// 32 rows are zero-padded.
//
// Global memory is addressed through buffer resources whose base is the chunk's first row and
// whose size covers the chunk's valid rows only, so the hardware range check makes rows at or
// beyond min(Q, T - t0) read as zero and drops their stores; offsets are per lane and
// chunk-relative (the scalar offset operand is always 0).
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

constexpr int SC_THREADS = 512;
constexpr int BS_LD = DSTATE + 16;  // B rows: 288 B (transposed reads conflict-free)
constexpr int XS_LD = HDIM;         // x rows: 160 B (transposed reads conflict-free)
constexpr int SI_LD = DSTATE + 8;   // S_in rows: 272 B
constexpr int YS_LD = HDIM + 8;     // staged output rows: 176 B (16-byte aligned, writes conflict-free)

// Member order keeps the tables, x and S_in below 64 KiB, so their reads take immediate
// offsets from one base register.
struct ScanSmem {
    float cum[QMAX];            // log2-scaled cumulative dt*A
    float dtv[QMAX];            // dt
    float Fv[QMAX];             // exp(cum_end(block of j) - cum_j) dt_j
    _Float16 Wh[QMAX];          // w_j = exp(cum_{L-1} - cum_j) dt_j (state-update weights)
    float wsum[4];
    uint16_t Xs[QMAX * XS_LD];  // x of the chunk, [j][p]
    uint16_t Si[HDIM * SI_LD];  // state at chunk start, [p][n]
    uint16_t Bs[QMAX * BS_LD];  // B of the chunk, [j][n]
    uint16_t Ys[8][16 * YS_LD]; // per wave: one 16-row bf16 output block, [i][p]
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Transposed read: lane (group g = lane/16, s = lane%16) addresses row r0 + s/4, columns
// c0 + 4*(s%4) .. +3 of a row-major fp16 tile; lane g*16 + i receives, for e = 0..3, element
// [r0 + e][c0 + i] where r0 is the group's own base row.
__device__ __forceinline__ uint2 ld_tr(const uint16_t *tile, int ld, int r0, int c0)
{
    const int s = threadIdx.x & 15;
    const uint16_t *p = tile + (r0 + (s >> 2)) * ld + c0 + 4 * (s & 3);
    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)p);
    return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ half8 ld_half8(const uint16_t *p)
{
    return __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ half8 cat(uint2 a, uint2 b)
{
    return __builtin_bit_cast(half8, make_uint4(a.x, a.y, b.x, b.y));
}

// DPP move of v (lanes whose source is invalid or whose row is masked off read 0)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ uint32_t pack_rne(float a, float b)
{
    half2v v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 w)
{
    return make_uint4(bf16x2_to_f16x2(w.x), bf16x2_to_f16x2(w.y), bf16x2_to_f16x2(w.z), bf16x2_to_f16x2(w.w));
}

constexpr int PB_VEC = QMAX * (DSTATE / 8) / SC_THREADS;  // 8 B vectors per thread
constexpr int PX_VEC = QMAX * (HDIM / 8) / SC_THREADS;    // 5 x vectors per thread

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Registers holding the next chunk while the current one is computed.
struct Prefetch {
    uint4 b[PB_VEC];
    uint4 x[PX_VEC];
    uint4 c[2][4];
    uint32_t dt;
};

// ------------------------------------------------- long-chunk operands (k_ssd_scanx)
// Chunks of at least XQ_MIN rows in sequences of at least XT_MIN positions take k_ssd_scanx.
// Its pre-pass writes, besides the C.B^T tiles, per (chunk, sequence, group) the chunk's B in
// the state update's operand order (NJ(L) steps of 32 rows x 8 state blocks x 64 lanes x 16 B)
// and its C in the operand order of C S_in^T (ceil(L/16) row blocks x 4 steps of 32 state
// columns x 64 lanes x 16 B), both fp16, and per (chunk, sequence, head) the tables over
// P = 32 NJ(L) positions: cum (log2 units), dt and F (fp32), then W (fp16).  All are laid out
// chunk-major like the tiles (full chunks at the Q stride, the last chunk at its own size).
constexpr int XQ_MIN = 128, XT_MIN = 64;

__host__ __device__ constexpr int nj_of(int L) { return (L + 31) >> 5; }
__host__ __device__ constexpr size_t btf_bytes(int L) { return (size_t)nj_of(L) * 8 * 1024; }
__host__ __device__ constexpr size_t tab_bytes(int L) { return ((size_t)nj_of(L) * 32 * 14 + 63) & ~(size_t)63; }
__host__ __device__ constexpr size_t cfr_bytes(int L) { return (size_t)((L + 15) >> 4) * 4 * 1024; }

// ------------------------------------------------------------------ C.B^T pre-pass

constexpr int CB_THREADS = 512;
constexpr int CB_LD = DSTATE + 8;  // bf16 B rows in LDS: 272 B (16-byte row reads conflict-free)

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// Tile pairs (2jp, 2jp + 1) of the row blocks I < nb: row block I holds ceil((I + 1) / 2) pairs.
__host__ __device__ constexpr int cb_pairs_before(int nb)
{
    return (nb & 1) ? ((nb + 1) / 2) * ((nb + 1) / 2) : (nb / 2) * (nb / 2 + 1);
}

__host__ __device__ constexpr int cb_pairs(int Q) { return cb_pairs_before((Q + 15) / 16); }

// first tile of (chunk ck of L rows, sequence b, group g)
__device__ __forceinline__ size_t cb_base(int ck, int Q, int L, int batch, int b, int g)
{
    return ((size_t)ck * batch * NGROUPS * cb_pairs(Q) + (size_t)(b * NGROUPS + g) * cb_pairs(L)) * 512;
}

// One work-group per (chunk, group, sequence): B rows of the chunk to LDS; wave w takes row
// blocks I = w and 15 - w (equal causal work when the chunk has 16 blocks) and for each J <= I
// computes the tile D = B_J C_I^T (D lane layout: rows j = 16J + 4q + r, column
// i = 16I + l16), which is the G layout the scan reads.  Diagonal tiles hold 0 above the
// diagonal (j > i): the causal mask.
// Tables of one (chunk, sequence, group) for its 16 heads: wave w takes heads 2w and 2w + 1, lane
// l positions 4l .. 4l + 3 of the chunk's P = 32 NJ(L) (dt = 0 past L).  ssd_tables_load issues
// the raw dt loads (positions past L clamped), ssd_tables computes and stores the tables.
__device__ __forceinline__ void ssd_tables_load(const uint16_t *__restrict__ dtr, long ld_dt, int T, int Q, int c,
                                                int g, int b, int L, int wave, int lane, uint16_t (&raw)[2][4])
{
    const uint16_t *dseq = dtr + ((size_t)b * T + (size_t)c * Q) * ld_dt;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            raw[k][r] = dseq[(size_t)min(4 * lane + r, L - 1) * ld_dt + g * HPG + 2 * wave + k];
}

__device__ __forceinline__ void ssd_tables(const uint16_t (&raw)[2][4], const float *__restrict__ dt_bias,
                                           const float *__restrict__ A_log, char *__restrict__ Tw, int Q, int c,
                                           int g, int b, int batch, int L, int wave, int lane)
{
    const int P = 32 * nj_of(L);
    const float LOG2E = 1.4426950408889634f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int h = g * HPG + 2 * wave + k;
        const float A2 = -expf(A_log[h]) * LOG2E;  // dt*A in log2 units
        const float dtb = dt_bias[h];
        float dt[4], s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * lane + r;
            dt[r] = j < L ? softplus_fast(bf16_to_f32(raw[k][r]) + dtb) : 0.f;
            s[r] = (r ? s[r - 1] : 0.f) + dt[r] * A2;
        }
        // inclusive sum of the lane totals over the wave (row shifts, then the row ends
        // broadcast into the following rows); the exclusive sum is the previous lane's
        float v = s[3];
        v += dpp_f<0x111, 0xF>(v);  // row_shr:1
        v += dpp_f<0x112, 0xF>(v);  // row_shr:2
        v += dpp_f<0x114, 0xF>(v);  // row_shr:4
        v += dpp_f<0x118, 0xF>(v);  // row_shr:8
        v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
        v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
        float ex = __shfl(v, (lane + 63) & 63, 64);
        if (lane == 0) ex = 0.f;
        float cum[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) cum[r] = ex + s[r];
        // cumulative value at the end of the position's 16-row block (position 16 m + 15 is
        // lane 4 m + 3, r = 3) and at the chunk end (a_j = 0 for j >= L)
        const float cend = __shfl(cum[3], lane | 3, 64);
        const float cl = __shfl(cum[3], P / 4 - 1, 64);
        if (4 * lane < P) {
            char *tb = Tw + (size_t)c * batch * NHEADS * tab_bytes(Q) + (size_t)(b * NHEADS + h) * tab_bytes(L);
            float F[4];
            _Float16 W[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                F[r] = __builtin_amdgcn_exp2f(cend - cum[r]) * dt[r];
                W[r] = (_Float16)(__builtin_amdgcn_exp2f(cl - cum[r]) * dt[r]);
            }
            reinterpret_cast<float4 *>(tb)[lane] = make_float4(cum[0], cum[1], cum[2], cum[3]);
            reinterpret_cast<float4 *>(tb + 4 * P)[lane] = make_float4(dt[0], dt[1], dt[2], dt[3]);
            reinterpret_cast<float4 *>(tb + 8 * P)[lane] = make_float4(F[0], F[1], F[2], F[3]);
            reinterpret_cast<uint2 *>(tb + 12 * P)[lane] =
                make_uint2(__builtin_bit_cast(uint32_t, half2v{W[0], W[1]}), __builtin_bit_cast(uint32_t, half2v{W[2], W[3]}));
        }
    }
}

// Long-chunk operands (EXT).  For k_ssd_scanx the pre-pass also writes, per (chunk, sequence,
// group), B in the operand order of the state update, and per (chunk, sequence, head) the chunk's
// discretisation tables; see k_ssd_scanx for their layouts.
template <bool EXT>
__global__ __launch_bounds__(CB_THREADS) void k_ssd_cb(const uint16_t *__restrict__ xc, int T, int Q,
                                                      uint16_t *__restrict__ Gw, const uint16_t *__restrict__ dtr,
                                                      long ld_dt, const float *__restrict__ dt_bias,
                                                      const float *__restrict__ A_log, char *__restrict__ Bfw,
                                                      char *__restrict__ Cfw, char *__restrict__ Tw)
{
    __shared__ __attribute__((aligned(16))) uint16_t Bs[QMAX * CB_LD];
    // EXT: two work-groups per (chunk, group, sequence): role 0 the tiles and C fragments, role 1
    // the B fragments and the tables (whose dt loads go out first, so the table arithmetic runs
    // while B is still arriving)
    const int role = EXT ? (int)blockIdx.z & 1 : 0;
    const int c = blockIdx.x, g = blockIdx.y, b = EXT ? blockIdx.z >> 1 : blockIdx.z;
    const int batch = EXT ? gridDim.z >> 1 : gridDim.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int t0 = c * Q, L = min(Q, T - t0), nb = (L + 15) >> 4;
    const uint32_t XROW = CONVDIM * 2;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xc + ((size_t)b * T + t0) * CONVDIM), 0, (int)((uint32_t)L * XROW), 0x00020000);

    uint16_t raw[2][4];
    if (EXT && role == 1) ssd_tables_load(dtr, ld_dt, T, Q, c, g, b, L, wave, lane, raw);
    const int Ib[2] = {wave, 15 - wave};
    uint4 cq[2][4];
    if (role == 0)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                cq[bi][ks] = bload16(rx, (uint32_t)(16 * Ib[bi] + l16) * XROW + (OFF_C + g * DSTATE + 32 * ks + 8 * q4) * 2, 0);
    // B rows to LDS: every load issued before the first LDS write (rows past L read as zero)
    {
        const int nrows = role == 1 ? 32 * nj_of(L) : 16 * nb;
        constexpr int NV = QMAX * 16 / CB_THREADS;
        uint4 bv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + CB_THREADS * i, row = v >> 4, pc = v & 15;
            bv[i] = bload16(rx, (uint32_t)row * XROW + (OFF_B + g * DSTATE + 8 * pc) * 2, 0);
        }
        if (EXT && role == 1) ssd_tables(raw, dt_bias, A_log, Tw, Q, c, g, b, batch, L, wave, lane);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + CB_THREADS * i, row = v >> 4, pc = v & 15;
            if (row < nrows) *reinterpret_cast<uint4 *>(&Bs[row * CB_LD + 8 * pc]) = bv[i];
        }
    }
    __syncthreads();

    if (EXT && role == 1) {
        // B fragment (jp, state block n = wave): lane (q, i) holds B[32 jp + 4 q + e][16 n + i] for
        // e < 4 and B[32 jp + 16 + 4 q + e - 4][16 n + i] for e >= 4, as fp16 (exact in range)
        char *bf = Bfw + (size_t)c * batch * NGROUPS * btf_bytes(Q) + (size_t)(b * NGROUPS + g) * btf_bytes(L);
        for (int jp = 0; jp < nj_of(L); ++jp) {
            const uint2 lo = ld_tr(Bs, CB_LD, 32 * jp + 4 * q4, 16 * wave);
            const uint2 hi = ld_tr(Bs, CB_LD, 32 * jp + 16 + 4 * q4, 16 * wave);
            *reinterpret_cast<uint4 *>(bf + ((size_t)(jp * 8 + wave) * 64 + lane) * 16) =
                make_uint4(bf16x2_to_f16x2(lo.x), bf16x2_to_f16x2(lo.y), bf16x2_to_f16x2(hi.x), bf16x2_to_f16x2(hi.y));
        }
        return;
    }

    uint16_t *Gc = Gw + cb_base(c, Q, L, batch, b, g) + lane * 8;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
        const int I = Ib[bi];
        if (I >= nb) continue;
        uint16_t *gI = Gc + cb_pairs_before(I) * 512;
        // two tiles per step: independent accumulation chains
        for (int J = 0; J <= I; J += 2) {
            const int J1 = min(J + 1, I);
            floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
            const uint16_t *s0 = &Bs[(16 * J + l16) * CB_LD + 8 * q4];
            const uint16_t *s1 = &Bs[(16 * J1 + l16) * CB_LD + 8 * q4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8v cf = __builtin_bit_cast(bf16x8v, cq[bi][ks]);
                a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4 *>(s0 + 32 * ks)), cf, a0, 0, 0, 0);
                a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4 *>(s1 + 32 * ks)), cf, a1, 0, 0, 0);
            }
            if (J == I)
#pragma unroll
                for (int r = 0; r < 4; ++r) a0[r] = 4 * q4 + r > l16 ? 0.f : a0[r];
            if (J1 == I)
#pragma unroll
                for (int r = 0; r < 4; ++r) a1[r] = 4 * q4 + r > l16 ? 0.f : a1[r];
            // pair J / 2: lane l's 4 values of tile J, then its 4 values of tile J + 1
            if (J + 1 <= I)
                *reinterpret_cast<uint4 *>(gI + (J >> 1) * 512) =
                    make_uint4(pack_rne(a0[0], a0[1]), pack_rne(a0[2], a0[3]), pack_rne(a1[0], a1[1]), pack_rne(a1[2], a1[3]));
            else
                *reinterpret_cast<uint2 *>(gI + (J >> 1) * 512) = make_uint2(pack_rne(a0[0], a0[1]), pack_rne(a0[2], a0[3]));
        }
    }
    if constexpr (EXT) {
        // C fragment (row block I, step ks): lane (q, i) holds C[16 I + i][32 ks + 8 q .. + 7]
        char *cfw = Cfw + (size_t)c * batch * NGROUPS * cfr_bytes(Q) + (size_t)(b * NGROUPS + g) * cfr_bytes(L);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
            if (Ib[bi] < nb)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    *reinterpret_cast<uint4 *>(cfw + ((size_t)(Ib[bi] * 4 + ks) * 64 + lane) * 16) = bf16x8_to_f16x8(cq[bi][ks]);
    }
}

// ------------------------------------------------------------------------- scan

template <int YT>
__global__ __launch_bounds__(SC_THREADS, 1) void k_ssd_scan(const uint16_t *__restrict__ xc,
                                                            const uint16_t *__restrict__ dtr, long ld_dt,
                                                            int T, int Q, const float *__restrict__ dt_bias,
                                                            const float *__restrict__ A_log,
                                                            const float *__restrict__ Dp, const float *h0,
                                                            float *hT, void *__restrict__ y,
                                                            const uint16_t *__restrict__ Gw)
{
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    ScanSmem &sm = *reinterpret_cast<ScanSmem *>(smem_raw);
    constexpr int YB = YT == BF16 ? 2 : 4;

    const int g = blockIdx.x % NGROUPS;
    const int rr = blockIdx.x / NGROUPS;
    const int h = g * HPG + rr % HPG;
    const int b = rr / HPG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;

    const float LOG2E = 1.4426950408889634f;
    const float A2 = -expf(A_log[h]) * LOG2E;  // dt*A in log2 units
    const float dtb = dt_bias[h];
    const float Dh = Dp[h];
    // D on the diagonal of the diagonal tile: lane (i = l16, j = 4q4 + r) holds D where j == i
    float dsel[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dsel[r] = 4 * q4 + r == l16 ? Dh : 0.f;

    // Rows of this sequence; a chunk's buffer resource starts at its first row.
    const uint32_t XROW = CONVDIM * 2, YROW = DINNER * YB, DROW = (uint32_t)ld_dt * 2;
    const char *xseq = reinterpret_cast<const char *>(xc + (size_t)b * T * CONVDIM);
    const char *dseq = reinterpret_cast<const char *>(dtr + (size_t)b * T * ld_dt);
    char *yseq = reinterpret_cast<char *>(y) + (size_t)b * T * YROW;
    auto rsrc = [](const char *p, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, (int)bytes, 0x00020000);
    };

    // output blocks of this wave
    const int I0 = wave, I1 = 15 - wave;
    // per-lane offsets inside a chunk: B row (tid/16) + 32i, 16 B piece tid%16; x row tid/2,
    // half row tid%2 as 5 x 16 B; C rows of blocks I0, I1; dt row tid
    const uint32_t vb = (uint32_t)(tid >> 4) * XROW + (OFF_B + g * DSTATE + 8 * (tid & 15)) * 2;
    const uint32_t vx = (uint32_t)(tid >> 1) * XROW + (h * HDIM + 40 * (tid & 1)) * 2;
    const uint32_t vc0 = (uint32_t)(16 * I0 + l16) * XROW + (OFF_C + g * DSTATE + 8 * q4) * 2;
    const uint32_t vc1 = (uint32_t)(16 * I1 + l16) * XROW + (OFF_C + g * DSTATE + 8 * q4) * 2;
    const uint32_t vdt = (uint32_t)tid * DROW + h * 2;

    auto prefetch_bx = [&](Prefetch &pf, int t0) {
        const uint32_t rows = (uint32_t)min(Q, T - t0);
        const __amdgpu_buffer_rsrc_t rx = rsrc(xseq + (size_t)t0 * XROW, rows * XROW);
        const __amdgpu_buffer_rsrc_t rd = rsrc(dseq + (size_t)t0 * DROW, rows * DROW);
#pragma unroll
        for (int i = 0; i < PB_VEC; ++i) pf.b[i] = bload16(rx, vb + (uint32_t)i * 32 * XROW, 0);
#pragma unroll
        for (int e = 0; e < PX_VEC; ++e) pf.x[e] = bload16(rx, vx + 16 * e, 0);
        pf.dt = __builtin_amdgcn_raw_buffer_load_b16(rd, vdt, 0, 0);
    };
    auto prefetch_c = [&](Prefetch &pf, int t0) {
        const uint32_t rows = (uint32_t)min(Q, T - t0);
        const __amdgpu_buffer_rsrc_t rx = rsrc(xseq + (size_t)t0 * XROW, rows * XROW);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            pf.c[0][ks] = bload16(rx, vc0 + 64 * ks, 0);
            pf.c[1][ks] = bload16(rx, vc1 + 64 * ks, 0);
        }
    };
    auto prefetch = [&](Prefetch &pf, int t0) {
        prefetch_bx(pf, t0);
        prefetch_c(pf, t0);
    };

    // State: st[pb] holds S[16pb + 4q4 + r][16 wave + l16], r = 0..3.
    floatx4 st[5];
    {
        const float *S0 = h0 ? h0 + ((size_t)b * NHEADS + h) * HDIM * DSTATE : nullptr;
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st[pb][r] = S0 ? S0[(16 * pb + 4 * q4 + r) * DSTATE + 16 * wave + l16] : 0.f;
    }

    Prefetch pf;
    prefetch(pf, 0);

    for (int t0 = 0, ck = 0; t0 < T; t0 += Q, ++ck) {
        const int L = min(Q, T - t0);
        const int LR = (L + 31) & ~31;

        // ---- 1. chunk to LDS; discretisation, cumulative sum, decay table; S_in
        float dtt = 0.f, a = 0.f;
        if (tid < L) {
            dtt = softplus_fast(bf16_to_f32((uint16_t)pf.dt) + dtb);
            a = dtt * A2;
        }
        // inclusive prefix sum over the wave: row shifts within 16-lane rows, then the row ends
        // broadcast into the following rows
        float v = a;
        v += dpp_f<0x111, 0xF>(v);  // row_shr:1
        v += dpp_f<0x112, 0xF>(v);  // row_shr:2
        v += dpp_f<0x114, 0xF>(v);  // row_shr:4
        v += dpp_f<0x118, 0xF>(v);  // row_shr:8
        v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
        v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
        if (lane == 63 && wave < 4) sm.wsum[wave] = v;
#pragma unroll
        for (int i = 0; i < PB_VEC; ++i)
            *reinterpret_cast<uint4 *>(&sm.Bs[((tid >> 4) + 32 * i) * BS_LD + 8 * (tid & 15)]) =
                bf16x8_to_f16x8(pf.b[i]);
#pragma unroll
        for (int e = 0; e < PX_VEC; ++e)
            *reinterpret_cast<uint4 *>(&sm.Xs[(tid >> 1) * XS_LD + 40 * (tid & 1) + 8 * e]) =
                bf16x8_to_f16x8(pf.x[e]);
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.Si[(16 * pb + 4 * q4 + r) * SI_LD + 16 * wave + l16] =
                    __builtin_bit_cast(uint16_t, (_Float16)st[pb][r]);
        __syncthreads();
        // cumulative value at the chunk end (a_j = 0 for j >= L)
        const float cl = (sm.wsum[0] + sm.wsum[1]) + (sm.wsum[2] + sm.wsum[3]);
        if (tid < QMAX) {
            for (int w = 0; w < wave; ++w) v += sm.wsum[w];
            // cumulative value at the end of this lane's 16-row block
            const float cend = __shfl(v, lane | 15, 64);
            sm.cum[tid] = v;
            sm.dtv[tid] = dtt;
            sm.Fv[tid] = __builtin_amdgcn_exp2f(cend - v) * dtt;
            sm.Wh[tid] = (_Float16)(__builtin_amdgcn_exp2f(cl - v) * dtt);
        }
        const int t1 = t0 + Q;
        __syncthreads();
        // the next chunk's B, x and dt rows (their registers were consumed by step 1)
        if (t1 < T) prefetch_bx(pf, t1);

        // ---- 3. outputs of blocks I0, I1
        const int nblk = (L + 15) >> 4;
        const __amdgpu_buffer_rsrc_t ry = rsrc(yseq + (size_t)t0 * YROW, (uint32_t)L * YROW);
        const uint16_t *Gc = Gw + cb_base(ck, Q, L, gridDim.x / NHEADS, b, g) + lane * 8;
#pragma unroll 1
        for (int bi = 0; bi < 2; ++bi) {
            const int I = bi == 0 ? I0 : I1;
            if (I >= nblk) continue;
            // the block's G tiles J = 0..I, loaded three pairs ahead of their use (the first
            // three while C S_in^T runs; loads past I re-read tile I and are unused)
            const uint16_t *gI = Gc + cb_pairs_before(I) * 512;
            auto gload = [&](int jp) { return *reinterpret_cast<const uint4 *>(gI + min(jp, I >> 1) * 512); };
            // window of pairs jp, jp + 1, jp + 2
            uint4 g0 = gload(0), g1 = gload(1), g2 = gload(2);
            __builtin_amdgcn_sched_barrier(0);
            half8 cfb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                cfb[ks] = __builtin_bit_cast(half8, bf16x8_to_f16x8(bi == 0 ? pf.c[0][ks] : pf.c[1][ks]));
            const int ia = 16 * I + l16;
            floatx4 acc[5];
#pragma unroll
            for (int pb = 0; pb < 5; ++pb) {
                acc[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        ld_half8(&sm.Si[(16 * pb + l16) * SI_LD + 32 * ks + 8 * q4]), cfb[ks], acc[pb], 0, 0, 0);
            }
            // acc[pb][r] = Y^T[p = 16pb + 4q4 + r][i = ia]
            const float ci = sm.cum[ia];
            const float ei = __builtin_amdgcn_exp2f(ci);
#pragma unroll
            for (int pb = 0; pb < 5; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pb][r] *= ei;

            // gt[r] = G[i = ia][j = 16J + 4q4 + r]
            auto gtile = [&](const uint2 gv) {
                const half2v lo = __builtin_bit_cast(half2v, gv.x), hi = __builtin_bit_cast(half2v, gv.y);
                return floatx4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
            };
            // below the diagonal: exp(cum_i - cum_j) = exp(cum_i - cum_end(J)) exp(cum_end(J) - cum_j);
            // the factor is rounded to fp16 and multiplied into the fp16 tile (packed)
            auto offdiag = [&](int J, const uint2 gv) {
                const float eJ = __builtin_amdgcn_exp2f(ci - sm.cum[16 * J + 15]);
                const float4 F = *reinterpret_cast<const float4 *>(&sm.Fv[16 * J + 4 * q4]);
                const half2v f01 = __builtin_bit_cast(half2v, pack_rne(eJ * F.x, eJ * F.y));
                const half2v f23 = __builtin_bit_cast(half2v, pack_rne(eJ * F.z, eJ * F.w));
                const half2v m01 = __builtin_bit_cast(half2v, gv.x) * f01;
                const half2v m23 = __builtin_bit_cast(half2v, gv.y) * f23;
                return make_uint2(__builtin_bit_cast(uint32_t, m01), __builtin_bit_cast(uint32_t, m23));
            };
            // the diagonal block (its tile is already 0 for j > i, where the clamped exponent
            // keeps the factor finite), plus the skip term D x_i on j == i
            auto diag = [&](const uint2 gv) {
                const floatx4 gt = gtile(gv);
                float m[4];
                const float4 cj = *reinterpret_cast<const float4 *>(&sm.cum[16 * I + 4 * q4]);
                const float4 dj = *reinterpret_cast<const float4 *>(&sm.dtv[16 * I + 4 * q4]);
                const float cja[4] = {cj.x, cj.y, cj.z, cj.w}, dja[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    m[r] = gt[r] * __builtin_amdgcn_exp2f(fminf(ci - cja[r], 0.f)) * dja[r] + dsel[r];
                return make_uint2(pack_rne(m[0], m[1]), pack_rne(m[2], m[3]));
            };
            // m: the scaled tiles 2jp, 2jp + 1, B operand (column i, k = j); the A operand is
            // X^T[p][j] with j = 32jp + 4q4 + e (e < 4) and 32jp + 16 + 4q4 + (e - 4)
            auto apply = [&](int jp, const uint2 ma, const uint2 mb) {
                const half8 mf = __builtin_bit_cast(half8, make_uint4(ma.x, ma.y, mb.x, mb.y));
#pragma unroll
                for (int pb = 0; pb < 5; ++pb) {
                    const half8 xf = cat(ld_tr(sm.Xs, XS_LD, 32 * jp + 4 * q4, 16 * pb),
                                         ld_tr(sm.Xs, XS_LD, 32 * jp + 16 + 4 * q4, 16 * pb));
                    acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf, mf, acc[pb], 0, 0, 0);
                }
            };
            // pairs of 16-column blocks strictly below the diagonal
            const int npair = I >> 1;
#pragma unroll 1
            for (int jp = 0; jp < npair; ++jp) {
                const uint4 nx = gload(jp + 3);
                apply(jp, offdiag(2 * jp, make_uint2(g0.x, g0.y)), offdiag(2 * jp + 1, make_uint2(g0.z, g0.w)));
                g0 = g1;
                g1 = g2;
                g2 = nx;
            }
            // the pair that holds the diagonal block
            if (I & 1)
                apply(npair, offdiag(I - 1, make_uint2(g0.x, g0.y)), diag(make_uint2(g0.z, g0.w)));
            else
                apply(npair, diag(make_uint2(g0.x, g0.y)), make_uint2(0u, 0u));
            // store y (the skip term is in the diagonal).  bf16 output goes through the wave's
            // LDS block so that each 16-byte store covers consecutive columns of one row.
            if (YT == BF16) {
                uint16_t *ys = sm.Ys[wave];
#pragma unroll
                for (int pb = 0; pb < 5; ++pb)
                    *reinterpret_cast<uint2 *>(&ys[l16 * YS_LD + 16 * pb + 4 * q4]) =
                        make_uint2(pack_bf16x2(acc[pb][0], acc[pb][1]), pack_bf16x2(acc[pb][2], acc[pb][3]));
#pragma unroll
                for (int e = 0; e < 3; ++e) {
                    const int c = lane + 64 * e;  // 16-byte piece: row c / 10, columns 8 (c % 10) ..
                    if (c < 160) {
                        const int ri = c / 10, cc = c - 10 * ri;
                        const uint4 v = *reinterpret_cast<const uint4 *>(&ys[ri * YS_LD + 8 * cc]);
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), ry,
                            (uint32_t)(16 * I + ri) * YROW + (uint32_t)(h * HDIM + 8 * cc) * 2, 0, 0);
                    }
                }
            } else {
                const uint32_t rowoff = (uint32_t)ia * YROW + (uint32_t)(h * HDIM + 4 * q4) * YB;
#pragma unroll
                for (int pb = 0; pb < 5; ++pb) {
                    const u32x4v w4 = {__float_as_uint(acc[pb][0]), __float_as_uint(acc[pb][1]),
                                       __float_as_uint(acc[pb][2]), __float_as_uint(acc[pb][3])};
                    __builtin_amdgcn_raw_buffer_store_b128(w4, ry, rowoff + 16 * pb * YB, 0, 0);
                }
            }
        }
        // ---- 2. the next chunk into registers (free once this chunk's outputs are done;
        // the loads land during step 4)
        if (t1 < T) prefetch_c(pf, t1);

        // ---- 4. state: S = exp(cum_{L-1}) S + x^T (w B) over this wave's 16 columns
        const float dec = __builtin_amdgcn_exp2f(cl);
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[pb][r] *= dec;
        for (int ks = 0; ks < (LR >> 5); ++ks) {
            const int j0 = 32 * ks + 8 * q4;
            half8 bfr = cat(ld_tr(sm.Bs, BS_LD, j0, 16 * wave), ld_tr(sm.Bs, BS_LD, j0 + 4, 16 * wave));
            bfr *= *reinterpret_cast<const half8 *>(&sm.Wh[j0]);
#pragma unroll
            for (int pb = 0; pb < 5; ++pb) {
                const half8 af = cat(ld_tr(sm.Xs, XS_LD, j0, 16 * pb), ld_tr(sm.Xs, XS_LD, j0 + 4, 16 * pb));
                st[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bfr, st[pb], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    if (hT) {
        float *Sg = hT + ((size_t)b * NHEADS + h) * HDIM * DSTATE;
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sg[(16 * pb + 4 * q4 + r) * DSTATE + 16 * wave + l16] = st[pb][r];
    }
}

// --------------------------------------------------------------- long-chunk scan
//
// k_ssd_scanx: the same decomposition (one work-group of 8 waves per (sequence, head), the
// head's fp32 state in registers, wave w owning output blocks w and 15 - w and state columns
// 16w .. 16w+15), arranged so that a wave never waits on the HBM stream:
//  - x of the next chunk goes to LDS by DMA (buffer loads that write LDS, double-buffered),
//    together with the chunk's tables from the pre-pass, so no registers hold it;
//  - every L2 operand of a chunk (its C rows, the B fragments of the state update, the C.B^T
//    pairs of both output blocks) is loaded into registers at the end of the previous chunk,
//    before the next DMA is issued: a wave's loads complete in issue order, so waiting for
//    them never waits for the DMA;
//  - the state update and both output blocks run in one loop over 32-row steps of the chunk,
//    so each x^T fragment read from LDS feeds up to 15 matrix-core products (5 for the state,
//    5 per output block) instead of 5.
// Per chunk: [DMA of the next chunk issued] x converted to fp16 in place, S_in to LDS, state
// decayed | barrier | C S_in^T for both blocks, the 32-row loop, y stores, the next chunk's L2
// operands | wait for this wave's DMA | barrier.
// s_waitcnt with only the vector-memory counter limited (expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void;

// Work-group barrier for LDS data only: this wave's LDS operations complete (lgkmcnt 0), then
// s_barrier.  __syncthreads() would also wait for the vector-memory counter, i.e. for a DMA
// into the other LDS buffer still in flight.  The empty asm statements with a memory clobber
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int YT>
__global__ __launch_bounds__(SC_THREADS, 1) void k_ssd_scanx(const uint16_t *__restrict__ xc, int T, int Q,
                                                             const float *__restrict__ Dp, const float *h0,
                                                             float *hT, void *__restrict__ y,
                                                             const uint16_t *__restrict__ Gw,
                                                             const char *__restrict__ Bfw,
                                                             const char *__restrict__ Cfw,
                                                             const char *__restrict__ Tw)
{
    // LDS: x of a chunk ([j][p], bf16 as loaded, fp16 once converted) and its tables (cum, dt,
    // F over P positions, then W), double-buffered as separate arrays so that the compiler can
    // tell the buffer being filled by DMA from the one being read; S_in ([p][n], fp16); per
    // wave, one 16-row bf16 output block.
    __shared__ __attribute__((aligned(16))) uint16_t Xs0[QMAX * HDIM], Xs1[QMAX * HDIM];
    __shared__ __attribute__((aligned(16))) uint32_t Tab0[1024], Tab1[1024];
    __shared__ __attribute__((aligned(16))) uint16_t Si[HDIM * SI_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Ys[8][16 * YS_LD];
    constexpr int YB = YT == BF16 ? 2 : 4;

    const int g = blockIdx.x % NGROUPS;
    const int rr = blockIdx.x / NGROUPS;
    const int h = g * HPG + rr % HPG;
    const int b = rr / HPG;
    const int batch = gridDim.x / NHEADS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int nch = (T + Q - 1) / Q;
    const float Dh = Dp[h];

    const uint32_t XROW = CONVDIM * 2, YROW = DINNER * YB;
    const char *xseq = reinterpret_cast<const char *>(xc + (size_t)b * T * CONVDIM);
    char *yseq = reinterpret_cast<char *>(y) + (size_t)b * T * YROW;
    auto rsrc = [](const char *p, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, (int)bytes, 0x00020000);
    };
    const int I0 = wave, I1 = 15 - wave;

    // A chunk's L2 operands, in registers: the C fragments of blocks I0 and I1 (B operand of
    // C S_in^T), the B fragments of the state update (state block = wave), the C.B^T pairs of
    // block I0 (at most 4) and I1 (at most 8).  The next chunk's B fragments and pairs are loaded
    // while this one is computed, each right after its register's last use here, so that the
    // chunk's L2 traffic spreads over its matrix-core work; its C fragments (not held through the
    // 32-row loop, for registers) after the loop.  Every load is unconditional (indices clamped
    // into the chunk's data): NL2 of them follow the next chunk's DMA.
    uint4 cf[2][4], bt[8], gp0[4], gp1[8];
    constexpr int NL2 = 8 + 8 + 4 + 8;
    struct Src {
        __amdgpu_buffer_rsrc_t rb, rg;
        uint32_t og0, og1;  // row-block offsets of the C.B^T pairs
        int ng0, ng1, nj1;  // last pair index of blocks I0 and I1, last 32-row step
    };
    auto src = [&](int ck) {
        const int L = min(Q, T - ck * Q), nb = (L + 15) >> 4;
        const size_t cb = (size_t)ck * batch * NGROUPS, grp = (size_t)b * NGROUPS + g;
        Src r;
        r.rb = rsrc(Bfw + cb * btf_bytes(Q) + grp * btf_bytes(L), (uint32_t)btf_bytes(L));
        r.rg = rsrc(reinterpret_cast<const char *>(Gw + cb_base(ck, Q, L, batch, b, g)), (uint32_t)cb_pairs(L) * 1024);
        const int Ia = min(I0, nb - 1), Ib = min(I1, nb - 1);
        r.og0 = (uint32_t)cb_pairs_before(Ia) * 1024;
        r.og1 = (uint32_t)cb_pairs_before(Ib) * 1024;
        r.ng0 = Ia >> 1;
        r.ng1 = Ib >> 1;
        r.nj1 = nj_of(L) - 1;
        return r;
    };
    const uint32_t vl = (uint32_t)lane * 16, vb = (uint32_t)(wave * 64 + lane) * 16;
    auto load_c = [&](int ck) {
        const int L = min(Q, T - ck * Q), nb = (L + 15) >> 4;
        const size_t cb = (size_t)ck * batch * NGROUPS, grp = (size_t)b * NGROUPS + g;
        const __amdgpu_buffer_rsrc_t rc = rsrc(Cfw + cb * cfr_bytes(Q) + grp * cfr_bytes(L), (uint32_t)cfr_bytes(L));
        const uint32_t oc0 = (uint32_t)min(I0, nb - 1) * 4096, oc1 = (uint32_t)min(I1, nb - 1) * 4096;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            cf[0][ks] = bload16(rc, vl, oc0 + 1024 * ks);
            cf[1][ks] = bload16(rc, vl, oc1 + 1024 * ks);
        }
    };
    auto load_b = [&](const Src &r, int jp) { bt[jp] = bload16(r.rb, vb, (uint32_t)min(jp, r.nj1) * 8192); };
    auto load_g0 = [&](const Src &r, int jp) { gp0[jp] = bload16(r.rg, vl, r.og0 + (uint32_t)min(jp, r.ng0) * 1024); };
    auto load_g1 = [&](const Src &r, int jp) { gp1[jp] = bload16(r.rg, vl, r.og1 + (uint32_t)min(jp, r.ng1) * 1024); };

    // x rows of chunk ck (head h's 160 bytes each) and its tables to LDS (Xd, Td): 5 DMA loads
    // of 1 KiB per wave for x (pieces 64 k + lane of 16 B, k = wave + 8 m; rows at or past L,
    // and every row of a chunk past the last, read as zero) and one for the tables (waves w and
    // w + 4 load the same KiB)
    auto dma = [&](int ck, uint16_t *Xd, uint32_t *Td) {
        const int t0 = ck * Q, L = ck < nch ? min(Q, T - t0) : 0;
        const __amdgpu_buffer_rsrc_t rx = rsrc(xseq + (size_t)min(t0, T - 1) * XROW, (uint32_t)L * XROW);
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const int k = wave + 8 * m, p = 64 * k + lane, row = p / 10, pc = p - 10 * row;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)&Xd[k * 512], 16,
                                                     (uint32_t)row * XROW + (uint32_t)(h * HDIM + 8 * pc) * 2, 0, 0, 0);
        }
        const int ckc = min(ck, nch - 1), Lc = min(Q, T - ckc * Q);
        const char *tb = Tw + (size_t)ckc * batch * NHEADS * tab_bytes(Q) + (size_t)(b * NHEADS + h) * tab_bytes(Lc);
        const __amdgpu_buffer_rsrc_t rt = rsrc(tb, ck < nch ? (uint32_t)tab_bytes(Lc) : 0u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_void *)&Td[(wave & 3) * 256], 16,
                                                 (uint32_t)((wave & 3) * 64 + lane) * 16, 0, 0, 0);
    };

    // State, as the transposed accumulator of the state update: st[pb] holds
    // S[16pb + l16][16 wave + 4q4 + r], r = 0..3 (four consecutive state columns of one row).
    floatx4 st[5];
    {
        const float *S0 = h0 ? h0 + ((size_t)b * NHEADS + h) * HDIM * DSTATE : nullptr;
#pragma unroll
        for (int pb = 0; pb < 5; ++pb) {
            const float4 v = S0 ? *reinterpret_cast<const float4 *>(&S0[(16 * pb + l16) * DSTATE + 16 * wave + 4 * q4])
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            st[pb] = floatx4{v.x, v.y, v.z, v.w};
        }
    }

    // outputs of blocks I0 and I1 of a chunk (Y^T, lane: column 16 I + l16, rows 16 pb + 4 q4 + r)
    floatx4 a0[5], a1[5];

    // y of chunk ck (the skip term is in the diagonal tiles).  bf16 output goes through the
    // wave's LDS rows so that each 16-byte store covers 8 consecutive columns of one row.  Called
    // at the start of the next chunk, while no DMA into LDS is in flight.
    auto store_y = [&](int ck) {
        const int t0 = ck * Q, L = min(Q, T - t0), nb = (L + 15) >> 4;
        const __amdgpu_buffer_rsrc_t ry = rsrc(yseq + (size_t)t0 * YROW, (uint32_t)L * YROW);
        auto store = [&](int I, const floatx4 *acc) {
            if (YT == BF16) {
                uint16_t *ys = Ys[wave];
#pragma unroll
                for (int pb = 0; pb < 5; ++pb)
                    *reinterpret_cast<uint2 *>(&ys[l16 * YS_LD + 16 * pb + 4 * q4]) =
                        make_uint2(pack_bf16x2(acc[pb][0], acc[pb][1]), pack_bf16x2(acc[pb][2], acc[pb][3]));
#pragma unroll
                for (int e = 0; e < 3; ++e) {
                    const int c = lane + 64 * e;  // 16-byte piece: row c / 10, columns 8 (c % 10) ..
                    if (c < 160) {
                        const int ri = c / 10, cc = c - 10 * ri;
                        const uint4 v = *reinterpret_cast<const uint4 *>(&ys[ri * YS_LD + 8 * cc]);
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), ry,
                            (uint32_t)(16 * I + ri) * YROW + (uint32_t)(h * HDIM + 8 * cc) * 2, 0, 0);
                    }
                }
            } else {
                const uint32_t rowoff = (uint32_t)(16 * I + l16) * YROW + (uint32_t)(h * HDIM + 4 * q4) * YB;
#pragma unroll
                for (int pb = 0; pb < 5; ++pb) {
                    const u32x4v w4 = {__float_as_uint(acc[pb][0]), __float_as_uint(acc[pb][1]),
                                       __float_as_uint(acc[pb][2]), __float_as_uint(acc[pb][3])};
                    __builtin_amdgcn_raw_buffer_store_b128(w4, ry, rowoff + 16 * pb * YB, 0, 0);
                }
            }
        };
        if (I0 < nb) store(I0, a0);
        if (I1 < nb) store(I1, a1);
    };

    // one chunk: reads x and the tables from (Xs, Tb), fills (Xn, Tn) with the next chunk
    auto chunk = [&](int ck, uint16_t *Xs, uint32_t *Tb, uint16_t *Xn, uint32_t *Tn) {
        const int t0 = ck * Q, L = min(Q, T - t0), nb = (L + 15) >> 4, NJ = nj_of(L), P = 32 * NJ;
        if (ck > 0) store_y(ck - 1);
        const Src nx = src(min(ck + 1, nch - 1));  // the last chunk re-loads its own operands, unused

        // ---- x to fp16 in place (rows < P; rows at or past L are zero), S_in, decay
        for (int e = tid; e < 10 * P; e += SC_THREADS) {
            uint4 *px = reinterpret_cast<uint4 *>(&Xs[8 * e]);
            *px = bf16x8_to_f16x8(*px);
        }
        const float *cum = reinterpret_cast<const float *>(Tb);
        const float *dtv = cum + P, *Fv = cum + 2 * P;
        const _Float16 *Wh = reinterpret_cast<const _Float16 *>(cum + 3 * P);
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
            *reinterpret_cast<uint2 *>(&Si[(16 * pb + l16) * SI_LD + 16 * wave + 4 * q4]) =
                make_uint2(pack_rne(st[pb][0], st[pb][1]), pack_rne(st[pb][2], st[pb][3]));
        const float dec = __builtin_amdgcn_exp2f(cum[P - 1]);
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[pb][r] *= dec;
        // the next chunk's DMA, after this wave's LDS writes of the chunk (with a DMA into LDS in
        // flight, the compiler would make them wait for it)
        __builtin_amdgcn_sched_barrier(0);
        dma(ck + 1, Xn, Tn);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();

        // ---- Y^T = S_in C^T for both blocks (S_in fragments shared), scaled by exp(cum_i)
        const bool v0 = I0 < nb, v1 = I1 < nb;
        const int ia0 = 16 * I0 + l16, ia1 = 16 * I1 + l16;
#pragma unroll
        for (int pb = 0; pb < 5; ++pb) {
            a0[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
            a1[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const half8 sf = ld_half8(&Si[(16 * pb + l16) * SI_LD + 32 * ks + 8 * q4]);
                a0[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf, __builtin_bit_cast(half8, cf[0][ks]), a0[pb], 0, 0, 0);
                if (v1) a1[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf, __builtin_bit_cast(half8, cf[1][ks]), a1[pb], 0, 0, 0);
            }
        }
        const float ci0 = cum[ia0], ci1 = v1 ? cum[ia1] : 0.f;
        {
            const float e0 = __builtin_amdgcn_exp2f(ci0), e1 = __builtin_amdgcn_exp2f(ci1);
#pragma unroll
            for (int pb = 0; pb < 5; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a0[pb][r] *= e0;
                    a1[pb][r] *= e1;
                }
        }

        // scaled C.B^T tiles (B operand: column i, k = j), as in k_ssd_scan
        auto offdiag = [&](float ci, int J, const uint32_t gx, const uint32_t gy) {
            const float eJ = __builtin_amdgcn_exp2f(ci - cum[16 * J + 15]);
            const float4 F = *reinterpret_cast<const float4 *>(&Fv[16 * J + 4 * q4]);
            const half2v f01 = __builtin_bit_cast(half2v, pack_rne(eJ * F.x, eJ * F.y));
            const half2v f23 = __builtin_bit_cast(half2v, pack_rne(eJ * F.z, eJ * F.w));
            const half2v m01 = __builtin_bit_cast(half2v, gx) * f01;
            const half2v m23 = __builtin_bit_cast(half2v, gy) * f23;
            return make_uint2(__builtin_bit_cast(uint32_t, m01), __builtin_bit_cast(uint32_t, m23));
        };
        auto diag = [&](float ci, int I, const uint32_t gx, const uint32_t gy) {
            const half2v lo = __builtin_bit_cast(half2v, gx), hi = __builtin_bit_cast(half2v, gy);
            const float gt[4] = {(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
            const float4 cj = *reinterpret_cast<const float4 *>(&cum[16 * I + 4 * q4]);
            const float4 dj = *reinterpret_cast<const float4 *>(&dtv[16 * I + 4 * q4]);
            const float cja[4] = {cj.x, cj.y, cj.z, cj.w}, dja[4] = {dj.x, dj.y, dj.z, dj.w};
            float m[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                m[r] = gt[r] * __builtin_amdgcn_exp2f(fminf(ci - cja[r], 0.f)) * dja[r] + (4 * q4 + r == l16 ? Dh : 0.f);
            return make_uint2(pack_rne(m[0], m[1]), pack_rne(m[2], m[3]));
        };
        // pair jp of block I: both tiles below the diagonal, or the pair that holds it
        auto pair = [&](float ci, int I, int jp, const uint4 gv) {
            uint2 ma, mb;
            if (jp < (I >> 1)) {
                ma = offdiag(ci, 2 * jp, gv.x, gv.y);
                mb = offdiag(ci, 2 * jp + 1, gv.z, gv.w);
            } else if (I & 1) {
                ma = offdiag(ci, I - 1, gv.x, gv.y);
                mb = diag(ci, I, gv.z, gv.w);
            } else {
                ma = diag(ci, I, gv.x, gv.y);
                mb = make_uint2(0u, 0u);
            }
            return __builtin_bit_cast(half8, make_uint4(ma.x, ma.y, mb.x, mb.y));
        };

        // ---- 32-row steps: x^T fragments (k = j in the order {4q + e, 16 + 4q + e}) feed the
        // state update and both output blocks; each operand register is re-loaded with the next
        // chunk's after its use
#pragma unroll
        for (int jp = 0; jp < 8; ++jp) {
            if (jp < NJ) {
                half8 xf[5];
#pragma unroll
                for (int pb = 0; pb < 5; ++pb)
                    xf[pb] = cat(ld_tr(Xs, XS_LD, 32 * jp + 4 * q4, 16 * pb), ld_tr(Xs, XS_LD, 32 * jp + 16 + 4 * q4, 16 * pb));
                const uint2 wlo = *reinterpret_cast<const uint2 *>(&Wh[32 * jp + 4 * q4]);
                const uint2 whi = *reinterpret_cast<const uint2 *>(&Wh[32 * jp + 16 + 4 * q4]);
                const half8 bw = __builtin_bit_cast(half8, bt[jp]) * cat(wlo, whi);
                // S^T += (w B)^T x: the B fragment is the A operand (rows: state columns), x the B
#pragma unroll
                for (int pb = 0; pb < 5; ++pb) st[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bw, xf[pb], st[pb], 0, 0, 0);
                if (jp < 4 && v0 && jp <= (I0 >> 1)) {
                    const half8 m = pair(ci0, I0, jp, gp0[jp < 4 ? jp : 0]);
#pragma unroll
                    for (int pb = 0; pb < 5; ++pb) a0[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf[pb], m, a0[pb], 0, 0, 0);
                }
                if (v1 && jp <= (I1 >> 1)) {
                    const half8 m = pair(ci1, I1, jp, gp1[jp]);
#pragma unroll
                    for (int pb = 0; pb < 5; ++pb) a1[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf[pb], m, a1[pb], 0, 0, 0);
                }
            }
            load_b(nx, jp);
            if (jp < 4) load_g0(nx, jp);
            load_g1(nx, jp);
        }
        load_c(min(ck + 1, nch - 1));

        // ---- this wave's share of the next chunk's DMA (issued before the NL2 loads above)
        wait_vm<NL2>();
        __syncthreads();
    };

    {
        const Src s0 = src(0);
        load_c(0);
#pragma unroll
        for (int jp = 0; jp < 8; ++jp) {
            load_b(s0, jp);
            if (jp < 4) load_g0(s0, jp);
            load_g1(s0, jp);
        }
    }
    dma(0, Xs0, Tab0);
    wait_vm<0>();
    __syncthreads();
#pragma unroll 1
    for (int ck = 0; ck < nch; ck += 2) {
        chunk(ck, Xs0, Tab0, Xs1, Tab1);
        if (ck + 1 < nch) chunk(ck + 1, Xs1, Tab1, Xs0, Tab0);
    }
    store_y(nch - 1);

    if (hT) {
        float *Sg = hT + ((size_t)b * NHEADS + h) * HDIM * DSTATE;
#pragma unroll
        for (int pb = 0; pb < 5; ++pb)
            *reinterpret_cast<float4 *>(&Sg[(16 * pb + l16) * DSTATE + 16 * wave + 4 * q4]) =
                make_float4(st[pb][0], st[pb][1], st[pb][2], st[pb][3]);
    }
}

static bool use_scanx(int T, int Q) { return Q >= XQ_MIN && T >= XT_MIN; }

static size_t cb_ws_bytes(int batch, int T, int Q)
{
    const int full = T / Q, last = T - full * Q;
    const size_t pairs = (size_t)full * cb_pairs(Q) + (last ? cb_pairs(last) : 0);
    return (size_t)batch * NGROUPS * pairs * 512 * sizeof(uint16_t);
}

size_t ssd_scan_ws_bytes(int batch, int T, int Q)
{
    size_t n = cb_ws_bytes(batch, T, Q);
    if (use_scanx(T, Q)) {
        const int full = T / Q, last = T - full * Q;
        n += (size_t)batch * NGROUPS * ((size_t)full * btf_bytes(Q) + (last ? btf_bytes(last) : 0));
        n += (size_t)batch * NGROUPS * ((size_t)full * cfr_bytes(Q) + (last ? cfr_bytes(last) : 0));
        n += (size_t)batch * NHEADS * ((size_t)full * tab_bytes(Q) + (last ? tab_bytes(last) : 0));
    }
    return n;
}

// the kernel with its dynamic LDS limit raised once (above 64 KiB it must be set explicitly)
template <class K>
static hipError_t raise_lds(K kern, size_t smem, bool &done)
{
    if (done) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess) done = true;
    return e;
}

hipError_t launch_ssd_scan(const uint16_t *xc, const uint16_t *dtr, long ld_dt, int T, int Q,
                           const float *dt_bias, const float *A_log, const float *D,
                           const float *h0, float *hT, void *y, int y_t, int batch, uint16_t *Gws,
                           hipStream_t st)
{
    const int nch = (T + Q - 1) / Q;
    const dim3 grid(batch * NHEADS), block(SC_THREADS);
    if (use_scanx(T, Q)) {
        char *Bf = reinterpret_cast<char *>(Gws) + cb_ws_bytes(batch, T, Q);
        const int full = T / Q, last = T - full * Q;
        char *Cf = Bf + (size_t)batch * NGROUPS * ((size_t)full * btf_bytes(Q) + (last ? btf_bytes(last) : 0));
        char *Tb = Cf + (size_t)batch * NGROUPS * ((size_t)full * cfr_bytes(Q) + (last ? cfr_bytes(last) : 0));
        k_ssd_cb<true><<<dim3(nch, NGROUPS, batch * 2), CB_THREADS, 0, st>>>(xc, T, Q, Gws, dtr, ld_dt, dt_bias, A_log,
                                                                          Bf, Cf, Tb);
        if (y_t == BF16)
            k_ssd_scanx<BF16><<<grid, block, 0, st>>>(xc, T, Q, D, h0, hT, y, Gws, Bf, Cf, Tb);
        else
            k_ssd_scanx<F32><<<grid, block, 0, st>>>(xc, T, Q, D, h0, hT, y, Gws, Bf, Cf, Tb);
        return hipGetLastError();
    }
    k_ssd_cb<false><<<dim3(nch, NGROUPS, batch), CB_THREADS, 0, st>>>(xc, T, Q, Gws, nullptr, 0, nullptr, nullptr,
                                                                       nullptr, nullptr, nullptr);
    const size_t smem = sizeof(ScanSmem);
    static bool set[2] = {false, false};
    if (y_t == BF16) {
        const hipError_t e = raise_lds(k_ssd_scan<BF16>, smem, set[0]);
        if (e != hipSuccess) return e;
        k_ssd_scan<BF16><<<grid, block, smem, st>>>(xc, dtr, ld_dt, T, Q, dt_bias, A_log, D, h0, hT, y, Gws);
    } else {
        const hipError_t e = raise_lds(k_ssd_scan<F32>, smem, set[1]);
        if (e != hipSuccess) return e;
        k_ssd_scan<F32><<<grid, block, smem, st>>>(xc, dtr, ld_dt, T, Q, dt_bias, A_log, D, h0, hT, y, Gws);
    }
    return hipGetLastError();
}

}  // namespace nh
