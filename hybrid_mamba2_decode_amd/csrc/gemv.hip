// gemv.hip -- W4 dequantising matrix-vector products of the per-position block on gfx950.
//
// The per-position block streams 82.9 MB of packed 4-bit weights per layer and does a few
// hundred MFLOP, so it is bound by HBM; the aim is every weight byte read exactly once with
// 128-bit loads, enough bytes in flight per CU to cover HBM latency, and a dequantisation
// cheap enough in VALU issue slots to hide under the loads.
//
// Layout.  LPR lanes own one output row (LPR = 32 or 64), so a wave works on 64/LPR rows at
// a time; lane li of a row handles 16-byte chunks (32 nibbles, half a quantisation group)
// c = li, li + LPR, ...  Its activations are the same for every row it visits, so they are
// staged once per work-group in LDS and then held in registers for the whole kernel.
//
// Dequantisation.  For a packed word w (nibbles q0..q7 of k = 8j .. 8j+7), with the fp16
// magic 0x6400 (1024.0, whose unit in the last place is 1):
//   (w      & 0x000F000F) | 0x64006400 = fp16 pair (1024 + q0,    1024 + q4)
//   (w      & 0x00F000F0) | 0x64006400 = fp16 pair (1024 + 16 q1, 1024 + 16 q5)
//   (w >> 8 & 0x000F000F) | 0x64006400 = fp16 pair (1024 + q2,    1024 + q6)
//   (w >> 8 & 0x00F000F0) | 0x64006400 = fp16 pair (1024 + 16 q3, 1024 + 16 q7)
// i.e. one shift and four v_and_or_b32 per word; v_dot2_f32_f16 multiplies each pair with the
// matching activation pair (fp16 holds the bf16 activations exactly).  With dA collecting the
// even k and dB the odd k of a chunk,
//   sum_k q_k x_k = dA + dB / 16 - (1024 sum_even x + 64 sum_odd x)
// and the affine map W = s q + b of the chunk's group adds s * that + b * sum x.
// Every product is exact and accumulation is fp32.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

#include <type_traits>

namespace nh {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}

// The same operation in plain code, for results that feed a matrix-core instruction: a VALU
// write of a register that an MFMA then reads as its A or B operand needs two wait states,
// which the compiler inserts only for instructions it can see (not for inline assembly).
__device__ __forceinline__ uint32_t and_or_mf(uint32_t a, uint32_t m, uint32_t c) { return (a & m) | c; }

// A value the compiler keeps in a vector register without knowing it (so that and_or_mf of two
// such masks is one v_and_or_b32: with constants it takes two instructions).
__device__ __forceinline__ uint32_t opaque_v(uint32_t x)
{
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// Sum over aligned groups of LPR lanes (LPR = 16, 32 or 64), in every lane of the group.
template <int LPR>
__device__ __forceinline__ float row_sum(float v)
{
    static_assert(LPR == 16 || LPR == 32 || LPR == 64, "row_sum: 16, 32 or 64 lanes");
    v = row16_sum(v);
    if (LPR >= 32) v = xor16_sum(v);
    if (LPR >= 64) v = xor32_sum(v);
    return v;
}

// Activations of one 16-byte chunk: 16 fp16 pairs (k, k+4) in extraction order, the offset
// 1024 sum_even + 64 sum_odd, and the plain sum.  A scaled chunk (make_chunk_scaled) holds its
// values times 2^-k and mul = 2^k, which the consumer applies to the chunk's dot product.
struct ActChunk {
    uint32_t p[16];
    float off, sum, mul;
};
constexpr int ACT_WORDS = 20;  // 80-byte slots: 16-byte reads, conflict-free across lanes

// Build one chunk from 32 bf16-exact floats v[0..31] into its 80-byte LDS slot (16-byte
// aligned: five 16-byte writes).
__device__ __forceinline__ void make_chunk(const float *v, uint32_t *dst)
{
    float se = 0.f, so = 0.f;
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = v[8 * j + e], hi = v[8 * j + e + 4];
            w[4 * j + e] = pack_f16x2(lo, hi);
            if (e & 1) so += lo + hi; else se += lo + hi;
        }
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int j = 0; j < 4; ++j) d4[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
    d4[4] = make_uint4(__float_as_uint(fmaf(1024.f, se, 64.f * so)), __float_as_uint(se + so), 0x3F800000u, 0u);
}

// A chunk of any bf16 values: the 32 values are scaled by 2^-k so that the largest magnitude m
// lies in [2^14, 2^15) (k = floor(log2 m) - 14, kept in [-100, 113]); the scaling is exact, every
// bf16 value of the chunk down to 2^-31 m is exact in fp16, and mul = 2^k restores the scale in
// fp32 after the dot products.  Relative rounding is the same as for an unscaled chunk.
__device__ __forceinline__ void make_chunk_scaled(const float *v, uint32_t *dst)
{
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(v[e]));
    const int ex = (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127;
    const int k = min(max(ex - 14, -100), 113);
    const float inv = __uint_as_float((uint32_t)(127 - k) << 23), mul = __uint_as_float((uint32_t)(127 + k) << 23);
    float u[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) u[e] = v[e] * inv;
    make_chunk(u, dst);
    dst[18] = __float_as_uint(mul);
}

// The raw words of one 32-value chunk of x (bf16 bits or fp32), loaded as they are (so that a
// caller can issue the loads early and unpack later); fp32 values are rounded to bf16 when
// unpacked, the GEMV's activation precision.
template <int XT>
struct XChunk {
    static constexpr int NW = XT == BF16 ? 4 : 8;
    uint4 r[NW];
    __device__ __forceinline__ void load(const void *x, size_t chunk)
    {
        const uint4 *src = XT == BF16
            ? reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + chunk * 32)
            : reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(x) + chunk * 32);
#pragma unroll
        for (int j = 0; j < NW; ++j) r[j] = src[j];
    }
    __device__ __forceinline__ void unpack(float (&v)[32]) const
    {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const uint4 w = r[j];
            if constexpr (XT == BF16) {
                v[8 * j + 0] = bf16lo(w.x); v[8 * j + 1] = bf16hi(w.x); v[8 * j + 2] = bf16lo(w.y);
                v[8 * j + 3] = bf16hi(w.y); v[8 * j + 4] = bf16lo(w.z); v[8 * j + 5] = bf16hi(w.z);
                v[8 * j + 6] = bf16lo(w.w); v[8 * j + 7] = bf16hi(w.w);
            } else {
                v[4 * j + 0] = round_bf16(__uint_as_float(w.x)); v[4 * j + 1] = round_bf16(__uint_as_float(w.y));
                v[4 * j + 2] = round_bf16(__uint_as_float(w.z)); v[4 * j + 3] = round_bf16(__uint_as_float(w.w));
            }
        }
    }
};

template <int LPR>
struct GemvShape {
    static constexpr int RPG = 64 / LPR;  // rows per wave-instruction
};

// Values an epilogue loads one stage ahead, kept exactly as loaded (16-bit values as 16-bit
// values, so not even a zero-extension is attached to the load): arithmetic on them before their
// stage is computed would make the wave wait for every load issued before them, the next
// stage's weights included.  Loads are unconditional for the same reason (a branch would make
// the compiler's waits conservative where the paths join).
struct EpiPre {
    uint16_t h[4];
    uint32_t w[2];
};

// y[b][n] = acc + res[b][n]
struct EpiStore {
    void *y;
    const void *res;
    int y_t, res_t, n;
    // The residual is read through one buffer resource per dtype; the one not in use (and both
    // when there is no residual) has no records, so its load returns zero without touching memory.
    __device__ __forceinline__ EpiPre prefetch(int row, int b) const
    {
        const uint32_t i = (uint32_t)(b * n + row);
        const auto r16 = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(res), 0,
                                                           (res && res_t == BF16) ? 0x7FFFFFFF : 0, 0x00020000);
        const auto r32 = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(res), 0,
                                                           (res && res_t != BF16) ? 0x7FFFFFFF : 0, 0x00020000);
        EpiPre p;
        p.h[0] = __builtin_amdgcn_raw_buffer_load_b16(r16, 2u * i, 0, 0);
        p.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r32, 4u * i, 0, 0);
        return p;
    }
    __device__ __forceinline__ void operator()(int row, int b, float v, const EpiPre &p) const
    {
        const size_t i = (size_t)b * n + row;
        v += res_t == BF16 ? bf16lo(p.h[0]) : __uint_as_float(p.w[0]);
        if (y_t == BF16)
            reinterpret_cast<uint16_t *>(y)[i] = f32_to_bf16(v);
        else
            reinterpret_cast<float *>(y)[i] = v;
    }
};

// in_proj rows of the per-position block: z | xBC | dt_raw.  The in_proj output is a bf16
// storage point; xBC channels immediately run the causal conv step (state row 0 oldest,
// tap 3 newest) and SiLU, and the conv state shifts by one position.  The conv state, taps
// and bias of a row are prefetched together with the row's weights.
struct EpiInProjStep {
    uint16_t *z, *xc, *dtr, *cs;
    const uint16_t *cw, *cb;
    __device__ __forceinline__ EpiPre prefetch(int n, int b) const
    {
        const int c = min(max(n - DINNER, 0), CONVDIM - 1);
        const uint16_t *st = cs + (size_t)b * (CONVK - 1) * CONVDIM + c;
        const uint2 w = *reinterpret_cast<const uint2 *>(cw + 4 * (size_t)c);
        EpiPre p;
        p.h[0] = st[0];
        p.h[1] = st[CONVDIM];
        p.h[2] = st[2 * CONVDIM];
        p.h[3] = cb[c];
        p.w[0] = w.x;
        p.w[1] = w.y;
        return p;
    }
    __device__ __forceinline__ void operator()(int n, int b, float acc, const EpiPre &p) const
    {
        const uint16_t vb = f32_to_bf16(acc);
        if (n < DINNER) {
            z[(size_t)b * DINNER + n] = vb;
        } else if (n < DINNER + CONVDIM) {
            const int c = n - DINNER;
            uint16_t *st = cs + (size_t)b * (CONVK - 1) * CONVDIM + c;
            float a = bf16lo(p.h[3]);
            a = fmaf(bf16lo(p.w[0]), bf16lo(p.h[0]), a);
            a = fmaf(bf16hi(p.w[0]), bf16lo(p.h[1]), a);
            a = fmaf(bf16lo(p.w[1]), bf16lo(p.h[2]), a);
            a = fmaf(bf16hi(p.w[1]), bf16_to_f32(vb), a);
            xc[(size_t)b * CONVDIM + c] = f32_to_bf16(silu(a));
            st[0] = p.h[1];
            st[CONVDIM] = p.h[2];
            st[2 * CONVDIM] = vb;
        } else {
            dtr[(size_t)b * NHEADS + (n - DINNER - CONVDIM)] = vb;
        }
    }
};

// MLP up projection: h[b][n] = bf16(relu(acc)^2), the activation between the two projections.
struct EpiReluSq {
    uint16_t *h;
    int n;
    __device__ __forceinline__ EpiPre prefetch(int, int) const { return EpiPre{}; }
    __device__ __forceinline__ void operator()(int row, int b, float acc, const EpiPre &) const
    {
        const float r = fmaxf(acc, 0.f);
        h[(size_t)b * n + row] = f32_to_bf16(r * r);
    }
};

// One pipeline stage: RG row groups of 64/LPR rows, CPL chunks per lane.
template <int RG, int CPL>
struct Stage {
    uint4 q[RG][CPL];
    uint16_t s[RG][CPL], b[RG][CPL];  // bf16 bits, widened where used
};

template <int RG, int CPL>
__device__ __forceinline__ void load_stage(Stage<RG, CPL> &st, __amdgpu_buffer_rsrc_t rq,
                                           __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rb,
                                           const uint32_t *qoff, const uint32_t *soff, uint32_t row0,
                                           uint32_t rpg, uint32_t rowbytes, uint32_t kg2)
{
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const uint32_t row = row0 + r * rpg;
        const uint32_t qb = row * rowbytes, sb = row * kg2;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            st.q[r][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[i] + qb, 0, 0));
            st.s[r][i] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[i] + sb, 0, 0);
            st.b[r][i] = __builtin_amdgcn_raw_buffer_load_b16(rb, soff[i] + sb, 0, 0);
        }
    }
}

// One 16-byte chunk of a row against its activations: acc + s * (q . a) + b * sum(a).
template <bool SC = false>
__device__ __forceinline__ float chunk_dot(uint4 q, uint32_t sbits, uint32_t bbits, const ActChunk &a, float acc,
                                           uint32_t mlo, uint32_t mhi, uint32_t magic)
{
    const uint32_t wq[4] = {q.x, q.y, q.z, q.w};
    float dA = 0.f, dB = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = wq[j], wh = w >> 8;
        dA = dot2h(and_or(w, mlo, magic), a.p[4 * j + 0], dA);
        dB = dot2h(and_or(w, mhi, magic), a.p[4 * j + 1], dB);
        dA = dot2h(and_or(wh, mlo, magic), a.p[4 * j + 2], dA);
        dB = dot2h(and_or(wh, mhi, magic), a.p[4 * j + 3], dB);
    }
    const float t = fmaf(dB, 0.0625f, dA) - a.off;
    const float sc = __uint_as_float(sbits << 16), bi = __uint_as_float(bbits << 16);
    if constexpr (SC)
        return fmaf(fmaf(sc, t, bi * a.sum), a.mul, acc);
    else
        return fmaf(sc, t, fmaf(bi, a.sum, acc));
}

template <int LPR, int CPL, int NB, int RG, class Epi, bool SC>
__device__ __forceinline__ void compute_stage(const Stage<RG, CPL> &st, const ActChunk (&a)[NB][CPL],
                                              const Epi &epi, const EpiPre &pre, int row0, int n_out,
                                              int li, uint32_t mlo, uint32_t mhi, uint32_t magic)
{
    constexpr int RPG = GemvShape<LPR>::RPG;
    float acc[RG][NB];
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                s = chunk_dot<SC>(st.q[r][i], st.s[r][i], st.b[r][i], a[b][i], s, mlo, mhi, magic);
            acc[r][b] = row_sum<LPR>(s);
        }
    // lane li = r*NB + b of each row finishes (row, b); rows are row0 + r*RPG
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (li == r * NB + b) v = acc[r][b];
    const int er = li / NB, eb = li % NB;
    const int row = row0 + er * RPG;
    if (li < RG * NB && row < n_out) epi(row, eb, v, pre);
}

// One activation chunk from its 80-byte LDS slot (five 16-byte reads).
__device__ __forceinline__ void chunk_from_lds(ActChunk &a, const uint32_t *src)
{
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 w = s4[j];
        a.p[4 * j] = w.x;
        a.p[4 * j + 1] = w.y;
        a.p[4 * j + 2] = w.z;
        a.p[4 * j + 3] = w.w;
    }
    const uint4 t = s4[4];
    a.off = __uint_as_float(t.x);
    a.sum = __uint_as_float(t.y);
    a.mul = __uint_as_float(t.z);
}

// Activations staged in LDS: [NB][nch][ACT_WORDS] words.
template <int LPR, int CPL, int NB>
__device__ __forceinline__ void act_from_lds(ActChunk (&a)[NB][CPL], const uint32_t *lds, int nch, int li)
{
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = li + LPR * i;
            if (c < nch) {
                chunk_from_lds(a[b][i], lds + ((size_t)b * nch + c) * ACT_WORDS);
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) a[b][i].p[j] = 0u;
                a[b][i].off = 0.f;
                a[b][i].sum = 0.f;
                a[b][i].mul = 1.f;
            }
        }
}

// The streaming loop.  Construction issues the first stage's loads, so a kernel can build
// its activations (LDS staging, pre-norm, gated norm) while those loads are in flight.
// SC: the activations are scaled chunks (make_chunk_scaled).
template <int LPR, int CPL, int NB, int RG, class Epi, bool SC = false>
struct GemvRunner {
    static constexpr int RPG = GemvShape<LPR>::RPG;
    static constexpr int ROWS = RG * RPG;  // rows per wave per stage
    const W4 W;
    const Epi epi;
    int sub, li, er, eb, stride, n0, nlim;
    uint32_t rowbytes, kg2, qoff[CPL], soff[CPL];
    __amdgpu_buffer_rsrc_t rq, rs, rb;
    Stage<RG, CPL> A, B;
    EpiPre pa, pb;

    // threads: the work-group size, a compile-time constant at every call site (blockDim would
    // be a load from the dispatch arguments whose wait also covers every load issued before it)
    // issue_now false: the first stage is left for issue_first() (a caller whose wave has other
    // loads to receive first)
    __device__ __forceinline__ GemvRunner(const W4 &W_, const Epi &epi_, int threads, bool issue_now = true)
        : W(W_), epi(epi_)
    {
        const int lane = threadIdx.x & 63;
        sub = lane / LPR;
        li = lane % LPR;
        // Rows are split into one contiguous slab per XCD (work-group i runs on XCD i mod 8), so
        // the cache lines that neighbouring rows share (row boundaries of the packed weights and
        // of the 140-byte scale rows) are fetched by one L2 only.  Inside a slab the XCD's waves
        // are numbered across work-groups first, so the leftover rows of an uneven split land one
        // per work-group.
        const int nx = (gridDim.x & 7) == 0 ? 8 : 1;
        const int xcd = blockIdx.x % nx;
        const int wave = __builtin_amdgcn_readfirstlane(
            (int)((threadIdx.x >> 6) * (gridDim.x / nx) + blockIdx.x / nx));
        const int nwaves = (gridDim.x / nx) * (threads >> 6);
        const int slab = (((W.n + nx - 1) / nx + ROWS - 1) / ROWS) * ROWS;
        const int nch = W.k >> 5;
        rowbytes = (uint32_t)W.k / 2;
        kg2 = (uint32_t)(W.k >> 6) * 2;
        rq = __builtin_amdgcn_make_buffer_rsrc((void *)W.q, 0, (int)((uint32_t)W.n * rowbytes), 0x00020000);
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)W.s, 0, (int)((uint32_t)W.n * kg2), 0x00020000);
        rb = __builtin_amdgcn_make_buffer_rsrc((void *)W.b, 0, (int)((uint32_t)W.n * kg2), 0x00020000);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t c = (uint32_t)min(li + LPR * i, nch - 1);
            qoff[i] = sub * rowbytes + 16u * c;
            soff[i] = sub * kg2 + 2u * (c >> 1);
        }
        er = min(li / NB, RG - 1);
        eb = li % NB;
        stride = nwaves * ROWS;
        n0 = xcd * slab + wave * ROWS;
        nlim = min(W.n, (xcd + 1) * slab);
        // unconditional (rows past the matrix read zero through the buffer range check): a
        // branch here would make the compiler's wait before the first use of any earlier load
        // also cover this stage's loads
        if (issue_now) issue_first();
    }

    __device__ __forceinline__ void issue_first()
    {
        load_stage<RG, CPL>(A, rq, rs, rb, qoff, soff, (uint32_t)min(n0, W.n), RPG, rowbytes, kg2);
        pa = epi.prefetch(min(n0 + er * RPG + sub, W.n - 1), eb);
    }

    __device__ __forceinline__ void run(const ActChunk (&a)[NB][CPL])
    {
        const uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
        if (n0 >= nlim) return;
        auto ld = [&](Stage<RG, CPL> &st, EpiPre &pe, int n) {
            load_stage<RG, CPL>(st, rq, rs, rb, qoff, soff, (uint32_t)n, RPG, rowbytes, kg2);
            pe = epi.prefetch(min(n + er * RPG + sub, W.n - 1), eb);
        };
        // The loop body holds no conditional load: the compiler's wait before a stage's first use
        // then counts exactly the next stage's loads (where a conditional load's path joins, it
        // would wait for everything).  Scheduling barriers keep those first uses inside the
        // compute blocks.  The last one or two stages are peeled.
        const int nst = (nlim - n0 + stride - 1) / stride;  // stages of this wave, A holds the first
        int n = n0, i = 0;
        for (; i + 2 < nst; i += 2, n += 2 * stride) {
            ld(B, pb, n + stride);
            __builtin_amdgcn_sched_barrier(0);
            compute_stage<LPR, CPL, NB, RG, Epi, SC>(A, a, epi, pa, n + sub, nlim, li, mlo, mhi, magic);
            ld(A, pa, n + 2 * stride);
            __builtin_amdgcn_sched_barrier(0);
            compute_stage<LPR, CPL, NB, RG, Epi, SC>(B, a, epi, pb, n + stride + sub, nlim, li, mlo, mhi, magic);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (i + 1 < nst) {
            ld(B, pb, n + stride);
            __builtin_amdgcn_sched_barrier(0);
            compute_stage<LPR, CPL, NB, RG, Epi, SC>(A, a, epi, pa, n + sub, nlim, li, mlo, mhi, magic);
            __builtin_amdgcn_sched_barrier(0);
            compute_stage<LPR, CPL, NB, RG, Epi, SC>(B, a, epi, pb, n + stride + sub, nlim, li, mlo, mhi, magic);
        } else {
            compute_stage<LPR, CPL, NB, RG, Epi, SC>(A, a, epi, pa, n + sub, nlim, li, mlo, mhi, magic);
        }
    }
};

// The in_proj rows have K = 4480, i.e. 140 chunks, which do not split evenly over 64 lanes.
// Lane l covers chunks l and l + 64 of every row (128 chunks); the remaining 12 chunks of R
// rows are covered by one further load in which lane l takes chunk 128 + l % 12 of row l / 12
// (lanes 12 R .. 63 idle, with zero activations).  A stage of R rows thus needs 2R + 1 loads
// per lane instead of 3R.
//
// Each wave owns one contiguous block of RW = R NS rows (NS stages, fully unrolled, two stages
// in flight).  Row results collect in lanes (one lane per row and batch row), and the
// epilogue, with its conv-state prefetch, runs once per wave at the end: no stores sit among
// the streaming loads, and the epilogue's branches are uniform (block boundaries are multiples
// of 8, as are the z | xBC | dt_raw boundaries).
constexpr int IP_NCH = HIDDEN / 32;       // 140
constexpr int IP_TAIL = IP_NCH - 128;     // 12
constexpr uint32_t IP_ROWB = HIDDEN / 2;  // packed bytes per row
constexpr uint32_t IP_GRPB = HIDDEN / 32; // scale bytes per row (70 bf16)

template <int R>
struct IpStage {
    uint4 q[R][2], qt;
    uint16_t s[R][2], b[R][2], st, bt;  // bf16 bits, widened where used
};

template <int NB>
struct InProjShape {
    static constexpr int R = NB == 1 ? 2 : 1;        // rows per stage
    static constexpr int NS = NB == 1 ? 4 : 8;       // stages per wave
    static constexpr int RW = R * NS;                // rows per wave
    static constexpr int NT = NB == 1 ? 768 : 256;   // threads per work-group
    static_assert(IP_TAIL * R <= 64 && RW * NB <= 64, "stage or block too large for one wave");
};

// Work-groups run on XCD (index mod 8); the blocks are split into one contiguous range per XCD.
template <int NB>
static inline int inproj_grid(int n)
{
    using S = InProjShape<NB>;
    const int nblk = (n + S::RW - 1) / S::RW, bx = (nblk + 7) / 8, wpg = S::NT / 64;
    return 8 * ((bx + wpg - 1) / wpg);
}

// Cache policy of the packed-weight loads of the K = 4480 kernels: non-temporal.  Each weight
// byte is read once per call.  Measured over working sets well beyond the 256 MB last-level
// cache (27 layers, 2.4 GB; four heads, 2.6 GB): in_proj 4% and the head 8% faster than with
// the plain policy.  Over smaller rotations the gain looks larger (the cache then keeps part
// of the rotation), which is not the per-position decode's case.
constexpr int NT_LOAD = 2;  // the nt bit of the buffer instructions' cache-policy operand

// Loads and row sums of R-row stages in the K = 4480 chunk layout above.  Rows past the
// matrix are clamped to its last row (a branch would make the compiler's waits conservative).
template <int R>
struct IpRows {
    int li, nmax, rt;
    uint32_t toff, tsoff;
    __amdgpu_buffer_rsrc_t rq, rs, rbias;

    __device__ __forceinline__ void init(const W4 &W)
    {
        li = threadIdx.x & 63;
        nmax = W.n - 1;
        rq = __builtin_amdgcn_make_buffer_rsrc((void *)W.q, 0, (int)((uint32_t)W.n * IP_ROWB), 0x00020000);
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)W.s, 0, (int)((uint32_t)W.n * IP_GRPB), 0x00020000);
        rbias = __builtin_amdgcn_make_buffer_rsrc((void *)W.b, 0, (int)((uint32_t)W.n * IP_GRPB), 0x00020000);
        rt = min(li / IP_TAIL, R - 1);
        const uint32_t tc = 128u + (uint32_t)(li % IP_TAIL);
        toff = 16u * tc;
        tsoff = 2u * (tc >> 1);
    }

    __device__ __forceinline__ void load(IpStage<R> &g, int n) const
    {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t row = (uint32_t)min(n + r, nmax);  // wave-uniform
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                g.q[r][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rq, 16u * (li + 64 * i), row * IP_ROWB, NT_LOAD));
                g.s[r][i] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2u * ((li + 64 * i) >> 1), row * IP_GRPB, 0);
                g.b[r][i] = __builtin_amdgcn_raw_buffer_load_b16(rbias, 2u * ((li + 64 * i) >> 1), row * IP_GRPB, 0);
            }
        }
        const uint32_t trow = (uint32_t)min(n + rt, nmax);
        g.qt = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, trow * IP_ROWB + toff, 0, NT_LOAD));
        g.st = __builtin_amdgcn_raw_buffer_load_b16(rs, trow * IP_GRPB + tsoff, 0, 0);
        g.bt = __builtin_amdgcn_raw_buffer_load_b16(rbias, trow * IP_GRPB + tsoff, 0, 0);
    }

    // the R row sums of a stage for every batch row, complete in every lane
    template <int NB>
    __device__ __forceinline__ void sums(const IpStage<R> &g, const ActChunk (&am)[NB][2],
                                         const ActChunk (&at)[NB], float (&out)[R][NB]) const
    {
        const uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
        float tail[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) tail[b] = chunk_dot(g.qt, g.st, g.bt, at[b], 0.f, mlo, mhi, magic);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float s = rt == r ? tail[b] : 0.f;
                s = chunk_dot(g.q[r][0], g.s[r][0], g.b[r][0], am[b][0], s, mlo, mhi, magic);
                s = chunk_dot(g.q[r][1], g.s[r][1], g.b[r][1], am[b][1], s, mlo, mhi, magic);
                out[r][b] = row_sum<64>(s);
            }
    }
};

template <int NB, class Epi = EpiInProjStep, class S = InProjShape<NB>>
struct InProjBlock {
    static constexpr int R = S::R, NS = S::NS, RW = S::RW;
    const Epi epi;
    IpRows<R> io;
    int rb;
    bool active;
    IpStage<R> st[2];
    EpiPre pe;

    // stage k of the block: its R row sums go to lanes (k R + r) NB + b
    __device__ __forceinline__ void compute(const IpStage<R> &g, int k, const ActChunk (&am)[NB][2],
                                            const ActChunk (&at)[NB], float &v) const
    {
        float sm[R][NB];
        io.template sums<NB>(g, am, at, sm);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (io.li == (k * R + r) * NB + b) v = sm[r][b];
    }

    // Issues the epilogue prefetch and the first stage (unconditionally, rows clamped: a
    // branch here would make the compiler's wait before the first use of any earlier load
    // also cover these loads; idle waves read the last row, which the cache holds).
    __device__ __forceinline__ InProjBlock(const W4 &W, const Epi &e) : epi(e)
    {
        io.init(W);
        const int xcd = blockIdx.x & 7;
        const int wave = __builtin_amdgcn_readfirstlane(
            (int)((threadIdx.x >> 6) * (gridDim.x >> 3) + (blockIdx.x >> 3)));
        const int nblk = (W.n + RW - 1) / RW, bx = (nblk + 7) / 8;
        const int blk = xcd * bx + wave;
        active = wave < bx && blk < nblk;
        rb = min(blk, nblk - 1) * RW;
        io.load(st[0], rb);
        pe = epi.prefetch(min(rb + min(io.li / NB, RW - 1), io.nmax), io.li % NB);
    }

    // a block whose first row and activity the caller chose (rows past the matrix are clamped)
    __device__ __forceinline__ InProjBlock(const W4 &W, const Epi &e, int row0, bool act) : epi(e)
    {
        io.init(W);
        active = act;
        rb = row0;
        io.load(st[0], rb);
        pe = epi.prefetch(min(rb + min(io.li / NB, RW - 1), io.nmax), io.li % NB);
    }

    __device__ __forceinline__ void run(const ActChunk (&am)[NB][2], const ActChunk (&at)[NB])
    {
        if (!active) return;
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            if (k + 1 < NS) io.load(st[(k + 1) & 1], rb + (k + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            compute(st[k & 1], k, am, at, v);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int row = rb + io.li / NB;
        if (io.li < RW * NB && row <= io.nmax) epi(row, io.li % NB, v, pe);
    }
};

// Pre-norm of the per-position kernels whose K is the hidden size.  Four threads build each
// 32-value chunk: item i = 4 c + j (chunk c, quarter j) covers values 8 j .. 8 j + 7 of chunk c of
// every batch row, i.e. the packed pairs p[4 j .. 4 j + 3], and the quarter's share of the chunk
// sums, which the four consecutive lanes add up.  issue() sends the raw loads (a wave's loads
// complete in issue order, so issued before the caller's weight stages they are all the
// pre-norm waits for); finish() sums the squares over the work-group and writes
// u = bf16(x / rms(x) * w) to LDS in the activation format.
template <int NB, int XT, int NT>
struct PreNorm {
    static constexpr int NCH = HIDDEN / 32, NI = 4 * NCH, NW = NT / 64;
    static constexpr int M = (NI + NT - 1) / NT;     // items per thread
    static constexpr int XW = XT == BF16 ? 1 : 2;    // 16-byte words per 8 values
    uint4 xr[M][NB][XW], wq[M];

    // item m of this thread (rows past the last item re-read it: unconditional loads)
    __device__ __forceinline__ static int item(int m) { return min((int)threadIdx.x + NT * m, NI - 1); }

    __device__ __forceinline__ void issue(const void *x, const uint16_t *nw)
    {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int it = item(m);
            wq[m] = *reinterpret_cast<const uint4 *>(nw + 8 * it);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int w = 0; w < XW; ++w)
                    xr[m][b][w] = XT == BF16
                        ? *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + (size_t)b * HIDDEN + 8 * it)
                        : *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(x) + (size_t)b * HIDDEN + 8 * it + 4 * w);
        }
    }

    // value e (0..7) of item m, batch row b
    __device__ __forceinline__ float xval(int m, int b, int e) const
    {
        if (XT == BF16) {
            const uint4 r = xr[m][b][0];
            const uint32_t u = e < 2 ? r.x : e < 4 ? r.y : e < 6 ? r.z : r.w;
            return (e % 2) == 0 ? bf16lo(u) : bf16hi(u);
        } else {
            const uint4 r = xr[m][b][e / 4];
            return __uint_as_float((e % 4) == 0 ? r.x : (e % 4) == 1 ? r.y : (e % 4) == 2 ? r.z : r.w);
        }
    }
    __device__ __forceinline__ float wval(int m, int e) const
    {
        const uint4 r = wq[m];
        const uint32_t u = e < 2 ? r.x : e < 4 ? r.y : e < 6 ? r.z : r.w;
        return (e % 2) == 0 ? bf16lo(u) : bf16hi(u);
    }

    __device__ __forceinline__ void finish(float eps, uint32_t *act_lds, float (&red)[NB][NW])
    {
        // sum of squares per batch row
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float ss = 0.f;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if ((int)threadIdx.x + NT * m < NI)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = xval(m, b, e);
                        ss = fmaf(v, v, ss);
                    }
            ss = wave_sum(ss);
            if ((threadIdx.x & 63) == 0) red[b][threadIdx.x >> 6] = ss;
        }
        __syncthreads();
        // normalised, bf16-rounded quarters of chunks
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float tot = 0.f;
#pragma unroll
            for (int i = 0; i < NW; ++i) tot += red[b][i];
            const float r = 1.0f / sqrtf(tot / (float)HIDDEN + eps);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int it = (int)threadIdx.x + NT * m, c = it >> 2, j = it & 3;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = round_bf16(xval(m, b, e) * r * wval(m, e));
                // pairs (k, k + 4) of the quarter; even and odd sums of the quarter
                float se = (v[0] + v[4]) + (v[2] + v[6]), so = (v[1] + v[5]) + (v[3] + v[7]);
                se += dpp_mov<0xB1>(se);  // quad_perm [1,0,3,2]
                so += dpp_mov<0xB1>(so);
                se += dpp_mov<0x4E>(se);  // quad_perm [2,3,0,1]
                so += dpp_mov<0x4E>(so);
                if (it < NI) {
                    uint32_t *dst = act_lds + ((size_t)b * NCH + c) * ACT_WORDS;
                    reinterpret_cast<uint4 *>(dst)[j] =
                        make_uint4(pack_f16x2(v[0], v[4]), pack_f16x2(v[1], v[5]), pack_f16x2(v[2], v[6]), pack_f16x2(v[3], v[7]));
                    if (j == 0)
                        reinterpret_cast<uint4 *>(dst)[4] =
                            make_uint4(__float_as_uint(fmaf(1024.f, se, 64.f * so)), __float_as_uint(se + so), 0x3F800000u, 0u);
                }
            }
        }
        __syncthreads();
    }
};

// The activation source of the K = hidden kernels without a pre-norm: the bf16 rows of x go to
// LDS in the activation format as they are, with PreNorm's interface (thread t < 140 owns
// chunk t of every batch row).
template <int NB, int NT, int XT>
struct PlainAct {
    static constexpr int NCH = HIDDEN / 32, NW = NT / 64;
    bool own;
    XChunk<XT> xr[NB];

    __device__ __forceinline__ void issue(const void *x, const uint16_t *)
    {
        own = (int)threadIdx.x < NCH;
        if (own) {
#pragma unroll
            for (int b = 0; b < NB; ++b) xr[b].load(x, (size_t)b * NCH + threadIdx.x);
        }
    }

    __device__ __forceinline__ void finish(float, uint32_t *act_lds, float (&)[NB][NW])
    {
        if (own) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float v[32];
                xr[b].unpack(v);
                make_chunk_scaled(v, act_lds + ((size_t)b * NCH + threadIdx.x) * ACT_WORDS);
            }
        }
        __syncthreads();
    }
};

// Activations of the lane's chunks in the K = 4480 layout: l and l + 64 of every row, and
// its tail chunk 128 + l % 12 (zero for lanes beyond the R rows' tails).
template <int NB, int R>
__device__ __forceinline__ void act_hidden(ActChunk (&am)[NB][2], ActChunk (&at)[NB], const uint32_t *act_lds)
{
    constexpr int NCH = HIDDEN / 32;
    const int l = threadIdx.x & 63;
    const bool tail = l < IP_TAIL * R;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            chunk_from_lds(am[b][i], act_lds + ((size_t)b * NCH + l + 64 * i) * ACT_WORDS);
        }
        chunk_from_lds(at[b], act_lds + ((size_t)b * NCH + 128 + l % IP_TAIL) * ACT_WORDS);
        if (!tail) {
#pragma unroll
            for (int j = 0; j < 16; ++j) at[b].p[j] = 0u;
            at[b].off = 0.f;
            at[b].sum = 0.f;
            at[b].mul = 1.f;
        }
    }
}

// ---------------------------------------------- batched rows on the matrix cores
//
// For 2 to 4 batch rows the dot products go to v_mfma_f32_4x4x4_16b_f16, which runs 16
// independent 4x4x4 products: for block b (lanes 4b .. 4b+3) lane 4b+i supplies row i of A
// (4 values of K), lane 4b+j column j of B, and lane 4b+j receives column j of D (register v
// holding row v).  Here block b is a K-range -- chunks b, b + 16, ... (32 K each; 140 per row,
// so blocks 12-15 have 8 and the rest 9) -- A's rows are the batch rows (lane 4b+i holds batch
// row i's activations, zero for i >= NB) and B's columns are 4 weight rows (lane 4b+j holds
// row j's packed words).  A stage is thus 4 rows, and the dequantisation (one shift and four
// v_and_or per word) is shared by all batch rows instead of repeated per row.
//
// Per chunk: D gathers the even nibbles (1024 + q) and D' the odd ones (1024 + 16 q) as in
// chunk_dot, and acc += s (D + D'/16).  The activation constants of the magic offset and of
// the bias are per (chunk, batch row) and live in the A lanes, so they enter through
// v_mfma_f32_4x4x1_16b_f32, which broadcasts them over the columns: D starts at -off, and
// E += sum_x b.  After the 9 chunks the 16 blocks' partials are summed across lanes (DPP row
// rotations, then two shuffles).  The same kernel serves the plain W4 GEMV of K = 4480 at
// batch 3 and 4.
constexpr int MF_CH = 9;    // chunks per lane and row
constexpr int MF_WGS = 256;  // work-groups of the batched in_proj: one per CU, 32 per XCD

struct MfStage {
    uint4 q[MF_CH];
    uint16_t s[MF_CH], b[MF_CH];
    EpiPre pe;
};

typedef _Float16 h4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h4v h4_of(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(h4v, make_uint2(lo, hi));
}

// NORM: the activations are the pre-norm u = bf16(x / rms(x) * nw) of x (XT: its dtype);
// otherwise x is bf16 and used as it is.  Epi: the row epilogue (in_proj's split and conv
// step, or a plain store).
template <int NB, int XT, bool NORM, class Epi>
__global__ __launch_bounds__(256, 1) void k_w4_mf(W4 W, const void *__restrict__ x, const uint16_t *__restrict__ nw,
                                                  float eps, Epi epi, uint32_t *zero_ptr, int nzero)
{
    constexpr int NT = 256, NW = NT / 64, NCH = HIDDEN / 32;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    __shared__ float red[NB][NW];
    if (blockIdx.x == 0 && (int)threadIdx.x < nzero) zero_ptr[threadIdx.x] = 0u;
    std::conditional_t<NORM, PreNorm<NB, XT, NT>, PlainAct<NB, NT, XT>> pn;
    pn.issue(x, nw);
    __builtin_amdgcn_sched_barrier(0);

    const int lane = threadIdx.x & 63, kb = lane >> 2, q4 = lane & 3;
    const int nmax = W.n - 1;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)W.q, 0, (int)((uint32_t)W.n * IP_ROWB), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)W.s, 0, (int)((uint32_t)W.n * IP_GRPB), 0x00020000);
    const __amdgpu_buffer_rsrc_t rbi = __builtin_amdgcn_make_buffer_rsrc((void *)W.b, 0, (int)((uint32_t)W.n * IP_GRPB), 0x00020000);
    // this wave's 4-row stages [s0, s1): an even split per XCD, then per wave inside the XCD
    const int nst = (W.n + 3) / 4;
    const int xcd = blockIdx.x & 7, nwx = (int)(gridDim.x >> 3) * NW;
    const int wx = __builtin_amdgcn_readfirstlane((int)((blockIdx.x >> 3) * NW + (threadIdx.x >> 6)));
    const int xs = (int)((long)nst * xcd / 8), xn = (int)((long)nst * (xcd + 1) / 8) - xs;
    const int s0 = xs + (int)((long)xn * wx / nwx), s1 = xs + (int)((long)xn * (wx + 1) / nwx);
    // lanes 0-15 finish (row 4 s + (lane & 3), batch lane >> 2) of each stage
    const int eb = min(lane >> 2, NB - 1);
    // the row differs between the four lanes of a block, so the whole offset goes in the
    // per-lane operand (a per-lane scalar offset would become a loop over its values)
    auto load = [&](MfStage &g, int st) {
        const uint32_t row = (uint32_t)min(4 * st + q4, nmax);
#pragma unroll
        for (int t = 0; t < MF_CH; ++t) {
            const uint32_t c = (uint32_t)min(kb + 16 * t, NCH - 1);
            g.q[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, row * IP_ROWB + 16u * c, 0, NT_LOAD));
            g.s[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * IP_GRPB + 2u * (c >> 1), 0, 0);
            g.b[t] = __builtin_amdgcn_raw_buffer_load_b16(rbi, row * IP_GRPB + 2u * (c >> 1), 0, 0);
        }
        g.pe = epi.prefetch(min(4 * st + q4, nmax), eb);
    };
    // The first stage is issued after the pre-norm.  Issued before it (one or two stages), the
    // weight loads delay the arrival of x, which every work-group reads, by about as much as
    // they overlap: 21.6 to 24 us at batch 4 against 21.6.
    pn.finish(eps, act_lds, red);
    MfStage A, B;
    load(A, min(s0, nst - 1));
    // activations: batch row q4 (zero beyond NB), chunks kb + 16 t (zero beyond the row);
    // the offset constant is kept negated for the f32 products
    ActChunk a[MF_CH];
#pragma unroll
    for (int t = 0; t < MF_CH; ++t) {
        const int c = kb + 16 * t;
        if (q4 < NB && c < NCH) {
            chunk_from_lds(a[t], act_lds + ((size_t)q4 * NCH + c) * ACT_WORDS);
            a[t].off = -a[t].off;
            if constexpr (!NORM) a[t].sum *= a[t].mul;  // scaled chunks: the bias term in true scale
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) a[t].p[j] = 0u;
            a[t].off = 0.f;
            a[t].sum = 0.f;
            a[t].mul = 1.f;
        }
    }
    const uint32_t mlo = opaque_v(0x000F000Fu), mhi = opaque_v(0x00F000F0u), magic = opaque_v(0x64006400u);
    auto step = [&](const MfStage &g, int st) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f}, E = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < MF_CH; ++t) {
            // D starts at -off (batch row i's offset in every column): D + D'/16 is then the
            // chunk's sum of a q itself, so a one-hot x gives s q + b with one rounding
            const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
            floatx4 D = __builtin_amdgcn_mfma_f32_4x4x1f32(a[t].off, 1.0f, zero, 0, 0, 0), D2 = zero;
            const uint32_t wq[4] = {g.q[t].x, g.q[t].y, g.q[t].z, g.q[t].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t wd = wq[w], wh = wd >> 8;
                const uint32_t d0 = and_or_mf(wd, mlo, magic), d1 = and_or_mf(wd, mhi, magic);
                const uint32_t d2 = and_or_mf(wh, mlo, magic), d3 = and_or_mf(wh, mhi, magic);
                D = __builtin_amdgcn_mfma_f32_4x4x4f16(h4_of(a[t].p[4 * w], a[t].p[4 * w + 2]), h4_of(d0, d2), D, 0, 0, 0);
                D2 = __builtin_amdgcn_mfma_f32_4x4x4f16(h4_of(a[t].p[4 * w + 1], a[t].p[4 * w + 3]), h4_of(d1, d3), D2, 0, 0, 0);
            }
            const float sc = __uint_as_float((uint32_t)g.s[t] << 16), bi = __uint_as_float((uint32_t)g.b[t] << 16);
            if constexpr (NORM) {
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, fmaf(D2[v], 0.0625f, D[v]), acc[v]);
            } else {
                // scaled chunks: batch row v's 2^k, broadcast over the columns like the offset
                const floatx4 Mb = __builtin_amdgcn_mfma_f32_4x4x1f32(a[t].mul, 1.0f, zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc * Mb[v], fmaf(D2[v], 0.0625f, D[v]), acc[v]);
            }
            E = __builtin_amdgcn_mfma_f32_4x4x1f32(a[t].sum, bi, E, 0, 0, 0);
        }
        float tot[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float u = acc[v] + E[v];
            u += dpp_mov<0x124>(u);  // row_ror:4
            u += dpp_mov<0x128>(u);  // row_ror:8
            u = xor32_sum(xor16_sum(u));
            tot[v] = u;
        }
        const int bsel = lane >> 2;
        const float mine = bsel == 0 ? tot[0] : bsel == 1 ? tot[1] : bsel == 2 ? tot[2] : tot[3];
        const int row = 4 * st + q4;
        if (lane < 4 * NB && row <= nmax) epi(row, bsel, mine, g.pe);
    };
    // two stages per iteration with no conditional load: loads past the wave's last stage
    // re-read that stage (the cache holds it), and only the second compute is conditional
    if (s1 > s0) {
        const int last = s1 - 1;
        for (int st = s0; st < s1; st += 2) {
            load(B, min(st + 1, last));
            __builtin_amdgcn_sched_barrier(0);
            step(A, st);
            load(A, min(st + 2, last));
            __builtin_amdgcn_sched_barrier(0);
            if (st + 1 < s1) step(B, st + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ------------------------------------ batched rows on the matrix cores, activations in LDS
//
// The same 4x4x4 block layout as k_w4_mf for any K: the NB activation rows stay in LDS (the
// work-group builds them once) and each lane reads its A operand chunk by chunk, so K is not
// limited by registers.  LDS slot c NB + b holds chunk c of batch row b: the four lanes of a
// block (batch rows 0..3 of one chunk) read consecutive 80-byte slots, which are
// conflict-free.  A 4-row stage is cut into slices of CH chunk slots per lane-block
// (block b takes chunks b + 16 t); the (stage, slice) units are streamed with the next unit's
// loads in flight, and after a stage's last slice the 16 blocks' partials are summed across
// lanes.  One work-group of 8 waves per CU.  SC: the chunks are scaled (make_chunk_scaled).
constexpr int MFL_NT = 512;

template <int CH>
struct MflUnit {
    uint4 q[CH];
    uint16_t s[CH], b[CH];
};

// x [NB][k] bf16 as scaled chunks.  issue() loads a thread's chunks (chunk it = b nch + c
// for it = thread, thread + NT, ...; at most MAXC per thread) before the caller's first weight
// loads, so that they do not queue behind them; finish() builds the LDS slots.
template <int NB, int NT, int MAXC, int XT>
struct ActPlainK {
    const void *x;
    XChunk<XT> r[MAXC];
    __device__ __forceinline__ void issue(int nch)
    {
        // unconditional (indices clamped): after a conditional load the compiler's wait for its
        // registers would also wait for every load issued after it, the weight stream included
#pragma unroll
        for (int i = 0; i < MAXC; ++i) r[i].load(x, (size_t)min((int)threadIdx.x + NT * i, NB * nch - 1));
    }
    __device__ __forceinline__ void finish(uint32_t *act_lds, int nch)
    {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            const int it = threadIdx.x + NT * i;
            if (it < NB * nch) {
                float v[32];
                r[i].unpack(v);
                const int b = it / nch, c = it - b * nch;
                make_chunk_scaled(v, act_lds + (size_t)(c * NB + b) * ACT_WORDS);
            }
        }
        __syncthreads();
    }
};

template <int NB, int CH, bool SC, class Act, class Epi>
__global__ __launch_bounds__(MFL_NT, 1) void k_w4_mfl(W4 W, Act act_in, Epi epi)
{
    Act act = act_in;
    constexpr int NW = MFL_NT / 64;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    const int lane = threadIdx.x & 63, kb = lane >> 2, q4 = lane & 3;
    const int nch = W.k >> 5, nmax = W.n - 1;
    const uint32_t rowbytes = (uint32_t)W.k / 2, kg2 = (uint32_t)(W.k >> 6) * 2;
    const int nsl = ((nch + 15) / 16 + CH - 1) / CH;  // slices per stage
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)W.q, 0, (int)((uint32_t)W.n * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)W.s, 0, (int)((uint32_t)W.n * kg2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rbi = __builtin_amdgcn_make_buffer_rsrc((void *)W.b, 0, (int)((uint32_t)W.n * kg2), 0x00020000);
    // this wave's 4-row stages [s0, s1): an even split per XCD, then per wave inside the XCD
    const int nst = (W.n + 3) / 4;
    const int xcd = blockIdx.x & 7, nwx = (int)(gridDim.x >> 3) * NW;
    const int wx = __builtin_amdgcn_readfirstlane((int)((blockIdx.x >> 3) * NW + (threadIdx.x >> 6)));
    const int xs = (int)((long)nst * xcd / 8), xn = (int)((long)nst * (xcd + 1) / 8) - xs;
    const int s0 = xs + (int)((long)xn * wx / nwx), s1 = xs + (int)((long)xn * (wx + 1) / nwx);
    const int eb = min(lane >> 2, NB - 1);
    const int nu = (s1 - s0) * nsl;  // (stage, slice) units of this wave

    // unit u = (stage s0 + u / nsl, slice u % nsl); loads past the wave's last unit re-read it
    auto load = [&](MflUnit<CH> &g, int u) {
        u = min(u, max(nu - 1, 0));
        const int st = s0 + u / nsl, sl = u % nsl;
        const uint32_t row = (uint32_t)min(4 * st + q4, nmax);
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const uint32_t c = (uint32_t)min(kb + 16 * (CH * sl + t), nch - 1);
            g.q[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, row * rowbytes + 16u * c, 0, NT_LOAD));
            g.s[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * kg2 + 2u * (c >> 1), 0, 0);
            g.b[t] = __builtin_amdgcn_raw_buffer_load_b16(rbi, row * kg2 + 2u * (c >> 1), 0, 0);
        }
    };
    MflUnit<CH> A, B;
    act.issue(nch);
    EpiPre pe = epi.prefetch(min(4 * min(s0, nst - 1) + q4, nmax), eb);
    load(A, 0);
    // slot NB nch: a zero chunk, read by the lanes with no activation (batch rows beyond NB,
    // chunks past the row), so that every lane's LDS read is unconditional
    uint32_t *zslot = act_lds + (size_t)NB * nch * ACT_WORDS;
    if (threadIdx.x < ACT_WORDS) zslot[threadIdx.x] = threadIdx.x == 18 ? 0x3F800000u : 0u;
    act.finish(act_lds, nch);
    if (nu == 0) return;

    const uint32_t mlo = opaque_v(0x000F000Fu), mhi = opaque_v(0x00F000F0u), magic = opaque_v(0x64006400u);
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    floatx4 acc = zero, E = zero;
    auto unit = [&](const MflUnit<CH> &g, int u) {
        const int st = s0 + u / nsl, sl = u % nsl;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            // the A operand: batch row q4's chunk (zero beyond NB and past the row)
            const int c = kb + 16 * (CH * sl + t);
            ActChunk a;
            chunk_from_lds(a, q4 < NB && c < nch ? act_lds + ((size_t)c * NB + q4) * ACT_WORDS : zslot);
            floatx4 D = __builtin_amdgcn_mfma_f32_4x4x1f32(-a.off, 1.0f, zero, 0, 0, 0), D2 = zero;
            const uint32_t wq[4] = {g.q[t].x, g.q[t].y, g.q[t].z, g.q[t].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t wd = wq[w], wh = wd >> 8;
                const uint32_t d0 = and_or_mf(wd, mlo, magic), d1 = and_or_mf(wd, mhi, magic);
                const uint32_t d2 = and_or_mf(wh, mlo, magic), d3 = and_or_mf(wh, mhi, magic);
                D = __builtin_amdgcn_mfma_f32_4x4x4f16(h4_of(a.p[4 * w], a.p[4 * w + 2]), h4_of(d0, d2), D, 0, 0, 0);
                D2 = __builtin_amdgcn_mfma_f32_4x4x4f16(h4_of(a.p[4 * w + 1], a.p[4 * w + 3]), h4_of(d1, d3), D2, 0, 0, 0);
            }
            const float sc = __uint_as_float((uint32_t)g.s[t] << 16), bi = __uint_as_float((uint32_t)g.b[t] << 16);
            if constexpr (SC) {
                const floatx4 Mb = __builtin_amdgcn_mfma_f32_4x4x1f32(a.mul, 1.0f, zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc * Mb[v], fmaf(D2[v], 0.0625f, D[v]), acc[v]);
                E = __builtin_amdgcn_mfma_f32_4x4x1f32(a.sum * a.mul, bi, E, 0, 0, 0);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, fmaf(D2[v], 0.0625f, D[v]), acc[v]);
                E = __builtin_amdgcn_mfma_f32_4x4x1f32(a.sum, bi, E, 0, 0, 0);
            }
        }
        if (sl == nsl - 1) {
            float tot[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x = acc[v] + E[v];
                x += dpp_mov<0x124>(x);  // row_ror:4
                x += dpp_mov<0x128>(x);  // row_ror:8
                x = xor32_sum(xor16_sum(x));
                tot[v] = x;
            }
            const int bsel = lane >> 2;
            const float mine = bsel == 0 ? tot[0] : bsel == 1 ? tot[1] : bsel == 2 ? tot[2] : tot[3];
            const int row = 4 * st + q4;
            if (lane < 4 * NB && row <= nmax) epi(row, bsel, mine, pe);
            pe = epi.prefetch(min(4 * min(st + 1, nst - 1) + q4, nmax), eb);
            acc = zero;
            E = zero;
        }
    };
    // two units per iteration with no conditional load; only the second compute is conditional
    for (int u = 0; u < nu; u += 2) {
        load(B, u + 1);
        __builtin_amdgcn_sched_barrier(0);
        unit(A, u);
        load(A, u + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < nu) unit(B, u + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ----------------------------- batched out_proj, split over K by the gated-norm groups
//
// At batch 2..4 the gated norm + out_proj (4480 x 10240) runs split over K by the eight
// gated-norm groups of 1280 channels: work-group i takes group g = i mod 8 (so each XCD streams
// one group's weight columns and holds one group's activations) and rows [140 (i / 8), +140).
// It builds only its group's NB x 40 activation chunks, where a work-group over the whole of K
// builds NB x 320 (at batch 4 that build, from every work-group's 160 KB of g w, took most of the
// full-K kernel's time).  The group's rstd needs only its own 32 per-(head, half) sums of
// squares.  Each 4-row stage runs on the 4x4x4 matrix-core blocks as in k_w4_mfl (block kb takes
// chunks kb, kb + 16, kb + 32 of the group's 40; the third is zero for kb >= 8).  The eight
// groups' partial sums go to the workspace ([group][batch row][row] fp32) and k_sk_reduce adds
// them in group order, then the residual: the result does not depend on timing.
constexpr int SK_ROWS = HIDDEN / 32, SK_NCH = GNORM / 32, SK_STAGES = SK_ROWS / 4, SK_NT = 512;

struct SkUnit {
    uint4 q[3];
    uint16_t s[3], b[3];
};

template <int NB>
__global__ __launch_bounds__(SK_NT, 1) void k_outproj_sk(W4 W, const float *__restrict__ gate,
                                                         const float *__restrict__ part, float eps,
                                                         float *__restrict__ partial)
{
    __shared__ __attribute__((aligned(16))) uint32_t act[(NB * SK_NCH + 1) * ACT_WORDS];
    __shared__ float rstd[NB];
    const int g = blockIdx.x & 7, row0 = SK_ROWS * (int)(blockIdx.x >> 3);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb = lane >> 2, q4 = lane & 3;
    const uint32_t rowbytes = (uint32_t)W.k / 2, kg2 = (uint32_t)(W.k >> 6) * 2;
    const int s0 = SK_STAGES * wave / 8, s1 = SK_STAGES * (wave + 1) / 8;  // this wave's stages
    const int nu = s1 - s0;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)W.q, 0, (int)((uint32_t)W.n * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)W.s, 0, (int)((uint32_t)W.n * kg2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rbi = __builtin_amdgcn_make_buffer_rsrc((void *)W.b, 0, (int)((uint32_t)W.n * kg2), 0x00020000);

    // stage u of this wave: lane (kb, q4) loads row row0 + 4 (s0 + u) + q4, chunks kb + 16 t of the
    // group's 40 (the third clamped for kb >= 8 and unused); past the last stage: re-read it
    auto load = [&](SkUnit &un, int u) {
        const uint32_t row = (uint32_t)(row0 + 4 * (s0 + min(u, nu - 1)) + q4);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const uint32_t c = (uint32_t)(SK_NCH * g + min(kb + 16 * t, SK_NCH - 1));
            un.q[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, row * rowbytes + 16u * c, 0, NT_LOAD));
            un.s[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * kg2 + 2u * (c >> 1), 0, 0);
            un.b[t] = __builtin_amdgcn_raw_buffer_load_b16(rbi, row * kg2 + 2u * (c >> 1), 0, 0);
        }
    };

    // prologue loads first: the group's sums of squares (thread t < 32 NB: batch row t / 32) and
    // the g w values of one chunk per thread (t < 40 NB: batch row t / 40, chunk t % 40)
    const int pb = min(tid >> 5, NB - 1), cb = min(tid / SK_NCH, NB - 1), cc = tid % SK_NCH;
    const float pv = part[pb * NHEADS * 2 + 32 * g + (tid & 31)];
    float4 gv[8];
    {
        const float4 *gp = reinterpret_cast<const float4 *>(gate + (size_t)cb * DINNER + GNORM * g + 32 * cc);
#pragma unroll
        for (int j = 0; j < 8; ++j) gv[j] = gp[j];
    }
    SkUnit A, B;
    load(A, 0);
    // slot NB * 40: a zero chunk for the lanes with no activation (batch rows past NB, chunks
    // past the group's 40), so that every LDS read is unconditional
    uint32_t *zslot = act + NB * SK_NCH * ACT_WORDS;
    if (tid < ACT_WORDS) zslot[tid] = tid == 18 ? 0x3F800000u : 0u;
    if (tid < 32 * NB) {
        const float tot = row_sum<32>(pv);
        if ((tid & 31) == 0) rstd[tid >> 5] = 1.0f / sqrtf(tot / (float)GNORM + eps);
    }
    __syncthreads();
    if (tid < SK_NCH * NB) {
        const float r = rstd[cb];
        float v[32];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[4 * j] = round_bf16(gv[j].x * r);
            v[4 * j + 1] = round_bf16(gv[j].y * r);
            v[4 * j + 2] = round_bf16(gv[j].z * r);
            v[4 * j + 3] = round_bf16(gv[j].w * r);
        }
        make_chunk(v, act + (size_t)(cc * NB + cb) * ACT_WORDS);
    }
    __syncthreads();
    if (nu == 0) return;

    const uint32_t mlo = opaque_v(0x000F000Fu), mhi = opaque_v(0x00F000F0u), magic = opaque_v(0x64006400u);
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    auto unit = [&](const SkUnit &un, int u) {
        floatx4 acc = zero, E = zero;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            // the A operand: batch row q4's chunk (zero beyond NB and past the group's chunks)
            const int c = kb + 16 * t;
            ActChunk a;
            chunk_from_lds(a, q4 < NB && c < SK_NCH ? act + ((size_t)c * NB + q4) * ACT_WORDS : zslot);
            floatx4 D = __builtin_amdgcn_mfma_f32_4x4x1f32(-a.off, 1.0f, zero, 0, 0, 0), D2 = zero;
            const uint32_t wq[4] = {un.q[t].x, un.q[t].y, un.q[t].z, un.q[t].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t wd = wq[w], wh = wd >> 8;
                const uint32_t d0 = and_or_mf(wd, mlo, magic), d1 = and_or_mf(wd, mhi, magic);
                const uint32_t d2 = and_or_mf(wh, mlo, magic), d3 = and_or_mf(wh, mhi, magic);
                D = __builtin_amdgcn_mfma_f32_4x4x4f16(h4_of(a.p[4 * w], a.p[4 * w + 2]), h4_of(d0, d2), D, 0, 0, 0);
                D2 = __builtin_amdgcn_mfma_f32_4x4x4f16(h4_of(a.p[4 * w + 1], a.p[4 * w + 3]), h4_of(d1, d3), D2, 0, 0, 0);
            }
            const float sc = __uint_as_float((uint32_t)un.s[t] << 16), bi = __uint_as_float((uint32_t)un.b[t] << 16);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, fmaf(D2[v], 0.0625f, D[v]), acc[v]);
            E = __builtin_amdgcn_mfma_f32_4x4x1f32(a.sum, bi, E, 0, 0, 0);
        }
        // the 16 blocks' partials: lane (kb, q4) ends with batch row kb's sum for row q4
        float tot[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float x = acc[v] + E[v];
            x += dpp_mov<0x124>(x);  // row_ror:4
            x += dpp_mov<0x128>(x);  // row_ror:8
            x = xor32_sum(xor16_sum(x));
            tot[v] = x;
        }
        const int bsel = lane >> 2;
        const float mine = bsel == 0 ? tot[0] : bsel == 1 ? tot[1] : bsel == 2 ? tot[2] : tot[3];
        if (lane < 4 * NB)
            partial[(size_t)(g * NB + bsel) * HIDDEN + row0 + 4 * (s0 + u) + q4] = mine;
    };
    // two stages per iteration with no conditional load; only the second compute is conditional
    for (int u = 0; u < nu; u += 2) {
        load(B, u + 1);
        __builtin_amdgcn_sched_barrier(0);
        unit(A, u);
        load(A, u + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < nu) unit(B, u + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// y[b][row] = sum over the eight groups of partial[g][b][row] (in group order) + res[b][row]
template <int NB>
__global__ __launch_bounds__(256) void k_sk_reduce(const float *__restrict__ partial, EpiStore epi)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= NB * HIDDEN) return;
    const int b = i / HIDDEN, row = i - b * HIDDEN;
    const EpiPre pe = epi.prefetch(row, b);
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < NGROUPS; ++g) v += partial[(size_t)(g * NB + b) * HIDDEN + row];
    epi(row, b, v, pe);
}

size_t mfl_lds_bytes(int batch, int k) { return ((size_t)batch * (k / 32) + 1) * ACT_WORDS * 4; }

// chunk slots per lane-block and slice for K = 32 nch: the fewest slots, then the largest CH
static inline int mfl_ch(int k)
{
    const int mch = (k / 32 + 15) / 16;
    int best = 10, slots = 1 << 30;
    for (int ch : {10, 9, 8, 4}) {
        const int sl = (mch + ch - 1) / ch * ch;
        if (sl < slots) { slots = sl; best = ch; }
    }
    return best;
}

// the kernel with its dynamic LDS limit raised once (above 64 KiB it must be set explicitly)
template <int NB, int CH, bool SC, class Act, class Epi>
static hipError_t launch_mfl_ch(const W4 &W, const Act &a, const Epi &e, size_t lds, hipStream_t st)
{
    static size_t allowed = 64 * 1024;  // raised to the largest size asked for so far
    if (lds > allowed) {
        const hipError_t r = hipFuncSetAttribute((const void *)k_w4_mfl<NB, CH, SC, Act, Epi>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (r != hipSuccess) return r;
        allowed = lds;
    }
    launch_k(k_w4_mfl<NB, CH, SC, Act, Epi>, dim3(MF_WGS), dim3(MFL_NT), lds, st, W, a, e);
    return hipGetLastError();
}

template <int NB, bool SC, class Act, class Epi>
static hipError_t launch_mfl(const W4 &W, const Act &a, const Epi &e, hipStream_t st)
{
    const size_t lds = mfl_lds_bytes(NB, W.k);
    switch (mfl_ch(W.k)) {
    case 10: return launch_mfl_ch<NB, 10, SC>(W, a, e, lds, st);
    case 9: return launch_mfl_ch<NB, 9, SC>(W, a, e, lds, st);
    case 8: return launch_mfl_ch<NB, 8, SC>(W, a, e, lds, st);
    default: return launch_mfl_ch<NB, 4, SC>(W, a, e, lds, st);
    }
}

// Work-groups of four waves per CU for the generic GEMV: three or two at batch 1 while the
// activations (CPL chunks of 18 registers per lane) leave room, one above: with 8 chunks per
// lane (K above 10240, e.g. an MLP down projection of K = 15680) two per CU spilled.
constexpr int gemv_wgs_per_cu(int nb, int cpl) { return nb == 1 ? (cpl <= 3 ? 3 : cpl <= 5 ? 2 : 1) : 1; }

// ------------------------------------------------------------------ kernels

template <int LPR, int CPL, int NB, int RG, int XT>
__global__ __launch_bounds__(256, gemv_wgs_per_cu(NB, CPL)) void k_gemv(W4 W, const void *__restrict__ x, EpiStore epi)
{
    GemvRunner<LPR, CPL, NB, RG, EpiStore, true> run(W, epi, 256);
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    const int nch = W.k >> 5;
    for (int it = threadIdx.x; it < NB * nch; it += 256) {  // chunk it = b nch + c
        XChunk<XT> xc;
        xc.load(x, (size_t)it);
        float v[32];
        xc.unpack(v);
        make_chunk_scaled(v, act_lds + (size_t)it * ACT_WORDS);
    }
    __syncthreads();
    ActChunk a[NB][CPL];
    act_from_lds<LPR, CPL, NB>(a, act_lds, nch, (threadIdx.x & 63) % LPR);
    run.run(a);
}

// Fused pre-norm + in_proj + conv step: the work-group normalises the input rows into LDS
// (u = bf16(x / rms(x) * w)), then streams its share of in_proj rows.
template <int NB, int XT>
__global__ __launch_bounds__(InProjShape<NB>::NT, 1) void k_inproj_step(W4 W, const void *__restrict__ x,
                                                                    const uint16_t *__restrict__ nw, float eps,
                                                                    EpiInProjStep epi, uint32_t *zero_ptr,
                                                                    int nzero)
{
    constexpr int NT = InProjShape<NB>::NT, R = InProjShape<NB>::R;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    __shared__ float red[NB][NT / 64];
    if (blockIdx.x == 0 && (int)threadIdx.x < nzero) zero_ptr[threadIdx.x] = 0u;
    PreNorm<NB, XT, NT> pn;
    pn.issue(x, nw);
    __builtin_amdgcn_sched_barrier(0);
    InProjBlock<NB> run(W, epi);
    pn.finish(eps, act_lds, red);
    ActChunk am[NB][2], at[NB];
    act_hidden<NB, R>(am, at, act_lds);
    run.run(am, at);
}

// Fused gated RMSNorm + out_proj + residual for the per-position block at batch 1 (batches
// 2..4 take the split over norm groups above).  The work-group forms
// o = bf16((g w) / rms_group(g)) straight into the LDS activation format from g w (the gate
// product g = bf16(y) * silu(z) times the norm weight) and the per-(head, half) sums of squares
// of g, both left by the SSM step, while the first stage of out_proj weights is already in
// flight; o never goes to memory.
__global__ __launch_bounds__(512, 1) void k_outproj_step(W4 W, const float *__restrict__ gate,
                                                         const float *__restrict__ part, float eps,
                                                         EpiStore epi)
{
    constexpr int NB = 1, LPR = 64, NCH = DINNER / 32, CPL = NCH / LPR, RG = 1, NT = 512;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    __shared__ float rstd[NGROUPS];
    // The prologue's loads go out alone on waves 0..3 (one per-(head, half) sum of squares per
    // thread, 32 of which make a group, and the chunks' g w values: chunks t and t + 256);
    // waves 4..7 issue their first weight stage at once, so their rows stream while the
    // activations are built.  Waves 0..3 start streaming after the first barrier: issued
    // together, the prologue loads would queue behind their weight loads.
    constexpr int PW = 256, GC = (NCH + PW - 1) / PW;
    const bool early = threadIdx.x >= PW;
    GemvRunner<LPR, CPL, NB, RG, EpiStore> run(W, epi, NT, early);
    float4 gv0[GC][8];
    if (!early) {
        const float pv = part[threadIdx.x];
#pragma unroll
        for (int k = 0; k < GC; ++k) {
            const int c = min((int)threadIdx.x + PW * k, NCH - 1);
            const float4 *gp = reinterpret_cast<const float4 *>(gate + 32 * c);
#pragma unroll
            for (int j = 0; j < 8; ++j) gv0[k][j] = gp[j];
        }
        const float tot = row_sum<32>(pv);  // 32 consecutive entries = one group
        if ((threadIdx.x & 31) == 0) rstd[threadIdx.x / 32] = 1.0f / sqrtf(tot / (float)GNORM + eps);
    }
    __syncthreads();
    if (!early) {
        run.issue_first();
#pragma unroll
        for (int k = 0; k < GC; ++k) {
            const int c = (int)threadIdx.x + PW * k;
            if (c < NCH) {
                const float r = rstd[(32 * c) / GNORM];
                float v[32];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v[4 * j] = round_bf16(gv0[k][j].x * r);
                    v[4 * j + 1] = round_bf16(gv0[k][j].y * r);
                    v[4 * j + 2] = round_bf16(gv0[k][j].z * r);
                    v[4 * j + 3] = round_bf16(gv0[k][j].w * r);
                }
                make_chunk(v, act_lds + (size_t)c * ACT_WORDS);
            }
        }
    }
    __syncthreads();
    ActChunk a[NB][CPL];
    act_from_lds<LPR, CPL, NB>(a, act_lds, NCH, (threadIdx.x & 63) % LPR);
    run.run(a);
}

// ----------------------------------------------------------------- attention q / k / v
//
// The q, k and v projections of an attention layer share one input, u = RMSNorm(x) w, so one
// launch computes all three (5120 + 1024 + 1024 rows of K = hidden): the pre-norm and the
// K = 4480 row layout of in_proj, 4-row blocks spread over 8-wave work-groups, each block inside
// one of the three matrices.  The epilogue stores q (bf16) and
// appends k and v (bf16) to the key/value cache, [batch][kv_heads][max_len][head_dim], at the
// sequence's position; a position outside 0 .. max_len - 1 stores nothing (the attention
// kernels then write NaN outputs for that sequence).
constexpr int ATT_HEADS = 40, ATT_KV = 8, ATT_HD = 128;
constexpr int ATT_QD = ATT_HEADS * ATT_HD, ATT_KD = ATT_KV * ATT_HD;  // 5120, 1024

// Batch 1 and 2: 4-row blocks (1792 of them), so that 8-wave work-groups still cover 224 CUs.
// Batch 3 and 4 need the registers of 4-wave work-groups: in_proj's 8-row blocks.
template <int NB>
struct AttnQkvShape {
    static constexpr int R = NB == 1 ? 2 : 1, RW = NB <= 2 ? 4 : 8, NS = RW / R, NT = NB <= 2 ? 512 : 256;
};

struct EpiAttnQKV {
    uint16_t *q, *kc, *vc;
    const int *pos;
    int max_len, base;  // base: the first global row (q | k | v) of the wave's matrix
    __device__ __forceinline__ EpiPre prefetch(int, int b) const
    {
        EpiPre p;
        p.w[0] = (uint32_t)pos[b];
        return p;
    }
    __device__ __forceinline__ void operator()(int n, int b, float acc, const EpiPre &p) const
    {
        const uint16_t vb = f32_to_bf16(acc);
        const int gn = base + n;
        if (gn < ATT_QD) {
            q[(size_t)b * ATT_QD + gn] = vb;
            return;
        }
        const int t = (int)p.w[0];
        if (t < 0 || t >= max_len) return;
        const int r = (gn - ATT_QD) % ATT_KD, kvh = r / ATT_HD, d = r % ATT_HD;
        uint16_t *dst = gn < ATT_QD + ATT_KD ? kc : vc;
        dst[(((size_t)b * ATT_KV + kvh) * max_len + t) * ATT_HD + d] = vb;
    }
};

template <int NB, int XT>
__global__ __launch_bounds__(AttnQkvShape<NB>::NT, 1) void k_attn_qkv(W4 Wq, W4 Wk, W4 Wv, const void *__restrict__ x,
                                                                  const uint16_t *__restrict__ nw, float eps,
                                                                  EpiAttnQKV epi)
{
    using S = AttnQkvShape<NB>;
    constexpr int NT = S::NT, R = S::R;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    __shared__ float red[NB][NT / 64];
    PreNorm<NB, XT, NT> pn;
    pn.issue(x, nw);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's block: one contiguous range of blocks per XCD, as in_proj
    const int xcd = blockIdx.x & 7;
    const int wave = __builtin_amdgcn_readfirstlane((int)((threadIdx.x >> 6) * (gridDim.x >> 3) + (blockIdx.x >> 3)));
    constexpr int NBLK = (ATT_QD + 2 * ATT_KD) / S::RW;
    const int bx = (NBLK + 7) / 8, blk = xcd * bx + wave;
    const bool active = wave < bx && blk < NBLK;
    const int row = min(blk, NBLK - 1) * S::RW;  // the three matrices' sizes are multiples of RW
    const int which = row < ATT_QD ? 0 : row < ATT_QD + ATT_KD ? 1 : 2;
    const int base = which == 0 ? 0 : which == 1 ? ATT_QD : ATT_QD + ATT_KD;
    EpiAttnQKV e = epi;
    e.base = base;
    InProjBlock<NB, EpiAttnQKV, S> run(which == 0 ? Wq : which == 1 ? Wk : Wv, e, row - base, active);
    pn.finish(eps, act_lds, red);
    ActChunk am[NB][2], at[NB];
    act_hidden<NB, R>(am, at, act_lds);
    run.run(am, at);
}

hipError_t launch_attn_qkv(const W4 &Wq, const W4 &Wk, const W4 &Wv, const void *x, int x_t, const uint16_t *norm_w,
                           float eps, int batch, uint16_t *q, uint16_t *kc, uint16_t *vc, const int *pos, int max_len,
                           hipStream_t st)
{
    EpiAttnQKV e{q, kc, vc, pos, max_len, 0};
    const size_t lds = (size_t)batch * (HIDDEN / 32) * ACT_WORDS * 4;
#define NH_LAUNCH(NB)                                                                                           \
    {                                                                                                           \
        using S = AttnQkvShape<NB>;                                                                             \
        constexpr int NBLK = (ATT_QD + 2 * ATT_KD) / S::RW, WPG = S::NT / 64;                                  \
        const int bx = (NBLK + 7) / 8, grid = 8 * ((bx + WPG - 1) / WPG);                                      \
        if (x_t == BF16)                                                                                        \
            launch_k(k_attn_qkv<NB, BF16>, dim3(grid), dim3(S::NT), lds, st, Wq, Wk, Wv, x, norm_w, eps, e);      \
        else                                                                                                    \
            launch_k(k_attn_qkv<NB, F32>, dim3(grid), dim3(S::NT), lds, st, Wq, Wk, Wv, x, norm_w, eps, e);       \
    }
    switch (batch) {
    case 1: NH_LAUNCH(1); break;
    case 2: NH_LAUNCH(2); break;
    case 3: NH_LAUNCH(3); break;
    default: NH_LAUNCH(4); break;
    }
#undef NH_LAUNCH
    return hipGetLastError();
}

// Pre-norm + MLP up projection (K = hidden) + squared ReLU: the in_proj kernel's structure
// with the activation as its epilogue.
// At batch 1 the work-groups have 8 waves instead of in_proj's 12: the 15680 rows make 1960
// blocks of 8, which 12-wave work-groups spread over only 168 CUs.
template <int NB>
struct MlpUpShape {
    static constexpr int NT = NB == 1 ? 512 : InProjShape<NB>::NT;
};

template <int NB, int XT>
__global__ __launch_bounds__(MlpUpShape<NB>::NT, 1) void k_mlp_up_step(W4 W, const void *__restrict__ x,
                                                                   const uint16_t *__restrict__ nw, float eps,
                                                                   EpiReluSq epi)
{
    constexpr int NT = MlpUpShape<NB>::NT, R = InProjShape<NB>::R;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    __shared__ float red[NB][NT / 64];
    PreNorm<NB, XT, NT> pn;
    pn.issue(x, nw);
    __builtin_amdgcn_sched_barrier(0);
    InProjBlock<NB, EpiReluSq> run(W, epi);
    pn.finish(eps, act_lds, red);
    ActChunk am[NB][2], at[NB];
    act_hidden<NB, R>(am, at, act_lds);
    run.run(am, at);
}

// Final norm + one W4 output head + greedy id.  The head has K = hidden, so it shares the
// in_proj chunk layout and pre-norm; its 131072 rows are R-row stages split into one
// contiguous range per XCD and, inside it, one contiguous range per wave (so rows that share
// scale cache lines stay in one L2).  A wave streams its range with two stages in flight,
// keeps the best (logit, row) of each batch row, and the work-group's best goes to
// part_v / part_i [NB][gridDim.x] for k_head_finish.  Logits are stored only on request.
//
// Greedy order: (v, n) beats (bv, bn) when v is not NaN and (bn < 0 or v > bv or
// (v == bv and n < bn)); it is a total order on the candidates, so any reduction tree gives
// the smallest row among those with the largest logit.
__device__ __forceinline__ bool greedy_better(float v, int n, float bv, int bn)
{
    return n >= 0 && v == v && (bn < 0 || v > bv || (v == bv && n < bn));
}

constexpr int HEAD_WGS = 256;  // work-groups of the head kernel: 32 per XCD

template <int NB, int XT>
__global__ __launch_bounds__(InProjShape<NB>::NT, 1) void k_head_step(W4 W, const void *__restrict__ x,
                                                                  const uint16_t *__restrict__ nw, float eps,
                                                                  float *__restrict__ logits,
                                                                  float *__restrict__ part_v,
                                                                  int *__restrict__ part_i)
{
    constexpr int NT = InProjShape<NB>::NT, R = InProjShape<NB>::R, NW = NT / 64;
    extern __shared__ __attribute__((aligned(16))) uint32_t act_lds[];
    __shared__ float red[NB][NW];
    __shared__ float wv[NB][NW];
    __shared__ int wi[NB][NW];
    PreNorm<NB, XT, NT> pn;
    pn.issue(x, nw);
    __builtin_amdgcn_sched_barrier(0);
    IpRows<R> io;
    io.init(W);
    // this wave's stages [s0, s1): an even split per XCD, then per wave inside the XCD
    const long nst = (W.n + R - 1) / R;
    const int xcd = blockIdx.x & 7, nwx = (int)(gridDim.x >> 3) * NW;
    const int wx = __builtin_amdgcn_readfirstlane((int)((blockIdx.x >> 3) * NW + (threadIdx.x >> 6)));
    const long xs = nst * xcd / 8, xn = nst * (xcd + 1) / 8 - xs;
    const int s0 = (int)(xs + xn * wx / nwx), s1 = (int)(xs + xn * (wx + 1) / nwx);
    IpStage<R> A, B;
    io.load(A, min(s0, (int)nst - 1) * R);
    pn.finish(eps, act_lds, red);
    ActChunk am[NB][2], at[NB];
    act_hidden<NB, R>(am, at, act_lds);

    float bv[NB];
    int bi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        bv[b] = -INFINITY;
        bi[b] = -1;
    }
    auto step = [&](const IpStage<R> &g, int s) {
        float sm[R][NB];
        io.template sums<NB>(g, am, at, sm);
        float mine = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int n = s * R + r;
                const float v = sm[r][b];
                if (n < W.n && greedy_better(v, n, bv[b], bi[b])) {
                    bv[b] = v;
                    bi[b] = n;
                }
                if (io.li == r * NB + b) mine = v;
            }
        const int n = s * R + io.li / NB;
        if (logits && io.li < R * NB && n < W.n) logits[(size_t)(io.li % NB) * W.n + n] = mine;
    };
    // no conditional load in the loop (see GemvRunner::run); the last one or two stages peeled
    const int cnt = s1 - s0;
    if (cnt > 0) {
        int s = s0, i = 0;
        for (; i + 2 < cnt; i += 2, s += 2) {
            io.load(B, (s + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            step(A, s);
            io.load(A, (s + 2) * R);
            __builtin_amdgcn_sched_barrier(0);
            step(B, s + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (i + 1 < cnt) {
            io.load(B, (s + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            step(A, s);
            __builtin_amdgcn_sched_barrier(0);
            step(B, s + 1);
        } else {
            step(A, s);
        }
    }
    const int wave = threadIdx.x >> 6;
    if (io.li == 0)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            wv[b][wave] = bv[b];
            wi[b][wave] = bi[b];
        }
    __syncthreads();
    if ((int)threadIdx.x < NB) {
        const int b = threadIdx.x;
        float v = wv[b][0];
        int n = wi[b][0];
        for (int w = 1; w < NW; ++w)
            if (greedy_better(wv[b][w], wi[b][w], v, n)) {
                v = wv[b][w];
                n = wi[b][w];
            }
        part_v[b * gridDim.x + blockIdx.x] = v;
        part_i[b * gridDim.x + blockIdx.x] = n;
    }
}

// The greedy id of each batch row from the work-groups' partial results: one work-group of
// 256 threads, one partial per thread, then wave and work-group reductions in greedy order.
__global__ __launch_bounds__(256) void k_head_finish(const float *__restrict__ part_v,
                                                     const int *__restrict__ part_i, int nparts,
                                                     int batch, int *__restrict__ ids)
{
    __shared__ float sv[4];
    __shared__ int si[4];
    for (int b = 0; b < batch; ++b) {
        float v = -INFINITY;
        int n = -1;
        for (int t = threadIdx.x; t < nparts; t += 256)
            if (greedy_better(part_v[b * nparts + t], part_i[b * nparts + t], v, n)) {
                v = part_v[b * nparts + t];
                n = part_i[b * nparts + t];
            }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float ov = __shfl_xor(v, o, 64);
            const int on = __shfl_xor(n, o, 64);
            if (greedy_better(ov, on, v, n)) {
                v = ov;
                n = on;
            }
        }
        if ((threadIdx.x & 63) == 0) {
            sv[threadIdx.x >> 6] = v;
            si[threadIdx.x >> 6] = n;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < 4; ++w)
                if (greedy_better(sv[w], si[w], v, n)) {
                    v = sv[w];
                    n = si[w];
                }
            ids[b] = n;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ launchers

static int cu_count()
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

// Persistent grid: at most wgs_per_cu work-groups of four waves per CU, each wave walking stages.
static int gemv_grid(int n, int rows_per_stage, int wgs_per_cu)
{
    const int stages = (n + rows_per_stage - 1) / rows_per_stage;
    const int g = (stages + 3) / 4;
    const int cap = wgs_per_cu * cu_count();
    return g < cap ? g : cap;
}

template <int LPR, int CPL, int NB, int RG, int XT>
static hipError_t run_gemv(const W4 &W, const void *x, EpiStore e, hipStream_t st)
{
    const size_t lds = (size_t)NB * (W.k >> 5) * ACT_WORDS * 4;
    const int grid = gemv_grid(W.n, RG * (64 / LPR), gemv_wgs_per_cu(NB, CPL));
    k_gemv<LPR, CPL, NB, RG, XT><<<dim3(grid), dim3(256), lds, st>>>(W, x, e);
    return hipGetLastError();
}

template <int NB, int XT>
static hipError_t gemv_nb(const W4 &W, const void *x, EpiStore e, hipStream_t st)
{
    const int nch = W.k >> 5;
    if (nch <= 32) return run_gemv<32, 1, NB, 2, XT>(W, x, e, st);
    if (nch <= 64) return run_gemv<64, 1, NB, 2, XT>(W, x, e, st);
    if (nch <= 128) return run_gemv<64, 2, NB, 2, XT>(W, x, e, st);
    if (nch <= 192) return run_gemv<64, 3, NB, (NB == 1 ? 2 : 1), XT>(W, x, e, st);
    if (nch <= 256) return run_gemv<64, 4, NB, 1, XT>(W, x, e, st);
    // batch 4 above K = 5120 and batch 2-3 above K = 10240 go to the matrix-core kernel
    if constexpr (NB <= 3)
        if (nch <= 320) return run_gemv<64, 5, NB, 1, XT>(W, x, e, st);
    if constexpr (NB == 1) return run_gemv<64, 8, NB, 1, XT>(W, x, e, st);
    return hipErrorInvalidValue;
}

template <int XT>
static hipError_t launch_gemv_t(const W4 &W, const void *x, int batch, EpiStore e, hipStream_t st)
{
    // K = hidden at batch 3 and 4: the matrix-core kernel of the batched in_proj
    if (W.k == HIDDEN && batch >= 3) {
        const size_t lds = (size_t)batch * (HIDDEN / 32) * ACT_WORDS * 4;
        if (batch == 3)
            launch_k(k_w4_mf<3, XT, false, EpiStore>, dim3(MF_WGS), dim3(256), lds, st, W, x,
                     (const uint16_t *)nullptr, 0.f, e, (uint32_t *)nullptr, 0);
        else
            launch_k(k_w4_mf<4, XT, false, EpiStore>, dim3(MF_WGS), dim3(256), lds, st, W, x,
                     (const uint16_t *)nullptr, 0.f, e, (uint32_t *)nullptr, 0);
        return hipGetLastError();
    }
    // The matrix-core kernel with the activations in LDS where the per-row kernel's registers
    // run out: K above 10240 at batch 2 to 4 (per-row: 28 / 90 / 164 us at K = 15680 against
    // 18-19 us) and K above 5120 at batch 4 (K = 10240: 27.5 against 15.5 us).  Elsewhere the
    // per-row kernel is faster (the matrix-core kernel's activation build takes about 7 us).
    // K up to 16384, i.e. 512 chunks per row: at most NB chunks per thread.
    if (batch >= 2 && (W.k > 10240 || (batch == 4 && W.k > 5120))) {
        switch (batch) {
        case 2: return launch_mfl<2, true>(W, ActPlainK<2, MFL_NT, 2, XT>{x}, e, st);
        case 3: return launch_mfl<3, true>(W, ActPlainK<3, MFL_NT, 3, XT>{x}, e, st);
        default: return launch_mfl<4, true>(W, ActPlainK<4, MFL_NT, 4, XT>{x}, e, st);
        }
    }
    switch (batch) {
    case 1: return gemv_nb<1, XT>(W, x, e, st);
    case 2: return gemv_nb<2, XT>(W, x, e, st);
    case 3: return gemv_nb<3, XT>(W, x, e, st);
    default: return gemv_nb<4, XT>(W, x, e, st);
    }
}

hipError_t launch_gemv(const W4 &W, const void *x, int x_t, int batch, const void *res, int res_t,
                       void *y, int y_t, hipStream_t st)
{
    EpiStore e{y, res, y_t, res_t, W.n};
    return x_t == BF16 ? launch_gemv_t<BF16>(W, x, batch, e, st) : launch_gemv_t<F32>(W, x, batch, e, st);
}

size_t outproj_partial_floats(int batch) { return batch > 1 ? (size_t)NGROUPS * batch * HIDDEN : 0; }

hipError_t launch_outproj_step(const W4 &W, const float *gate, const float *part,
                               float eps, int batch, const void *res, int res_t, void *out, int out_t,
                               float *partial, hipStream_t st)
{
    EpiStore e{out, res, out_t, res_t, W.n};
    if (batch == 1) {
        // one work-group of 8 waves per CU
        const size_t lds = (size_t)(DINNER / 32) * ACT_WORDS * 4;
        const int grid = min(cu_count(), (W.n + 7) / 8);
        launch_k(k_outproj_step, dim3(grid), dim3(512), lds, st, W, gate, part, eps, e);
        return hipGetLastError();
    }
    // batch 2..4: split over the gated-norm groups, then the ordered sum
    const dim3 grid(NGROUPS * (HIDDEN / SK_ROWS)), rgrid((batch * HIDDEN + 255) / 256);
    switch (batch) {
    case 2:
        launch_k(k_outproj_sk<2>, grid, dim3(SK_NT), 0, st, W, gate, part, eps, partial);
        launch_k(k_sk_reduce<2>, rgrid, dim3(256), 0, st, (const float *)partial, e);
        break;
    case 3:
        launch_k(k_outproj_sk<3>, grid, dim3(SK_NT), 0, st, W, gate, part, eps, partial);
        launch_k(k_sk_reduce<3>, rgrid, dim3(256), 0, st, (const float *)partial, e);
        break;
    default:
        launch_k(k_outproj_sk<4>, grid, dim3(SK_NT), 0, st, W, gate, part, eps, partial);
        launch_k(k_sk_reduce<4>, rgrid, dim3(256), 0, st, (const float *)partial, e);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_inproj_step(const W4 &W, const void *x, int x_t, const uint16_t *norm_w,
                              float eps, int batch, uint16_t *z, uint16_t *xc, uint16_t *dtr,
                              uint16_t *conv_state, const uint16_t *conv_w,
                              const uint16_t *conv_b, uint32_t *zero_ptr, int nzero,
                              hipStream_t st)
{
    EpiInProjStep e{z, xc, dtr, conv_state, conv_w, conv_b};
    const size_t lds = (size_t)batch * (HIDDEN / 32) * ACT_WORDS * 4;
#define NH_LAUNCH(NB)                                                                                      \
    {                                                                                                      \
        const int grid = inproj_grid<NB>(W.n);                                                             \
        const dim3 blk(InProjShape<NB>::NT);                                                               \
        if (x_t == BF16)                                                                                   \
            launch_k(k_inproj_step<NB, BF16>, dim3(grid), blk, lds, st, W, x, norm_w, eps, e, zero_ptr, nzero); \
        else                                                                                               \
            launch_k(k_inproj_step<NB, F32>, dim3(grid), blk, lds, st, W, x, norm_w, eps, e, zero_ptr, nzero);  \
    }
#define NH_LAUNCH_MF(NB)                                                                                   \
    {                                                                                                      \
        if (x_t == BF16)                                                                                   \
            launch_k(k_w4_mf<NB, BF16, true, EpiInProjStep>, dim3(MF_WGS), dim3(256), lds, st, W, x, norm_w, eps, e, \
                     zero_ptr, nzero);                                                                     \
        else                                                                                               \
            launch_k(k_w4_mf<NB, F32, true, EpiInProjStep>, dim3(MF_WGS), dim3(256), lds, st, W, x, norm_w, eps, e, \
                     zero_ptr, nzero);                                                                     \
    }
    // the matrix-core kernel from batch 3 on (at batch 2 the per-row kernel is 1 us faster)
    switch (batch) {
    case 1: NH_LAUNCH(1); break;
    case 2: NH_LAUNCH(2); break;
    case 3: NH_LAUNCH_MF(3); break;
    default: NH_LAUNCH_MF(4); break;
    }
#undef NH_LAUNCH
#undef NH_LAUNCH_MF
    return hipGetLastError();
}

hipError_t launch_mlp_up_step(const W4 &W, const void *x, int x_t, const uint16_t *norm_w, float eps, int batch,
                              uint16_t *h, hipStream_t st)
{
    EpiReluSq e{h, W.n};
    const size_t lds = (size_t)batch * (HIDDEN / 32) * ACT_WORDS * 4;
#define NH_LAUNCH(NB)                                                                                      \
    {                                                                                                      \
        constexpr int RW = InProjShape<NB>::RW, WPG = MlpUpShape<NB>::NT / 64;                             \
        const int bx = ((W.n + RW - 1) / RW + 7) / 8, grid = 8 * ((bx + WPG - 1) / WPG);                   \
        const dim3 blk(MlpUpShape<NB>::NT);                                                                \
        if (x_t == BF16)                                                                                   \
            launch_k(k_mlp_up_step<NB, BF16>, dim3(grid), blk, lds, st, W, x, norm_w, eps, e);             \
        else                                                                                               \
            launch_k(k_mlp_up_step<NB, F32>, dim3(grid), blk, lds, st, W, x, norm_w, eps, e);              \
    }
    switch (batch) {
    case 1: NH_LAUNCH(1); break;
    case 2: NH_LAUNCH(2); break;
    case 3: NH_LAUNCH(3); break;
    default: NH_LAUNCH(4); break;
    }
#undef NH_LAUNCH
    return hipGetLastError();
}

size_t head_ws_bytes(int batch) { return (size_t)batch * HEAD_WGS * (sizeof(float) + sizeof(int)); }

hipError_t launch_head(const W4 &W, const void *x, int x_t, const uint16_t *norm_w, float eps, int batch,
                       float *logits, int *ids, void *ws, hipStream_t st)
{
    float *pv = reinterpret_cast<float *>(ws);
    int *pi = reinterpret_cast<int *>(pv + (size_t)batch * HEAD_WGS);
    const size_t lds = (size_t)batch * (HIDDEN / 32) * ACT_WORDS * 4;
#define NH_LAUNCH(NB)                                                                                   \
    {                                                                                                   \
        const dim3 blk(InProjShape<NB>::NT);                                                            \
        if (x_t == BF16)                                                                                \
            launch_k(k_head_step<NB, BF16>, dim3(HEAD_WGS), blk, lds, st, W, x, norm_w, eps, logits, pv, pi); \
        else                                                                                            \
            launch_k(k_head_step<NB, F32>, dim3(HEAD_WGS), blk, lds, st, W, x, norm_w, eps, logits, pv, pi);  \
    }
    switch (batch) {
    case 1: NH_LAUNCH(1); break;
    case 2: NH_LAUNCH(2); break;
    case 3: NH_LAUNCH(3); break;
    default: NH_LAUNCH(4); break;
    }
#undef NH_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_head_finish<<<dim3(1), dim3(256), 0, st>>>(pv, pi, HEAD_WGS, batch, ids);
    return hipGetLastError();
}

}  // namespace nh
