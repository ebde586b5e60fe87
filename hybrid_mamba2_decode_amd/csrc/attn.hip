// attn.hip -- decode attention of the hybrid stack's attention layers (gfx950).
//
// One new query position per sequence attends over its key/value cache, positions
// 0 .. pos[b] (the new k and v already appended at pos[b]).  Grouped-query attention as the
// issue page "feat(nemotron_voicechat): ... offline duplex inference #1374", section
// "config.json" sets it: 40 query heads of 128 on 8 key/value heads, query head h reading
// key/value head h / 5; scores q . k / sqrt(128), softmax over every cached position.
//
// The cache stream is the HBM cost (512 bytes of k and v per position and key/value head), so
// the positions are split over work-groups: grid (split, kv head, sequence).  A work-group
// owns one key/value head -- its five query heads share every k and v read -- and a range of
// positions, walked in 64-position tiles with an online softmax (running maximum and sum per
// head, in base 2); it leaves (max, sum, unnormalised output) per head, and k_attn_combine
// merges the splits into o = bf16(sum_s e_s acc_s / sum_s e_s l_s), e_s = 2^(m_s - max_s m_s).
#include "nh_device.hpp"
#include "nh_kernels.hpp"

#include <algorithm>

namespace nh {

namespace {

constexpr int HEADS = 40, KVH = 8, HD = 128, REP = HEADS / KVH;  // 5 query heads per kv head
constexpr int TILE = 64;                                         // positions per tile
constexpr int PART = 16 + REP * HD;                              // floats per (split, kv head): m, l, acc
constexpr int MAX_SPLIT = 64;

// Positions per split for a cache of L positions: a multiple of the tile.  Split s owns
// [s c, min(L, (s + 1) c)); splits past L own nothing.
__device__ __forceinline__ int split_len(int L, int nsplit)
{
    const int c = (L + nsplit - 1) / nsplit;
    return (c + TILE - 1) / TILE * TILE;
}

typedef __bf16 bf16x2t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2t, a), __builtin_bit_cast(bf16x2t, b), c, false);
}

__device__ __forceinline__ float dot8(uint4 a, uint4 b, float c)
{
    c = dot2(a.x, b.x, c);
    c = dot2(a.y, b.y, c);
    c = dot2(a.z, b.z, c);
    return dot2(a.w, b.w, c);
}

// One tile's loads for a lane: its k piece (score role) and its four value rows (value role),
// positions clamped into the split's range so that every load stays in it.
struct TileRegs {
    uint4 k[4], v[4];
};

__device__ __forceinline__ void load_tile(TileRegs &r, const uint16_t *kp, const uint16_t *vp, int t0, int plast,
                                          int t)
{
    const int pk = min(t0 + (t >> 2), plast);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.k[j] = *reinterpret_cast<const uint4 *>(kp + (size_t)pk * HD + 8 * ((t & 3) + 4 * j));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pv = min(t0 + (t >> 4) + 16 * i, plast);
        r.v[i] = *reinterpret_cast<const uint4 *>(vp + (size_t)pv * HD + 8 * (t & 15));
    }
}

// Thread roles inside a 256-thread work-group, per tile:
//   scores:  position p = t / 4 of the tile, dims 8 (t % 4 + 4 j) .. + 7 for j < 4 (the quad
//            reads the 256-byte k row as four 64-byte pieces); quad sums give q_h . k_p.
//   weights: the quad's lane i computes 2^(s - m) for query head i (lane 0 also head 4).
//   values:  dims 8 (t % 16) .. + 7 over positions t / 16 + 16 i, i < 4 (16 lanes read one
//            256-byte value row).
// The next tile's loads are issued before the current tile is computed.
__global__ __launch_bounds__(256) void k_attn_decode(const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
                                                     const uint16_t *__restrict__ vc, const int *__restrict__ pos,
                                                     int max_len, float *__restrict__ part)
{
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z, nsplit = gridDim.x;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    // the five query heads' dims of this lane (score role), bf16 pairs; issued before the
    // position is known
    const int dq = t & 3;
    uint4 qv[REP][4];
#pragma unroll
    for (int h = 0; h < REP; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qv[h][j] = *reinterpret_cast<const uint4 *>(q + (size_t)b * HEADS * HD + (g * REP + h) * HD + 8 * (dq + 4 * j));
    const int P = pos[b];
    if (P < 0 || P >= max_len) return;  // the combine writes NaN for this sequence
    const int L = P + 1, c = split_len(L, nsplit);
    const int p0 = s * c, p1 = min(L, p0 + c);
    if (p0 >= p1) return;  // nothing here; the combine reads only the splits below L

    __shared__ float wl[2][REP][TILE];  // softmax weights of a tile (double-buffered)
    __shared__ float rm[2][4][REP];     // per-wave tile maxima of the scores
    __shared__ __attribute__((aligned(16))) float red[4][REP * HD];  // final cross-wave sums of acc
    __shared__ float redl[4][REP];      // and of l

    const size_t kvbase = ((size_t)b * KVH + g) * max_len * HD;
    const uint16_t *kp = kc + kvbase, *vp = vc + kvbase;

    // log2(e) / sqrt(128): scores in base 2
    const float scale = 1.4426950408889634f * 0.08838834764831845f;
    float m[REP], l[REP], acc[REP][8];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    TileRegs cur, nxt;
    load_tile(nxt, kp, vp, p0, p1 - 1, t);
    int buf = 0;
    for (int t0 = p0; t0 < p1; t0 += TILE, buf ^= 1) {
        cur = nxt;
        load_tile(nxt, kp, vp, t0 + TILE, p1 - 1, t);  // past the range: clamped re-reads of the last row
        const int pk = t0 + (t >> 2);
        float sc[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) a = dot8(qv[h][j], cur.k[j], a);
            a += dpp_mov<0xB1>(a);  // quad_perm [1,0,3,2]
            a += dpp_mov<0x4E>(a);  // quad_perm [2,3,0,1]
            sc[h] = pk < p1 ? a * scale : -INFINITY;
        }
        // tile maximum per head: over the wave, then over the four waves
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            const float v = wave_max(sc[h]);  // the quad's lanes hold equal values
            if (lane == 0) rm[buf][wave][h] = v;
        }
        __syncthreads();
        float alpha[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            const float tm = fmaxf(fmaxf(rm[buf][0][h], rm[buf][1][h]), fmaxf(rm[buf][2][h], rm[buf][3][h]));
            const float mn = fmaxf(m[h], tm);  // finite: every tile holds a position
            alpha[h] = exp2f(m[h] - mn);
            m[h] = mn;
        }
        // weights of position pk: lane dq takes head dq, lane 0 also head 4; l collects them
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            l[h] *= alpha[h];
            if (dq == (h & 3)) {
                const float w = exp2f(sc[h] - m[h]);  // 0 past the range
                wl[buf][h][t >> 2] = w;
                l[h] += w;
            }
        }
        __syncthreads();
        // values
#pragma unroll
        for (int h = 0; h < REP; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 vr = cur.v[i];
            const float v8[8] = {bf16lo(vr.x), bf16hi(vr.x), bf16lo(vr.y), bf16hi(vr.y),
                                 bf16lo(vr.z), bf16hi(vr.z), bf16lo(vr.w), bf16hi(vr.w)};
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                const float w = wl[buf][h][(t >> 4) + 16 * i];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, v8[e], acc[h][e]);
            }
        }
    }

    // acc over the 16 position groups: the wave's four (lanes 16 apart), then the four waves
#pragma unroll
    for (int h = 0; h < REP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[h][e];
            v = xor32_sum(xor16_sum(v));
            acc[h][e] = v;
        }
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            float4 *d4 = reinterpret_cast<float4 *>(&red[wave][h * HD + 8 * lane]);
            d4[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
            d4[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        }
    }
#pragma unroll
    for (int h = 0; h < REP; ++h) {
        const float lw = wave_sum(l[h]);
        if (lane == 0) redl[wave][h] = lw;
    }
    __syncthreads();
    float *dst = part + (((size_t)b * KVH + g) * nsplit + s) * PART;
    if (t < REP) {
        float mv = m[0];
#pragma unroll
        for (int h = 1; h < REP; ++h) mv = t == h ? m[h] : mv;
        dst[t] = mv;
        dst[REP + t] = redl[0][t] + redl[1][t] + redl[2][t] + redl[3][t];
    }
    for (int e = t; e < REP * HD; e += 256) dst[16 + e] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
}

// o[b][h * 128 + d] = bf16(sum_s e_s acc_s[d] / sum_s e_s l_s) over the splits that hold
// positions; NaN for a sequence whose position is outside the cache.  One wave per query head:
// lane s holds split s's maximum and sum (the splits' loads all in flight at once), lane d
// sums dims d and d + 64.
__global__ __launch_bounds__(64) void k_attn_combine(const float *__restrict__ part, const int *__restrict__ pos,
                                                     int max_len, int nsplit, uint16_t *__restrict__ o)
{
    const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int g = hq / REP, h = hq % REP;
    const float *src = part + ((size_t)b * KVH + g) * nsplit * PART;
    const int P = pos[b];
    uint16_t *dst = o + (size_t)b * HEADS * HD + hq * HD;
    if (P < 0 || P >= max_len) {
        dst[lane] = dst[lane + 64] = 0x7FC0;  // NaN
        return;
    }
    const int L = P + 1, c = split_len(L, nsplit), ns = (L + c - 1) / c;  // 1 .. 64
    const bool have = lane < ns;
    const float ms = have ? src[(size_t)lane * PART + h] : -INFINITY;
    const float ls = have ? src[(size_t)lane * PART + REP + h] : 0.f;
    const float M = wave_max(ms);
    const float es = have ? exp2f(ms - M) : 0.f;
    const float den = wave_sum(es * ls);
    float n0 = 0.f, n1 = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sj = min(s0 + j, ns - 1);  // past ns: weight 0, an in-range row re-read
            const float e = s0 + j < ns ? __shfl(es, sj, 64) : 0.f;
            const float *a = src + (size_t)sj * PART + 16 + h * HD;
            n0 = fmaf(e, a[lane], n0);
            n1 = fmaf(e, a[lane + 64], n1);
        }
    }
    dst[lane] = f32_to_bf16(n0 / den);
    dst[lane + 64] = f32_to_bf16(n1 / den);
}

// Splits per (sequence, kv head): about 512 work-groups in all (two per CU), at most one split
// per tile of the cache.
int max_splits(int batch) { return std::max(1, std::min((512 + 8 * batch - 1) / (8 * batch), MAX_SPLIT)); }

int attn_splits(int batch, int max_len)
{
    const int tiles = (max_len + TILE - 1) / TILE;
    return std::max(1, std::min(max_splits(batch), tiles));
}

}  // namespace

size_t attn_part_bytes(int batch) { return (size_t)batch * KVH * max_splits(batch) * PART * sizeof(float); }

hipError_t launch_attn_decode(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, const int *pos, int max_len,
                              int batch, float *part, uint16_t *o, hipStream_t st)
{
    const int ns = attn_splits(batch, max_len);
    launch_k(k_attn_decode, dim3(ns, KVH, batch), dim3(256), 0, st, q, kc, vc, pos, max_len, part);
    launch_k(k_attn_combine, dim3(HEADS, batch), dim3(64), 0, st, (const float *)part, pos, max_len, ns, o);
    return hipGetLastError();
}

}  // namespace nh
