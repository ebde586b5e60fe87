// rows.hip -- row-wise kernels of the sequence (full-history) path on gfx950:
// RMSNorm, gated RMSNorm, the causal conv over T positions and the bf16 -> fp16 staging
// of matrix-core operands.  All are HBM-streaming kernels with 128-bit accesses.
#include "nh_device.hpp"
#include "nh_kernels.hpp"

namespace nh {

// Sum over the 8 lanes that hold one 64-element quantisation group (8 values each).
__device__ __forceinline__ float group8_sum(float v)
{
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);  // row_half_mirror: the other quad of the 8 lanes
    return v;
}

// Eight consecutive values of y (bf16 bits or fp32) at element offset i.
template <int YT>
__device__ __forceinline__ void load_y8(const void *y, size_t i, float (&v)[8])
{
    if constexpr (YT == BF16) {
        const uint4 t = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(y) + i);
        const uint32_t a[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16lo(a[e]);
            v[2 * e + 1] = bf16hi(a[e]);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(y) + i);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ __forceinline__ float block_sum256(float v, float *red)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return t;
}

// Store eight values that are already bf16-exact, as bf16 bits (kind 0) or as fp16 bits
// (kind 1, the W4 matrix product's operand format: the eight values in pair order
// (0,4) (1,5) (2,6) (3,7), the order in which that product dequantises a packed weight word).
__device__ __forceinline__ void store8(uint16_t *dst, const float *v, int kind)
{
    uint4 o;
    if (kind == 0) {
        o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        o.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
        o.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    } else {
        o.x = pack_f16x2(v[0], v[4]);
        o.y = pack_f16x2(v[1], v[5]);
        o.z = pack_f16x2(v[2], v[6]);
        o.w = pack_f16x2(v[3], v[7]);
    }
    *reinterpret_cast<uint4 *>(dst) = o;
}

template <int XT>
__device__ __forceinline__ void ld8(const void *x, size_t e, float *v)
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

// ---------------------------------------------------------------- RMSNorm
// One work-group per row; d % 64 == 0, d <= 256*8*MAXV.
constexpr int RN_MAXV = 4;

template <int XT>
__global__ __launch_bounds__(256) void k_rmsnorm(const void *__restrict__ x,
                                                 const uint16_t *__restrict__ w,
                                                 uint16_t *__restrict__ u, int kind,
                                                 float *__restrict__ su, int d, float eps)
{
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    const int nv = d >> 3;
    float v[RN_MAXV][8];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < RN_MAXV; ++i) {
        const int vi = threadIdx.x + 256 * i;
        if (vi < nv) {
            ld8<XT>(x, row * d + 8 * vi, v[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
        }
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < RN_MAXV; ++i) {
        const int vi = threadIdx.x + 256 * i;
        float s = 0.f;
        if (vi < nv) {
            uint4 ww = *reinterpret_cast<const uint4 *>(w + 8 * vi);
            const float w8[8] = {bf16lo(ww.x), bf16hi(ww.x), bf16lo(ww.y), bf16hi(ww.y),
                                 bf16lo(ww.z), bf16hi(ww.z), bf16lo(ww.w), bf16hi(ww.w)};
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = round_bf16(v[i][e] * r * w8[e]);
                s += o[e];
            }
            store8(u + row * d + 8 * vi, o, kind);
        }
        // 256 is a multiple of 8, so the 8 lanes of a group share the same i.
        s = group8_sum(s);
        if (su && vi < nv && (vi & 7) == 0) su[(size_t)(vi >> 3) * gridDim.x + row] = s;
    }
}

hipError_t launch_rmsnorm(const void *x, int x_t, const uint16_t *w, uint16_t *u, int out_kind,
                          float *su, int rows, int d, float eps, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    dim3 grid(rows), block(256);
    if (x_t == BF16)
        k_rmsnorm<BF16><<<grid, block, 0, st>>>(x, w, u, out_kind, su, d, eps);
    else
        k_rmsnorm<F32><<<grid, block, 0, st>>>(x, w, u, out_kind, su, d, eps);
    return hipGetLastError();
}

// ---------------------------------------------------------- gated RMSNorm
// One work-group per (row, group of channels).  g = y * silu(z); out = g / rms(g) * w.
template <int YT>
__global__ __launch_bounds__(256) void k_rmsnorm_gated(const void *__restrict__ y,
                                                       const uint16_t *__restrict__ z, long ld_z,
                                                       const uint16_t *__restrict__ w,
                                                       uint16_t *__restrict__ out, int kind,
                                                       float *__restrict__ su, int d, int group,
                                                       float eps)
{
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    const int j = blockIdx.y;
    const int nv = group >> 3;
    const size_t base = (size_t)j * group;
    float gv[RN_MAXV][8];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < RN_MAXV; ++i) {
        const int vi = threadIdx.x + 256 * i;
        if (vi < nv) {
            float yv[8];
            load_y8<YT>(y, row * d + base + 8 * vi, yv);
            const uint4 zz = *reinterpret_cast<const uint4 *>(z + row * ld_z + base + 8 * vi);
            const uint32_t za[4] = {zz.x, zz.y, zz.z, zz.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gv[i][2 * e] = yv[2 * e] * silu(bf16lo(za[e]));
                gv[i][2 * e + 1] = yv[2 * e + 1] * silu(bf16hi(za[e]));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += gv[i][e] * gv[i][e];
        }
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)group + eps);
#pragma unroll
    for (int i = 0; i < RN_MAXV; ++i) {
        const int vi = threadIdx.x + 256 * i;
        float s = 0.f;
        if (vi < nv) {
            const uint4 ww = *reinterpret_cast<const uint4 *>(w + base + 8 * vi);
            const float w8[8] = {bf16lo(ww.x), bf16hi(ww.x), bf16lo(ww.y), bf16hi(ww.y),
                                 bf16lo(ww.z), bf16hi(ww.z), bf16lo(ww.w), bf16hi(ww.w)};
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = round_bf16(gv[i][e] * r * w8[e]);
                s += o[e];
            }
            store8(out + row * d + base + 8 * vi, o, kind);
        }
        s = group8_sum(s);
        if (su && vi < nv && (vi & 7) == 0) su[(size_t)((base >> 6) + (vi >> 3)) * gridDim.x + row] = s;
    }
}

// The same with one wave per (row, group) for groups of at most 2048 channels: the group's
// sum of squares is a wave reduction (no LDS, no barrier), and a work-group of four waves
// takes four consecutive (row, group) units.  Same products and rounding points as above; the
// sum of squares is accumulated in another order.
constexpr int RG_MAXI = 4;  // 16-byte vectors per lane: group <= 64 * 8 * RG_MAXI

template <int YT>
__global__ __launch_bounds__(256) void k_rmsnorm_gated_w(const void *__restrict__ y,
                                                         const uint16_t *__restrict__ z, long ld_z,
                                                         const uint16_t *__restrict__ w,
                                                         uint16_t *__restrict__ out, int kind,
                                                         float *__restrict__ su, int rows, int d,
                                                         int group, float eps)
{
    const int ng = d / group;
    const int unit = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if ((long)unit >= (long)rows * ng) return;  // wave-uniform; the kernel has no barrier
    const size_t row = unit / ng;
    const int j = unit - (int)row * ng, lane = threadIdx.x & 63, nv = group >> 3;
    const size_t base = (size_t)j * group;
    float gv[RG_MAXI][8];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < RG_MAXI; ++i) {
        const int vi = lane + 64 * i;
        if (vi < nv) {
            float yv[8];
            load_y8<YT>(y, row * d + base + 8 * vi, yv);
            const uint4 zz = *reinterpret_cast<const uint4 *>(z + row * ld_z + base + 8 * vi);
            const uint32_t za[4] = {zz.x, zz.y, zz.z, zz.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gv[i][2 * e] = yv[2 * e] * silu(bf16lo(za[e]));
                gv[i][2 * e + 1] = yv[2 * e + 1] * silu(bf16hi(za[e]));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += gv[i][e] * gv[i][e];
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)group + eps);
#pragma unroll
    for (int i = 0; i < RG_MAXI; ++i) {
        const int vi = lane + 64 * i;
        float s = 0.f;
        if (vi < nv) {
            const uint4 ww = *reinterpret_cast<const uint4 *>(w + base + 8 * vi);
            const float w8[8] = {bf16lo(ww.x), bf16hi(ww.x), bf16lo(ww.y), bf16hi(ww.y),
                                 bf16lo(ww.z), bf16hi(ww.z), bf16lo(ww.w), bf16hi(ww.w)};
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = round_bf16(gv[i][e] * r * w8[e]);
                s += o[e];
            }
            store8(out + row * d + base + 8 * vi, o, kind);
        }
        // 64 is a multiple of 8, so the 8 lanes of a 64-channel group share the same i
        s = group8_sum(s);
        if (su && vi < nv && (vi & 7) == 0) su[(size_t)((base >> 6) + (vi >> 3)) * rows + row] = s;
    }
}

hipError_t launch_rmsnorm_gated(const void *y, int y_t, const uint16_t *z, long ld_z,
                                const uint16_t *w, uint16_t *out, int out_kind, float *su,
                                int rows, int d, int group, float eps, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (group <= 64 * 8 * RG_MAXI) {
        const dim3 grid((unsigned)(((long)rows * (d / group) + 3) / 4)), block(256);
        if (y_t == BF16)
            k_rmsnorm_gated_w<BF16><<<grid, block, 0, st>>>(y, z, ld_z, w, out, out_kind, su, rows, d, group, eps);
        else
            k_rmsnorm_gated_w<F32><<<grid, block, 0, st>>>(y, z, ld_z, w, out, out_kind, su, rows, d, group, eps);
    } else {
        dim3 grid(rows, d / group), block(256);
        if (y_t == BF16)
            k_rmsnorm_gated<BF16><<<grid, block, 0, st>>>(y, z, ld_z, w, out, out_kind, su, d, group, eps);
        else
            k_rmsnorm_gated<F32><<<grid, block, 0, st>>>(y, z, ld_z, w, out, out_kind, su, d, group, eps);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------- conv over T
// Thread per (sequence, channel, block of CT positions): causal depthwise conv, kernel 4,
// tap 3 on the newest input, left context from the carried state (row 0 oldest) or zeros.
constexpr int CT = 16;

__global__ __launch_bounds__(256) void k_conv_seq(const uint16_t *__restrict__ xbc, long ld, int T,
                                                  const uint16_t *__restrict__ s_in,
                                                  uint16_t *__restrict__ s_out,
                                                  const uint16_t *__restrict__ w,
                                                  const uint16_t *__restrict__ bias,
                                                  uint16_t *__restrict__ out, int channels)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int t0 = blockIdx.y * CT;
    const int b = blockIdx.z;
    if (c >= channels) return;
    const uint16_t *xb = xbc + (size_t)b * T * ld;
    const uint16_t *si = s_in ? s_in + (size_t)b * (CONVK - 1) * channels : nullptr;
    auto in = [&](int tau) -> float {
        if (tau >= 0) return bf16_to_f32(xb[(size_t)tau * ld + c]);
        return si ? bf16_to_f32(si[(size_t)(tau + CONVK - 1) * channels + c]) : 0.f;
    };
    const uint2 wv = *reinterpret_cast<const uint2 *>(w + 4 * (size_t)c);
    const float w0 = bf16lo(wv.x), w1 = bf16hi(wv.x), w2 = bf16lo(wv.y), w3 = bf16hi(wv.y);
    const float bb = bf16_to_f32(bias[c]);
    float x0 = in(t0 - 3), x1 = in(t0 - 2), x2 = in(t0 - 1);
    const int tend = min(T, t0 + CT);
    for (int t = t0; t < tend; ++t) {
        const float x3 = bf16_to_f32(xb[(size_t)t * ld + c]);
        float a = fmaf(w0, x0, bb);
        a = fmaf(w1, x1, a);
        a = fmaf(w2, x2, a);
        a = fmaf(w3, x3, a);
        out[((size_t)b * T + t) * channels + c] = f32_to_bf16(silu(a));
        x0 = x1; x1 = x2; x2 = x3;
    }
    if (s_out && tend == T) {
        uint16_t *so = s_out + (size_t)b * (CONVK - 1) * channels;
        for (int r = 0; r < CONVK - 1; ++r) {
            const int tau = T - (CONVK - 1) + r;
            uint16_t v;
            if (tau >= 0)
                v = xb[(size_t)tau * ld + c];
            else
                v = si ? si[(size_t)(tau + CONVK - 1) * channels + c] : (uint16_t)0;
            so[(size_t)r * channels + c] = v;
        }
    }
}

// The same conv with 8 channels per thread (16-byte loads and stores of each position's
// row) and CT8 positions per thread; the products are summed in the same order, so the
// results equal k_conv_seq's.  Needs channels and ld multiples of 8 and 16-byte aligned rows.
constexpr int CT8 = 32;

__device__ __forceinline__ void unpack_bf16x8(uint4 r, float (&v)[8])
{
    v[0] = bf16lo(r.x); v[1] = bf16hi(r.x); v[2] = bf16lo(r.y); v[3] = bf16hi(r.y);
    v[4] = bf16lo(r.z); v[5] = bf16hi(r.z); v[6] = bf16lo(r.w); v[7] = bf16hi(r.w);
}

__global__ __launch_bounds__(256) void k_conv_seq8(const uint16_t *__restrict__ xbc, long ld, int T,
                                                   const uint16_t *__restrict__ s_in,
                                                   uint16_t *__restrict__ s_out,
                                                   const uint16_t *__restrict__ w,
                                                   const uint16_t *__restrict__ bias,
                                                   uint16_t *__restrict__ out, int channels)
{
    const int c = 8 * (blockIdx.x * 256 + threadIdx.x);
    const int t0 = blockIdx.y * CT8;
    const int b = blockIdx.z;
    if (c >= channels) return;
    const uint16_t *xb = xbc + (size_t)b * T * ld + c;
    const uint16_t *si = s_in ? s_in + (size_t)b * (CONVK - 1) * channels + c : nullptr;
    auto row = [&](int tau) -> uint4 {
        if (tau >= 0) return *reinterpret_cast<const uint4 *>(xb + (size_t)tau * ld);
        if (si) return *reinterpret_cast<const uint4 *>(si + (size_t)(tau + CONVK - 1) * channels);
        return make_uint4(0u, 0u, 0u, 0u);
    };
    float wt[8][4], bb[8];
    {
        const uint4 *wp = reinterpret_cast<const uint4 *>(w + 4 * (size_t)c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // channels 2q and 2q + 1, taps 0..3 each
            const uint4 r = wp[q];
            wt[2 * q][0] = bf16lo(r.x); wt[2 * q][1] = bf16hi(r.x); wt[2 * q][2] = bf16lo(r.y); wt[2 * q][3] = bf16hi(r.y);
            wt[2 * q + 1][0] = bf16lo(r.z); wt[2 * q + 1][1] = bf16hi(r.z);
            wt[2 * q + 1][2] = bf16lo(r.w); wt[2 * q + 1][3] = bf16hi(r.w);
        }
        unpack_bf16x8(*reinterpret_cast<const uint4 *>(bias + c), bb);
    }
    float x0[8], x1[8], x2[8];
    unpack_bf16x8(row(t0 - 3), x0);
    unpack_bf16x8(row(t0 - 2), x1);
    unpack_bf16x8(row(t0 - 1), x2);
    const int tend = min(T, t0 + CT8);
    uint16_t *ob = out + ((size_t)b * T) * channels + c;
    for (int t = t0; t < tend; t += 4) {
        // the rows of up to four positions are loaded before any of them is used
        uint4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = row(min(t + u, tend - 1));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t + u >= tend) break;
            float x3[8], o[8];
            unpack_bf16x8(r[u], x3);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = fmaf(wt[e][0], x0[e], bb[e]);
                a = fmaf(wt[e][1], x1[e], a);
                a = fmaf(wt[e][2], x2[e], a);
                a = fmaf(wt[e][3], x3[e], a);
                o[e] = silu(a);
                x0[e] = x1[e];
                x1[e] = x2[e];
                x2[e] = x3[e];
            }
            store8(ob + (size_t)(t + u) * channels, o, 0);
        }
    }
    if (s_out && tend == T) {
        uint16_t *so = s_out + (size_t)b * (CONVK - 1) * channels + c;
#pragma unroll
        for (int q = 0; q < CONVK - 1; ++q)
            *reinterpret_cast<uint4 *>(so + (size_t)q * channels) = row(T - (CONVK - 1) + q);
    }
}

hipError_t launch_conv_seq(const uint16_t *xbc, long ld, int T, const uint16_t *state_in,
                           uint16_t *state_out, const uint16_t *w, const uint16_t *b,
                           uint16_t *out, int batch, int channels, hipStream_t st)
{
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    if (channels % 8 == 0 && ld % 8 == 0 && al16(xbc) && al16(w) && al16(b) && al16(out) &&
        (!state_in || al16(state_in)) && (!state_out || al16(state_out))) {
        dim3 grid((channels / 8 + 255) / 256, (T + CT8 - 1) / CT8, batch), block(256);
        k_conv_seq8<<<grid, block, 0, st>>>(xbc, ld, T, state_in, state_out, w, b, out, channels);
    } else {
        dim3 grid((channels + 255) / 256, (T + CT - 1) / CT, batch), block(256);
        k_conv_seq<<<grid, block, 0, st>>>(xbc, ld, T, state_in, state_out, w, b, out, channels);
    }
    return hipGetLastError();
}

// ------------------------------------------------------- bf16 -> fp16 bits
// The W4 matrix product's operand format: fp16 bits, each 8-value chunk in pair order
// (0,4) (1,5) (2,6) (3,7); plus the sum of each row's 64-value groups, [group][row].
__global__ __launch_bounds__(256) void k_to_f16(const uint16_t *__restrict__ x,
                                                uint16_t *__restrict__ xh, float *__restrict__ su,
                                                size_t nvec, int kvec)
{
    const size_t v = (size_t)blockIdx.x * 256 + threadIdx.x;
    float s = 0.f;
    if (v < nvec) {
        const uint4 w = *reinterpret_cast<const uint4 *>(x + 8 * v);
        uint4 o;
        o.x = pack_f16x2(bf16lo(w.x), bf16lo(w.z));
        o.y = pack_f16x2(bf16hi(w.x), bf16hi(w.z));
        o.z = pack_f16x2(bf16lo(w.y), bf16lo(w.w));
        o.w = pack_f16x2(bf16hi(w.y), bf16hi(w.w));
        *reinterpret_cast<uint4 *>(xh + 8 * v) = o;
        s = sum_bf16x8(w);
    }
    s = group8_sum(s);
    // kvec % 8 == 0, so a group never straddles two rows; su is [group][row]
    if (v < nvec && (v & 7) == 0) {
        const size_t gi = v >> 3, kg = (size_t)kvec >> 3;
        su[(gi % kg) * (nvec / kvec) + gi / kg] = s;
    }
}

hipError_t launch_to_f16(const uint16_t *x, uint16_t *xh, float *su, int M, int K, hipStream_t st)
{
    const size_t nvec = (size_t)M * K / 8;
    dim3 grid((unsigned)((nvec + 255) / 256)), block(256);
    k_to_f16<<<grid, block, 0, st>>>(x, xh, su, nvec, K / 8);
    return hipGetLastError();
}

}  // namespace nh
