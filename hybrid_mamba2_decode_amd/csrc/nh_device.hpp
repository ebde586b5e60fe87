// nh_device.hpp -- device helpers shared by the libnhmamba kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nh {

// Nemotron-H mixer dimensions (text_config of the issue page "feat(nemotron_voicechat):
// ... #1374", section "config.json").
constexpr int HIDDEN = 4480;
constexpr int NHEADS = 128;
constexpr int HDIM = 80;
constexpr int DSTATE = 128;
constexpr int NGROUPS = 8;
constexpr int CONVK = 4;
constexpr int DINNER = NHEADS * HDIM;                        // 10240
constexpr int CONVDIM = DINNER + 2 * NGROUPS * DSTATE;       // 12288
constexpr int NIN = 2 * DINNER + 2 * NGROUPS * DSTATE + NHEADS;  // 22656
constexpr int HPG = NHEADS / NGROUPS;                        // 16 heads per B/C group
constexpr int GNORM = DINNER / NGROUPS;                      // 1280 channels per gated-norm group
constexpr int OFF_B = DINNER;                                // B inside x|B|C
constexpr int OFF_C = DINNER + NGROUPS * DSTATE;             // C inside x|B|C
constexpr int QMAX = 256;                                    // largest scan chunk

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest bf16, ties to even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two floats -> packed bf16 pair (low half = lo), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
    const bf16x2n v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// Two floats that are exactly representable in fp16 -> packed fp16x2 (round toward
// zero is exact for them; values below the fp16 normal range are truncated).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Packed bf16x2 word -> packed fp16x2 word (exact inside the fp16 range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) { return pack_f16x2(bf16lo(w), bf16hi(w)); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ float sum_bf16x8(uint4 v)
{
    return ((bf16lo(v.x) + bf16hi(v.x)) + (bf16lo(v.y) + bf16hi(v.y))) +
           ((bf16lo(v.z) + bf16hi(v.z)) + (bf16lo(v.w) + bf16hi(v.w)));
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

__device__ __forceinline__ float softplus(float v) { return fmaxf(v, 0.0f) + log1pf(__expf(-fabsf(v))); }

// softplus with a short log1p: max(v, 0) + log1p(y), y = exp(-|v|) in (0, 1]; below 2^-6 a
// 4-term series (truncation < y^5 / 5), above it the hardware logarithm of 1 + y (whose
// argument is then >= 1.0156, so its absolute error is a small relative one).  About 1e-6
// relative; used where dt is computed per position in bulk.
__device__ __forceinline__ float softplus_fast(float v)
{
    const float y = __expf(-fabsf(v));
    const float ser = y * (1.0f - y * (0.5f - y * (1.0f / 3.0f - 0.25f * y)));
    return fmaxf(v, 0.0f) + (y < 0.015625f ? ser : __logf(1.0f + y));
}

// Cross-lane moves: DPP inside rows of 16 lanes; across rows, the swap instructions of this
// target, which exchange rows 0/2 with rows 1/3 (16-lane swap) or lanes 0-31 with 32-63
// (32-lane swap) between two registers.  Given the same register twice, the two results hold
// the value and its partner's, so their sum is v[i] + v[i ^ 16] (or ^ 32), equal in both lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor16_sum(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over the 16 lanes of each row (quad swaps, half-row and row mirrors), in every lane.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    return v;
}

// Sum over the 64 lanes, the same value in every lane.
__device__ __forceinline__ float wave_sum(float v) { return xor32_sum(xor16_sum(row16_sum(v))); }

// The same for the maximum.
__device__ __forceinline__ float xor16_max(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
    return xor32_max(xor16_max(v));
}

// Sum over aligned groups of 32 lanes (lanes 0-31 and 32-63 separately).
__device__ __forceinline__ float half_wave_sum(float v) { return xor16_sum(row16_sum(v)); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 128-bit load / store.
__device__ __forceinline__ uint4 ld_nt(const uint4 *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 ld_nt(const float4 *p)
{
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt(float4 v, float4 *p)
{
    const floatx4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<floatx4 *>(p));
}

}  // namespace nh
