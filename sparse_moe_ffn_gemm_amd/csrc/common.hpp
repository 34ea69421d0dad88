// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kBlock = 128;          // quantisation block / group edge
constexpr float kFp8Max = 448.0f;    // largest finite OCP e4m3 value

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; inputs are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp32 -> IEEE half bits, round to nearest even, saturated to +-65504 (the expert-output
// buffer: 11 significant bits, a quarter of a bf16 output ulp after the gate sum).
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  f = fminf(fmaxf(f, -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Scale of a group with absolute maximum `amax`: fp32(amax / 448) with an IEEE
// (correctly rounded) division, 1 for an all-zero group.
__device__ __forceinline__ float group_scale(float amax) {
  return amax > 0.0f ? amax / kFp8Max : 1.0f;
}

// Two e4m3 codes (OCP fn, round to nearest even) of v0/s and v1/s, clamped to +-448,
// packed into the low 16 bits.  The quotient is an IEEE division so that the code is
// the one the fp32 quantisation rule defines.
__device__ __forceinline__ uint32_t encode2(float v0, float v1, float s) {
  float q0 = fminf(fmaxf(v0 / s, -kFp8Max), kFp8Max);
  float q1 = fminf(fmaxf(v1 / s, -kFp8Max), kFp8Max);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false)) & 0xFFFFu;
}

// Four codes packed little-endian into one dword.
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3, float s) {
  return encode2(v0, v1, s) | (encode2(v2, v3, s) << 16);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// v from the lane `CTRL` names inside this lane's row of 16 (a DPP row rotation).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over each aligned group of `W` lanes (W a power of two <= 64).  Groups of 16 are
// DPP rows: four rotations (by 8, 4, 2, 1 lanes) leave the row maximum in every lane
// without a round trip through LDS.
template <int W>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (W == 16) {
    v = fmaxf(v, dpp_row<0x128>(v));
    v = fmaxf(v, dpp_row<0x124>(v));
    v = fmaxf(v, dpp_row<0x122>(v));
    v = fmaxf(v, dpp_row<0x121>(v));
  } else {
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  }
  return v;
}

// Stores and loads at device scope (the sc1 cache policy) when COH: data that workgroups of
// one launch hand to each other after a counter says it is complete, visible across the
// XCDs' L2 caches without cache-wide write-back or invalidation.
template <bool COH, typename T>
__device__ __forceinline__ void store_c(T* p, T v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COH, typename T>
__device__ __forceinline__ T load_c(const T* p) {
  if constexpr (COH)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// Quantises columns [col, col + 8) of one 1x128 group of a bf16 row (16 lanes of a DPP row
// cover the group; `in` is false for lanes past the row's end) and returns the group's
// scale, the same in all 16 lanes.  Codes go to codes_row + col.
template <bool COH = false>
__device__ __forceinline__ float quantize_group16(const uint16_t* row, int col, bool in,
                                                  uint8_t* codes_row) {
  float f[8];
  float amax = 0.0f;
  if (in) {
    const uint4 raw = *reinterpret_cast<const uint4*>(row + col);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32(static_cast<uint16_t>(wds[i] & 0xFFFFu));
      f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(wds[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = group_max<16>(amax);
  const float s = group_scale(amax);
  if (in) {
    const uint64_t lo = encode4(f[0], f[1], f[2], f[3], s);
    const uint64_t hi = encode4(f[4], f[5], f[6], f[7], s);
    store_c<COH>(reinterpret_cast<uint64_t*>(codes_row + col), lo | (hi << 32));
  }
  return s;
}

// ---- MXFP8 (OCP microscaling): 1x32 blocks along K, E8M0 scale = exponent + 127 ----
constexpr int kMxBlock = 32;

// E8M0 code of a 32-block with absolute maximum `amax`: exponent floor(log2(amax)) - 8
// (the block maximum lands in [256, 512) before the e4m3 rounding), clamped below at
// -127 (a subnormal amax has exponent field 0 and lands there), 0 for an all-zero block.
// floor(log2) of a normal fp32 value is its exponent field - 127; the largest (127)
// gives 119, so no upper clamp is needed.
__device__ __forceinline__ int mx_scale_code(float amax) {
  if (!(amax > 0.0f)) return 127;
  const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
  return max(ex - 8, -127) + 127;
}

// 2^-(code - 127), a normal fp32 power of two for every code in [0, 246].
__device__ __forceinline__ float mx_inv_scale(int code) {
  return __uint_as_float(static_cast<uint32_t>(254 - code) << 23);
}

// Four e4m3 codes of v * m (m a power of two: the product is exact), clamped to +-448,
// round to nearest even, packed little-endian.
__device__ __forceinline__ uint32_t encode4_mul(float v0, float v1, float v2, float v3, float m) {
  const float q0 = fminf(fmaxf(v0 * m, -kFp8Max), kFp8Max);
  const float q1 = fminf(fmaxf(v1 * m, -kFp8Max), kFp8Max);
  const float q2 = fminf(fmaxf(v2 * m, -kFp8Max), kFp8Max);
  const float q3 = fminf(fmaxf(v3 * m, -kFp8Max), kFp8Max);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false)) & 0xFFFFu;
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, 0, false)) & 0xFFFFu;
  return lo | (hi << 16);
}

// MX-quantises columns [col, col + 8) of one 32-block of a bf16 row (4 aligned lanes cover
// the block; `in` is false for lanes past the row's end, whose codes are not written) and
// returns the block's E8M0 code, the same in all 4 lanes.  Codes go to codes_row + col.
template <bool COH = false>
__device__ __forceinline__ int quantize_mx8(const uint16_t* row, int col, bool in,
                                            uint8_t* codes_row) {
  float f[8];
  float amax = 0.0f;
  if (in) {
    const uint4 raw = *reinterpret_cast<const uint4*>(row + col);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32(static_cast<uint16_t>(wds[i] & 0xFFFFu));
      f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(wds[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = group_max<4>(amax);
  const int code = mx_scale_code(amax);
  if (in) {
    const float m = mx_inv_scale(code);
    const uint64_t lo = encode4_mul(f[0], f[1], f[2], f[3], m);
    const uint64_t hi = encode4_mul(f[4], f[5], f[6], f[7], m);
    store_c<COH>(reinterpret_cast<uint64_t*>(codes_row + col), lo | (hi << 32));
  }
  return code;
}

// ---- MXFP4 weights: e2m1 elements (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) in MX blocks ----

// E8M0 code of an MXFP4 block: floor(log2(amax)) - 2 (the block maximum lands in [4, 8)),
// clamped below at -127, 0 for an all-zero block.
__device__ __forceinline__ int mx4_scale_code(float amax) {
  if (!(amax > 0.0f)) return 127;
  const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
  return max(ex - 2, -127) + 127;
}

// e2m1 code of u (an exactly scaled value): the nearest magnitude, ties to the even code,
// clamped to 6, counted against the midpoints (a tie sits on its midpoint and goes down
// when the lower code is even: 0.25, 1.25, 2.5, 5; up when it is odd: 0.75, 1.75, 3.5);
// the sign bit kept.
__device__ __forceinline__ uint32_t e2m1_code(float u) {
  const float m = fabsf(u);
  const uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
                     (m >= 3.5f) + (m > 5.0f);
  return c | ((__float_as_uint(u) >> 28) & 8u);
}

}  // namespace moe
