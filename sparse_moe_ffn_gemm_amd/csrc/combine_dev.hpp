// The gate-weighted combine of one column quad (combine.hip), shared with the fused decode
// kernel (fused.hip).
#pragma once

#include "common.hpp"

namespace moe {

// out[t, c .. c + 3] = sum_j gates[t, j] * y[inv[t k + j], c .. c + 3], summed in fp32 in j
// order (deterministic) and rounded once to bf16; the k 8-byte loads of y are issued before
// the sum.  `rows` bounds the y rows (an out-of-range inv entry reads row 0).  COH: gates,
// inv and y are read with device-coherent loads (written by other workgroups of the same
// launch).
template <bool COH = false>
__device__ __forceinline__ void combine_quad(const uint16_t* __restrict__ y,
                                             const float* __restrict__ gates,
                                             const int32_t* __restrict__ inv, int rows, int t,
                                             int c, int H, int top_k,
                                             uint16_t* __restrict__ out) {
  float g[8];
  uint2 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g[j] = 0.f;
    v[j] = make_uint2(0u, 0u);
    if (j < top_k) {
      g[j] = load_c<COH>(gates + static_cast<size_t>(t) * top_k + j);
      int r = load_c<COH>(inv + static_cast<size_t>(t) * top_k + j);
      if (static_cast<unsigned>(r) >= static_cast<unsigned>(rows)) r = 0;   // never read past y
      const uint16_t* row = y + static_cast<size_t>(r) * H;
      if constexpr (COH) {
        const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(row + c),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v[j] = make_uint2(static_cast<uint32_t>(u), static_cast<uint32_t>(u >> 32));
      } else {
        v[j] = *reinterpret_cast<const uint2*>(row + c);
      }
    }
  }
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < top_k) {
      s.x = fmaf(g[j], f16_to_f32(static_cast<uint16_t>(v[j].x & 0xFFFFu)), s.x);
      s.y = fmaf(g[j], f16_to_f32(static_cast<uint16_t>(v[j].x >> 16)), s.y);
      s.z = fmaf(g[j], f16_to_f32(static_cast<uint16_t>(v[j].y & 0xFFFFu)), s.z);
      s.w = fmaf(g[j], f16_to_f32(static_cast<uint16_t>(v[j].y >> 16)), s.w);
    }
  }
  uint2 o;
  o.x = static_cast<uint32_t>(f32_to_bf16(s.x)) | (static_cast<uint32_t>(f32_to_bf16(s.y)) << 16);
  o.y = static_cast<uint32_t>(f32_to_bf16(s.z)) | (static_cast<uint32_t>(f32_to_bf16(s.w)) << 16);
  *reinterpret_cast<uint2*>(out + static_cast<size_t>(t) * H + c) = o;
}

}  // namespace moe
