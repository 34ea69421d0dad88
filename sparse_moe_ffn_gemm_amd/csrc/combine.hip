// Gate-weighted unpermute-combine.
//
// "GPT-OSS on day 0", section "Kernels -> MoE": combine performs the weighted
// accumulation of the experts' outputs per token; "Hosting Qwen on Blackwell",
// section "Expert Parallel": the local combine aggregates the contributions of the
// experts a token was routed to.  out[t] = sum_j gates[t,j] * y[inv[t*k+j]], summed in
// fp32 in j order (deterministic) and rounded once to bf16.  y is stored in fp16.
#include "kernels.hpp"

namespace moe {

// Workgroup (t, c): token t, columns [1024 c, 1024 c + 1024); each lane owns one column
// quad and issues the k 16-byte loads of its y rows before summing them in j order
// (deterministic), then stores 8 bytes of out.  Several workgroups per token keep enough
// loads in flight for small batches.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int H,
                                                      int top_k, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int rows = static_cast<int>(gridDim.x) * top_k;
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= H) return;
  float g[8];
  uint2 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g[j] = 0.f;
    v[j] = make_uint2(0u, 0u);
    if (j < top_k) {
      g[j] = gates[static_cast<size_t>(t) * top_k + j];
      int r = inv[static_cast<size_t>(t) * top_k + j];
      if (static_cast<unsigned>(r) >= static_cast<unsigned>(rows)) r = 0;   // never read past y
      const uint16_t* row = y + static_cast<size_t>(r) * H;
      v[j] = *reinterpret_cast<const uint2*>(row + c);
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

void launch_combine(const uint16_t* y, const float* gates, const int32_t* inv, int T, int H,
                    int top_k, uint16_t* out, hipStream_t st) {
  combine_kernel<<<dim3(T, ceil_div(H, 1024)), dim3(256), 0, st>>>(y, gates, inv, H, top_k, out);
}

}  // namespace moe
