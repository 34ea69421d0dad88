// Gate-weighted unpermute-combine.
//
// "GPT-OSS on day 0", section "Kernels -> MoE": combine performs the weighted
// accumulation of the experts' outputs per token; "Hosting Qwen on Blackwell",
// section "Expert Parallel": the local combine aggregates the contributions of the
// experts a token was routed to.  out[t] = sum_j gates[t,j] * y[inv[t*k+j]], summed in
// fp32 in j order (deterministic) and rounded once to bf16.
#include "kernels.hpp"

namespace moe {

// One workgroup per token; each lane owns column quads (16-byte loads of y, 8-byte
// stores of out), so every y row is streamed once, fully coalesced.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int H,
                                                      int top_k, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  float g[8];
  const float* rows[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g[j] = 0.f;
    rows[j] = y;
    if (j < top_k) {
      g[j] = gates[static_cast<size_t>(t) * top_k + j];
      rows[j] = y + static_cast<size_t>(inv[static_cast<size_t>(t) * top_k + j]) * H;
    }
  }
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < top_k) {
        const float4 v = *reinterpret_cast<const float4*>(rows[j] + c);
        s.x = fmaf(g[j], v.x, s.x);
        s.y = fmaf(g[j], v.y, s.y);
        s.z = fmaf(g[j], v.z, s.z);
        s.w = fmaf(g[j], v.w, s.w);
      }
    }
    uint2 o;
    o.x = static_cast<uint32_t>(f32_to_bf16(s.x)) | (static_cast<uint32_t>(f32_to_bf16(s.y)) << 16);
    o.y = static_cast<uint32_t>(f32_to_bf16(s.z)) | (static_cast<uint32_t>(f32_to_bf16(s.w)) << 16);
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(t) * H + c) = o;
  }
}

void launch_combine(const float* y, const float* gates, const int32_t* inv, int T, int H,
                    int top_k, uint16_t* out, hipStream_t st) {
  combine_kernel<<<dim3(T), dim3(256), 0, st>>>(y, gates, inv, H, top_k, out);
}

}  // namespace moe
