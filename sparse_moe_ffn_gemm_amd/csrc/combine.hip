// Gate-weighted unpermute-combine.
//
// "GPT-OSS on day 0", section "Kernels -> MoE": combine performs the weighted
// accumulation of the experts' outputs per token; "Hosting Qwen on Blackwell",
// section "Expert Parallel": the local combine aggregates the contributions of the
// experts a token was routed to.  out[t] = sum_j gates[t,j] * y[inv[t*k+j]], summed in
// fp32 in j order (deterministic) and rounded once to bf16.  y is stored in fp16.
#include "combine_dev.hpp"
#include "kernels.hpp"

namespace moe {

// Workgroup (t, c): token t, columns [1024 c, 1024 c + 1024); each lane owns one column
// quad.  Several workgroups per token keep enough loads in flight for small batches.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int H,
                                                      int top_k, uint16_t* __restrict__ out) {
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= H) return;
  combine_quad(y, gates, inv, static_cast<int>(gridDim.x) * top_k, blockIdx.x, c, H, top_k, out);
}

void launch_combine(const uint16_t* y, const float* gates, const int32_t* inv, int T, int H,
                    int top_k, uint16_t* out, hipStream_t st) {
  combine_kernel<<<dim3(T, ceil_div(H, 1024)), dim3(256), 0, st>>>(y, gates, inv, H, top_k, out);
}

}  // namespace moe
