// FP8 e4m3 quantisers: 128x128 weight blocks and 1x128 activation groups, and the
// MXFP8 variant (1x32 blocks along K with E8M0 scales) for both.
//
// "GPT-OSS on day 0", section "On Hopper": FP8 with 128x128 block scaling is the
// weight scheme; "Hosting Qwen on Blackwell", section "Quantization": the weights
// are converted once, statically, and the MXFP8 (microscaling) format is the one its
// Blackwell deployment takes.  The activation side uses per-token 1x128 groups (a
// design choice of this implementation) with the same rounding rule, or 1x32 MX blocks.
//
// MX scale layout: a row of K elements has K/32 blocks; its E8M0 codes are stored in a
// row of 4 ceil(K/128) bytes (whole dwords per 128-wide K-step, what the GEMMs stage),
// the bytes past K/32 holding 127 (scale 1).
#include "kernels.hpp"

namespace moe {

// One workgroup (256 lanes) per 128x128 block.  Lane (r, c4) owns column quad c4 of
// rows r, r+8, ..., r+120: 16 float4 loads, kept in registers between the amax pass
// and the encode pass, so the source is read exactly once.
__global__ __launch_bounds__(256) void quantize_weights_kernel(const float* __restrict__ w, int N,
                                                               int K, uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales) {
  const int KB = ceil_div(K, kBlock), NB = ceil_div(N, kBlock);
  const long blk = blockIdx.x;
  const int kb = static_cast<int>(blk % KB);
  const int nb = static_cast<int>((blk / KB) % NB);
  const long e = blk / (static_cast<long>(KB) * NB);
  const int c4 = threadIdx.x & 31, r = threadIdx.x >> 5;
  const int col = kb * kBlock + c4 * 4;
  const size_t mat = static_cast<size_t>(N) * K;
  const float* src = w + e * mat;
  float4 v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = nb * kBlock + r + 8 * i;
    if (row < N && col < K) {
      v[i] = *reinterpret_cast<const float4*>(src + static_cast<size_t>(row) * K + col);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = group_scale(amax);
  uint8_t* dst = codes + e * mat;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = nb * kBlock + r + 8 * i;
    if (row < N && col < K)
      *reinterpret_cast<uint32_t*>(dst + static_cast<size_t>(row) * K + col) =
          encode4(v[i].x, v[i].y, v[i].z, v[i].w, s);
  }
  if (threadIdx.x == 0) scales[blk] = s;
}

// 16 lanes per 1x128 group, 8 bf16 per lane; a workgroup covers 16 groups.
__global__ __launch_bounds__(256) void quantize_act_kernel(const uint16_t* __restrict__ x, int T,
                                                           int H, uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  const int KB = ceil_div(H, kBlock);
  const long g = static_cast<long>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = g < static_cast<long>(T) * KB;
  const long t = live ? g / KB : 0;
  const int kb = live ? static_cast<int>(g % KB) : 0;
  const int col = kb * kBlock + sub * 8;
  const bool in = live && col < H;
  const float s = quantize_group16(x + t * H, col, in, codes + t * H);
  if (live && sub == 0) scales[g] = s;
}

// MXFP8: 4 lanes per 32-block, 8 elements per lane; a workgroup covers 64 block slots
// of the padded scale rows (slots past K/32 write the pad code 127 and no elements).
// Weights are fp32 [rows, K] (rows a multiple of 16); their scales are stored in 16-row
// x 128-K tiles, as the GEMMs read them.
__global__ __launch_bounds__(256) void quantize_weights_mx_kernel(const float* __restrict__ w,
                                                                  long rows, int K,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  const int RS = 4 * ceil_div(K, kBlock);               // scale bytes per row
  const long slot = static_cast<long>(blockIdx.x) * 64 + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool live = slot < rows * RS;
  const long row = live ? slot / RS : 0;
  const int blk = live ? static_cast<int>(slot % RS) : 0;
  const int col = blk * kMxBlock + sub * 8;
  const bool in = live && col < K;
  float f[8];
  float amax = 0.0f;
  if (in) {
    const float4 a0 = *reinterpret_cast<const float4*>(w + row * K + col);
    const float4 a1 = *reinterpret_cast<const float4*>(w + row * K + col + 4);
    f[0] = a0.x; f[1] = a0.y; f[2] = a0.z; f[3] = a0.w;
    f[4] = a1.x; f[5] = a1.y; f[6] = a1.z; f[7] = a1.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = group_max<4>(amax);
  const int code = mx_scale_code(amax);
  if (in) {
    const float m = mx_inv_scale(code);
    uint2 q;
    q.x = encode4_mul(f[0], f[1], f[2], f[3], m);
    q.y = encode4_mul(f[4], f[5], f[6], f[7], m);
    *reinterpret_cast<uint2*>(codes + row * K + col) = q;
  }
  // weight scales in 16-row x 128-K tiles: row r of tile (row / 16, blk / 4) at byte 4 r
  if (live && sub == 0)
    scales[((row >> 4) * (RS / 4) + (blk >> 2)) * 64 + (row & 15) * 4 + (blk & 3)] = static_cast<uint8_t>(code);
}

// Activations bf16 [T, H], the same block slots (scale rows per token).
__global__ __launch_bounds__(256) void quantize_act_mx_kernel(const uint16_t* __restrict__ x, int T,
                                                              int H, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  const int RS = 4 * ceil_div(H, kBlock);
  const long slot = static_cast<long>(blockIdx.x) * 64 + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool live = slot < static_cast<long>(T) * RS;
  const long t = live ? slot / RS : 0;
  const int blk = live ? static_cast<int>(slot % RS) : 0;
  const int col = blk * kMxBlock + sub * 8;
  const int code = quantize_mx8(x + t * H, col, live && col < H, codes + t * H);
  if (live && sub == 0) scales[slot] = static_cast<uint8_t>(code);
}

// MXFP4 weights: the same block slots, stored in 16-row x 128-K tiles (the order in which
// the GEMMs stream them): tile (n16, j) of a matrix is 1024 code bytes, row r of the tile
// at byte 64 r holding K [128 j, 128 j + 128) two codes per byte (element 2i in the low
// nibble of byte i), K past the row zero; and 64 scale bytes, row r's four E8M0 codes of
// the K-block at byte 4 r (pads 127).  Rows are counted over all E matrices (N is a
// multiple of 16, so no tile straddles two experts).
__global__ __launch_bounds__(256) void quantize_weights_mxfp4_kernel(const float* __restrict__ w,
                                                                     long rows, int K,
                                                                     uint8_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ scales) {
  const int KB = ceil_div(K, kBlock), RS = 4 * KB;
  const long slot = static_cast<long>(blockIdx.x) * 64 + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool live = slot < rows * RS;
  const long row = live ? slot / RS : 0;
  const int blk = live ? static_cast<int>(slot % RS) : 0;
  const int col = blk * kMxBlock + sub * 8;
  const bool in = live && col < K;
  float f[8];
  float amax = 0.0f;
  if (in) {
    const float4 a0 = *reinterpret_cast<const float4*>(w + row * K + col);
    const float4 a1 = *reinterpret_cast<const float4*>(w + row * K + col + 4);
    f[0] = a0.x; f[1] = a0.y; f[2] = a0.z; f[3] = a0.w;
    f[4] = a1.x; f[5] = a1.y; f[6] = a1.z; f[7] = a1.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = group_max<4>(amax);
  const int code = mx4_scale_code(amax);
  const long tile = (row >> 4) * KB + (blk >> 2);   // the row's 16-row tile, its K-block
  const int rr = static_cast<int>(row & 15);
  if (live) {
    uint32_t q = 0;
    if (in) {
      const float m = mx_inv_scale(code);
#pragma unroll
      for (int i = 0; i < 8; ++i) q |= e2m1_code(f[i] * m) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(codes + tile * 1024 + rr * 64 + (blk & 3) * 16 + sub * 4) = q;
    if (sub == 0) scales[tile * 64 + rr * 4 + (blk & 3)] = static_cast<uint8_t>(code);
  }
}

void launch_quantize_weights_mxfp4(const float* w, int E, int N, int K, uint8_t* codes,
                                   uint8_t* scales, hipStream_t st) {
  const long rows = static_cast<long>(E) * N;
  const long slots = rows * 4 * ceil_div(K, kBlock);
  quantize_weights_mxfp4_kernel<<<dim3(static_cast<unsigned>((slots + 63) / 64)), dim3(256), 0,
                                  st>>>(w, rows, K, codes, scales);
}

void launch_quantize_weights_mx(const float* w, int E, int N, int K, uint8_t* codes,
                                uint8_t* scales, hipStream_t st) {
  const long rows = static_cast<long>(E) * N;
  const long slots = rows * 4 * ceil_div(K, kBlock);
  quantize_weights_mx_kernel<<<dim3(static_cast<unsigned>((slots + 63) / 64)), dim3(256), 0, st>>>(
      w, rows, K, codes, scales);
}

void launch_quantize_act_mx(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales,
                            hipStream_t st) {
  const long slots = static_cast<long>(T) * 4 * ceil_div(H, kBlock);
  quantize_act_mx_kernel<<<dim3(static_cast<unsigned>((slots + 63) / 64)), dim3(256), 0, st>>>(
      x, T, H, codes, scales);
}

void launch_quantize_weights(const float* w, int E, int N, int K, uint8_t* codes, float* scales,
                             hipStream_t st) {
  const long blocks = static_cast<long>(E) * ceil_div(N, kBlock) * ceil_div(K, kBlock);
  quantize_weights_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(w, N, K, codes,
                                                                                    scales);
}

void launch_quantize_act(const uint16_t* x, int T, int H, uint8_t* codes, float* scales,
                         hipStream_t st) {
  const long groups = static_cast<long>(T) * ceil_div(H, kBlock);
  quantize_act_kernel<<<dim3(static_cast<unsigned>((groups + 15) / 16)), dim3(256), 0, st>>>(
      x, T, H, codes, scales);
}

}  // namespace moe
