// Grouped FP8 GEMMs of the experts on the gfx950 matrix cores.
//
// "GPT-OSS on day 0", section "On Hopper": FP8 with 128x128 block scaling and
// experts with biases; section "Kernels -> MoE": the bias enters the GEMM as the
// accumulator's starting value once per output tile (here it is added in the
// epilogue, which gives the same sum); section "Performance Tweaks": launch shapes
// are specialised for the hidden size 2880 rather than reused from 7168.
//
// Both GEMMs are "NT": A [rows, K] and B [N, K] are K-contiguous, the natural
// operand order of v_mfma_f32_16x16x128_f8f6f4 (lane l supplies 32 consecutive K
// bytes of row l%16 for K-quarter l/16, for A and B alike).  One K-step is one
// 128-wide scale block: each 16x16 sub-tile's MFMA result of that step is folded
// into the fp32 accumulator with the product of the row's activation scale and the
// sub-tile's weight block scale (block-scale promotion; the weight scale is
// uniform over every wave's column range by construction of the tiling).
//
// gemm1: rows of expert e gathered from xq through perm; the 256-wide B tile holds
//   128 gate rows and the matching 128 up rows of w13, so SwiGLU pairs (j, I+j) sit
//   in the same lane; the epilogue adds b13, applies silu(gate)*up and requantises
//   each 1x128 group of h (row amax across lanes and waves) to e4m3.
// gemm2: rows of h in dispatch order, B = w2 [H, I]; the epilogue adds b2 and stores
//   y in fp32.
#include "kernels.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 128-byte LDS rows; the 16-byte chunk index is XOR-swizzled with the row so that
// the 16 rows one MFMA operand read touches spread over all banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int g) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, 2 * g));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, 2 * g + 1));
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <int BM, int BN, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(const GemmArgs a) {
  constexpr int WTM = BM / WM, SM = WTM / 16;
  constexpr int WTN = BN / WN, SN = WTN / 16;
  constexpr int NG = SN / 2;                  // gemm1: gate (= up) sub-tiles per wave
  constexpr int GW = WTN / 2;                 // gemm1: gate columns per wave
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int A_CH = (BM * 8 + 255) / 256;  // 16-byte chunks per lane and K-step
  constexpr int B_CH = BN * 8 / 256;
  static_assert(WM * WN == 4, "four waves");
  static_assert(SM >= 1 && SN >= 1, "sub-tiles");
  static_assert(!SWIGLU || (BN == 256 && SN % 2 == 0 && GW <= 64), "gemm1 tile");
  static_assert(SWIGLU || WTN <= 128, "gemm2 wave columns inside one scale block");

  __shared__ __align__(16) uint8_t smem[2 * (A_BYTES + B_BYTES)];
  __shared__ float sA[2][BM];
  __shared__ int rowsrc[BM];
  __shared__ float red[SWIGLU ? WN : 1][BM];

  if (static_cast<int>(blockIdx.x) >= *a.num_tiles) return;
  const MTile mt = a.tiles[blockIdx.x];
  const int nt = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K, N = a.N, I = a.I;
  const int KB = ceil_div(K, kBlock), NBs = ceil_div(N, kBlock);
  const int e = mt.expert;
  const uint8_t* Bexp = a.B + static_cast<size_t>(e) * N * K;
  const float* Bsc = a.B_scale + static_cast<size_t>(e) * NBs * KB;

  for (int r = tid; r < BM; r += 256) {
    const int p = mt.row_begin + r;
    int src = -1;
    if (p < mt.row_end) src = SWIGLU ? a.perm[p] / a.top_k : p;
    rowsrc[r] = src;
  }

  // global B rows of this lane's load chunks (-1: outside the matrix)
  int brow[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int br = (tid + 256 * i) >> 3;
    int g = -1;
    if (SWIGLU) {
      const int j = nt * 128 + (br & 127);
      if (j < I) g = (br >> 7) * I + j;
    } else {
      const int col = nt * BN + br;
      if (col < N) g = col;
    }
    brow[i] = g;
  }

  // weight block-scale rows of this wave's column groups (-1: the group is empty)
  int sb_row0, sb_row1;
  if (SWIGLU) {
    const int j0 = nt * 128 + wn * GW;
    sb_row0 = j0 < I ? j0 / kBlock : -1;
    sb_row1 = j0 < I ? (I + j0) / kBlock : -1;
  } else {
    const int c0 = nt * BN + wn * WTN;
    sb_row0 = c0 < N ? c0 / kBlock : -1;
    sb_row1 = sb_row0;
  }
  __syncthreads();

  uint4 ra[A_CH], rb[B_CH];
  float rsa = 0.f;
  auto gload = [&](int kt) {
    const int k0 = kt * kBlock;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + 256 * i;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q < BM * 8) {
        const int src = rowsrc[q >> 3], kk = k0 + (q & 7) * 16;
        if (src >= 0 && kk < K)
          v = *reinterpret_cast<const uint4*>(a.A + static_cast<size_t>(src) * K + kk);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int kk = k0 + ((tid + 256 * i) & 7) * 16;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (brow[i] >= 0 && kk < K)
        v = *reinterpret_cast<const uint4*>(Bexp + static_cast<size_t>(brow[i]) * K + kk);
      rb[i] = v;
    }
    if (tid < BM) {
      const int src = rowsrc[tid];
      rsa = src >= 0 ? a.A_scale[static_cast<size_t>(src) * KB + kt] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* As = smem + buf * (A_BYTES + B_BYTES);
    uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + 256 * i;
      if (q < BM * 8) *reinterpret_cast<uint4*>(As + swz(q >> 3, q & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + 256 * i;
      *reinterpret_cast<uint4*>(Bs + swz(q >> 3, q & 7)) = rb[i];
    }
    if (tid < BM) sA[buf][tid] = rsa;
  };

  v4f acc[SM][SN];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int n = 0; n < SN; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};

  // B-tile row of sub-tile n of this wave
  auto sub_brow = [&](int n) {
    if (SWIGLU) return n < NG ? wn * GW + 16 * n : 128 + wn * GW + 16 * (n - NG);
    return wn * WTN + 16 * n;
  };

  gload(0);
  sstore(0);
  __syncthreads();
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < KB; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KB) gload(kt + 1);
    const uint8_t* As = smem + cur * (A_BYTES + B_BYTES);
    const uint8_t* Bs = As + A_BYTES;
    const float sb0 = sb_row0 >= 0 ? Bsc[sb_row0 * KB + kt] : 0.f;
    const float sb1 = sb_row1 >= 0 ? Bsc[sb_row1 * KB + kt] : 0.f;
    v8i af[SM];
    float s0[SM][4], s1[SM][4];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const int r0 = wm * WTM + 16 * m;
      af[m] = lds_frag(As, r0 + (lane & 15), lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sa = sA[cur][r0 + 4 * (lane >> 4) + i];
        s0[m][i] = sa * sb0;
        s1[m][i] = sa * sb1;
      }
    }
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const v8i bfr = lds_frag(Bs, sub_brow(n) + (lane & 15), lane >> 4);
      const bool second = SWIGLU && n >= NG;
#pragma unroll
      for (int m = 0; m < SM; ++m) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bfr, zero, 0, 0, 0,
                                                                       0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[m][n][i] = fmaf(p[i], second ? s1[m][i] : s0[m][i], acc[m][n][i]);
      }
    }
    if (kt + 1 < KB) sstore(cur ^ 1);
    __syncthreads();
  }

  const int rbase = wm * WTM + 4 * (lane >> 4);   // + 16 m + i
  if constexpr (SWIGLU) {
    const uint16_t* bias = a.bias ? a.bias + static_cast<size_t>(e) * N : nullptr;
    float hv[SM][NG][4];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int j = nt * 128 + wn * GW + 16 * n + (lane & 15);
      const bool ok = j < I;
      const float bg = (ok && bias) ? bf16_to_f32(bias[j]) : 0.f;
      const float bu = (ok && bias) ? bf16_to_f32(bias[I + j]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[m][n][i] + bg;
          const float u = acc[m][n + NG][i] + bu;
          hv[m][n][i] = ok ? g / (1.0f + expf(-g)) * u : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < SM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.f;
#pragma unroll
        for (int n = 0; n < NG; ++n) mx = fmaxf(mx, fabsf(hv[m][n][i]));
        mx = group_max<16>(mx);
        if ((lane & 15) == 0) red[wn][rbase + 16 * m + i] = mx;
      }
    __syncthreads();
    uint8_t* hs = smem;   // [BM][128] staging of the codes
    const int KBI = ceil_div(I, kBlock);
#pragma unroll
    for (int m = 0; m < SM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + 16 * m + i;
        float amax = red[0][r];
#pragma unroll
        for (int w = 1; w < WN; ++w) amax = fmaxf(amax, red[w][r]);
        const float s = group_scale(amax);
#pragma unroll
        for (int n = 0; n < NG; ++n)
          hs[r * 128 + wn * GW + 16 * n + (lane & 15)] =
              static_cast<uint8_t>(encode2(hv[m][n][i], 0.f, s) & 0xFFu);
        const int p = mt.row_begin + r;
        if (wn == 0 && (lane & 15) == 0 && p < mt.row_end)
          a.h_scale[static_cast<size_t>(p) * KBI + nt] = s;
      }
    __syncthreads();
    for (int q = tid; q < BM * 8; q += 256) {
      const int r = q >> 3, c = q & 7;
      const int p = mt.row_begin + r, col = nt * 128 + c * 16;
      if (p < mt.row_end && col < I)
        *reinterpret_cast<uint4*>(a.h_out + static_cast<size_t>(p) * I + col) =
            *reinterpret_cast<const uint4*>(hs + r * 128 + c * 16);
    }
  } else {
    const uint16_t* bias = a.bias ? a.bias + static_cast<size_t>(e) * N : nullptr;
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const int col = nt * BN + wn * WTN + 16 * n + (lane & 15);
      if (col >= N) continue;
      const float b = bias ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = mt.row_begin + rbase + 16 * m + i;
          if (p < mt.row_end) a.y_out[static_cast<size_t>(p) * N + col] = acc[m][n][i] + b;
        }
    }
  }
}

int gemm_tile_rows(long rows, int E) {
  const long avg = rows / (E > 0 ? E : 1);
  if (avg <= 24) return 16;
  if (avg <= 96) return 64;
  return 128;
}

template <bool SWIGLU>
static void launch_gemm(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  const int ntiles = SWIGLU ? ceil_div(a.I, 128) : ceil_div(a.N, 256);
  const dim3 grid(max_tiles, ntiles);
  switch (bm) {
    case 16: grouped_gemm_kernel<16, 256, 1, 4, SWIGLU><<<grid, dim3(256), 0, st>>>(a); break;
    case 64: grouped_gemm_kernel<64, 256, 1, 4, SWIGLU><<<grid, dim3(256), 0, st>>>(a); break;
    default: grouped_gemm_kernel<128, 256, 2, 2, SWIGLU><<<grid, dim3(256), 0, st>>>(a); break;
  }
}

void launch_gemm1(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  launch_gemm<true>(a, bm, max_tiles, st);
}
void launch_gemm2(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  launch_gemm<false>(a, bm, max_tiles, st);
}

}  // namespace moe
