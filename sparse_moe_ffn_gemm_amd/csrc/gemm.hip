// Grouped FP8 GEMMs of the experts on the gfx950 matrix cores.
//
// "GPT-OSS on day 0", section "On Hopper": FP8 with 128x128 block scaling and
// experts with biases; section "Kernels -> MoE": the bias enters the GEMM as the
// accumulator's starting value once per output tile (here it is added in the
// epilogue, which gives the same sum); section "Performance Tweaks": launch shapes
// are specialised for the hidden size 2880 rather than reused from 7168.
//
// Both GEMMs are "NT": A [rows, K] and B [N, K] are K-contiguous, the natural
// operand order of v_mfma_f32_16x16x128_f8f6f4 (lane l supplies 32 K bytes of row
// l%16, for A and B alike).  One K-step is one
// 128-wide scale block: each 16x16 sub-tile's MFMA result of that step is folded
// into the fp32 accumulator with the product of the row's activation scale and the
// sub-tile's weight block scale (block-scale promotion; the weight scale is uniform
// over every wave's column range by construction of the tiling).  Promoting every
// 128 products also bounds the error of the matrix cores' own fp8 accumulation.
//
// Memory pipeline: tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging) through a ring of STAGES K-steps,
// so STAGES-1 K-steps of loads are in flight while one is multiplied.  LDS rows are
// 128 bytes; the 16-byte chunk c of row r is stored in slot c ^ (r & 7), which each lane
// realises by choosing the global chunk it fetches.  A fragment lane (row r, K-quarter g)
// takes chunks g and g + 4 of its row rather than 2g and 2g + 1: the MFMA only needs the
// A and B lanes to agree on which K values they hold, and with this pairing the 128-bit
// fragment reads spread over all LDS banks (measured: about 1.4x the read bandwidth of
// the adjacent-chunk pairing).  Out-of-range chunks (K tail, N tail, rows past the
// expert's segment) are fetched from a zero block.
//
// Work order: blocks are numbered so that each XCD (blocks are dealt round-robin to
// the 8 XCDs) receives a contiguous range of (n-tile, m-tile) pairs with m-tiles
// fastest, so the M-tiles that share an expert's weight tile run together on one XCD
// and its L2 serves the repeated weight reads.
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
typedef __attribute__((address_space(3))) void lds_void;

__device__ __align__(16) const uint8_t kZeroChunk[64] = {0};
__device__ __align__(16) const float kZeroScale[4] = {0.f, 0.f, 0.f, 0.f};

__device__ __forceinline__ int swz_key(int row) { return row & 7; }

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ swz_key(row)) << 4);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int g) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, g));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, g + 4));
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// LDS address (32-bit) of a shared-memory pointer.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void*)(p)));
}

// One wave-wide direct load: lane l's 16 (or 4) bytes land at lds + l * 16 (or 4).  The
// loads are issued as inline assembly so that the compiler neither inserts its own
// conservative vmcnt(0) waits before LDS reads nor moves LDS reads across the explicit
// wait + barrier below; `lds` must be wave-uniform (it goes to M0).
__device__ __forceinline__ void load_lds16(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_addr(lds)) : "memory", "m0");
}
// Same with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte offset, so
// that advancing along K touches only the scalar base.
__device__ __forceinline__ void load_lds16_s(unsigned off, const void* base, const void* lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_addr(lds)) : "memory", "m0");
}
__device__ __forceinline__ void load_lds4(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds_addr(lds)) : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier without the memory fences of __syncthreads (the ring's loads are
// waited for explicitly); the "memory" clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

template <int BM, int BN, int WM, int WN, bool SWIGLU, int STAGES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(const GemmArgs a, int max_tiles,
                                                           int ntiles, int grid) {
  constexpr int WTM = BM / WM, SM = WTM / 16;
  constexpr int WTN = BN / WN, SN = WTN / 16;
  constexpr int NG = SN / 2;                  // gemm1: gate (= up) sub-tiles per wave
  constexpr int GW = WTN / 2;                 // gemm1: gate columns per wave
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  constexpr int AROWS = BM / 4;               // A rows each wave fetches per stage
  constexpr int A_INSTR = AROWS >= 8 ? AROWS / 8 : 1;
  constexpr int BROWS = BN / 4;
  constexpr int B_INSTR = BROWS / 8;
  constexpr int LOADS = A_INSTR + B_INSTR + 1;   // vmem instructions per wave and stage
  static_assert(WM * WN == 4, "four waves");
  static_assert(SM >= 1 && SN >= 1, "sub-tiles");
  static_assert(AROWS % 8 == 0 || AROWS == 4, "A rows per wave");
  static_assert(AROWS + 2 <= 64, "one scale load per wave");
  static_assert(!SWIGLU || (BN == 256 && SN % 2 == 0 && GW <= 64), "gemm1 tile");
  static_assert(SWIGLU || WTN <= 128, "gemm2 wave columns inside one scale block");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) < 64, "pipeline depth");

  __shared__ __align__(16) uint8_t smem[STAGES * STAGE];
  __shared__ __align__(16) float sA[STAGES][4][64];
  __shared__ int rowsrc[BM];
  __shared__ float red[SWIGLU ? WN : 1][BM];

  // ---- which tile: XCD-contiguous logical order, m-tiles fastest ----
  const int b = blockIdx.x;
  const int per_xcd = grid / 8;
  const int L = (b % 8) * per_xcd + b / 8;
  const int mti = L % max_tiles, nt = L / max_tiles;
  if (nt >= ntiles || mti >= *a.num_tiles) return;
  MTile mt = a.tiles[mti];
  mt.expert = __builtin_amdgcn_readfirstlane(mt.expert);
  mt.row_begin = __builtin_amdgcn_readfirstlane(mt.row_begin);
  mt.row_end = __builtin_amdgcn_readfirstlane(mt.row_end);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
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
  __syncthreads();

  // ---- per-lane fetch descriptors (constant over K) ----
  // A: wave w fetches rows [w*AROWS, (w+1)*AROWS); lane -> (row, slot) of an 8-row group
  const int a_slot = lane & 7, a_r8 = lane >> 3;
  // Rows outside the tile are redirected to row 0 (finite codes that only feed output
  // rows/columns that are never stored); only the ragged K tail needs real zeros.
  const uint8_t* a_src[A_INSTR];
  bool a_ok[A_INSTR];
  unsigned a_off[A_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int row = wave * AROWS + i * 8 + a_r8;
    const bool live = AROWS >= 8 || lane < 32;
    const int src = live ? rowsrc[row] : -1;
    a_ok[i] = src >= 0;
    a_off[i] = static_cast<unsigned>(src < 0 ? 0 : src) * K + ((a_slot ^ swz_key(row)) << 4);
    a_src[i] = a.A + a_off[i];
  }
  const uint8_t* b_src[B_INSTR];
  bool b_ok[B_INSTR];
  unsigned b_off[B_INSTR];
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    const int br = wave * BROWS + i * 8 + a_r8;
    int g = -1;
    if (SWIGLU) {
      const int j = nt * 128 + (br & 127);
      if (j < I) g = (br >> 7) * I + j;
    } else {
      const int col = nt * BN + br;
      if (col < N) g = col;
    }
    b_ok[i] = g >= 0;
    b_off[i] = static_cast<unsigned>(g < 0 ? 0 : g) * K + ((a_slot ^ swz_key(br)) << 4);
    b_src[i] = Bexp + b_off[i];
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
  // scale fetch of one K-step, one instruction per wave: lanes [0, AROWS) take the
  // activation scales of the wave's A rows, lanes AROWS and AROWS+1 the two weight block
  // scales of the wave's column groups
  const float* s_ptr = kZeroScale;
  bool s_live = false;
  if (lane < AROWS) {
    const int src = rowsrc[wave * AROWS + lane];
    s_live = src >= 0;
    s_ptr = a.A_scale + static_cast<size_t>(src < 0 ? 0 : src) * KB;
  } else if (lane < AROWS + 2) {
    const int row = lane == AROWS ? sb_row0 : sb_row1;
    s_live = row >= 0;
    s_ptr = Bsc + static_cast<size_t>(row < 0 ? 0 : row) * KB;
  }

  auto issue = [&](int kt) {   // all loads of K-step kt into ring slot kt % STAGES
    uint8_t* As = smem + (kt % STAGES) * STAGE;
    uint8_t* Bs = As + A_BYTES;
    const int k0 = kt * kBlock;
    if (k0 + kBlock <= K) {      // full K-step: scalar base + constant lane offsets
      const uint8_t* abase = a.A + k0;
      const uint8_t* bbase = Bexp + k0;
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i)
        if (AROWS >= 8 || lane < 32) load_lds16_s(a_off[i], abase, As + (wave * AROWS + i * 8) * 128);
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) load_lds16_s(b_off[i], bbase, Bs + (wave * BROWS + i * 8) * 128);
      if (lane < AROWS + 2) {
        const void* src = s_live ? static_cast<const void*>(s_ptr + kt) : kZeroScale;
        load_lds4(src, &sA[kt % STAGES][wave][0]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      const int row0 = wave * AROWS + i * 8;
      const int kk = k0 + ((a_slot ^ swz_key(row0 + a_r8)) << 4);
      const void* src = (a_ok[i] && kk < K) ? static_cast<const void*>(a_src[i] + k0) : kZeroChunk;
      if (AROWS >= 8 || lane < 32) load_lds16(src, As + row0 * 128);
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      const int row0 = wave * BROWS + i * 8;
      const int kk = k0 + ((a_slot ^ swz_key(row0 + a_r8)) << 4);
      const void* src = (b_ok[i] && kk < K) ? static_cast<const void*>(b_src[i] + k0) : kZeroChunk;
      load_lds16(src, Bs + row0 * 128);
    }
    if (lane < AROWS + 2) {
      const void* src = s_live ? static_cast<const void*>(s_ptr + kt) : kZeroScale;
      load_lds4(src, &sA[kt % STAGES][wave][0]);
    }
  };

  v4f acc[SM][SN];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int n = 0; n < SN; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};

  auto sub_brow = [&](int n) {
    if (SWIGLU) return n < NG ? wn * GW + 16 * n : 128 + wn * GW + 16 * (n - NG);
    return wn * WTN + 16 * n;
  };

  // prologue: STAGES-1 K-steps in flight
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KB) issue(s);

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f pcar[SM];                     // last column's partial, promoted in the next step
  float scar[SM][4];
#pragma unroll
  for (int m = 0; m < SM; ++m) {
    pcar[m] = zero;
#pragma unroll
    for (int i = 0; i < 4; ++i) scar[m][i] = 0.f;
  }
  for (int kt = 0; kt < KB; ++kt) {
    // wait until this wave's loads of step kt have landed, then for every wave's
    if (kt + STAGES - 2 < KB) {
      wait_vmcnt<LOADS * (STAGES - 2)>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_only();
    // the slot consumed in step kt-1 is free: refill it with step kt+STAGES-1
    if (kt + STAGES - 1 < KB) issue(kt + STAGES - 1);

    const int slot = kt % STAGES;
    const uint8_t* As = smem + slot * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    // fragment and scale reads of this step, issued together
    const float sb0 = sA[slot][wave][AROWS];
    const float sb1 = sA[slot][wave][AROWS + 1];
    v8i af[SM];
    float4 sa4[SM];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const int rw0 = wm * WTM + 16 * m;
      af[m] = lds_frag(As, rw0 + (lane & 15), lane >> 4);
      const int r = rw0 + 4 * (lane >> 4);          // 4 consecutive rows, one wave segment
      sa4[m] = *reinterpret_cast<const float4*>(&sA[slot][r / AROWS][r % AROWS]);
    }
    v8i bq0 = lds_frag(Bs, sub_brow(0) + (lane & 15), lane >> 4);
    v8i bq1 = lds_frag(Bs, sub_brow(SN > 1 ? 1 : 0) + (lane & 15), lane >> 4);
    // the previous step's last column, deferred to overlap the reads above
    if (kt > 0) {
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][SN - 1][i] = fmaf(pcar[m][i], scar[m][i], acc[m][SN - 1][i]);
    }
    float s0[SM][4], s1[SM][4];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const float sa[4] = {sa4[m].x, sa4[m].y, sa4[m].z, sa4[m].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0[m][i] = sa[i] * sb0;
        s1[m][i] = sa[i] * sb1;
      }
    }
    // Software pipeline over the n sub-tiles, pinned with scheduling fences: each MFMA
    // of column n+1 is followed by the four FMAs that fold the (finished) partial of
    // column n; B fragments are read two columns ahead.
    v4f pc[SM], pn[SM];
#pragma unroll
    for (int m = 0; m < SM; ++m)
      pc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bq0, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const bool second = SWIGLU && n >= NG;
      const v8i bn = bq1;
      if (n + 2 < SN) bq1 = lds_frag(Bs, sub_brow(n + 2) + (lane & 15), lane >> 4);
      if (n + 1 < SN) {
#pragma unroll
        for (int m = 0; m < SM; ++m) {
          __builtin_amdgcn_sched_barrier(0);
          pn[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bn, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m][n][i] = fmaf(pc[m][i], second ? s1[m][i] : s0[m][i], acc[m][n][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < SM; ++m) pc[m] = pn[m];
      } else {
#pragma unroll
        for (int m = 0; m < SM; ++m) {
          pcar[m] = pc[m];
#pragma unroll
          for (int i = 0; i < 4; ++i) scar[m][i] = second ? s1[m][i] : s0[m][i];
        }
      }
    }
  }
  // the last step's last column
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][SN - 1][i] = fmaf(pcar[m][i], scar[m][i], acc[m][SN - 1][i]);
  __syncthreads();   // every wave is done with the ring before its LDS is reused

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
      const float bv = bias ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = mt.row_begin + rbase + 16 * m + i;
          if (p < mt.row_end) a.y_out[static_cast<size_t>(p) * N + col] = acc[m][n][i] + bv;
        }
    }
  }
}

// ------------------------------------------------------------------------------------
// Large-group variant: 256 x 256 workgroup tile, eight waves in a 4 (M) x 2 (N) grid,
// each wave 64 x 128 (4 x 8 sub-tiles of 16 x 16), two waves per SIMD so that one wave's
// promotion FMAs and LDS reads overlap the other's MFMAs.  The LDS ring holds two K-steps
// (2 x 64 KB): the loads of step k+1 are in flight while step k is multiplied.  Wave rows
// that lie entirely past the M-tile's rows skip their MFMAs (a short last tile of an
// expert costs only its live rows).  Two K-steps of lookahead do not cover the latency of
// a weight tile that comes from HBM, so each step also touches, PF K-steps ahead, the
// cache lines of the A and B rows it will load then (a one-dword direct-to-LDS load per
// line into a scratch area), which brings them into L2 early.
// ------------------------------------------------------------------------------------
template <bool SWIGLU, int PF>
__global__ __launch_bounds__(512) void grouped_gemm256_kernel(const GemmArgs a, int max_tiles,
                                                              int ntiles, int grid) {
  constexpr int BM = 256, BN = 256, WN = 2;
  constexpr int SM = 4, SN = 8, NG = 4, GW = 64;     // gemm1: 64 gate + 64 up columns/wave
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  constexpr int ROWS_PER_WAVE = 32;                  // A and B rows each wave fetches
  constexpr int LOADS = 4 + 4 + 1;                   // vmem instructions per wave and step

  __shared__ __align__(16) uint8_t smem[2 * STAGE];
  __shared__ __align__(16) float sS[2][8][64];      // per wave: 32 A-row scales, 4 B scales
  __shared__ int rowsrc[BM];
  __shared__ float red[WN][BM];
  __shared__ __align__(16) float pf_sink[8][64];    // destination of the L2 touches

  const int b = blockIdx.x;
  const int L = (b % 8) * (grid / 8) + b / 8;
  const int mti = L % max_tiles, nt = L / max_tiles;
  if (nt >= ntiles || mti >= *a.num_tiles) return;
  MTile mt = a.tiles[mti];
  mt.expert = __builtin_amdgcn_readfirstlane(mt.expert);
  mt.row_begin = __builtin_amdgcn_readfirstlane(mt.row_begin);
  mt.row_end = __builtin_amdgcn_readfirstlane(mt.row_end);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, N = a.N, I = a.I;
  const int KB = ceil_div(K, kBlock), NBs = ceil_div(N, kBlock);
  const int e = mt.expert;
  const int live_rows = mt.row_end - mt.row_begin;
  const bool wave_live = wm * 64 < live_rows;
  const uint8_t* Bexp = a.B + static_cast<size_t>(e) * N * K;
  const float* Bsc = a.B_scale + static_cast<size_t>(e) * NBs * KB;

  for (int r = tid; r < BM; r += 512) {
    const int p = mt.row_begin + r;
    int src = -1;
    if (p < mt.row_end) src = SWIGLU ? a.perm[p] / a.top_k : p;
    rowsrc[r] = src;
  }
  __syncthreads();

  // ---- fetch descriptors: wave w fetches A rows and B rows [32 w, 32 w + 32) ----
  const int a_slot = lane & 7, a_r8 = lane >> 3;
  unsigned a_off[4], b_off[4];
  bool a_ok[4], b_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wave * ROWS_PER_WAVE + i * 8 + a_r8;
    const int src = rowsrc[row];
    a_ok[i] = src >= 0;
    a_off[i] = static_cast<unsigned>(src < 0 ? 0 : src) * K + ((a_slot ^ swz_key(row)) << 4);
    int g = -1;
    if (SWIGLU) {
      const int j = nt * 128 + (row & 127);
      if (j < I) g = (row >> 7) * I + j;
    } else {
      const int col = nt * BN + row;
      if (col < N) g = col;
    }
    b_ok[i] = g >= 0;
    b_off[i] = static_cast<unsigned>(g < 0 ? 0 : g) * K + ((a_slot ^ swz_key(row)) << 4);
  }
  // scale lanes: [0, 32) the activation scales of the wave's A rows; 32 + q the weight
  // block scale of column group q (gemm1: q = 2 wn' + {gate, up}; gemm2: q = wn')
  const float* s_ptr = kZeroScale;
  bool s_live = false;
  if (lane < 32) {
    const int src = rowsrc[wave * ROWS_PER_WAVE + lane];
    s_live = src >= 0;
    s_ptr = a.A_scale + static_cast<size_t>(src < 0 ? 0 : src) * KB;
  } else if (lane < 36) {
    const int q = lane - 32;
    int row = -1;
    if (SWIGLU) {
      const int j0 = nt * 128 + (q >> 1) * GW;
      if (j0 < I) row = ((q & 1) ? I + j0 : j0) / kBlock;
    } else if (q < 2) {
      const int c0 = nt * BN + q * 128;
      if (c0 < N) row = c0 / kBlock;
    }
    s_live = row >= 0;
    s_ptr = Bsc + static_cast<size_t>(row < 0 ? 0 : row) * KB;
  }

  auto issue = [&](int kt) {   // all loads of K-step kt into ring slot kt & 1
    uint8_t* As = smem + (kt & 1) * STAGE;
    uint8_t* Bs = As + A_BYTES;
    const int k0 = kt * kBlock;
    if (k0 + kBlock <= K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) load_lds16_s(a_off[i], a.A + k0, As + (wave * ROWS_PER_WAVE + i * 8) * 128);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_lds16_s(b_off[i], Bexp + k0, Bs + (wave * ROWS_PER_WAVE + i * 8) * 128);
    } else {                     // ragged K tail: chunks past K come from zeros
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * ROWS_PER_WAVE + i * 8 + a_r8;
        const int kk = k0 + ((a_slot ^ swz_key(row)) << 4);
        const void* src = (a_ok[i] && kk < K) ? static_cast<const void*>(a.A + a_off[i] + k0) : kZeroChunk;
        load_lds16(src, As + (wave * ROWS_PER_WAVE + i * 8) * 128);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * ROWS_PER_WAVE + i * 8 + a_r8;
        const int kk = k0 + ((a_slot ^ swz_key(row)) << 4);
        const void* src = (b_ok[i] && kk < K) ? static_cast<const void*>(Bexp + b_off[i] + k0) : kZeroChunk;
        load_lds16(src, Bs + (wave * ROWS_PER_WAVE + i * 8) * 128);
      }
    }
    if (lane < 36) {
      const void* src = s_live ? static_cast<const void*>(s_ptr + kt) : kZeroScale;
      load_lds4(src, &sS[kt & 1][wave][0]);
    }
  };

  // L2 touch of K-step kt: lanes [0, 32) the A rows, lanes [32, 64) the B rows of this
  // wave's fetch range; the first and the last dword of each row's 128-byte chunk (the
  // chunk may straddle two cache lines)
  const uint8_t* pf_row;
  {
    const int row = wave * ROWS_PER_WAVE + (lane & 31);
    if (lane < 32) {
      const int src = rowsrc[row];
      pf_row = a.A + static_cast<size_t>(src < 0 ? 0 : src) * K;
    } else {
      int g = 0;
      if (SWIGLU) {
        const int j = nt * 128 + (row & 127);
        if (j < I) g = (row >> 7) * I + j;
      } else {
        const int col = nt * BN + row;
        if (col < N) g = col;
      }
      pf_row = Bexp + static_cast<size_t>(g) * K;
    }
  }
  auto touch = [&](int kt) {
    const int k0 = kt * kBlock;
    const int k1 = min(k0 + kBlock, K) - 4;
    load_lds4(pf_row + k0, &pf_sink[wave][0]);
    load_lds4(pf_row + k1, &pf_sink[wave][0]);
  };

  auto sub_brow = [&](int n) {
    if (SWIGLU) return n < NG ? wn * GW + 16 * n : 128 + wn * GW + 16 * (n - NG);
    return wn * 128 + 16 * n;
  };

  v4f acc[SM][SN];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int n = 0; n < SN; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  if constexpr (PF > 1) {
    for (int d = 1; d < PF && d < KB; ++d) touch(d);
  }
  issue(0);
  for (int kt = 0; kt < KB; ++kt) {
    // this wave's loads of step kt have landed (the two L2 touches issued after them in
    // the previous step may still be in flight) ...
    if (PF > 1 && kt > 0 && kt - 1 + PF < KB) {
      wait_vmcnt<2>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_only();           // ... and every wave's; step kt-1's slot is free
    if (kt + 1 < KB) issue(kt + 1);
    if (PF > 1 && kt + PF < KB) touch(kt + PF);
    if (!wave_live) continue;

    const int slot = kt & 1;
    const uint8_t* As = smem + slot * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    float sb0, sb1;
    if (SWIGLU) {
      sb0 = sS[slot][0][32 + 2 * wn];
      sb1 = sS[slot][0][33 + 2 * wn];
    } else {
      sb0 = sS[slot][0][32 + wn];
      sb1 = sb0;
    }
    v8i af[SM];
    float s0[SM][4], s1[SM][4];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const int rw0 = wm * 64 + 16 * m;
      af[m] = lds_frag(As, rw0 + (lane & 15), lane >> 4);
      const int r = rw0 + 4 * (lane >> 4);
      const float4 sa = *reinterpret_cast<const float4*>(&sS[slot][r >> 5][r & 31]);
      s0[m][0] = sa.x * sb0; s0[m][1] = sa.y * sb0; s0[m][2] = sa.z * sb0; s0[m][3] = sa.w * sb0;
      if (SWIGLU) {
        s1[m][0] = sa.x * sb1; s1[m][1] = sa.y * sb1; s1[m][2] = sa.z * sb1; s1[m][3] = sa.w * sb1;
      }
    }
    // Software pipeline over the 32 products (column-major): product j goes to partial
    // j % 3 and is folded into its accumulator two products later, so the FMAs never wait
    // for the MFMA just issued; B fragments are read one column ahead.
    v8i bq[2];
    bq[0] = lds_frag(Bs, sub_brow(0) + (lane & 15), lane >> 4);
    v4f pp[3];
#pragma unroll
    for (int j = 0; j < SM * SN + 2; ++j) {
      if (j < SM * SN) {
        const int n = j / SM, m = j % SM;
        if (m == 0 && n + 1 < SN) bq[(n + 1) & 1] = lds_frag(Bs, sub_brow(n + 1) + (lane & 15), lane >> 4);
        pp[j % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bq[n & 1], zero, 0, 0, 0, 0, 0, 0);
      }
      if (j >= 2) {
        const int q = j - 2, n = q / SM, m = q % SM;
        const bool second = SWIGLU && n >= NG;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][n][i] = fmaf(pp[q % 3][i], second ? s1[m][i] : s0[m][i], acc[m][n][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();   // every wave is done with the ring before its LDS is reused

  const int rbase = wm * 64 + 4 * (lane >> 4);   // + 16 m + i
  if constexpr (SWIGLU) {
    const int KBI = ceil_div(I, kBlock);
    const uint16_t* bias = a.bias ? a.bias + static_cast<size_t>(e) * N : nullptr;
    float hv[SM][NG][4];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int j = nt * 128 + wn * GW + 16 * n + (lane & 15);
      const bool ok = j < I;
      const float bg = (bias && ok) ? bf16_to_f32(bias[j]) : 0.f;
      const float bu = (bias && ok) ? bf16_to_f32(bias[I + j]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[m][n][i] + bg;
          const float u = acc[m][n + NG][i] + bu;
          const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          hv[m][n][i] = ok ? h : 0.f;
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
    uint8_t* hs = smem;   // h codes of the tile, [256][128], staged for 16-byte stores
#pragma unroll
    for (int m = 0; m < SM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + 16 * m + i;
        const float s = group_scale(fmaxf(red[0][r], red[1][r]));
#pragma unroll
        for (int n = 0; n < NG; ++n)
          hs[r * 128 + wn * GW + 16 * n + (lane & 15)] =
              static_cast<uint8_t>(encode2(hv[m][n][i], 0.f, s) & 0xFFu);
        const int p = mt.row_begin + r;
        if (wn == 0 && (lane & 15) == 0 && p < mt.row_end)
          a.h_scale[static_cast<size_t>(p) * KBI + nt] = s;
      }
    __syncthreads();
    for (int q = tid; q < BM * 8; q += 512) {
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
      const int col = nt * BN + wn * 128 + 16 * n + (lane & 15);
      if (col >= N) continue;
      const float bv = bias ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = mt.row_begin + rbase + 16 * m + i;
          if (p < mt.row_end) a.y_out[static_cast<size_t>(p) * N + col] = acc[m][n][i] + bv;
        }
    }
  }
}

constexpr int kGemmPrefetch = 0;   // K-steps between the L2 touch and the use of a chunk

int gemm_tile_rows(long rows, int E) {
  const long avg = rows / (E > 0 ? E : 1);
  if (avg <= 24) return 16;
  if (avg <= 96) return 64;
  if (avg <= 160) return 128;
  return 256;
}

template <bool SWIGLU>
static void launch_gemm(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  const int ntiles = SWIGLU ? ceil_div(a.I, 128) : ceil_div(a.N, 256);
  const long total = static_cast<long>(max_tiles) * ntiles;
  const int grid = static_cast<int>((total + 7) / 8 * 8);
  if (bm == 256) {
    grouped_gemm256_kernel<SWIGLU, kGemmPrefetch><<<grid, 512, 0, st>>>(a, max_tiles, ntiles, grid);
    return;
  }
  switch (bm) {
    case 16:
      grouped_gemm_kernel<16, 256, 1, 4, SWIGLU, 4><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      break;
    case 64:
      grouped_gemm_kernel<64, 256, 1, 4, SWIGLU, 3><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      break;
    default:
      grouped_gemm_kernel<128, 256, 2, 2, SWIGLU, 3><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      break;
  }
}

void launch_gemm1(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  launch_gemm<true>(a, bm, max_tiles, st);
}
void launch_gemm2(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  launch_gemm<false>(a, bm, max_tiles, st);
}

}  // namespace moe
