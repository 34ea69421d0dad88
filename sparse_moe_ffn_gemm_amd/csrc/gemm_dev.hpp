// Device building blocks of the grouped FP8 GEMMs (gemm.hip), shared with the fused decode
// kernel (fused.hip): LDS layout helpers, direct-to-LDS loads, the tile order, and the
// row-run tile body.  The layouts and the kernels' design are described in gemm.hip.
#pragma once

#include "kernels.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

static __device__ __align__(16) const uint8_t kZeroChunk[64] = {0};
static __device__ __align__(16) const float kZeroScale[4] = {0.f, 0.f, 0.f, 0.f};

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

// MXFP4 weight tiles in LDS: 16 rows x 64 bytes (1 KB, one tile of the tiled storage per
// K-step), 16-byte chunk c of row r in slot c ^ ((r >> 1) & 3), so the rows that one read
// phase serves fall in distinct banks.  The e2m1 fragment of lane (row r, group g) is the
// row's chunk g (K [32 g, 32 g + 32)), in the low four dwords of the operand.
__device__ __forceinline__ int swz4_key(int row) { return (row >> 1) & 3; }

__device__ __forceinline__ v8i lds_frag4(const uint8_t* base, int row, int g) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 64 + ((g ^ swz4_key(row)) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
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

// Device-coherent variants of the direct-to-LDS loads (COH = true: the sc1 cache policy,
// as store_c / load_c in common.hpp).
template <bool COH>
__device__ __forceinline__ void load_lds16_c(const void* g, const void* lds) {
  if constexpr (COH)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1"
                 :: "v"(g), "s"(lds_addr(lds)) : "memory", "m0");
  else
    load_lds16(g, lds);
}
template <bool COH>
__device__ __forceinline__ void load_lds4_c(const void* g, const void* lds) {
  if constexpr (COH)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off sc1"
                 :: "v"(g), "s"(lds_addr(lds)) : "memory", "m0");
  else
    load_lds4(g, lds);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Tile L of the expert-major order (an expert's M-tiles fastest, then its n-tiles) of
// `ntiles` n-tiles per M-tile.  The expert e with off[e] * ntiles <= L < off[e+1] * ntiles:
// off is non-decreasing, so e + 1 is the number of experts with off[e] * ntiles <= L,
// counted by ballots over one round of independent loads (E <= 256).
// `eto`: the expert_tile_off table, in global memory or a workgroup's LDS copy.
__device__ __forceinline__ void tile_of(const GemmArgs& a, const int32_t* eto, int ntiles, int L,
                                        int& nt, MTile& mt) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
#pragma unroll
  for (int base = 0; base < 256; base += 64) {
    if (base < a.E) {
      const int idx = base + lane;
      const bool le = idx < a.E && eto[idx] * ntiles <= L;
      cnt += __builtin_popcountll(__ballot(le));
    }
  }
  const int lo = __builtin_amdgcn_readfirstlane(cnt - 1);
  const int t0 = eto[lo];
  const int mcount = eto[lo + 1] - t0;
  const int local = L - t0 * ntiles;
  nt = local / mcount;
  mt = a.tiles[t0 + local % mcount];
  mt.expert = __builtin_amdgcn_readfirstlane(mt.expert);
  mt.row_begin = __builtin_amdgcn_readfirstlane(mt.row_begin);
  mt.row_end = __builtin_amdgcn_readfirstlane(mt.row_end);
}

// Which tile this workgroup of a one-tile-per-workgroup launch computes: the expert-major
// order cut into eight contiguous ranges, one per XCD (blocks are dealt to the XCDs round-
// robin), so the concurrent workgroups of an XCD share the expert's activation rows
// across n-tiles and each weight tile across the expert's M-tiles in their L2.  False
// for blocks past the device-side tile count.
__device__ __forceinline__ bool pick_tile(const GemmArgs& a, int ntiles, int& nt, MTile& mt) {
  const int total = __builtin_amdgcn_readfirstlane(*a.num_tiles) * ntiles;
  const int per_xcd = (total + 7) / 8;
  const int b = blockIdx.x;
  if (b / 8 >= per_xcd) return false;
  const int L = (b % 8) * per_xcd + b / 8;
  if (L >= total) return false;
  tile_of(a, a.expert_tile_off, ntiles, L, nt, mt);
  return true;
}

// Workgroup barrier without the memory fences of __syncthreads (the ring's loads are
// waited for explicitly); the "memory" clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// ------------------------------------------------------------------------------------
// Row-run streaming variant for decode-sized groups (M-tiles of at most 16 rows), the
// HBM-bound case: every weight byte feeds only the tile's 16 rows.  The weight stream
// is laid out for DRAM locality: HBM throughput of a read stream grows with the
// contiguous run fetched from each weight row at a time (measured with register loads
// over rows of 2880 bytes: about 4.1 TB/s for 128-byte runs, 5.4 TB/s for 512 and
// 6.4 TB/s for about 1 KB).  So each wave owns ONE 16-row weight sub-tile and walks its
// rows in bursts of KS K-blocks (KS x 128 contiguous bytes per row), NB (two) bursts in
// flight in registers, with no barrier in the K loop.  The tile's 16 activation rows
// (all of K) and their scales are staged in LDS once, fetched while the first weight
// bursts are in flight.
//
// A workgroup is eight waves over 16 rows x 128 output columns, wave w taking columns
// [16w, 16w+16).  gemm1: the wave streams the 16 gate rows and then the 16 matching up
// rows of w13, so each lane ends with the gate and up sums of the same four columns
// and the workgroup's 128 columns are exactly one 1x128 group of h.  gemm2: the wave
// streams 16 rows of w2.  All sixteen rows of a sub-tile share one 128-row scale block.
//
// K tail (K a multiple of 64): the staged activation tile holds zeros past K, and the
// weight fragment's upper half re-reads its lower half in a half-filled last block, so
// the extra products vanish.  Bursts padded past the last K-block re-read that block
// (L2 hits) and are scaled by zero.  Rows past the tile's end are staged from its first
// row; their outputs are never stored.
// ------------------------------------------------------------------------------------
// FP4 (with MX): the weights are MXFP4, stored in 16-row x 128-K tiles (1024 code bytes,
// row r at byte 64 r, K past the row zero; 64 scale bytes, row r's four E8M0 codes at byte
// 4 r), so a wave's sub-tile is one contiguous run of KB tiles and each burst reads KS
// whole kilobytes; scattered per-row pieces and per-row scale words streamed about 30 %
// slower.  The matrix cores take an e2m1 first operand, whose lane (r, g) holds the 32
// consecutive K values [32 g, 32 g + 32) of row r in 16 bytes (element 2j in the low
// nibble), against the e4m3 activation fragment.
//
// One M-tile (mt) x n-tile (nt) of the row-run variant by a workgroup of NW waves;
// dyn_lds: the tile's LDS (rowrun_lds_bytes(K)).  Every thread must call it.
//
// COH: the activation tile (x codes through perm, or h) and its scales are read and the
// tile's outputs (h and its scales, or y) are written with device-coherent accesses
// (load_c, load_lds16_c, store_c), for a launch whose workgroups hand them to each other.
// WIDE (gemm2 only): each wave streams two 16-row sub-tiles of w2, 128 rows apart, so the
// workgroup covers 256 output columns (n-tile nt: [256 nt, 256 nt + 256)); every column's
// sum is formed exactly as in the 128-column tile.
template <bool SWIGLU, int KS, bool MX = false, bool FP4 = false, int NW = 8, bool RAW = false,
          int NB = 2, bool COH = false, bool WIDE = false>
__device__ __forceinline__ void rowrun_tile(const GemmArgs& a, const int nt, const MTile& mt,
                                            uint8_t* dyn_lds) {
  static_assert(MX || !FP4, "MXFP4 weights take E8M0 scales");
  // NW = 2 (MX only: h blocks of 32 columns are wave pairs; the block-scaled 1x128 groups
  // need all eight waves): 32-column workgroups, four times as many, for launches that
  // would otherwise leave most CUs idle
  static_assert(NW == 8 || (MX && NW == 2), "workgroup width");
  constexpr int WAVES = NW;
  static_assert(!(SWIGLU && WIDE), "wide tiles are gemm2 tiles");
  constexpr int NSUB = (SWIGLU || WIDE) ? 2 : 1;   // weight sub-tiles per wave (gate, up)
  // B rows of sub-tile 1 past those of sub-tile 0: the up half of w13, or 128 rows of w2
  const int s1_rows = SWIGLU ? a.I : 128;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, N = a.N, I = a.I;
  const int KB = ceil_div(K, kBlock), NBs = ceil_div(N, kBlock);
  const int e = mt.expert;
  const int r = lane & 15, g = lane >> 4;
  // LDS: activation tile [KB][16][128] (chunk-swizzled rows), its scales [KB4][16]
  // (KB rounded up to the 4 blocks one scale fetch covers), and the gemm1 row-amax
  // exchange [8][16]
  uint8_t* sA = dyn_lds;
  float* sSa = reinterpret_cast<float*>(dyn_lds + KB * 2048);
  float* red = sSa + ceil_div(KB, 4) * 64;

  const int c0 = nt * 16 * WAVES * (WIDE ? 2 : 1) + 16 * wave;   // the wave's first output column
  const bool live = c0 < (SWIGLU ? I : N);   // I, N multiples of 64: all 16 or none
  const bool live1 = WIDE ? c0 + 128 < N : live;   // the wide tile's second sub-tile

  // ---- the wave's weight stream: sub-tile s, K-block j, in bursts of KS blocks ----
  const uint8_t* Bexp = a.B + static_cast<size_t>(e) * N * (FP4 ? KB * 64 : K);
  const float* Bsc = a.B_scale + static_cast<size_t>(e) * NBs * KB;
  const int bps = ceil_div(KB, KS);          // bursts per sub-tile
  const int nb = (live1 ? NSUB : 1) * bps;   // bursts of the wave (sub-tile major)
  const int nbp = (nb + NB - 1) / NB * NB;   // padded to the NB-slot ring
  unsigned b_off[NSUB];
  float sbg[NSUB];                           // lane j: weight block scale of K-block j
  const uint8_t* bmx[NSUB];                  // MX: the lane's E8M0 codes in the scale tiles
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const bool ls = s == 1 ? live1 : live;   // dead sub-tiles address row 0
    const int row = ls ? (s == 1 ? s1_rows : 0) + c0 + r : r;
    b_off[s] = FP4 ? static_cast<unsigned>(row - r) * KB * 64 + 64 * r + 16 * g
                   : static_cast<unsigned>(row) * K + 16 * g;
    if constexpr (MX) {
      // the tile row's 4 codes of K-block 0 (64 bytes per K-block)
      bmx[s] = a.B_mx + (static_cast<size_t>(e) * N + (row - r)) * (4 * KB) + 4 * r;
      sbg[s] = 0.f;
    } else {
      const int brow = (row - r) / kBlock;
      sbg[s] = (ls && lane < KB) ? Bsc[static_cast<size_t>(brow) * KB + lane] : 0.f;
    }
  }

  v8i ring[NB][KS];
  uint32_t xring[NB][KS];   // MXFP8: the burst's weight scale words (byte g is the lane's)
  auto issue = [&](int b, v8i (&bq)[KS], uint32_t (&xq)[KS]) {
    const int bb = b < nb ? b : nb - 1;
    const int s = bb / bps, j0 = (bb % bps) * KS;
    const unsigned bo = (NSUB == 2 && s == 1) ? b_off[NSUB - 1] : b_off[0];
    if constexpr (MX) {
      const uint8_t* xr = (NSUB == 2 && s == 1) ? bmx[NSUB - 1] : bmx[0];
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const int jj = j0 + t < KB ? j0 + t : KB - 1;
        xq[t] = *reinterpret_cast<const uint32_t*>(xr + 64 * jj);
      }
    }
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int jj = j0 + t < KB ? j0 + t : KB - 1;
      if constexpr (FP4) {
        // one 1024-byte tile per K-step (a half-filled last block holds zero codes past K)
        const uint4 lo = *reinterpret_cast<const uint4*>(Bexp + jj * 1024 + bo);
        bq[t] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
      } else {
        const unsigned hoff = (jj + 1) * kBlock <= K ? 64u : 0u;   // half block: re-read chunks 0-3
        const uint8_t* base = Bexp + jj * kBlock;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + bo);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + hoff + bo);
        bq[t] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
  };
  v4f acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int b, const v8i (&bq)[KS], const uint32_t (&xq)[KS]) {
    const bool bl = b < nb;
    const int bb = bl ? b : nb - 1;
    const int s = bb / bps, j0 = (bb % bps) * KS;
    const float sbs = (NSUB == 2 && s == 1) ? sbg[NSUB - 1] : sbg[0];
    if constexpr (MX) {
      // The matrix cores apply both E8M0 codes of the lane's block and accumulate in
      // place (the result register is the live accumulator, never a scale operand's);
      // blocks past K (padded bursts re-read the last one) are skipped: a wave-uniform
      // branch.
      v4f& ac = (NSUB == 2 && s == 1) ? acc[NSUB - 1] : acc[0];
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        if (bl && j0 + t < KB) {
          const int jj = j0 + t;
          const v8i af = lds_frag(sA + jj * 2048, r, g);
          const int xa = reinterpret_cast<const uint8_t*>(sSa)[4 * (jj * 16 + r) + g];
          const int xb = static_cast<int>((xq[t] >> (8 * g)) & 0xFFu);
          ac = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq[t], af, ac, FP4 ? 4 : 0, 0, 0, xb,
                                                                0, xa);
          // both scale operands stay live past the instruction, so its result registers
          // can never be allocated over them (the matrix core reads them late)
          asm volatile("" : "+v"(ac) : "v"(xa), "v"(xb));
        }
      }
      return;
    }
    v4f pr[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int jj = j0 + t < KB ? j0 + t : KB - 1;
      const v8i af = lds_frag(sA + jj * 2048, r, g);
      pr[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq[t], af, zero, 0, 0, 0, 0, 0, 0);
    }
    // each K-block's product folded into the accumulator in K order (the sum does not
    // depend on the burst length)
    float sc[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int j = j0 + t;
      const int jj = j < KB ? j : KB - 1;
      const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sbs), jj));
      sc[t] = (bl && j < KB) ? sSa[jj * 16 + r] * sb : 0.f;
    }
    if (NSUB == 2 && s == 1) {
#pragma unroll
      for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[NSUB - 1][i] = fmaf(pr[t][i], sc[t], acc[NSUB - 1][i]);
    } else {
#pragma unroll
      for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[0][i] = fmaf(pr[t][i], sc[t], acc[0][i]);
    }
  };

  // the first NB weight bursts go out before the activation rows are even located
  if (live) {
#pragma unroll
    for (int i = 0; i < NB; ++i) issue(i, ring[i], xring[i]);
  }
  // ---- stage the activation tile and its scales (all waves share the fetches) ----
  auto src_row = [&](int rr) {
    const int q = mt.row_begin + rr < mt.row_end ? mt.row_begin + rr : mt.row_begin;
    const int s = SWIGLU ? load_c<COH>(a.perm + q) / a.top_k : q;
    return static_cast<unsigned>(s) < static_cast<unsigned>(a.A_rows) ? s : 0;   // never read past A
  };
  {
    // fetch q: block q >> 1, rows 8 (q & 1) .. +8; lane -> row 8 (q & 1) + (lane >> 3),
    // LDS slot lane & 7 holding global chunk slot ^ (row & 7)
    const int rq = lane >> 3, slot = lane & 7;
    const unsigned off0 = static_cast<unsigned>(src_row(rq)) * K;
    const unsigned off1 = static_cast<unsigned>(src_row(8 + rq)) * K;
    for (int q = wave; q < 2 * KB; q += WAVES) {
      const int j = q >> 1, row = 8 * (q & 1) + rq;
      const int kk = j * kBlock + ((slot ^ swz_key(row)) << 4);
      const void* src = kk < K ? static_cast<const void*>(a.A + ((q & 1) ? off1 : off0) + kk)
                               : static_cast<const void*>(kZeroChunk);
      load_lds16_c<COH>(src, sA + j * 2048 + 8 * (q & 1) * 128);
    }
    // scales: fetch q covers blocks 4q .. 4q+3, lane -> block 4q + (lane >> 4), row lane & 15
    // (MXFP8: the row's 4-byte word of E8M0 codes of that block)
    const unsigned so = static_cast<unsigned>(src_row(r)) * KB;
    for (int q = wave; q < ceil_div(KB, 4); q += WAVES) {
      const int j = 4 * q + g;
      const void* src = j >= KB ? static_cast<const void*>(kZeroScale)
                        : MX ? static_cast<const void*>(a.A_mx + 4 * (so + j))
                             : static_cast<const void*>(a.A_scale + so + j);
      load_lds4_c<COH>(src, sSa + 64 * q);
    }
  }

  wait_vmcnt<0>();   // this wave's staging fetches (and its first bursts) have landed ...
  __syncthreads();   // ... and so have every wave's
  // the weight block scales have landed too: passing them through an empty asm makes them
  // values the compiler no longer tracks as outstanding loads, so it does not drain every
  // in-flight burst (vmcnt(0)) before their first use in each K-loop iteration
  if constexpr (!MX) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) asm volatile("" : "+v"(sbg[s]));
  }

  if (live) {
    for (int b0 = 0; b0 < nbp - NB; b0 += NB) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        compute(b0 + i, ring[i], xring[i]);
        issue(b0 + i + NB, ring[i], xring[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) compute(nbp - NB + i, ring[i], xring[i]);
  }

  // ---- epilogue: lane holds row r and the four columns c0 + 4g + i ----
  const int p = mt.row_begin + r;
  const int cq = c0 + 4 * g;
  if constexpr (RAW) {   // the fp32 accumulators (gate columns, then up columns I + ...)
    if (!live || p >= mt.row_end) return;
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
      if (s == 0 || live1)
        *reinterpret_cast<float4*>(a.c_raw + static_cast<size_t>(p) * N + (s == 1 ? s1_rows : 0) + cq) =
            make_float4(acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
    return;
  }
  const uint16_t* bias = a.bias ? a.bias + static_cast<size_t>(e) * N : nullptr;
  if constexpr (SWIGLU) {
    const int KBI = ceil_div(I, kBlock);
    float hv[4];
    float mx = 0.f;
    float bg[4] = {0.f, 0.f, 0.f, 0.f}, bu[4] = {0.f, 0.f, 0.f, 0.f};
    if (live && bias) {
      const uint2 g2 = *reinterpret_cast<const uint2*>(bias + cq);
      const uint2 u2 = *reinterpret_cast<const uint2*>(bias + I + cq);
      bg[0] = __uint_as_float(g2.x << 16); bg[1] = __uint_as_float(g2.x & 0xFFFF0000u);
      bg[2] = __uint_as_float(g2.y << 16); bg[3] = __uint_as_float(g2.y & 0xFFFF0000u);
      bu[0] = __uint_as_float(u2.x << 16); bu[1] = __uint_as_float(u2.x & 0xFFFF0000u);
      bu[2] = __uint_as_float(u2.y << 16); bu[3] = __uint_as_float(u2.y & 0xFFFF0000u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gv = acc[0][i] + bg[i];
      const float uv = acc[NSUB - 1][i] + bu[i];
      const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
      hv[i] = live ? h : 0.f;
      mx = fmaxf(mx, fabsf(hv[i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lane < 16) red[wave * 16 + lane] = mx;
    __syncthreads();
    if constexpr (MX) {
      // 1x32 MX blocks: waves 2q and 2q+1 hold the 32 columns of block q of the tile;
      // blocks past I (h = 0 there) get the pad code 127
      if (p >= mt.row_end) return;
      const float amax32 = fmaxf(red[(wave & ~1) * 16 + r], red[(wave | 1) * 16 + r]);
      const int code = mx_scale_code(amax32);
      if (live)
        store_c<COH>(reinterpret_cast<uint32_t*>(a.h_out + static_cast<size_t>(p) * I + cq),
                     encode4_mul(hv[0], hv[1], hv[2], hv[3], mx_inv_scale(code)));
      if ((wave & 1) == 0 && g == 0)
        store_c<COH>(a.h_mx + static_cast<size_t>(p) * 4 * KBI + (nt * 16 * WAVES + 16 * wave) / kMxBlock,
                     static_cast<uint8_t>(code));
      return;
    }
    if (!live || p >= mt.row_end) return;
    float amax = red[r];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) amax = fmaxf(amax, red[w * 16 + r]);
    const float sc = group_scale(amax);
    const float rs = __builtin_amdgcn_rcpf(sc);   // quotient: reciprocal plus one correction
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q0 = hv[i] * rs;
      const float q1 = fmaf(fmaf(-q0, sc, hv[i]), rs, q0);
      q[i] = fminf(fmaxf(q1, -kFp8Max), kFp8Max);
    }
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false)) & 0xFFFFu;
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], 0, false)) & 0xFFFFu;
    store_c<COH>(reinterpret_cast<uint32_t*>(a.h_out + static_cast<size_t>(p) * I + cq), lo | (hi << 16));
    if (wave == 0 && lane < 16) store_c<COH>(a.h_scale + static_cast<size_t>(p) * KBI + nt, sc);
  } else {
    if (p >= mt.row_end) return;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {   // (WIDE: sub-tile 1 holds columns 128 further on)
      if (!(s == 1 ? live1 : live)) continue;
      const int cs = cq + (s == 1 ? 128 : 0);
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
        const uint2 b2 = *reinterpret_cast<const uint2*>(bias + cs);
        bv[0] = __uint_as_float(b2.x << 16); bv[1] = __uint_as_float(b2.x & 0xFFFF0000u);
        bv[2] = __uint_as_float(b2.y << 16); bv[3] = __uint_as_float(b2.y & 0xFFFF0000u);
      }
      const uint64_t ylo = f32_to_f16_sat(acc[s][0] + bv[0]) |
                           (static_cast<uint32_t>(f32_to_f16_sat(acc[s][1] + bv[1])) << 16);
      const uint64_t yhi = f32_to_f16_sat(acc[s][2] + bv[2]) |
                           (static_cast<uint32_t>(f32_to_f16_sat(acc[s][3] + bv[3])) << 16);
      store_c<COH>(reinterpret_cast<uint64_t*>(a.y_out + static_cast<size_t>(p) * N + cs), ylo | (yhi << 32));
    }
  }
}

// Dynamic LDS bytes of rowrun_tile over K: the activation tile, its scales, the row-amax
// exchange.
__host__ __device__ inline size_t rowrun_lds_bytes(int K) {
  const int KB = ceil_div(K, kBlock);
  return static_cast<size_t>(KB) * 2048 + ceil_div(KB, 4) * 256 + 8 * 16 * 4;
}

}  // namespace moe
