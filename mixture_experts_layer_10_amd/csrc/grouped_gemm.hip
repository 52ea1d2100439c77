// Grouped expert GEMMs ("27. Mixture of experts", section "Dispatch": Experts.expert run on each
// expert's contiguous rows, which "a grouped GEMM kernel does as one launch"; stretch exercise 2:
// one program per (expert, output tile), driven by the row-offset prefix sum).
//
//   gate_up: h[p, i]   = silu(X[p] . G[g, i]) * (X[p] . G[g, I + i])   SwiGLU fused in the epilogue
//   down:    out[p, n] = h[p] . Dn[g, n]                               fp32 output
//
// Both operands are contiguous along K (weights stored [out, in]), so A and B tiles are loaded the
// same way: 16-byte vectors. Tiles are staged in LDS with an XOR swizzle of the 16-byte chunks
// (defined with each kernel), so the matrix-core operand reads (32 rows at one k offset) hit
// distinct banks. bf16 uses 32x32x16 matrix-core steps with
// fp32 accumulators; fp32 uses an LDS-tiled FMA kernel.
//
// Scheduling: persistent workgroups. Each builds, in LDS, the prefix sum over groups of
// ceil(rows_g / BM) * n_tiles from the device-side offsets (no host round trip), then walks the
// tile list. Tile t -> (group by binary search, m-tile, n-tile), n fastest, so neighbouring tiles
// share their A rows and their expert's weights. Workgroup w runs on XCD w % 8; the list is cut into
// runs of (grid / 8) consecutive tiles per XCD, so tiles that share data share an L2. The streaming
// kernel orders its list longest first (build_tile_lists) and deals it in alternate directions.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// Tile list shared by both kernels.
// ---------------------------------------------------------------------------------------------
// s_pref[g] = sum_{g' < g} tiles_of(g'), for g = 0..G (G <= 2 * NT); ends with a barrier.
template <int NT, typename F>
__device__ void tile_prefix_scan(F tiles_of, int G, int* s_pref, int* s_tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = 2 * tid < G ? tiles_of(2 * tid) : 0, v1 = 2 * tid + 1 < G ? tiles_of(2 * tid + 1) : 0;
  const int own = v0 + v1;
  int inc = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_tmp[w];
  const int excl = before + inc - own;
  if (2 * tid < G) s_pref[2 * tid] = excl;
  if (2 * tid + 1 < G) s_pref[2 * tid + 1] = excl + v0;
  // the total: groups at or past G contribute nothing, so the last thread's inclusive sum is it
  // (written separately because G may equal 2 * NT, one past the last slot the loop covers)
  if (tid == NT - 1) s_pref[G] = before + inc;
  __syncthreads();
}

// s_pref[g] = sum_{g' < g} ceil(rows_g' / BM) * n_tiles, for g = 0..G. G <= 2 * NT.
template <int NT>
__device__ void build_tile_prefix(const int32_t* offsets, int G, int64_t max_rows, int BM, int n_tiles,
                                  int* s_pref, int* s_tmp) {
  tile_prefix_scan<NT>(
      [&](int g) {
        const int64_t rows = offsets ? static_cast<int64_t>(offsets[g + 1] - offsets[g]) : max_rows;
        return static_cast<int>((rows + BM - 1) / BM) * n_tiles;
      },
      G, s_pref, s_tmp);
}

// Tile list of the streaming kernel, the most work first. A tile costs about the number of its
// 32-row blocks that hold rows (those without rows skip their matrix-core steps). The list holds
// first every tile whose BM / 32 blocks all hold rows (group order, m-tile, n-tile fastest), then
// each group's last m-tile where it is shorter, ordered by its number of row blocks, most first
// (equal counts in group order), n-tile fastest. Dealt out round by round, the list leaves the
// cheap tiles for the last rounds, which then end together instead of on whichever full tiles
// fall last in group order.
// s_pref[g] = sum_{g' < g} (full m-tiles of g') * n_tiles, s_pref[G] = their total;
// s_plist[i] = the group of short m-tile i in list order. Returns the number of short m-tiles.
// G <= 2 * NT; s_cnt holds 2 * NT / 64 * 8 ints. Ends with a barrier.
template <int NT, int BM>
__device__ int build_tile_lists(const int32_t* offsets, int G, int64_t max_rows, int n_tiles, int* s_pref,
                                int* s_plist, int* s_tmp, int* s_cnt) {
  constexpr int NW = NT / 64, LB = BM / 32;
  static_assert(LB <= 8, "eight block counts per slot");
  auto rows_of = [&](int g) -> int64_t {
    return offsets ? static_cast<int64_t>(offsets[g + 1] - offsets[g]) : max_rows;
  };
  tile_prefix_scan<NT>(
      [&](int g) {
        const int64_t c = rows_of(g), rem = c % BM;
        return static_cast<int>(c / BM + (rem > BM - 32 ? 1 : 0)) * n_tiles;
      },
      G, s_pref, s_tmp);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // groups g = tid + k NT; slot k NW + wave holds groups 64 (k NW + wave) .. + 63 (group order)
  int cls[2];
  uint64_t same[2] = {0, 0};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int g = tid + k * NT;
    cls[k] = 0;
    if (g < G) {
      const int64_t rem = rows_of(g) % BM;
      if (rem > 0 && rem <= BM - 32) cls[k] = static_cast<int>((rem + 31) / 32);
    }
#pragma unroll
    for (int L = 1; L < LB; ++L) {
      const uint64_t m = __ballot(cls[k] == L);
      if (cls[k] == L) same[k] = m;
      if (lane == 0) s_cnt[(k * NW + wave) * 8 + L] = __popcll(m);
    }
  }
  __syncthreads();
  int total[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int slot = 0; slot < 2 * NW; ++slot)
#pragma unroll
    for (int L = 1; L < LB; ++L) total[L] += s_cnt[slot * 8 + L];
  int n_short = 0;
#pragma unroll
  for (int L = 1; L < LB; ++L) n_short += total[L];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = cls[k];
    if (c == 0) continue;
    int rank = 0;
#pragma unroll
    for (int L = 1; L < LB; ++L)
      if (L > c) rank += total[L];
    for (int slot = 0; slot < k * NW + wave; ++slot) rank += s_cnt[slot * 8 + c];
    rank += __popcll(same[k] & ((1ull << lane) - 1));
    s_plist[rank] = tid + k * NT;
  }
  __syncthreads();
  return n_short;
}

__device__ __forceinline__ int find_group(const int* s_pref, int G, int t) {
  int lo = 0, hi = G;  // invariant: s_pref[lo] <= t < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int tile_of_round(int r, int w, int P) {
  if ((P & 7) == 0) {
    const int per = P >> 3;
    return (r * 8 + (w & 7)) * per + (w >> 3);
  }
  return r * P + w;
}

// ---------------------------------------------------------------------------------------------
// bf16 matrix-core kernel.
//   WM x WN waves; each wave owns TM x TN blocks of 32x32.
//   BM = WM*TM*32 rows of A per tile, BNB = WN*TN*32 rows of B (weight rows) per tile.
//   SwiGLU: TN == 2, block 0 of a wave reads gate rows, block 1 the matching up rows; the tile's
//   B rows are [gate i0 .. i0+BNB/2) then [up I+i0 .. I+i0+BNB/2), giving BNB/2 h columns.
// ---------------------------------------------------------------------------------------------
constexpr int kBK = 64;            // k per LDS stage (8 chunks of 16 bytes per row)

template <int WM, int TM, int WN, int TN, bool kSwiGLU>
struct BfCfg {
  static constexpr int BM = WM * TM * 32;
  static constexpr int BNB = WN * TN * 32;
  static constexpr int NT = WM * WN * 64;
  static constexpr int A_LD = BM * 8 / NT;     // 16-byte chunks of A each thread loads per stage
  static constexpr int B_LD = BNB * 8 / NT;
  static constexpr int OUT_COLS = kSwiGLU ? BNB / 2 : BNB;
  static_assert(!kSwiGLU || TN == 2, "SwiGLU pairs one gate block with one up block");
  static_assert(A_LD * NT == BM * 8 && B_LD * NT == BNB * 8, "tile must split evenly over threads");
};

// 128-byte rows (64 bf16). The LDS serves a 16-byte-per-lane read 16 lanes at a time over 64 banks
// (256 bytes), so 16 consecutive rows at one logical chunk must land in 16 distinct 16-byte slots
// of a 256-byte window: chunk c of row r sits at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

template <int WM, int TM, int WN, int TN, bool kSwiGLU>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmArgs a) {
  using C = BfCfg<WM, TM, WN, TN, kSwiGLU>;
  constexpr int BM = C::BM, BNB = C::BNB, NT = C::NT;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BNB * kBK];
  __shared__ int s_pref[1025];
  __shared__ int s_tmp[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int G = a.G;
  // K and the output width
  const int K = kSwiGLU ? a.D : a.I;
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int n_tiles = (NOUT + C::OUT_COLS - 1) / C::OUT_COLS;

  build_tile_prefix<NT>(a.offsets, G, a.max_rows, BM, n_tiles, s_pref, s_tmp);
  const int total = s_pref[G];
  const int P = gridDim.x;

  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  const int ksteps = (K + kBK - 1) / kBK;

  for (int r = 0;; ++r) {
    const int t = tile_of_round(r, blockIdx.x, P);
    if (r * P >= total) break;
    if (t >= total) continue;
    const int g = find_group(s_pref, G, t);
    const int local = t - s_pref[g];
    const int mt = local / n_tiles, nt = local - mt * n_tiles;
    const int64_t row0 = a.offsets ? a.offsets[g] : 0;
    const int64_t rows = a.offsets ? static_cast<int64_t>(a.offsets[g + 1]) - row0 : a.max_rows;
    if (rows <= 0) continue;           // cannot happen with a consistent prefix; never index row -1
    const int m0 = mt * BM;
    const int c0 = nt * C::OUT_COLS;   // first output column of the tile

    // Source rows for this thread's A and B chunks (fixed over k).
    const uint16_t* srcA[C::A_LD];
    int chA[C::A_LD];
#pragma unroll
    for (int j = 0; j < C::A_LD; ++j) {
      const int idx = tid + j * NT, rr = idx >> 3;
      chA[j] = idx & 7;
      const int64_t lr = min<int64_t>(m0 + rr, rows - 1);   // rows past the group: any valid row
      const int64_t p = row0 + lr;
      const int64_t src = a.row_index ? a.row_index[p] : p;
      srcA[j] = X + src * K + chA[j] * 8;
    }
    const uint16_t* srcB[C::B_LD];
    int chB[C::B_LD];
    const uint16_t* Wg = W + static_cast<int64_t>(g) * (kSwiGLU ? 2LL * a.I * a.D : static_cast<int64_t>(a.D) * a.I);
#pragma unroll
    for (int j = 0; j < C::B_LD; ++j) {
      const int idx = tid + j * NT, rr = idx >> 3;
      chB[j] = idx & 7;
      int wrow;
      if (kSwiGLU) {
        const int half = BNB / 2;
        const int ci = min(c0 + (rr % half), NOUT - 1);
        wrow = rr < half ? ci : a.I + ci;
      } else {
        wrow = min(c0 + rr, NOUT - 1);
      }
      srcB[j] = Wg + static_cast<int64_t>(wrow) * K + chB[j] * 8;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    u32x4 ra[C::A_LD], rb[C::B_LD];
    auto gload = [&](int ks) {
      const int kb = ks * kBK;
#pragma unroll
      for (int j = 0; j < C::A_LD; ++j)
        ra[j] = (kb + chA[j] * 8 < K) ? *reinterpret_cast<const u32x4*>(srcA[j] + kb) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < C::B_LD; ++j)
        rb[j] = (kb + chB[j] * 8 < K) ? *reinterpret_cast<const u32x4*>(srcB[j] + kb) : u32x4{0, 0, 0, 0};
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < C::A_LD; ++j) {
        const int rr = (tid + j * NT) >> 3;
        *reinterpret_cast<u32x4*>(&sA[buf][swz(rr, chA[j])]) = ra[j];
      }
#pragma unroll
      for (int j = 0; j < C::B_LD; ++j) {
        const int rr = (tid + j * NT) >> 3;
        *reinterpret_cast<u32x4*>(&sB[buf][swz(rr, chB[j])]) = rb[j];
      }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < ksteps) gload(ks + 1);
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        u32x4 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = (wm * TM + i) * 32 + (lane & 31);
          fa[i] = *reinterpret_cast<const u32x4*>(&sA[buf][swz(row, ch)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = kSwiGLU ? (j * (BNB / 2) + wn * 32 + (lane & 31)) : ((wn * TN + j) * 32 + (lane & 31));
          fb[j] = *reinterpret_cast<const u32x4*>(&sB[buf][swz(row, ch)]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
      }
      if (ks + 1 < ksteps) sstore(buf ^ 1);
      __syncthreads();
    }

    // Epilogue.
    if constexpr (kSwiGLU) {
      uint16_t* H = static_cast<uint16_t*>(a.out);
      const int col = c0 + wn * 32 + (lane & 31);
      if (col < NOUT) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rr = m0 + (wm * TM + i) * 32 + acc_row(e, lane);
            if (rr < rows) {
              const float gt = acc[i][0][e], up = acc[i][1][e];
              H[(row0 + rr) * NOUT + col] = f32_to_bf16(silu(gt) * up);
            }
          }
      }
    } else if (a.out_f16s) {
      // fp16 form: the 16 lanes of a DPP row hold 16 consecutive columns of one output row
      // (NOUT % 16 == 0, so a group is wholly in or out)
      const int64_t rb = f16s_row_bytes(NOUT);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = c0 + (wn * TN + j) * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float v = acc[i][j][e];
            float m = fabsf(v);
            m = fmaxf(m, xor16f<1>(m));
            m = fmaxf(m, xor16f<2>(m));
            m = fmaxf(m, xor16f<4>(m));
            m = fmaxf(m, xor16f<8>(m));
            const int ex = f16s_exp(m);
            const int rr = m0 + (wm * TM + i) * 32 + acc_row(e, lane);
            if (col < NOUT && rr < rows) {
              char* Ob = static_cast<char*>(a.out) + (row0 + rr) * rb;
              *reinterpret_cast<uint16_t*>(Ob + 2 * col) = f16_scaled(v, ex);
              if ((lane & 15) == 0) Ob[2 * NOUT + col / 16] = static_cast<char>(ex);
            }
          }
      }
    } else {
      float* O = static_cast<float*>(a.out);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = c0 + (wn * TN + j) * 32 + (lane & 31);
        if (col < NOUT) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int rr = m0 + (wm * TM + i) * 32 + acc_row(e, lane);
              if (rr < rows) O[(row0 + rr) * NOUT + col] = acc[i][j][e];
            }
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------------------------
// Streaming bf16 kernel (K % 128 == 0): tiles of 32 k-values (64-byte rows) move straight from
// global memory into LDS with global_load_lds (no register round trip), four stages deep, so three
// stages of loads are in flight while one is consumed. Chunk c of row r sits at c ^ ((r >> 2) & 3):
// 16 consecutive rows at one chunk cover a 256-byte window's 16 slots. One DMA instruction writes
// 64 lanes x 16 bytes = 16 rows contiguously, so the swizzle is applied to the global side: lane l
// fetches chunk (l & 3) ^ (((l >> 2) >> 2) & 3) of row l >> 2.
// 32-row blocks of a tile that lie past the group's last row skip their matrix-core steps: the
// k-loop is compiled once per number of such blocks a wave has live (chosen once per tile), with
// the DMA and wait depths fixed per position, so no branch sits between two barriers.
// Quantised weights (kQ = 8, 4 or FP8): each stage's weight blocks (64 kQ bytes of codes per 16 x 32)
// move with 4-byte-per-lane DMA; fragments are converted to bf16 exactly as they are read, and each
// output column is multiplied by its weight row's scale in the epilogue.
// ---------------------------------------------------------------------------------------------
constexpr int kSK = 32;

// f(integral_constant<L>) for L = min(live, LMAX): one compiled copy of a loop per live-block count.
template <int LMAX, typename F>
__device__ __forceinline__ void dispatch_live(int live, F&& f) {
  if constexpr (LMAX == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (live >= LMAX) f(std::integral_constant<int, LMAX>{});
    else dispatch_live<LMAX - 1>(live, f);
  }
}

// Byte offsets in a wave's 2 KB epilogue staging. A row's 16-byte chunks are rotated by an XOR with
// bits of the row, so that the 16 lanes writing one chunk of 16 consecutive rows hit 16 distinct
// 16-byte bank slots of a 256-byte window (unrotated, rows 128 or 64 bytes apart fall on 2 or 4
// slots: an 8- or 4-way bank conflict on every staging write); a row's chunks stay within it, so
// reads of whole consecutive rows stay conflict-free.
// fp16 form: 16 rows x 128 bytes, chunk c (0-7) of row r.
__device__ __forceinline__ int stage_f16s_at(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
// h: 32 rows x 64 bytes, chunk c (0-3) of row r.
__device__ __forceinline__ int stage_h_at(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

template <int WM, int TM, int WN, int TN, bool kSwiGLU, bool kPacked, int kQ = 0, bool kWKN = false, bool kBwd = false,
          bool kPipe = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_stream_kernel(GemmArgs a) {
  constexpr int BM = WM * TM * 32, BNB = WN * TN * 32, NT = WM * WN * 64, NW = WM * WN;
  // DMA instructions per wave per stage; with fewer 16-row A groups than waves (BM = 32), waves
  // repeat a group (identical bytes to the same LDS place), so every wave issues the same count
  constexpr int A_GROUPS = BM / 16;
  constexpr int A_INS = (A_GROUPS + NW - 1) / NW, B_INS = BNB / 16 / NW;
  constexpr int OUT_COLS = kSwiGLU ? BNB / 2 : BNB;
  constexpr int QS = kQ ? code_slot(kQ) : 16;              // bytes per lane slot of a weight block
  // LDS bytes of one 16 x 32 weight block; int4: 256 bytes of codes, then its 16 rows' group
  // multipliers (4 bytes per row, byte t for the slice of buffer t), repeated to fill 256 bytes
  constexpr bool kQ4 = kQ == kQInt4;
  constexpr int QB = kQ4 ? 512 : 64 * QS;
  constexpr int B_DMA = (QS == 8 || kQ4) ? 2 * B_INS : B_INS;   // weight DMA instructions per wave per stage
  constexpr int PER_STAGE = A_INS + B_DMA;
  static_assert(kQ == 0 || kPacked, "quantised weights use the packed block order");
  static_assert(!kWKN || (!kSwiGLU && !kPacked && kQ == 0 && BNB == 256), "[K][N] weights: bf16 down form, 256 columns");
  static_assert(!kBwd || (kSwiGLU && kQ == 0 && !kWKN), "SwiGLU backward: bf16 gate_up form");
  // bf16 weights enter the matrix cores as the row operand, so a lane's accumulators hold one token
  // and runs of four consecutive output columns (stored as one 8- or 16-byte vector); quantised
  // weights keep the activation rows there, so that a lane's outputs share one weight-row scale.
  constexpr bool kSwap = kQ == 0;
  constexpr bool kEarlyReads = true;
  static_assert(A_INS * NW == A_GROUPS || A_INS == 1, "A rows must split into 16-row DMA groups");
  static_assert(B_INS * 16 * NW == BNB, "B rows must split into 16-row DMA groups");
  static_assert(!kSwiGLU || TN % 2 == 0, "SwiGLU pairs gate blocks with up blocks");
  // one array per stage: the four buffers are distinct objects
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[BM * kSK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[BM * kSK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA2[BM * kSK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA3[BM * kSK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[BNB * QB / 32];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[BNB * QB / 32];
  __shared__ __attribute__((aligned(1024))) uint16_t sB2[BNB * QB / 32];
  __shared__ __attribute__((aligned(1024))) uint16_t sB3[BNB * QB / 32];
  __shared__ int s_pref[1025];
  __shared__ int s_off[1025];           // group row offsets (no global round trip per tile)
  __shared__ int s_tmp[16];
  __shared__ int s_plist[1024];         // groups of the short m-tiles, in list order
  __shared__ int s_cnt[2 * NW * 8];
  // pipelined loop with gathered rows: the next tile's BM row indices, staged by DMA a tile ahead
  __shared__ __attribute__((aligned(16))) int s_rows[BM];
  // epilogue staging, 2 KB per wave: the fp16-form outputs of down (16 rows x 128 bytes at a time,
  // stored 8 rows x 128 contiguous bytes per instruction) and gate_up's h (32 rows x 64 bytes,
  // stored 16 rows x 64 contiguous bytes per instruction)
  __shared__ __attribute__((aligned(16))) char s_stage[kSwap && !kBwd ? NW * 2048 : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int G = a.G;
  const int K = kSwiGLU ? a.D : a.I;
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int n_tiles = (NOUT + OUT_COLS - 1) / OUT_COLS;
  for (int g = tid; g <= G; g += NT)
    s_off[g] = a.offsets ? a.offsets[g] : (g == 0 ? 0 : static_cast<int>(a.max_rows));
  const int n_short = build_tile_lists<NT, BM>(a.offsets, G, a.max_rows, n_tiles, s_pref, s_plist, s_tmp, s_cnt);
  const int total_full = s_pref[G];
  const int total = total_full + n_short * n_tiles;
  const int P = gridDim.x;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  const int ksteps = K / kSK;                        // a multiple of 4
  const int lrow = lane >> 2;                         // row within a 16-row DMA group
  const int lch = (lane & 3) ^ ((lrow >> 2) & 3);     // logical chunk this lane fetches

  // LDS read offsets: fragment rows are 32-aligned + (lane & 31), so row bits 2..3 are lane bits
  // 2..3 and the chunk of k-step kk is (2 kk + (lane >> 5)) ^ ((lane >> 2) & 3).
  // Packed B: each 16-row group's 1 KB holds the fragment in lane order (row r16, 8-wide k chunk q
  // at (r16 + 16 q) * 8), so 16 lanes read 256 contiguous bytes.
  // Quantised B: the same block and slot in bytes (QB per block, kQ bytes per slot).
  const int rb0 = (kSwiGLU ? wn * (TN / 2) : wn * TN) * 32;
  int koA[2], koB[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int pc = ((2 * kk + (lane >> 5)) ^ ((lane >> 2) & 3)) << 3;
    koA[kk] = (wm * TM * 32 + (lane & 31)) * kSK + pc;
    if constexpr (kQ != 0)
      koB[kk] = (rb0 / 16 + ((lane >> 4) & 1)) * QB + ((lane & 15) + 16 * (2 * kk + (lane >> 5))) * QS;
    else
      koB[kk] = kPacked ? rb0 * kSK + ((lane >> 4) & 1) * 512 + (lane & 15) * 8 + (2 * kk + (lane >> 5)) * 128
                        : (rb0 + (lane & 31)) * kSK + pc;
  }
  const int R = kSwiGLU ? 2 * a.I : a.D;              // weight rows per group
  // [K][NOUT] weights: a stage holds 32 k-rows of the tile's 256 columns (512 bytes per row, 32-byte
  // chunks swizzled by (2 row) & 7); lds_tr_frag assembles each weight operand with two transpose
  // reads, in the layout of the plain read.
  constexpr int W3 = waitcnt_vm(3 * PER_STAGE), W2 = waitcnt_vm(2 * PER_STAGE), W1 = waitcnt_vm(PER_STAGE),
                W0 = waitcnt_vm(0);

  // The pipelined k-loop (plain bf16 weights, rows gathered or not): each k-slice's barrier sits in
  // its middle, so the next slice's first fragments are read while the current slice's second half
  // of matrix-core steps runs (see pipe_kloop). Gathered rows need at least 8 k-slices per tile (the
  // next tile's row indices are staged in LDS a tile ahead).
  const bool gather = a.row_index != nullptr;
  static_assert(!kPipe || (kQ == 0 && !kWKN && !kBwd), "the pipelined loop: plain bf16 weights");
  constexpr bool pipe = kPipe;

  // One tile's fixed data. make_tile reads the group table in LDS and, for gathered rows, the row
  // indices of its A rows (global loads whose values are first used when its DMA is issued; in the
  // pipelined loop, from s_rows).
  struct Tile {
    bool valid;
    int m0, c0, live;
    int64_t row0, rows;
    const uint16_t* srcA[A_INS];
    const uint16_t* srcB[B_INS];
    // pipelined loop: the same sources as byte offsets from X (A) and from the group's weights bB (B)
    uint32_t oA[A_INS], oB[B_INS];
    const char* bB;
    const char* srcQ[B_INS];          // quantised: this lane's code bytes of k-block 0 (int4: its
                                      // super-block slot)
    const char* srcM[kQ4 ? B_INS : 1];  // int4: its row's multipliers in super-block 0
    float sc[TN];                     // quantised: scale of each of this lane's output columns
  };
  // tile r of this workgroup: (valid, group, m-tile, n-tile) from the tables in LDS
  struct Coord {
    bool valid;
    int g, mt, nt;
  };
  auto tile_coord = [&](int r) {
    Coord C{};
    // round r deals tiles r P .. r P + P - 1, in alternate directions in alternate rounds (a
    // workgroup that drew a more expensive tile in one round draws a cheaper one in the next)
    const int t = tile_of_round(r, (r & 1) ? P - 1 - static_cast<int>(blockIdx.x) : static_cast<int>(blockIdx.x), P);
    C.valid = r * P < total && t < total;             // t grows with r: past the list, nothing follows
    if (!C.valid) return C;
    if (t < total_full) {
      C.g = find_group(s_pref, G, t);
      const int local = t - s_pref[C.g];
      C.mt = local / n_tiles;
      C.nt = local - C.mt * n_tiles;
    } else {
      const int u = t - total_full, i = u / n_tiles;
      C.g = min(max(s_plist[i], 0), G - 1);           // (a permutation of the short groups; kept in range)
      C.nt = u - i * n_tiles;
      C.mt = (s_off[C.g + 1] - s_off[C.g]) / BM;      // the group's last, short m-tile
    }
    C.g = __builtin_amdgcn_readfirstlane(C.g);        // uniform: the same tile in every lane
    C.mt = __builtin_amdgcn_readfirstlane(C.mt);
    C.nt = __builtin_amdgcn_readfirstlane(C.nt);
    return C;
  };
  // pipelined loop, gathered rows: DMA the BM row indices of tile r into s_rows (waves 0 .. BM / 64 - 1,
  // 4 bytes per lane; rows past the group repeat its last row)
  auto stage_rows = [&](int r) {
    const Coord C = tile_coord(r);
    if (!C.valid || wave >= BM / 64) return;
    const int64_t row0 = s_off[C.g], rows = static_cast<int64_t>(s_off[C.g + 1]) - row0;
    const int64_t lr = min<int64_t>(static_cast<int64_t>(C.mt) * BM + wave * 64 + lane, rows - 1);
    dma4(a.row_index + row0 + lr, s_rows + wave * 64);
  };
  auto make_tile = [&](int r) {
    Tile T;
    const Coord C = tile_coord(r);
    T.valid = C.valid;
    if (!T.valid) return T;
    const int g = C.g, mt = C.mt, nt = C.nt;
    T.row0 = s_off[g];
    T.rows = static_cast<int64_t>(s_off[g + 1]) - T.row0;   // > 0: empty groups own no tiles
    T.m0 = mt * BM;
    T.c0 = nt * OUT_COLS;
    // 32-row blocks of this wave that hold real rows (uniform across the wave)
    T.live = static_cast<int>(min<int64_t>(TM, max<int64_t>(0, (T.rows - T.m0 - wm * TM * 32 + 31) / 32)));
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int rr = ((wave * A_INS + j) % A_GROUPS) * 16 + lrow;
      const int64_t lr = min<int64_t>(T.m0 + rr, T.rows - 1);   // rows past the group read a valid row
      const int64_t p = T.row0 + lr;
      int64_t src = p;
      if (gather) {
        if constexpr (pipe) src = s_rows[rr];
        else src = a.row_index[p];
      }
      if constexpr (pipe) T.oA[j] = static_cast<uint32_t>((src * K + lch * 8) * 2);   // x below 4 GB (checked at launch)
      else T.srcA[j] = X + src * K + lch * 8;
    }
    const uint16_t* Wg = W + static_cast<int64_t>(g) * (kSwiGLU ? 2LL * a.I * a.D : static_cast<int64_t>(a.D) * a.I);
    if constexpr (kQ != 0) {
      // the weight row of this lane's column in block j (columns past the output width read a
      // valid row; their outputs are never stored)
      const float* S = reinterpret_cast<const float*>(static_cast<const char*>(a.w) + quant_code_bytes(G, R, K, code_bits(kQ))) +
                       static_cast<int64_t>(g) * R;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        constexpr int H = TN / 2;
        if (kSwiGLU) {
          const int col = min(T.c0 + (wn * H + (j < H ? j : j - H)) * 32 + (lane & 31), NOUT - 1);
          T.sc[j] = S[j < H ? col : a.I + col];
        } else {
          T.sc[j] = S[min(T.c0 + (wn * TN + j) * 32 + (lane & 31), NOUT - 1)];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      const int grp = wave * B_INS + j;
      if constexpr (kPacked) {
        // the group's 16 weight rows are one row block (c0, I and NOUT are multiples of 16): one
        // DMA instruction moves its 1 KB fragment of k-block ks contiguously
        int rb;
        if (kSwiGLU) {
          const int half = BNB / 32;                          // 16-row groups per half
          const int cb = min(T.c0 / 16 + grp % half, NOUT / 16 - 1);
          rb = grp < half ? cb : a.I / 16 + cb;
        } else {
          rb = min(T.c0 / 16 + grp, NOUT / 16 - 1);
        }
        if constexpr (kQ4) {
          const char* sp = static_cast<const char*>(a.w) + quant_code_bytes(g, R, K, 4) +
                           static_cast<int64_t>(rb) * (K / 128) * kQ4Super;
          T.srcQ[j] = sp + lane * 16;
          T.srcM[j] = sp + 1024 + 4 * (lane & 15);
        } else if constexpr (kQ != 0)
          T.srcQ[j] = static_cast<const char*>(a.w) + quant_code_bytes(g, R, K, code_bits(kQ)) +
                      static_cast<int64_t>(rb) * (K / kSK) * QB + lane * 4;
        else if constexpr (pipe)
          T.oB[j] = static_cast<uint32_t>((static_cast<int64_t>(rb) * (K / kSK) * 512 + lane * 8) * 2);
        else
          T.srcB[j] = Wg + static_cast<int64_t>(rb) * (K / kSK) * 512 + lane * 8;
      } else if constexpr (kWKN) {
        // weights [K][NOUT]: DMA group grp carries k-rows 2 grp and 2 grp + 1 of the stage (512 bytes
        // each); lane l fetches 16 bytes of row 2 grp + l / 32 into physical 32-byte chunk (l % 32) / 2,
        // which holds logical chunk ((l % 32) / 2) ^ ((2 row) & 7) (the transpose-read swizzle);
        // columns past NOUT read a valid chunk, and their outputs are never stored
        const int row = 2 * grp + (lane >> 5);
        const int chunk = ((lane & 31) >> 1) ^ ((2 * row) & 7);
        const int n = min(T.c0 + chunk * 16 + (lane & 1) * 8, NOUT - 8);
        T.srcB[j] = Wg + static_cast<int64_t>(row) * NOUT + n;
      } else {
        const int rr = grp * 16 + lrow;
        int wrow;
        if (kSwiGLU) {
          const int half = BNB / 2;
          const int ci = min(T.c0 + (rr % half), NOUT - 1);
          wrow = rr < half ? ci : a.I + ci;
        } else {
          wrow = min(T.c0 + rr, NOUT - 1);
        }
        if constexpr (pipe) T.oB[j] = static_cast<uint32_t>((static_cast<int64_t>(wrow) * K + lch * 8) * 2);
        else T.srcB[j] = Wg + static_cast<int64_t>(wrow) * K + lch * 8;
      }
    }
    T.bB = reinterpret_cast<const char*>(Wg);
    return T;
  };
  auto issue = [&](const Tile& T, int ks, uint16_t* sa, uint16_t* sb) {
    const int kb = ks * kSK;
    if constexpr (pipe) {
#pragma unroll
      for (int j = 0; j < A_INS; ++j) dma16_sv(X, T.oA[j] + kb * 2, sa + ((wave * A_INS + j) % A_GROUPS) * 512);
#pragma unroll
      for (int j = 0; j < B_INS; ++j)
        dma16_sv(T.bB, T.oB[j] + (kPacked ? ks * 1024 : kb * 2), sb + (wave * B_INS + j) * 512);
      return;
    }
#pragma unroll
    for (int j = 0; j < A_INS; ++j) dma16(T.srcA[j] + kb, sa + ((wave * A_INS + j) % A_GROUPS) * 512);
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      if constexpr (kQ4) {
        const int64_t so = static_cast<int64_t>(ks >> 2) * kQ4Super;
        char* dst = reinterpret_cast<char*>(sb) + (wave * B_INS + j) * QB;
        dma4(T.srcQ[j] + so + 4 * (ks & 3), dst);
        dma4(T.srcM[j] + so, dst + 256);
      } else if constexpr (kQ != 0) {
        const char* src = T.srcQ[j] + static_cast<int64_t>(ks) * QB;
        char* dst = reinterpret_cast<char*>(sb) + (wave * B_INS + j) * QB;
        dma4(src, dst);
        if constexpr (QS == 8) dma4(src + 256, dst + 256);
      } else {
        dma16(T.srcB[j] + (kWKN ? static_cast<int64_t>(kb) * NOUT : kPacked ? ks * 512 : kb), sb + (wave * B_INS + j) * 512);
      }
    }
  };

  // DMA instruction n of issue() alone (n < PER_STAGE, in issue()'s order)
  auto issue_one = [&](const Tile& T, int ks, uint16_t* sa, uint16_t* sb, int n) {
    if constexpr (pipe) {
      if (n < A_INS) dma16_sv(X, T.oA[n] + ks * kSK * 2, sa + ((wave * A_INS + n) % A_GROUPS) * 512);
      else dma16_sv(T.bB, T.oB[n - A_INS] + (kPacked ? ks * 1024 : ks * kSK * 2), sb + (wave * B_INS + n - A_INS) * 512);
      return;
    }
    if (n < A_INS) {
      dma16(T.srcA[n] + ks * kSK, sa + ((wave * A_INS + n) % A_GROUPS) * 512);
    } else if constexpr (kQ4) {
      const int b = n - A_INS, j = b / 2;
      const int64_t so = static_cast<int64_t>(ks >> 2) * kQ4Super;
      char* dst = reinterpret_cast<char*>(sb) + (wave * B_INS + j) * QB;
      if (b % 2 == 0) dma4(T.srcQ[j] + so + 4 * (ks & 3), dst);
      else dma4(T.srcM[j] + so, dst + 256);
    } else if constexpr (kQ != 0) {
      const int b = n - A_INS, j = QS == 8 ? b / 2 : b, half = QS == 8 ? b % 2 : 0;
      dma4(T.srcQ[j] + static_cast<int64_t>(ks) * QB + half * 256,
           reinterpret_cast<char*>(sb) + (wave * B_INS + j) * QB + half * 256);
    } else {
      const int j = n - A_INS;
      dma16(T.srcB[j] + (kWKN ? static_cast<int64_t>(ks) * kSK * NOUT : kPacked ? ks * 512 : ks * kSK),
            sb + (wave * B_INS + j) * 512);
    }
  };

  // wait for the oldest stage in flight while n later stages may stay in flight, then sync the
  // workgroup: after this the stage is visible to every wave and every wave has finished reading the
  // previous stage's buffer. Loads retire in order, so "at most n stages outstanding" implies the
  // stage has landed even with the previous tile's epilogue stores still counted. Inside a tile's
  // k-loop n = 2; its last group of four stages waits with 2, 2, 1, 0.
  // The wait includes lgkmcnt(0): the compiler may place matrix-core steps after the barrier, and the
  // fragment reads feeding them must not still be pending once other waves may refill the buffer.
  auto wait_stage = [&](auto Nc) __attribute__((always_inline)) {
    constexpr int n = decltype(Nc)::value;
    __builtin_amdgcn_s_waitcnt((n == 3 ? W3 : n == 2 ? W2 : n == 1 ? W1 : W0) & ~(0xF << 8));
    lds_barrier();
  };
  f32x16 acc[TM][TN];
  // One stage's matrix-core steps for the first L 32-row blocks of this wave; with kDma, stage dks
  // of tile T goes to (dsa, dsb), one DMA instruction after each group of steps (issued together,
  // the DMA instructions of all waves queue behind one another in the CU's load path and hold up
  // every wave's steps). L and kDma are compile-time, so no branch sits between the steps.
  auto compute = [&](auto Lc, auto Dc, const uint16_t* sa, const uint16_t* sb, const Tile& T, int dks, uint16_t* dsa,
                     uint16_t* dsb) __attribute__((always_inline)) {
    constexpr int L = decltype(Lc)::value;
    constexpr bool kDma = decltype(Dc)::value;
    // both k-steps' fragments are read first (the reads of the second overlap the first's steps)
    u32x4 fa[2][TM], fb[2][TN];
    // int4: this lane's group multiplier in each block (one per slice: buffer t holds slices t mod 4)
    uint32_t qm[kQ4 ? TN : 1];
    if constexpr (kQ4) {
      const int t = sb == sB0 ? 0 : sb == sB1 ? 1 : sb == sB2 ? 2 : 3;
      const char* mb = reinterpret_cast<const char*>(sb) + (rb0 / 16 + ((lane >> 4) & 1)) * QB + 256 + 4 * (lane & 15) + t;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        constexpr int H = TN / 2;
        const int rowoff = kSwiGLU ? (j < H ? j * 32 : BNB / 2 + (j - H) * 32) : j * 32;
        qm[j] = *reinterpret_cast<const uint8_t*>(mb + rowoff / 16 * QB);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < L; ++i) fa[kk][i] = *reinterpret_cast<const u32x4*>(&sa[koA[kk] + i * 32 * kSK]);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        constexpr int H = TN / 2;
        const int rowoff = kSwiGLU ? (j < H ? j * 32 : BNB / 2 + (j - H) * 32) : j * 32;
        if constexpr (kQ == kQInt8)
          fb[kk][j] = codes8_to_bf16(*reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(sb) + koB[kk] + rowoff / 16 * QB));
        else if constexpr (kQ == kQFp8)
          fb[kk][j] = codesf8_to_bf16(*reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(sb) + koB[kk] + rowoff / 16 * QB));
        else if constexpr (kQ4)
          fb[kk][j] = codes4m_to_bf16(*reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(sb) + koB[kk] + rowoff / 16 * QB), qm[j]);
        else if constexpr (kWKN)
          fb[kk][j] = lds_tr_frag<256>(sb, kk, rb0 + rowoff, lane);
        else
          fb[kk][j] = *reinterpret_cast<const u32x4*>(&sb[koB[kk] + rowoff * kSK]);
      }
    }
    if constexpr (kEarlyReads) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i < L) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = kSwap ? mfma32(fb[kk][j], fa[kk][i], acc[i][j]) : mfma32(fa[kk][i], fb[kk][j], acc[i][j]);
        }
        if (kDma && kk * TM + i < PER_STAGE) issue_one(T, dks, dsa, dsb, kk * TM + i);
      }
    }
#pragma unroll
    for (int n = 2 * TM; n < PER_STAGE; ++n)          // more instructions than groups (short tiles)
      if (kDma) issue_one(T, dks, dsa, dsb, n);
  };
  constexpr std::integral_constant<int, 0> n0{};
  constexpr std::integral_constant<int, 1> n1{};
  constexpr std::integral_constant<int, 2> n2{};
  constexpr std::true_type dma{};
  constexpr std::false_type no_dma{};

  // One tile's k-loop for L live 32-row blocks of this wave (a copy per L, chosen once per tile).
  // Every copy clears all accumulators, the skipped blocks too, so that each defines them all and
  // the register allocator keeps them in place across the copies.
  auto kloop = [&](auto Lc, const Tile& cur, Tile& nxt, int r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    int ks = 0;
    for (; ks + 4 < ksteps; ks += 4) {
      wait_stage(n2);
      compute(Lc, dma, sA0, sB0, cur, ks + 3, sA3, sB3);
      wait_stage(n2);
      compute(Lc, dma, sA1, sB1, cur, ks + 4, sA0, sB0);
      wait_stage(n2);
      compute(Lc, dma, sA2, sB2, cur, ks + 5, sA1, sB1);
      wait_stage(n2);
      compute(Lc, dma, sA3, sB3, cur, ks + 6, sA2, sB2);
    }
    // the last four stages: only the first still issues one of this tile's stages
    wait_stage(n2);
    nxt = make_tile(r + 1);
    compute(Lc, dma, sA0, sB0, cur, ks + 3, sA3, sB3);
    wait_stage(n2);
    compute(Lc, no_dma, sA1, sB1, cur, 0, sA0, sB0);
    wait_stage(n1);
    compute(Lc, no_dma, sA2, sB2, cur, 0, sA1, sB1);
    wait_stage(n0);                       // everything this wave issued has landed
    if (nxt.valid) {
      issue(nxt, 0, sA0, sB0);
      issue(nxt, 1, sA1, sB1);
      issue(nxt, 2, sA2, sB2);
    }
    compute(Lc, no_dma, sA3, sB3, cur, 0, sA2, sB2);
  };

  // ---- pipelined k-loop (kPipeKind) ----
  // Slice g (buffer g % 4) runs as: (a) read its second k-step's fragments F1; (b) the first k-step's
  // steps on F0 (read during the previous slice); (c) wait until stage g + 1 has landed (and F1 is in
  // registers), barrier; (d) read stage g + 1's first k-step into F0; (e) the second k-step's steps on
  // F1, with the DMA of stage g + 4 into buffer g % 4, which every wave finished reading before (c).
  // So the reads of a slice overlap the previous slice's steps instead of following its barrier.
  // Fragments of every block are read (a dead block's rows hold valid data; its steps are skipped).
  u32x4 fa0[pipe ? TM : 1], fb0[pipe ? TN : 1];
  auto read_half = [&](int kk, const uint16_t* sa, const uint16_t* sb, u32x4* fa, u32x4* fb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const u32x4*>(&sa[koA[kk] + i * 32 * kSK]);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      constexpr int H = TN / 2;
      const int rowoff = kSwiGLU ? (j < H ? j * 32 : BNB / 2 + (j - H) * 32) : j * 32;
      fb[j] = *reinterpret_cast<const u32x4*>(&sb[koB[kk] + rowoff * kSK]);
    }
  };
  // kDma: issue the DMA of stage dks of T (when dma_on, a uniform flag), one instruction per group
  auto steps_half = [&](auto Lc, const u32x4* fa, const u32x4* fb, auto Dc, const Tile& T, int dks, uint16_t* dsa,
                        uint16_t* dsb, bool dma_on = true) __attribute__((always_inline)) {
    constexpr int L = decltype(Lc)::value;
    constexpr bool kDma = decltype(Dc)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i < L) {
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
      }
      if (kDma && i < PER_STAGE && dma_on) issue_one(T, dks, dsa, dsb, i);
    }
#pragma unroll
    for (int n = TM; n < PER_STAGE; ++n)
      if (kDma && dma_on) issue_one(T, dks, dsa, dsb, n);
  };
  // one slice in buffer (sa, sb); Wc: the wait for the next slice's stage, HasNext: whether one
  // follows in this workgroup (then its buffer is (nsa, nsb)); Dc / T / dks: the DMA of (e)
  // wait_n: with a compile-time Wc, that wait; with Wc = -1, wait 2 when the next tile is valid (its
  // stages keep the count up) and w_last otherwise (the stream drains)
  auto pslice = [&](auto Lc, uint16_t* sa, uint16_t* sb, auto Wc, auto HasNext, const uint16_t* nsa,
                    const uint16_t* nsb, auto Dc, const Tile& T, int dks, bool dma_on = true, int w_last = 2)
                    __attribute__((always_inline)) {
    u32x4 fa1[TM], fb1[TN];
    read_half(1, sa, sb, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    steps_half(Lc, fa0, fb0, std::false_type{}, T, 0, sa, sb);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(HasNext)::value) {
      if constexpr (decltype(Wc)::value >= 0) {
        wait_stage(Wc);
      } else {
        if (dma_on || w_last == 2) __builtin_amdgcn_s_waitcnt(W2 & ~(0xF << 8));
        else if (w_last == 1) __builtin_amdgcn_s_waitcnt(W1 & ~(0xF << 8));
        else __builtin_amdgcn_s_waitcnt(W0 & ~(0xF << 8));
        lds_barrier();
      }
      read_half(0, nsa, nsb, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
    steps_half(Lc, fa1, fb1, Dc, T, dks, sa, sb, dma_on);
    __builtin_amdgcn_sched_barrier(0);      // the next slice's reads stay after these steps
  };
  constexpr std::integral_constant<int, 3> n3{};
  constexpr std::true_type yes{};
  constexpr std::false_type no{};
  // One tile's slices. Stages run four ahead: slice j issues stage j + 4 of this tile, and the last
  // four slices stage 0-3 of the next tile (made at the start of those four); the next tile's first
  // fragments are read after this tile's epilogue (so they are not live across it). The last tile
  // drains with waits 2, 1, 0.
  auto pipe_kloop = [&](auto Lc, const Tile& cur, Tile& nxt, int r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    if (gather) stage_rows(r + 1);          // the next tile's row indices, landed before its make_tile
    int ks = 0;
    for (; ks + 4 < ksteps; ks += 4) {
      pslice(Lc, sA0, sB0, n2, yes, sA1, sB1, dma, cur, ks + 4);
      pslice(Lc, sA1, sB1, n2, yes, sA2, sB2, dma, cur, ks + 5);
      pslice(Lc, sA2, sB2, n2, yes, sA3, sB3, dma, cur, ks + 6);
      pslice(Lc, sA3, sB3, n2, yes, sA0, sB0, dma, cur, ks + 7);
    }
    // the last four slices: stages 0-2 of the next tile if there is one; the last slice has no
    // barrier after its reads, so stage 3 (into its buffer) and the next tile's first fragments follow
    // the epilogue. Without a next tile: no DMA and waits 2, 1, 0.
    nxt = make_tile(r + 1);
    const bool nv = nxt.valid;
    constexpr std::integral_constant<int, -1> wsel{};
    pslice(Lc, sA0, sB0, n2, yes, sA1, sB1, dma, nxt, 0, nv);
    pslice(Lc, sA1, sB1, wsel, yes, sA2, sB2, dma, nxt, 1, nv, 1);
    pslice(Lc, sA2, sB2, wsel, yes, sA3, sB3, dma, nxt, 2, nv, 0);
    pslice(Lc, sA3, sB3, n0, no, sA0, sB0, no_dma, nxt, 0, false);
  };

  // Tiles are software-pipelined: the next tile's first three stages go out as soon as every wave
  // has passed the last stage's barrier (buffers 0-2 are free then), so their latency overlaps the
  // last k-slice and the epilogue stores instead of following them. (The pipelined loop instead
  // keeps four stages in flight across tile boundaries.)
  Tile cur;
  if constexpr (pipe) {
    if (gather) {
      stage_rows(0);
      wait_stage(n0);
    }
    cur = make_tile(0);
    if (cur.valid) {
      issue(cur, 0, sA0, sB0);
      issue(cur, 1, sA1, sB1);
      issue(cur, 2, sA2, sB2);
      issue(cur, 3, sA3, sB3);
      wait_stage(n3);
      read_half(0, sA0, sB0, fa0, fb0);
    }
  } else {
    cur = make_tile(0);
    if (cur.valid) {
      issue(cur, 0, sA0, sB0);
      issue(cur, 1, sA1, sB1);
      issue(cur, 2, sA2, sB2);
    }
  }
  for (int r = 0; cur.valid; ++r) {
    Tile nxt;
    nxt.valid = false;
    if constexpr (pipe)
      dispatch_live<TM>(cur.live, [&](auto Lc) __attribute__((always_inline)) { pipe_kloop(Lc, cur, nxt, r); });
    else
      dispatch_live<TM>(cur.live, [&](auto Lc) __attribute__((always_inline)) { kloop(Lc, cur, nxt, r); });
    // Epilogue. The next tile writes buffer 3 only after its first barrier, which every wave
    // reaches after finishing these reads of buffer 3.
    const int64_t row0 = cur.row0, rows = cur.rows;
    const int m0 = cur.m0, c0 = cur.c0;
    if constexpr (kQ != 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] *= cur.sc[j];
    }
    bool staged = false;
    if constexpr (kSwap && !kSwiGLU && !kBwd && TN == 2) {
      if (a.out_f16s && NOUT % 64 == 0) {
        // fp16 form, a wave's 64 columns whole (in or out): per 32-row block, each lane forms its
        // four 16-byte runs (see below), the rows of each half-block go through the wave's 2 KB of
        // LDS, and every lane then stores 16 bytes of one row: 8 rows x 128 contiguous bytes per
        // instruction. The row's four exponent bytes are contiguous and go as one 4-byte store.
        staged = true;
        char* st = s_stage + wave * 2048;
        const int hf = lane >> 5, r32 = lane & 31;
        const int wcol = c0 + wn * TN * 32;
        const int64_t RB = f16s_row_bytes(NOUT);
        char* O = static_cast<char*>(a.out);
        if (wcol < NOUT) {
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int rb = m0 + (wm * TM + i) * 32;            // first row of the block
            u32x4 run[TN][2];
            uint32_t exw = 0;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                const f32x16& c = acc[i][j];
                float m = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(c[8 * g + t]));
                m = fmaxf(m, __shfl_xor(m, 32, kWave));
                const int ex = f16s_exp(m);
                exw |= static_cast<uint32_t>(ex & 0xff) << (8 * (2 * j + g));
                // lane l < 32 holds columns 0-3 and 8-11 of the group, l + 32 columns 4-7 and
                // 12-15: one 8-byte exchange gives each a contiguous half (0-7 or 8-15)
                const int q0 = 2 * g;
                const u32x2 lo = u32x2{pack_f16x2_scaled(c[4 * q0], c[4 * q0 + 1], ex), pack_f16x2_scaled(c[4 * q0 + 2], c[4 * q0 + 3], ex)};
                const u32x2 hi = u32x2{pack_f16x2_scaled(c[4 * q0 + 4], c[4 * q0 + 5], ex), pack_f16x2_scaled(c[4 * q0 + 6], c[4 * q0 + 7], ex)};
                const u32x2 send = hf ? lo : hi;
                const u32x2 got = u32x2{static_cast<uint32_t>(__shfl_xor(static_cast<int>(send[0]), 32, kWave)),
                                        static_cast<uint32_t>(__shfl_xor(static_cast<int>(send[1]), 32, kWave))};
                run[j][g] = hf ? u32x4{got[0], got[1], hi[0], hi[1]} : u32x4{lo[0], lo[1], got[0], got[1]};
              }
            if (hf == 0 && rb + r32 < rows)
              *reinterpret_cast<uint32_t*>(O + (row0 + rb + r32) * RB + 2 * NOUT + wcol / 16) = exw;
#pragma unroll
            for (int ph = 0; ph < 2; ++ph) {
              if ((r32 >> 4) == ph) {                           // rows 16 ph .. 16 ph + 15 of the block
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                  for (int g = 0; g < 2; ++g)
                    *reinterpret_cast<u32x4*>(st + stage_f16s_at(r32 & 15, 4 * j + 2 * g + hf)) = run[j][g];
              }
#pragma unroll
              for (int it = 0; it < 2; ++it) {
                const int off = it * 1024 + lane * 16;
                const int r = rb + 16 * ph + (off >> 7);
                const u32x4 v = *reinterpret_cast<const u32x4*>(st + stage_f16s_at(off >> 7, (off >> 4) & 7));
                if (r < rows) *reinterpret_cast<u32x4*>(O + (row0 + r) * RB + 2 * wcol + (off & 127)) = v;
              }
            }
          }
        }
      }
    }
    if constexpr (kSwap && kSwiGLU && !kBwd && TN == 2) {
      if (NOUT % 32 == 0) {
        // h, a wave's 32 columns whole (in or out): per 32-row block each lane forms four 8-byte
        // runs (columns 8 q + 4 (lane / 32) .. + 3), the block's 32 rows x 64 bytes go through the
        // wave's 2 KB of LDS, and each lane then stores 16 bytes of one row, 16 rows x 64 contiguous
        // bytes per instruction
        staged = true;
        char* st = s_stage + wave * 2048;
        const int hf = lane >> 5, r32 = lane & 31;
        const int wcol = c0 + wn * 32;
        uint16_t* Hh = static_cast<uint16_t*>(a.out);
        if (wcol < NOUT) {
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int rb = m0 + (wm * TM + i) * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint16_t v[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) v[t] = f32_to_bf16(silu(acc[i][0][4 * q + t]) * acc[i][1][4 * q + t]);
              *reinterpret_cast<u32x2*>(st + stage_h_at(r32, q) + 8 * hf) =
                  u32x2{v[0] | (static_cast<uint32_t>(v[1]) << 16), v[2] | (static_cast<uint32_t>(v[3]) << 16)};
            }
#pragma unroll
            for (int it = 0; it < 2; ++it) {
              const int off = it * 1024 + lane * 16;
              const int r = rb + (off >> 6);
              const u32x4 v = *reinterpret_cast<const u32x4*>(st + stage_h_at(off >> 6, (off >> 4) & 3));
              if (r < rows)
                *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(Hh + (row0 + r) * NOUT + wcol) + (off & 63)) = v;
            }
          }
        }
      }
    }
    if (staged) {
      // stored above
    } else if constexpr (kSwap) {
      // block (i, j): token m0 + (wm TM + i) 32 + lane % 32; element e is output column
      // 8 (e / 4) + 4 (lane / 32) + e % 4 of the block
      const bool vec = NOUT % 4 == 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rr = m0 + (wm * TM + i) * 32 + (lane & 31);
        if (rr >= rows) continue;
        if constexpr (kBwd) {
          // SwiGLU backward of this row's columns (the formulas of swiglu_bwd_kernel); lanes l and
          // l ^ 32 hold the two halves of each 32-column block, so one exchange completes its dot
          const int64_t p = row0 + rr;
          uint16_t* Hrow = static_cast<uint16_t*>(a.out) + p * NOUT;
          uint16_t* DArow = static_cast<uint16_t*>(a.bwd_dab) + p * 2 * NOUT;
          const float* Grow = a.bwd_dhu + p * NOUT;
          const float wp = a.bwd_w[p];
          const int nb = (NOUT + 31) / 32;
          constexpr int H = TN / 2;
#pragma unroll
          for (int j = 0; j < H; ++j) {
            const int blk = c0 / 32 + wn * H + j;
            float dot = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = c0 + (wn * H + j) * 32 + 8 * q + 4 * (lane >> 5);
              const bool full = vec && col + 3 < NOUT;
              float g[4];
              if (full) {
                const f32x4 gv = *reinterpret_cast<const f32x4*>(Grow + col);
#pragma unroll
                for (int t = 0; t < 4; ++t) g[t] = gv[t];
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) g[t] = col + t < NOUT ? Grow[col + t] : 0.f;
              }
              uint16_t hv[4], dav[4], dbv[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const float av = acc[i][j][4 * q + t], bv = acc[i][j + H][4 * q + t];
                const float s = 1.0f / (1.0f + __expf(-av));
                hv[t] = f32_to_bf16(av * s * bv);
                dot = fmaf(g[t], bf16_to_f32(hv[t]), dot);
                const float dh = wp * g[t];
                dav[t] = f32_to_bf16(dh * bv * (s * (1.0f + av * (1.0f - s))));
                dbv[t] = f32_to_bf16(dh * av * s);
              }
              if (full) {
                *reinterpret_cast<u32x2*>(Hrow + col) = u32x2{hv[0] | (static_cast<uint32_t>(hv[1]) << 16),
                                                              hv[2] | (static_cast<uint32_t>(hv[3]) << 16)};
                *reinterpret_cast<u32x2*>(DArow + col) = u32x2{dav[0] | (static_cast<uint32_t>(dav[1]) << 16),
                                                               dav[2] | (static_cast<uint32_t>(dav[3]) << 16)};
                *reinterpret_cast<u32x2*>(DArow + NOUT + col) = u32x2{dbv[0] | (static_cast<uint32_t>(dbv[1]) << 16),
                                                                      dbv[2] | (static_cast<uint32_t>(dbv[3]) << 16)};
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (col + t < NOUT) {
                    Hrow[col + t] = hv[t];
                    DArow[col + t] = dav[t];
                    DArow[NOUT + col + t] = dbv[t];
                  }
              }
            }
            dot += __shfl_xor(dot, 32, 64);
            if (lane < 32 && blk < nb) a.bwd_dwp[p * nb + blk] = dot;
          }
        } else if constexpr (kSwiGLU) {
          uint16_t* Hrow = static_cast<uint16_t*>(a.out) + (row0 + rr) * NOUT;
          constexpr int H = TN / 2;
#pragma unroll
          for (int j = 0; j < H; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = c0 + (wn * H + j) * 32 + 8 * q + 4 * (lane >> 5);
              uint16_t v[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) v[t] = f32_to_bf16(silu(acc[i][j][4 * q + t]) * acc[i][j + H][4 * q + t]);
              if (vec && col + 3 < NOUT) {
                *reinterpret_cast<u32x2*>(Hrow + col) = u32x2{v[0] | (static_cast<uint32_t>(v[1]) << 16),
                                                              v[2] | (static_cast<uint32_t>(v[3]) << 16)};
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (col + t < NOUT) Hrow[col + t] = v[t];
              }
            }
        } else if (a.out_f16s) {
          // fp16 form: a 16-column group of this row is runs q = 2 g, 2 g + 1 of lanes l and l ^ 32
          // (the same row); its exponent comes from the pair's largest magnitude
          char* Ob = static_cast<char*>(a.out) + (row0 + rr) * f16s_row_bytes(NOUT);
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const f32x16& c = acc[i][j];
              float m = 0.f;
#pragma unroll
              for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(c[8 * g + t]));
              m = fmaxf(m, __shfl_xor(m, 32, kWave));
              const int ex = f16s_exp(m);
              const int gcol = c0 + (wn * TN + j) * 32 + 16 * g;   // NOUT % 16 == 0: in or out whole
              if (gcol < NOUT) {
                // lane l < 32 holds columns 0-3 and 8-11 of the group, l + 32 columns 4-7 and 12-15:
                // one exchange of 8 bytes gives each a contiguous half (0-7, or 8-15) to store as 16 bytes
                const int q0 = 2 * g;
                const u32x2 lo = u32x2{pack_f16x2_scaled(c[4 * q0], c[4 * q0 + 1], ex), pack_f16x2_scaled(c[4 * q0 + 2], c[4 * q0 + 3], ex)};
                const u32x2 hi = u32x2{pack_f16x2_scaled(c[4 * q0 + 4], c[4 * q0 + 5], ex), pack_f16x2_scaled(c[4 * q0 + 6], c[4 * q0 + 7], ex)};
                const bool upper = lane >= 32;
                const u32x2 send = upper ? lo : hi;
                const u32x2 got = u32x2{static_cast<uint32_t>(__shfl_xor(static_cast<int>(send[0]), 32, kWave)),
                                        static_cast<uint32_t>(__shfl_xor(static_cast<int>(send[1]), 32, kWave))};
                const u32x4 v = upper ? u32x4{got[0], got[1], hi[0], hi[1]} : u32x4{lo[0], lo[1], got[0], got[1]};
                *reinterpret_cast<u32x4*>(Ob + 2 * (gcol + 8 * (upper ? 1 : 0))) = v;
                if (lane < 32) Ob[2 * NOUT + gcol / 16] = static_cast<char>(ex);
              }
            }
        } else {
          float* Orow = static_cast<float*>(a.out) + (row0 + rr) * NOUT;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = c0 + (wn * TN + j) * 32 + 8 * q + 4 * (lane >> 5);
              const f32x16& c = acc[i][j];
              if (vec && col + 3 < NOUT) {
                *reinterpret_cast<f32x4*>(Orow + col) = f32x4{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (col + t < NOUT) Orow[col + t] = c[4 * q + t];
              }
            }
        }
      }
    } else if constexpr (kSwiGLU) {
      uint16_t* Hh = static_cast<uint16_t*>(a.out);
      constexpr int H = TN / 2;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const int col = c0 + (wn * H + j) * 32 + (lane & 31);
        if (col < NOUT) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int rr = m0 + (wm * TM + i) * 32 + acc_row(e, lane);
              if (rr < rows) Hh[(row0 + rr) * NOUT + col] = f32_to_bf16(silu(acc[i][j][e]) * acc[i][j + H][e]);
            }
        }
      }
    } else {
      float* O = static_cast<float*>(a.out);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = c0 + (wn * TN + j) * 32 + (lane & 31);
        if (col < NOUT) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int rr = m0 + (wm * TM + i) * 32 + acc_row(e, lane);
              if (rr < rows) O[(row0 + rr) * NOUT + col] = acc[i][j][e];
            }
        }
      }
    }
    if constexpr (pipe) {
      if (nxt.valid) {
        // stage 0 of the next tile landed (1 and 2 may stay in flight) and every wave is done with
        // buffer 3: its stage 3 goes there, then its first fragments are read
        wait_stage(n2);
        issue(nxt, 3, sA3, sB3);
        read_half(0, sA0, sB0, fa0, fb0);
      }
    }
    cur = nxt;
  }
}


// ---------------------------------------------------------------------------------------------
// Weight-streaming kernel for short groups (decode: a few rows per expert). Every weight byte is
// used by one wave only, so there is nothing to share through LDS: each wave owns one task =
// (group, 16 output columns) and streams that block's weight rows with nontemporal 16-byte loads
// straight into 16x16x32 matrix-core fragments (lane l: row l % 16, 16 bytes of k-group l / 16,
// i.e. 64 contiguous bytes per row per k-step), with the group's activation rows (tiny, L2-resident)
// loaded the same way. No barriers; U k-steps of loads are in flight per wave.
// MB = 16-row blocks per pass; groups with more rows take several passes over the weights.
// gate_up: a task holds 16 gate rows and the 16 matching up rows (SwiGLU in the epilogue).
// Requires K % 32 == 0.
// Quantised weights (kQ = 8 or 4 bits, packed block order): the integer codes go to the matrix
// cores exactly as bf16, and the lane's output column is multiplied by its row's scale in the
// epilogue (one scale per weight row, so it factors out of the dot product).
// ---------------------------------------------------------------------------------------------
template <int kQ> struct WRaw { typedef u32x4 T; };          // bf16: 8 values = 16 bytes per lane
template <> struct WRaw<8> { typedef u32x2 T; };              // int8: 8 codes = 8 bytes
template <> struct WRaw<4> { typedef uint32_t T; };           // int4: 8 codes = 4 bytes (prefill LDS slots)
template <> struct WRaw<kQFp8> { typedef u32x2 T; };          // fp8: 8 codes = 8 bytes

template <int kQ>
__device__ __forceinline__ u32x4 to_bf16_frag(typename WRaw<kQ>::T v) {
  if constexpr (kQ == kQInt8) return codes8_to_bf16(v);
  else if constexpr (kQ == kQInt4) return codes4_to_bf16(v);
  else if constexpr (kQ == kQFp8) return codesf8_to_bf16(v);
  else return v;
}

// Column blocks of 16 per task: quantised codes are smaller than bf16, so a task takes two column
// blocks to keep more weight bytes in flight per wave, and each activation fragment then feeds twice
// as many matrix-core steps (one block for MB = 4, whose accumulators would not fit the registers
// otherwise). Measured on the 64-token decode layer: two blocks beat one (int8 and int4) and four
// (int4, whose registers then allow one wave per SIMD only).
// bf16 with four slabs: two blocks as well, so that each activation fragment (rows re-read by
// every task of the expert) feeds twice the steps (measured on the 512-token, 60-expert layer:
// 0.316 -> 0.252 ms for both products; the gate_up form then loads one k-step per batch).
template <int kQ, int MB, bool kSwiGLU> constexpr int wstream_cols() {
  return (kQ && MB < 4) || (!kQ && MB == 4) ? 2 : 1;
}

template <int MB, bool kSwiGLU, bool kPacked, int kQ>
__device__ __forceinline__ void wstream_body(const GemmArgs& a) {
  static_assert(kQ == 0 || kPacked, "quantised weights use the packed block order");
  typedef typename WRaw<kQ>::T Raw;
  constexpr int CB = wstream_cols<kQ, MB, kSwiGLU>(); // column blocks per task
  constexpr int NS = kSwiGLU ? 2 : 1;        // weight blocks per column block (gate, up)
  constexpr int NB = CB * NS;                // weight blocks of 16 rows per task; block j: column
                                             // block j / NS, part j % NS
  constexpr int U = (MB == 4 && !kQ) ? (kSwiGLU ? 1 : 2) : 4;   // k-steps per load batch (two batches in flight)
  const int lane = threadIdx.x & 63;
  const int K = kSwiGLU ? a.D : a.I;
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int R = kSwiGLU ? 2 * a.I : a.D;     // weight rows per group
  const int ncb = (NOUT + 15) / 16;
  const int ntc = (ncb + CB - 1) / CB;       // tasks per group
  const int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (task >= static_cast<int64_t>(a.G) * ntc) return;
  const int g = static_cast<int>(task / ntc);
  const int cb0 = static_cast<int>(task - static_cast<int64_t>(g) * ntc) * CB;
  const int64_t row0 = a.offsets ? a.offsets[g] : 0;
  const int64_t rows = a.offsets ? static_cast<int64_t>(a.offsets[g + 1]) - row0 : a.max_rows;
  if (rows <= 0) return;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const int kg = (lane >> 4) * 8;            // this lane's k offset inside a 32-wide step
  int col[CB];                               // this lane's output column in each column block
#pragma unroll
  for (int c = 0; c < CB; ++c) col[c] = (cb0 + c) * 16 + (lane & 15);
  // wrow[j]: this lane's weight bytes of k-step 0 of block j; k-step ks is WSTEP bytes further.
  // packed: a column block's 16 rows are one row block; k-step ks of it is one block in lane order.
  // int4: a lane's slot of a super-block holds U = 4 k-steps of codes (16 bytes), and its row's four
  // group multipliers sit at moff from it (one 4-byte load per super-block)
  constexpr bool kQ4 = kQ == kQInt4;
  const char* wrow[NB];
  constexpr int WSTEP = kQ ? 64 * code_slot(kQ) : (kPacked ? 1024 : 64);
  const int moff = 1024 + 4 * (lane & 15) - lane * 16;
  const char* Wg = static_cast<const char*>(a.w) +
                   (kQ ? quant_code_bytes(g, R, K, code_bits(kQ)) : static_cast<int64_t>(g) * R * K * 2);
  float scl[NB];                             // quantised: the scale of each block's row for this lane
  const float* S = nullptr;
  if constexpr (kQ != 0)
    S = reinterpret_cast<const float*>(static_cast<const char*>(a.w) + quant_code_bytes(a.G, R, K, code_bits(kQ))) +
        static_cast<int64_t>(g) * R;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int cb = min(cb0 + j / NS, ncb - 1);
    const int up = (j % NS) * a.I;           // SwiGLU: the up rows follow the I gate rows
    if constexpr (kQ4) {
      wrow[j] = Wg + static_cast<int64_t>(up / 16 + cb) * (K / 128) * kQ4Super + lane * 16;
    } else if constexpr (kPacked) {
      constexpr int SLOT = kQ ? code_slot(kQ) : 16;   // bytes per lane slot
      wrow[j] = Wg + static_cast<int64_t>(up / 16 + cb) * (K / 32) * WSTEP + lane * SLOT;
    } else {
      wrow[j] = Wg + (static_cast<int64_t>(up + min(cb * 16 + (lane & 15), NOUT - 1)) * K + kg) * 2;
    }
    if constexpr (kQ != 0) scl[j] = S[up + min(cb * 16 + (lane & 15), NOUT - 1)];
  }
  const int ksteps = K / 32;

  for (int64_t m0 = 0; m0 < rows; m0 += 16 * MB) {
    const uint16_t* xrow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int64_t lr = min<int64_t>(m0 + b * 16 + (lane & 15), rows - 1);
      const int64_t p = row0 + lr;
      const int64_t src = a.row_index ? a.row_index[p] : p;
      xrow[b] = X + src * K + kg;
    }
    f32x4 acc[MB][NB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // register double buffer: the loads of the next U k-steps are issued before the matrix-core
    // steps of the current ones, so U k-steps of weight loads are always in flight
    Raw fb[2][kQ4 ? 1 : U][NB];
    u32x4 fq[2][kQ4 ? NB : 1];                   // int4: the super-block slots
    uint32_t fm[2][kQ4 ? NB : 1];                // int4: their rows' group multipliers
    u32x4 fa[2][U][MB];
    auto load = [&](int buf, int k0) {
      if constexpr (kQ4) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const char* sp = wrow[j] + static_cast<int64_t>(k0 / U) * kQ4Super;
          fq[buf][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sp));
          fm[buf][j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp + moff));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (!kQ4) {
#pragma unroll
          for (int j = 0; j < NB; ++j)
            fb[buf][u][j] = __builtin_nontemporal_load(reinterpret_cast<const Raw*>(wrow[j] + static_cast<int64_t>(k0 + u) * WSTEP));
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) fa[buf][u][b] = *reinterpret_cast<const u32x4*>(xrow[b] + (k0 + u) * 32);
      }
    };
    // int4: the words enter the matrix cores as the bf16 values 136 + code (two per byte permute);
    // a k-step's product with them, less 136 times the step's activation sums (one product with
    // ones, shared by the task's blocks), times the step's group multiplier, is added to the sums
    auto math = [&](int buf) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (kQ4) {
          constexpr uint32_t kOne2 = 0x3F803F80u;               // two bf16 ones
          f32x4 sum[MB];
#pragma unroll
          for (int b = 0; b < MB; ++b)
            sum[b] = mfma16(fa[buf][u][b], u32x4{kOne2, kOne2, kOne2, kOne2}, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const u32x4 w = codes4_biased_bf16(fq[buf][j][u]);
            const float mj = static_cast<float>((fm[buf][j] >> (8 * u)) & 0xffu);
#pragma unroll
            for (int b = 0; b < MB; ++b) {
              const f32x4 t = mfma16(fa[buf][u][b], w, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[b][j][e] = fmaf(mj, fmaf(-136.f, sum[b][e], t[e]), acc[b][j][e]);
              // the sums are formed here, not sunk to the end of the batch (which would keep every
              // step's products live at once)
              asm volatile("" : "+v"(acc[b][j]));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const u32x4 w = to_bf16_frag<kQ>(fb[buf][u][j]);
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[b][j] = mfma16(fa[buf][u][b], w, acc[b][j]);
          }
        }
      }
    };
    const int full = ksteps / U;                 // U-step batches
    int ks = full * U;
    if (full > 0) {
      load(0, 0);
      int q = 0;
      for (; q + 2 <= full; q += 2) {            // two batches per trip keeps the buffers static
        if (q + 1 < full) load(1, (q + 1) * U);
        math(0);
        if (q + 2 < full) load(0, (q + 2) * U);
        math(1);
      }
      if (q < full) math(0);                     // odd batch count: the last one sits in buffer 0
    }
    if constexpr (!kQ4) {                        // int4 has none (K % 128 == 0)
      for (; ks < ksteps; ++ks) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const u32x4 w = to_bf16_frag<kQ>(__builtin_nontemporal_load(reinterpret_cast<const Raw*>(wrow[j] + static_cast<int64_t>(ks) * WSTEP)));
#pragma unroll
          for (int b = 0; b < MB; ++b)
            acc[b][j] = mfma16(*reinterpret_cast<const u32x4*>(xrow[b] + ks * 32), w, acc[b][j]);
        }
      }
    }
    if constexpr (kQ != 0) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[b][j] *= scl[j];
    }
    if constexpr (!kSwiGLU && kQ == 0) {
      if (a.out_f16s) {
        // fp16 form: the 16 lanes of a DPP row hold one row's 16 columns of the task (NOUT % 16 == 0)
        const int64_t rb = f16s_row_bytes(NOUT);
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = acc[b][c][i];
              float m = fabsf(v);
              m = fmaxf(m, xor16f<1>(m));
              m = fmaxf(m, xor16f<2>(m));
              m = fmaxf(m, xor16f<4>(m));
              m = fmaxf(m, xor16f<8>(m));
              const int ex = f16s_exp(m);
              const int64_t rr = m0 + b * 16 + 4 * (lane >> 4) + i;
              if (rr < rows && col[c] < NOUT) {
                char* Ob = static_cast<char*>(a.out) + (row0 + rr) * rb;
                *reinterpret_cast<uint16_t*>(Ob + 2 * col[c]) = f16_scaled(v, ex);
                if ((lane & 15) == 0) Ob[2 * NOUT + col[c] / 16] = static_cast<char>(ex);
              }
            }
        continue;
      }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      if (col[c] >= NOUT) continue;
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t rr = m0 + b * 16 + 4 * (lane >> 4) + i;
          if (rr < rows) {
            if constexpr (kSwiGLU)
              static_cast<uint16_t*>(a.out)[(row0 + rr) * NOUT + col[c]] =
                  f32_to_bf16(silu(acc[b][c * NS][i]) * acc[b][c * NS + 1][i]);
            else
              static_cast<float*>(a.out)[(row0 + rr) * NOUT + col[c]] = acc[b][c][i];
          }
        }
    }
  }
}

template <int MB, bool kSwiGLU, bool kPacked, int kQ>
__global__ __launch_bounds__(256) void gemm_wstream_kernel(GemmArgs a) {
  wstream_body<MB, kSwiGLU, kPacked, kQ>(a);
}

// The four-slab bf16 gate_up form at two waves per SIMD: left to itself the compiler gives it 284
// registers (one wave per SIMD); it fits 256 without spills, and a second wave keeps more weight
// loads in flight.
template <bool kPacked>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_wstream2_kernel(GemmArgs a) {
  wstream_body<4, true, kPacked, 0>(a);
}

template <bool kSwiGLU, bool kPacked, int kQ = 0>
static void launch_wstream(const GemmArgs& a, hipStream_t st) {
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int64_t ncb = (NOUT + 15) / 16;
  auto grid = [&](int cb) { return static_cast<unsigned>((a.G * ((ncb + cb - 1) / cb) + 3) / 4); };
  const int64_t mean_rows = a.offsets ? a.max_rows / std::max(a.G, 1) : a.max_rows;
  if (mean_rows <= 8)
    gemm_wstream_kernel<1, kSwiGLU, kPacked, kQ><<<grid(wstream_cols<kQ, 1, kSwiGLU>()), 256, 0, st>>>(a);
  else if (mean_rows <= 20)
    gemm_wstream_kernel<2, kSwiGLU, kPacked, kQ><<<grid(wstream_cols<kQ, 2, kSwiGLU>()), 256, 0, st>>>(a);
  else if constexpr (kSwiGLU && kQ == 0)
    gemm_wstream2_kernel<kPacked><<<grid(wstream_cols<kQ, 4, kSwiGLU>()), 256, 0, st>>>(a);
  else
    gemm_wstream_kernel<4, kSwiGLU, kPacked, kQ><<<grid(wstream_cols<kQ, 4, kSwiGLU>()), 256, 0, st>>>(a);
}

// ---------------------------------------------------------------------------------------------
// fp32 kernel: 64 x 64 tiles, 256 threads, 4 x 4 register blocking, k step 16.
//   SwiGLU: B tile = 32 gate rows + the 32 matching up rows; each thread keeps 4 rows x 2 h columns
//   of gate and of up accumulators.
// ---------------------------------------------------------------------------------------------
template <bool kSwiGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BM = 64, BNB = 64, BK = 16, NT = 256;
  constexpr int OUT_COLS = kSwiGLU ? 32 : 64;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BNB + 4];
  __shared__ int s_pref[1025];
  __shared__ int s_tmp[16];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int G = a.G;
  const int K = kSwiGLU ? a.D : a.I;
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int n_tiles = (NOUT + OUT_COLS - 1) / OUT_COLS;
  build_tile_prefix<NT>(a.offsets, G, a.max_rows, BM, n_tiles, s_pref, s_tmp);
  const int total = s_pref[G];
  const int P = gridDim.x;
  const float* X = static_cast<const float*>(a.x);
  const float* W = static_cast<const float*>(a.w);

  for (int r = 0;; ++r) {
    const int t = tile_of_round(r, blockIdx.x, P);
    if (r * P >= total) break;
    if (t >= total) continue;
    const int g = find_group(s_pref, G, t);
    const int local = t - s_pref[g];
    const int mt = local / n_tiles, nt = local - mt * n_tiles;
    const int64_t row0 = a.offsets ? a.offsets[g] : 0;
    const int64_t rows = a.offsets ? static_cast<int64_t>(a.offsets[g + 1]) - row0 : a.max_rows;
    if (rows <= 0) continue;
    const int m0 = mt * BM, c0 = nt * OUT_COLS;
    const float* Wg = W + static_cast<int64_t>(g) * (kSwiGLU ? 2LL * a.I * a.D : static_cast<int64_t>(a.D) * a.I);

    // loader: thread -> (row = tid / 4, k quad = tid % 4)
    const int lr = tid >> 2, lq = tid & 3;
    const int64_t arow = min<int64_t>(m0 + lr, rows - 1);
    const int64_t ap = row0 + arow;
    const float* srcA = X + (a.row_index ? static_cast<int64_t>(a.row_index[ap]) : ap) * K + lq * 4;
    int wrow;
    if (kSwiGLU) {
      const int ci = min(c0 + (lr & 31), NOUT - 1);
      wrow = lr < 32 ? ci : a.I + ci;
    } else {
      wrow = min(c0 + lr, NOUT - 1);
    }
    const float* srcB = Wg + static_cast<int64_t>(wrow) * K + lq * 4;

    float acc[4][4] = {};
    for (int kb = 0; kb < K; kb += BK) {
      const bool ok = kb + lq * 4 < K;
      const f32x4 va = ok ? *reinterpret_cast<const f32x4*>(srcA + kb) : f32x4{0, 0, 0, 0};
      const f32x4 vb = ok ? *reinterpret_cast<const f32x4*>(srcB + kb) : f32x4{0, 0, 0, 0};
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sA[lq * 4 + q][lr] = va[q];
        sB[lq * 4 + q][lr] = vb[q];
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
        if (kSwiGLU) {
          bv[0] = sB[kk][tx * 2];
          bv[1] = sB[kk][tx * 2 + 1];
          bv[2] = sB[kk][32 + tx * 2];
          bv[3] = sB[kk][32 + tx * 2 + 1];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[j] = sB[kk][tx * 4 + j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      }
    }
    float* O = static_cast<float*>(a.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = m0 + ty * 4 + i;
      if (rr >= rows) continue;
      if (kSwiGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = c0 + tx * 2 + j;
          if (col < NOUT) O[(row0 + rr) * NOUT + col] = silu(acc[i][j]) * acc[i][2 + j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = c0 + tx * 4 + j;
          if (col < NOUT) O[(row0 + rr) * NOUT + col] = acc[i][j];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Launch: a persistent grid of at most one workgroup per CU (the bf16 kernels use > 80 KB of LDS).
// ---------------------------------------------------------------------------------------------
static int64_t tile_upper_bound(const GemmArgs& a, int BM, int n_tiles) {
  const int64_t m_tiles = a.offsets ? (a.max_rows / BM + std::min<int64_t>(a.G, a.max_rows)) : (a.max_rows + BM - 1) / BM;
  return m_tiles * n_tiles;
}

static unsigned persistent_grid(int64_t ub, int per_cu) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
  int64_t p = std::min<int64_t>(ub, cap);
  if (p >= 8) p &= ~int64_t(7);
  return static_cast<unsigned>(std::max<int64_t>(p, 1));
}

template <int WM, int TM, int WN, int TN, bool kSwiGLU>
static void launch_bf16(const GemmArgs& a, hipStream_t st) {
  using C = BfCfg<WM, TM, WN, TN, kSwiGLU>;
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int n_tiles = (NOUT + C::OUT_COLS - 1) / C::OUT_COLS;
  constexpr int lds = 2 * (C::BM + C::BNB) * kBK * 2;
  const unsigned grid = persistent_grid(tile_upper_bound(a, C::BM, n_tiles), lds <= 76 * 1024 ? 2 : 1);
  gemm_bf16_kernel<WM, TM, WN, TN, kSwiGLU><<<grid, C::NT, 0, st>>>(a);
}

template <int WM, int TM, int WN, int TN, bool kSwiGLU, bool kPacked, int kQ = 0, bool kWKN = false, bool kBwd = false,
          bool kPipe = false>
static void launch_stream(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = WM * TM * 32, BNB = WN * TN * 32;
  constexpr int out_cols = kSwiGLU ? BNB / 2 : BNB;
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int n_tiles = (NOUT + out_cols - 1) / out_cols;
  constexpr int lds = 4 * (BM * 2 + BNB * (kQ ? (kQ == kQInt4 ? 8 : code_bits(kQ)) : 16) / 8) * kSK;
  // Short-row tiles (few rows per group) are pure weight streams: one workgroup per tile lets the
  // dispatcher start a new tile wherever one finishes instead of running fixed rounds with a
  // half-empty last round. Tall tiles keep a persistent grid (one prologue per workgroup).
  const int64_t ub = tile_upper_bound(a, BM, n_tiles);
  const unsigned grid = BM <= 32 ? static_cast<unsigned>(std::max<int64_t>(ub, 1))
                                 : persistent_grid(ub, lds <= 76 * 1024 ? 2 : 1);
  gemm_stream_kernel<WM, TM, WN, TN, kSwiGLU, kPacked, kQ, kWKN, kBwd, kPipe><<<grid, WM * WN * 64, 0, st>>>(a);
}

template <bool kSwiGLU>
static void launch_f32(const GemmArgs& a, hipStream_t st) {
  const int NOUT = kSwiGLU ? a.I : a.D;
  const int out_cols = kSwiGLU ? 32 : 64;
  const int n_tiles = (NOUT + out_cols - 1) / out_cols;
  const unsigned grid = persistent_grid(tile_upper_bound(a, 64, n_tiles), 4);
  gemm_f32_kernel<kSwiGLU><<<grid, 256, 0, st>>>(a);
}

// Rows per group decide the tile height: few rows per expert (decode) -> 32-row tiles with wide
// weight tiles; many rows -> 256 x 256 tiles.
static bool small_rows_of(bool grouped, int64_t max_rows, int G) { return grouped ? max_rows <= 64LL * G : max_rows <= 64; }
static bool small_rows(const GemmArgs& a) { return small_rows_of(a.offsets != nullptr, a.max_rows, a.G); }

// Streaming path when K is a multiple of 128 (four 32-wide stages per loop trip); the
// register-staged kernel covers the other K.
static bool streamable(const GemmArgs& a, bool gate_up) { return ((gate_up ? a.D : a.I) % 128) == 0; }

// The packed layout is accepted only with bf16 and K % 128 == 0 (checked at the boundary), so it
// always has a streaming kernel.
template <bool kSwiGLU>
static void launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (!a.bf16) return launch_f32<kSwiGLU>(a, st);
  if constexpr (!kSwiGLU) {
    // [K][N] weights (set only where wkn_streamable holds)
    if (a.wkn) return launch_stream<2, 4, 4, 2, false, false, 0, true>(a, st);
  } else {
    // SwiGLU backward epilogue (set only where bwd_fusable holds)
    if (a.bwd_dab) return launch_stream<2, 4, 4, 2, true, false, 0, false, true>(a, st);
  }
  const int K = kSwiGLU ? a.D : a.I;
  const bool stream = streamable(a, kSwiGLU);
  if (a.qbits == 8) {
    if (small_rows(a)) return launch_wstream<kSwiGLU, true, 8>(a, st);
    return launch_stream<2, 4, 4, 2, kSwiGLU, true, 8>(a, st);
  }
  if (a.qbits == 4) {
    if (small_rows(a)) return launch_wstream<kSwiGLU, true, 4>(a, st);
    return launch_stream<2, 4, 4, 2, kSwiGLU, true, 4>(a, st);
  }
  if (a.qbits == kQFp8) {
    if (small_rows(a)) return launch_wstream<kSwiGLU, true, kQFp8>(a, st);
    return launch_stream<2, 4, 4, 2, kSwiGLU, true, kQFp8>(a, st);
  }
  // the pipelined k-loop where it applies: gathered rows need 8 k-slices per tile, and its 32-bit DMA
  // byte offsets need the activation rows (at most max_rows of them: a gather reads x [N, D] with
  // N <= max_rows) and one group's weights below 2 GB
  const bool pipe = (!a.row_index || K / kSK >= 8) && a.max_rows * K * 2 < (1LL << 31) &&
                    (kSwiGLU ? 2LL * a.I : static_cast<int64_t>(a.D)) * K * 2 < (1LL << 31);
  if (a.packed) {
    if (small_rows(a)) return launch_wstream<kSwiGLU, true>(a, st);
    if (pipe) return launch_stream<2, 4, 4, 2, kSwiGLU, true, 0, false, false, true>(a, st);
    return launch_stream<2, 4, 4, 2, kSwiGLU, true>(a, st);
  }
  if (small_rows(a) && K % 32 == 0) return launch_wstream<kSwiGLU, false>(a, st);
  if (small_rows(a)) return stream ? launch_stream<1, 1, 4, 2, kSwiGLU, false>(a, st) : launch_bf16<1, 1, 4, 2, kSwiGLU>(a, st);
  if (stream && pipe) return launch_stream<2, 4, 4, 2, kSwiGLU, false, 0, false, false, true>(a, st);
  return stream ? launch_stream<2, 4, 4, 2, kSwiGLU, false>(a, st) : launch_bf16<2, 4, 4, 2, kSwiGLU>(a, st);
}

bool bwd_fusable(bool bf16, bool grouped, int64_t max_rows, int G, int D, int I) {
  return bf16 && !small_rows_of(grouped, max_rows, G) && D % 128 == 0 && I % 4 == 0;
}

bool wkn_streamable(bool bf16, bool grouped, int64_t max_rows, int G, int k_in, int n_out) {
  return bf16 && !small_rows_of(grouped, max_rows, G) && k_in % 128 == 0 && n_out % 8 == 0;
}

void launch_gate_up(const GemmArgs& a, hipStream_t st) { launch_gemm<true>(a, st); }
void launch_down(const GemmArgs& a, hipStream_t st) { launch_gemm<false>(a, st); }

// ---------------------------------------------------------------------------------------------
// Packing: one wave per 16 x 32 fragment; lane l copies the 16 bytes of row l % 16, k-chunk l / 16.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n_frags,
                                                   int R, int K) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (f >= n_frags) return;
  const int lane = threadIdx.x & 63;
  const int KB = K / 32, RB = R / 16;
  const int64_t kb = f % KB;
  const int64_t grb = f / KB;                          // g * RB + rb
  const int64_t g = grb / RB, rb = grb - g * RB;
  const int64_t row = g * R + rb * 16 + (lane & 15);
  dst[f * 64 + lane] = src[(row * K + kb * 32 + (lane >> 4) * 8) / 8];
}

void launch_pack(const uint16_t* src, uint16_t* dst, int64_t G, int R, int K, hipStream_t st) {
  const int64_t n_frags = G * (R / 16) * (K / 32);
  if (n_frags <= 0) return;
  pack_kernel<<<static_cast<unsigned>((n_frags + 3) / 4), 256, 0, st>>>(reinterpret_cast<const u32x4*>(src),
                                                                        reinterpret_cast<u32x4*>(dst), n_frags, R, K);
}

}  // namespace moe
