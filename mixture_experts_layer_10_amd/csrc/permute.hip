// Grouping of the N*k assignments by expert: histogram -> prefix scan -> stable scatter
// ("27. Mixture of experts", section "Dispatch", grouped dispatch steps 1-2; stretch exercise 2,
//  the prefix-sum array of row offsets).
//
// Deterministic by construction: ranks come from ordered ballots inside a wave and ordered
// per-wave counts inside a round, never from atomics (LDS atomics only build counts, whose value
// does not depend on order).
// An expert id outside [0, E) (never produced by the router; possible from a caller's own ids) is
// treated as a dropped pair: it is not counted, takes no row and gets slot_pos -1, so no index
// derived from it reaches memory.
// Capacity limit ("Qwen3-VL + MoE: train to deploy", section "How the router and experts learn", the item on capacity limits): an expert keeps
// its first `capacity` assignments in assignment order. Counts and offsets cover the kept rows;
// since positions are handed out in assignment order, an assignment is kept exactly when its
// position falls before its expert's end offset, and a dropped one gets slot_pos -1.
#include "common.h"
#include "kernels.h"
#include "perm_block.h"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermRounds = kPermChunk / kPermThreads;   // assignments per thread and chunk
static_assert(kPermRounds * kPermThreads == kPermChunk, "a chunk is whole rounds");

int64_t permute_chunks(int64_t A) { return (A + kPermChunk - 1) / kPermChunk; }

// Pass 1: per-chunk expert histogram.
__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(PermuteArgs a) {
  __shared__ int s_cnt[512];
  const int E = a.E;
  for (int e = threadIdx.x; e < E; e += kPermThreads) s_cnt[e] = 0;
  __syncthreads();
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * kPermChunk;
  const int64_t hi = min<int64_t>(lo + kPermChunk, a.A);
  // every load of the chunk issued before the first count (one memory latency, not one per round)
  int ev[kPermRounds];
#pragma unroll
  for (int r = 0; r < kPermRounds; ++r) {
    const int64_t i = lo + r * kPermThreads + threadIdx.x;
    ev[r] = i < hi ? a.experts[i] : -1;
  }
#pragma unroll
  for (int r = 0; r < kPermRounds; ++r)
    if (static_cast<unsigned>(ev[r]) < static_cast<unsigned>(E)) atomicAdd(&s_cnt[ev[r]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) a.block_counts[blockIdx.x * static_cast<int64_t>(E) + e] = s_cnt[e];
}

// Pass 2 (one workgroup of 512 threads, one expert per thread): counts, offsets, and each chunk's
// starting row for each expert (written back over block_counts). With at most kScanRegs chunks a
// thread holds its expert's whole column in registers: one round of loads, one round of stores.
constexpr int kScanRegs = 128;

template <bool kInRegs>
__global__ __launch_bounds__(512) void perm_scan_kernel(PermuteArgs a, int n_chunks) {
  __shared__ int s_wave[8];
  const int E = a.E, e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int total = 0;
  int c[kInRegs ? kScanRegs : 1];
  if (e < E) {
    if constexpr (kInRegs) {
#pragma unroll
      for (int b = 0; b < kScanRegs; ++b) c[b] = b < n_chunks ? a.block_counts[static_cast<int64_t>(b) * E + e] : 0;
#pragma unroll
      for (int b = 0; b < kScanRegs; ++b) {      // exclusive running sum down the column
        const int v = c[b];
        c[b] = total;
        total += v;
      }
    } else {
      // eight chunk counts in flight at a time (each thread walks its own expert's column)
      int b = 0;
      for (; b + 8 <= n_chunks; b += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = a.block_counts[static_cast<int64_t>(b + u) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a.block_counts[static_cast<int64_t>(b + u) * E + e] = total;
          total += v[u];
        }
      }
      for (; b < n_chunks; ++b) {
        int32_t* p = a.block_counts + static_cast<int64_t>(b) * E + e;
        const int v = *p;
        *p = total;
        total += v;
      }
    }
    total = static_cast<int>(min<int64_t>(total, a.capacity));   // kept rows (chunk bases unchanged)
    a.counts[e] = total;
  }
  // exclusive scan of total over e: inclusive wave scan, then the wave totals
  int inc = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  const int excl = before + inc - total;
  if (e < E) {
    a.offsets[e] = excl;
    if constexpr (kInRegs) {
#pragma unroll
      for (int b = 0; b < kScanRegs; ++b)
        if (b < n_chunks) a.block_counts[static_cast<int64_t>(b) * E + e] = c[b] + excl;
    } else {
#pragma unroll 8
      for (int b = 0; b < n_chunks; ++b) a.block_counts[static_cast<int64_t>(b) * E + e] += excl;
    }
  }
  if (e == E - 1) a.offsets[E] = excl + total;
}

// Pass 3: stable scatter. Rounds of 256 assignments in order; inside a wave, the rank among equal
// experts comes from a ballot match; across the 4 waves of a round, from per-wave counts in LDS.
__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(PermuteArgs a, int nbits) {
  __shared__ int s_run[512];
  __shared__ int s_end[512];
  __shared__ int s_wcnt[4][512];
  const int E = a.E, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kPermThreads) {
    s_run[e] = a.block_counts[blockIdx.x * static_cast<int64_t>(E) + e];
    s_end[e] = a.offsets[e + 1];
    s_wcnt[0][e] = s_wcnt[1][e] = s_wcnt[2][e] = s_wcnt[3][e] = 0;
  }
  __syncthreads();
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * kPermChunk;
  const int64_t hi = min<int64_t>(lo + kPermChunk, a.A);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the chunk's expert ids, all loads issued before the first round
  int ev[kPermRounds];
#pragma unroll
  for (int r = 0; r < kPermRounds; ++r) {
    const int64_t i = lo + r * kPermThreads + tid;
    ev[r] = i < hi ? a.experts[i] : 0;
  }
#pragma unroll
  for (int r = 0; r < kPermRounds; ++r) {
    const int64_t base = lo + r * kPermThreads;
    if (base >= hi) break;                    // uniform: the chunk's last round is done
    const int64_t i = base + tid;
    const int e_in = ev[r];
    const bool in_range = static_cast<unsigned>(e_in) < static_cast<unsigned>(E);
    const bool valid = i < hi && in_range;
    const int e = valid ? e_in : 0;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t b = __ballot(set);
      m &= set ? b : ~b;
    }
    const int rank = __popcll(m & below);
    const int cnt = __popcll(m);
    if (valid && rank == 0) s_wcnt[wave][e] = cnt;
    __syncthreads();
    int pos = 0;
    if (valid) {
      pos = s_run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_run[e], cnt);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
    if (valid) {
      const bool kept = pos < s_end[e];
      if (kept) a.token_of[pos] = static_cast<int32_t>(i / a.k);
      a.slot_pos[i] = kept ? pos : -1;
    } else if (!in_range) {
      a.slot_pos[i] = -1;                     // an id outside [0, E): dropped
    }
  }
}

// Small batches (decode): one workgroup of 8 waves does the histogram, the scan and the stable
// scatter (perm_block512), instead of three launches whose fixed cost would dominate.
__global__ __launch_bounds__(512) void perm_small_kernel(PermuteArgs a, int nbits) { perm_block512(a, nbits); }

void launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int n_chunks = static_cast<int>(permute_chunks(a.A));
  int nbits = 1;
  while ((1 << nbits) < a.E) ++nbits;
  if (a.A <= kPermSmallMax) {
    perm_small_kernel<<<1, 512, 0, st>>>(a, nbits);
    return;
  }
  if (n_chunks > 0) perm_count_kernel<<<n_chunks, kPermThreads, 0, st>>>(a);
  if (n_chunks <= kScanRegs)
    perm_scan_kernel<true><<<1, 512, 0, st>>>(a, n_chunks);
  else
    perm_scan_kernel<false><<<1, 512, 0, st>>>(a, n_chunks);
  if (n_chunks > 0) perm_scatter_kernel<<<n_chunks, kPermThreads, 0, st>>>(a, nbits);
}

// Row gather: one wave per row, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ x, const int32_t* __restrict__ token_of,
                                                          const int32_t* __restrict__ n_valid, u32x4* __restrict__ x_perm,
                                                          int64_t rows, int64_t vecs) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows || row >= *n_valid) return;          // rows past the kept total hold no token
  const u32x4* src = x + static_cast<int64_t>(token_of[row]) * vecs;
  u32x4* dst = x_perm + row * vecs;
  for (int64_t v = threadIdx.x & 63; v < vecs; v += 64) dst[v] = src[v];
}

void launch_gather_rows(const void* x, const int32_t* token_of, const int32_t* n_valid, void* x_perm, int64_t rows,
                        int64_t row_bytes, hipStream_t st) {
  if (rows <= 0) return;
  const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
  gather_rows_kernel<<<grid, 256, 0, st>>>(static_cast<const u32x4*>(x), token_of, n_valid, static_cast<u32x4*>(x_perm),
                                           rows, row_bytes / 16);
}

}  // namespace moe
