// The grouping of a small batch (at most kPermSmallMax assignments) by one workgroup of 512
// threads: histogram, scan and stable scatter ("27. Mixture of experts", section "Dispatch", grouped
// dispatch steps 1-2), with ranks from ordered ballots and per-wave counts (deterministic).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermSmallMax = 8192;

// Must be called by all 512 threads of the workgroup.
__device__ __forceinline__ void perm_block512(const PermuteArgs& a, int nbits) {
  __shared__ int s_pos[512];         // counts, then each expert's next sorted position
  __shared__ int s_end[512];         // end of each expert's kept rows
  __shared__ int s_wcnt[8][512];
  __shared__ int s_wave[8];
  const int E = a.E, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t A = a.A;
  // the batch's expert ids, all loads issued at once (A <= kPermSmallMax: 16 per thread), used by
  // the count and by the scatter
  constexpr int RND = kPermSmallMax / 512;
  int ev[RND];
#pragma unroll
  for (int r = 0; r < RND; ++r) {
    const int64_t i = static_cast<int64_t>(r) * 512 + tid;
    ev[r] = i < A ? a.experts[i] : -1;
  }
  if (tid < E) s_pos[tid] = 0;
  for (int w = 0; w < 8; ++w)
    if (tid < E) s_wcnt[w][tid] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RND; ++r)
    if (static_cast<unsigned>(ev[r]) < static_cast<unsigned>(E)) atomicAdd(&s_pos[ev[r]], 1);
  __syncthreads();
  const int total = tid < E ? static_cast<int>(min<int64_t>(s_pos[tid], a.capacity)) : 0;   // kept rows
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
  if (tid < E) {
    a.counts[tid] = total;
    a.offsets[tid] = excl;
    s_pos[tid] = excl;
    s_end[tid] = excl + total;
  }
  if (tid == E - 1) a.offsets[E] = excl + total;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < RND; ++r) {
    const int64_t base = static_cast<int64_t>(r) * 512;
    if (base >= A) break;                     // uniform
    const int64_t i = base + tid;
    const int e_in = i < A ? ev[r] : 0;
    const bool in_range = static_cast<unsigned>(e_in) < static_cast<unsigned>(E);
    const bool valid = i < A && in_range;
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
      pos = s_pos[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_pos[e], cnt);
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

}  // namespace moe
