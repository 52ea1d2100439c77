// Weighted unpermute ("27. Mixture of experts", section "Dispatch", grouped step 4, and the
// shared-expert equation): y[n] = sum_j w[n, j] * out_perm[slot_pos[n*k + j]] (+ s[n] * shared[n]).
// A gather per token instead of an index_add scatter: no atomics, the fp32 sum runs in slot order
// j = 0..k-1 and is rounded once, so results are bitwise reproducible.
// One wave per token row; each lane handles 4 consecutive fp32 columns per 256-column stripe.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombineWaves = 4;

template <bool kOutBf16>
__global__ __launch_bounds__(kCombineWaves * 64) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kCombineWaves + (threadIdx.x >> 6);
  if (n >= a.N) return;
  const int D = a.D, k = a.k;
  for (int c = lane * 4; c < D; c += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float w = a.weights[n * k + j];
      const int64_t p = a.slot_pos[n * k + j];
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.out_perm + p * D + c);
      acc[0] = fmaf(w, v[0], acc[0]);
      acc[1] = fmaf(w, v[1], acc[1]);
      acc[2] = fmaf(w, v[2], acc[2]);
      acc[3] = fmaf(w, v[3], acc[3]);
    }
    if (a.shared_out) {
      const float s = a.shared_scale ? a.shared_scale[n] : 1.0f;
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.shared_out + n * D + c);
      acc[0] = fmaf(s, v[0], acc[0]);
      acc[1] = fmaf(s, v[1], acc[1]);
      acc[2] = fmaf(s, v[2], acc[2]);
      acc[3] = fmaf(s, v[3], acc[3]);
    }
    if constexpr (kOutBf16) {
      uint2 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + n * D + c) = o;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.y) + n * D + c) = acc;
    }
  }
}

void launch_combine(const CombineArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.N + kCombineWaves - 1) / kCombineWaves);
  if (a.out_bf16)
    combine_kernel<true><<<grid, kCombineWaves * 64, 0, st>>>(a);
  else
    combine_kernel<false><<<grid, kCombineWaves * 64, 0, st>>>(a);
}

}  // namespace moe
