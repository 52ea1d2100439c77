// Weighted unpermute ("27. Mixture of experts", section "Dispatch", grouped step 4, and the
// shared-expert equation): y[n] = sum_j w[n, j] * out_perm[slot_pos[n*k + j]] (+ s[n] * shared[n]).
// A gather per token instead of an index_add scatter: no atomics, the fp32 sum runs in slot order
// j = 0..k-1 and is rounded once, so results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {

// One workgroup per token: its k weights and slot rows go to LDS once, then each thread sums 4
// consecutive columns over the k rows, eight rows' loads in flight at a time. A pair dropped by a
// capacity limit (slot_pos -1) contributes nothing: its row is not read and adds zero.
template <bool kOutBf16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ float s_w[512];
  __shared__ int s_p[512];
  const int64_t n = blockIdx.x;
  const int D4 = a.D / 4, k = a.k, tid = threadIdx.x;
  for (int j = tid; j < k; j += 256) {
    const int p = a.slot_pos[n * k + j];
    s_w[j] = p >= 0 ? a.weights[n * k + j] : 0.f;
    s_p[j] = p;
  }
  __syncthreads();
  const f32x4* o = reinterpret_cast<const f32x4*>(a.out_perm);
  const float s = a.shared_out ? (a.shared_scale ? a.shared_scale[n] : 1.0f) : 0.0f;
  for (int c = tid; c < D4; c += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int j = 0;
    for (; j + 8 <= k; j += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = s_p[j + u] >= 0 ? __builtin_nontemporal_load(&o[static_cast<int64_t>(s_p[j + u]) * D4 + c]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = s_w[j + u];
        acc[0] = fmaf(w, v[u][0], acc[0]);
        acc[1] = fmaf(w, v[u][1], acc[1]);
        acc[2] = fmaf(w, v[u][2], acc[2]);
        acc[3] = fmaf(w, v[u][3], acc[3]);
      }
    }
    for (; j < k; ++j) {
      const f32x4 v = s_p[j] >= 0 ? __builtin_nontemporal_load(&o[static_cast<int64_t>(s_p[j]) * D4 + c]) : f32x4{0.f, 0.f, 0.f, 0.f};
      const float w = s_w[j];
      acc[0] = fmaf(w, v[0], acc[0]);
      acc[1] = fmaf(w, v[1], acc[1]);
      acc[2] = fmaf(w, v[2], acc[2]);
      acc[3] = fmaf(w, v[3], acc[3]);
    }
    if (a.shared_out) {
      const f32x4 v = reinterpret_cast<const f32x4*>(a.shared_out)[n * D4 + c];
      acc[0] = fmaf(s, v[0], acc[0]);
      acc[1] = fmaf(s, v[1], acc[1]);
      acc[2] = fmaf(s, v[2], acc[2]);
      acc[3] = fmaf(s, v[3], acc[3]);
    }
    if constexpr (kOutBf16) {
      uint2 ov;
      ov.x = pack_bf16x2(acc[0], acc[1]);
      ov.y = pack_bf16x2(acc[2], acc[3]);
      reinterpret_cast<uint2*>(a.y)[n * D4 + c] = ov;
    } else {
      reinterpret_cast<f32x4*>(a.y)[n * D4 + c] = acc;
    }
  }
}

void launch_combine(const CombineArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>(a.N);
  if (a.out_bf16)
    combine_kernel<true><<<grid, 256, 0, st>>>(a);
  else
    combine_kernel<false><<<grid, 256, 0, st>>>(a);
}

}  // namespace moe
