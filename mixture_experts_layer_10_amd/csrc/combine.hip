// Weighted unpermute ("27. Mixture of experts", section "Dispatch", grouped step 4, and the
// shared-expert equation): y[n] = sum_j w[n, j] * out_perm[slot_pos[n*k + j]] (+ s[n] * shared[n]),
// from fp32 expert outputs or from their fp16 form (fp16 values with a power-of-two exponent per
// 16 columns).
// A gather per token instead of an index_add scatter: no atomics, the fp32 sum runs in slot order
// j = 0..k-1 and is rounded once, so results are bitwise reproducible.
#include <algorithm>

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

// Expert outputs in the fp16 form (rows of f16s_row_bytes(D) bytes: D fp16 values, then one int8
// exponent per 16 columns): one thread per 16-column group of the token, 32 bytes of values and its
// exponent byte per slot row, eight rows' loads in flight. Each value is restored exactly
// (fp16 * 2^exp) and then summed as in combine_kernel: fp32, slot order, then the shared term.
// Plain (cached) loads: the rows were written by the down product just before, and nontemporal
// loads made the 16,384-token layer 12 us slower.
template <bool kOutBf16, int TPB>
__global__ __launch_bounds__(256) void combine_f16s_kernel(CombineArgs a) {
  __shared__ float s_w_all[TPB][512];
  __shared__ int s_p_all[TPB][512];
  // TPB tokens per workgroup, blockDim.x / TPB threads each
  const int per = blockDim.x / TPB, sub = threadIdx.x / per;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * TPB + sub;
  const int G = a.D / 16, k = a.k, tid = threadIdx.x - sub * per;
  float* s_w = s_w_all[sub];
  int* s_p = s_p_all[sub];
  if (n < a.N) {
    for (int j = tid; j < k; j += per) {
      const int p = a.slot_pos[n * k + j];
      s_w[j] = p >= 0 ? a.weights[n * k + j] : 0.f;
      s_p[j] = p;
    }
  }
  __syncthreads();
  if (n >= a.N) return;
  const int64_t RB = f16s_row_bytes(a.D);
  const char* base = reinterpret_cast<const char*>(a.out_perm);
  const float s = a.shared_out ? (a.shared_scale ? a.shared_scale[n] : 1.0f) : 0.0f;
  auto add_row = [&](float* acc, const u32x4* v, int ex, float w) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[8 * h + 2 * i] = fmaf(w, f16_unscale(static_cast<uint16_t>(v[h][i]), ex), acc[8 * h + 2 * i]);
        acc[8 * h + 2 * i + 1] = fmaf(w, f16_unscale(static_cast<uint16_t>(v[h][i] >> 16), ex), acc[8 * h + 2 * i + 1]);
      }
  };
  for (int g = tid; g < G; g += per) {
    float acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = 0.f;
    int j = 0;
    for (; j + 8 <= k; j += 8) {
      u32x4 v[8][2];
      int ex[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int p = s_p[j + u];
        if (p >= 0) {
          const char* r = base + static_cast<int64_t>(p) * RB;
          v[u][0] = *reinterpret_cast<const u32x4*>(r + 32 * g);
          v[u][1] = *reinterpret_cast<const u32x4*>(r + 32 * g + 16);
          ex[u] = static_cast<signed char>(r[2 * a.D + g]);
        } else {
          v[u][0] = v[u][1] = u32x4{0, 0, 0, 0};
          ex[u] = 0;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) add_row(acc, v[u], ex[u], s_w[j + u]);
    }
    for (; j < k; ++j) {
      const int p = s_p[j];
      if (p < 0) continue;                     // adds 0 * 0: nothing
      const char* r = base + static_cast<int64_t>(p) * RB;
      const u32x4 v[2] = {*reinterpret_cast<const u32x4*>(r + 32 * g), *reinterpret_cast<const u32x4*>(r + 32 * g + 16)};
      add_row(acc, v, static_cast<signed char>(r[2 * a.D + g]), s_w[j]);
    }
    if (a.shared_out) {
      const char* r = reinterpret_cast<const char*>(a.shared_out) + n * RB;
      const u32x4 v[2] = {*reinterpret_cast<const u32x4*>(r + 32 * g), *reinterpret_cast<const u32x4*>(r + 32 * g + 16)};
      add_row(acc, v, static_cast<signed char>(r[2 * a.D + g]), s);
    }
    if constexpr (kOutBf16) {
      u32x4* yv = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.y) + n * a.D + 16 * g);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        yv[h] = u32x4{pack_bf16x2(acc[8 * h], acc[8 * h + 1]), pack_bf16x2(acc[8 * h + 2], acc[8 * h + 3]),
                      pack_bf16x2(acc[8 * h + 4], acc[8 * h + 5]), pack_bf16x2(acc[8 * h + 6], acc[8 * h + 7])};
    } else {
      f32x4* yv = reinterpret_cast<f32x4*>(static_cast<float*>(a.y) + n * a.D + 16 * g);
#pragma unroll
      for (int h = 0; h < 4; ++h) yv[h] = f32x4{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
    }
  }
}

void launch_combine(const CombineArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>(a.N);
  if (a.in_f16s) {
    // a thread per 16-column group (up to 256 per token); two tokens per workgroup when a token
    // needs at most 128 threads
    const int per = std::min(256, (a.D / 16 + 63) / 64 * 64);
    if (per <= 128) {
      const unsigned grid2 = static_cast<unsigned>((a.N + 1) / 2);
      if (a.out_bf16)
        combine_f16s_kernel<true, 2><<<grid2, 2 * per, 0, st>>>(a);
      else
        combine_f16s_kernel<false, 2><<<grid2, 2 * per, 0, st>>>(a);
    } else {
      if (a.out_bf16)
        combine_f16s_kernel<true, 1><<<grid, per, 0, st>>>(a);
      else
        combine_f16s_kernel<false, 1><<<grid, per, 0, st>>>(a);
    }
    return;
  }
  if (a.out_bf16)
    combine_kernel<true><<<grid, 256, 0, st>>>(a);
  else
    combine_kernel<false><<<grid, 256, 0, st>>>(a);
}

}  // namespace moe
