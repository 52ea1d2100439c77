// Router load statistics and the Switch-style balance loss ("Qwen3-VL + MoE: train to deploy",
// section "How the router and experts learn", the item on an auxiliary balance loss, reading its N as the number of experts; "27. Mixture of
// experts", section "Dispatch", closing paragraph on expert load):
//   f_e  = counts[e] / (N k)                         fraction of assignments routed to e
//   P_e  = (1 / N) sum_n softmax(logits[n])_e        mean router probability of e (fp32 softmax)
//   loss = E * sum_e f_e P_e                          (the caller applies its coefficient)
// Deterministic: per-block partial sums in token order, then per expert a fixed-order fp64 sum of
// the blocks, then the loss sum in expert order. No atomics.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kStatTok = 32;      // tokens per block of the first pass (many blocks: latency-bound work)

int64_t stats_blocks(int64_t N) { return (N + kStatTok - 1) / kStatTok; }

// Pass 1: one workgroup of 4 waves per block of kStatTok tokens; a wave takes every fourth token,
// a lane experts lane + 64 j. Each wave sums its tokens' probabilities in token order into its own
// LDS row; the four rows are added in wave order and written to partial[block][E].
__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits, float* __restrict__ partial,
                                                            int64_t N, int E) {
  __shared__ float s_p[4][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = lane; e < 512; e += 64) s_p[wave][e] = 0.f;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kStatTok;
  const int64_t n1 = min<int64_t>(n0 + kStatTok, N);
  for (int64_t n = n0 + wave; n < n1; n += 4) {
    const float* l = logits + n * E;
    float v[8];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? l[e] : -INFINITY;
      m = fmaxf(m, v[j]);
    }
    m = wave_max_dpp(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? expf(v[j] - m) : 0.f;
      s += v[j];
    }
    s = wave_sum_dpp(s);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      if (e < E) s_p[wave][e] += v[j] / s;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    partial[static_cast<int64_t>(blockIdx.x) * E + e] = ((s_p[0][e] + s_p[1][e]) + s_p[2][e]) + s_p[3][e];
}

// Pass 2: one workgroup per expert. Thread t adds blocks t, t + 256, ... in order (fp64); the 256
// thread sums are added by a fixed pairwise tree in LDS.
__global__ __launch_bounds__(256) void stats_finish_kernel(const float* __restrict__ partial, const int32_t* __restrict__ counts,
                                                           float* __restrict__ f_out, float* __restrict__ P_out,
                                                           int64_t N, int E, int k, int64_t n_blocks) {
  __shared__ double s_sum[256];
  const int t = threadIdx.x, e = blockIdx.x;
  double sum = 0.0;
  for (int64_t b = t; b < n_blocks; b += 256) sum += static_cast<double>(partial[b * E + e]);
  s_sum[t] = sum;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) s_sum[t] += s_sum[t + h];
    __syncthreads();
  }
  if (t == 0) {
    // no tokens: no load and no probability mass (zeros rather than 0 / 0)
    P_out[e] = N > 0 ? static_cast<float>(s_sum[0] / static_cast<double>(N)) : 0.f;
    f_out[e] = N > 0 ? static_cast<float>(static_cast<double>(counts[e]) / (static_cast<double>(N) * k)) : 0.f;
  }
}

// Pass 3: loss = E * sum_e f_e P_e, the sum in expert order (fp64).
__global__ __launch_bounds__(64) void stats_loss_kernel(const float* __restrict__ f, const float* __restrict__ P,
                                                        float* __restrict__ loss_out, int E) {
  if (threadIdx.x != 0) return;
  double acc = 0.0;
  for (int e = 0; e < E; ++e) acc += static_cast<double>(f[e]) * static_cast<double>(P[e]);
  loss_out[0] = static_cast<float>(static_cast<double>(E) * acc);
}

void launch_stats(const float* logits, const int32_t* counts, float* f, float* P, float* loss, float* partial,
                  int64_t N, int E, int k, hipStream_t st) {
  const int64_t nb = stats_blocks(N);
  if (nb > 0) stats_partial_kernel<<<static_cast<unsigned>(nb), 256, 0, st>>>(logits, partial, N, E);
  stats_finish_kernel<<<E, 256, 0, st>>>(partial, counts, f, P, N, E, k, nb);
  stats_loss_kernel<<<1, 64, 0, st>>>(f, P, loss, E);
}

// Selection-bias nudge ("Qwen3-VL + MoE: train to deploy", section "How the router and experts learn", the item on balancing without a loss:
// overloaded experts get their bias lowered slightly, idle ones raised): one thread per expert,
// bias[e] -= gamma * sign(counts[e] - A / E), comparing counts[e] * E with A exactly in integers.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                                          float gamma, int64_t A, int E) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t load = static_cast<int64_t>(counts[e]) * E;
  const float sgn = load > A ? 1.f : (load < A ? -1.f : 0.f);
  bias[e] = bias[e] - gamma * sgn;
}

void launch_bias_update(const int32_t* counts, float* bias, float gamma, int64_t A, int E, hipStream_t st) {
  bias_update_kernel<<<static_cast<unsigned>((E + 255) / 256), 256, 0, st>>>(counts, bias, gamma, A, E);
}

}  // namespace moe
