// Router kernel: logits = x W_r^T, FP32 softmax over all experts, top-k with the lower index
// winning ties, optional renormalisation, optional shared-expert gate sigmoid(w_s . x).
// ("27. Mixture of experts", section "The router", steps 1-3 and the parity note; section
//  "The shared expert", its equation.)
//
// One workgroup (4 waves) owns 64 tokens and all E <= 512 experts, so the softmax never leaves the
// workgroup. bf16: the [64 x E] logits come from 32x32x16 matrix-core steps (bf16 products are exact
// in fp32, accumulation in fp32), written to LDS unrounded. fp32: plain FMA dot products.
// Selection: each wave walks 16 tokens; a lane holds experts lane, lane+64, ...; k rounds of a
// wave-wide (p, index) arg-max with ties to the lower index.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteTokens = 64;
constexpr int kRouteThreads = 256;

template <int EB, bool kBf16>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  constexpr int kCols = EB * 128;                 // padded expert columns held in LDS
  constexpr int kPer = kCols / kWave;             // logits per lane during selection
  __shared__ float s_logit[kRouteTokens * kCols];
  __shared__ float s_sel_p[4][512];
  __shared__ int s_sel_e[4][512];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRouteTokens;
  const int D = a.D, E = a.E;

  if constexpr (kBf16) {
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* w = static_cast<const uint16_t*>(a.w_router);
    f32x16 acc[2][EB];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int b = 0; b < EB; ++b) acc[r][b] = f32x16{};
    const int64_t r0 = min<int64_t>(n0 + (lane & 31), a.N - 1);
    const int64_t r1 = min<int64_t>(n0 + 32 + (lane & 31), a.N - 1);
    const uint16_t* xa0 = x + r0 * D;
    const uint16_t* xa1 = x + r1 * D;
    const uint16_t* wb[EB];
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      int e = (wave + 4 * b) * 32 + (lane & 31);
      wb[b] = w + static_cast<int64_t>(min(e, E - 1)) * D;   // columns >= E are masked later
    }
    const int koff = (lane >> 5) * 8;
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 16) {
      const int kk = k0 + koff;
      const bool ok = kk < D;                    // D % 8 == 0: a lane's 8 values are all in or out
      u32x4 a0 = ok ? *reinterpret_cast<const u32x4*>(xa0 + kk) : u32x4{0, 0, 0, 0};
      u32x4 a1 = ok ? *reinterpret_cast<const u32x4*>(xa1 + kk) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < EB; ++b) {
        if ((wave + 4 * b) * 32 < E) {
          u32x4 bv = ok ? *reinterpret_cast<const u32x4*>(wb[b] + kk) : u32x4{0, 0, 0, 0};
          acc[0][b] = mfma32(a0, bv, acc[0][b]);
          acc[1][b] = mfma32(a1, bv, acc[1][b]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int b = 0; b < EB; ++b) {
        const int col = (wave + 4 * b) * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) s_logit[(r * 32 + acc_row(i, lane)) * kCols + col] = acc[r][b][i];
      }
  } else {
    const float* x = static_cast<const float*>(a.x);
    const float* w = static_cast<const float*>(a.w_router);
    for (int idx = tid; idx < kRouteTokens * E; idx += kRouteThreads) {
      const int t = idx / E, e = idx - t * E;
      const int64_t n = min<int64_t>(n0 + t, a.N - 1);
      const f32x4* xr = reinterpret_cast<const f32x4*>(x + n * D);
      const f32x4* wr = reinterpret_cast<const f32x4*>(w + static_cast<int64_t>(e) * D);
      float s = 0.f;
      for (int d = 0; d < D / 4; ++d) {
        f32x4 u = xr[d], v = wr[d];
        s = fmaf(u[0], v[0], s);
        s = fmaf(u[1], v[1], s);
        s = fmaf(u[2], v[2], s);
        s = fmaf(u[3], v[3], s);
      }
      s_logit[t * kCols + e] = s;
    }
  }
  __syncthreads();

  const int k = a.k;
  for (int t = wave; t < kRouteTokens; t += 4) {
    const int64_t n = n0 + t;
    if (n >= a.N) break;
    float v[kPer];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane + kWave * j;
      v[j] = e < E ? s_logit[t * kCols + e] : -INFINITY;
      m = fmaxf(m, v[j]);
    }
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane + kWave * j;
      v[j] = e < E ? expf(v[j] - m) : 0.f;
      s += v[j];
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane + kWave * j;
      v[j] = e < E ? v[j] / s : -1.f;          // probabilities; -1 marks "not a candidate"
    }
    if (a.logits) {
      for (int e = lane; e < E; e += kWave) a.logits[n * E + e] = s_logit[t * kCols + e];
    }
    float kept_sum = 0.f;
    for (int r = 0; r < k; ++r) {
      float bp = -2.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {          // strict '>' keeps the lowest index of a lane
        if (v[j] > bp) { bp = v[j]; be = lane + kWave * j; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float op = __shfl_xor(bp, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (op > bp || (op == bp && oe < be)) { bp = op; be = oe; }
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (lane + kWave * j == be) v[j] = -1.f;
      kept_sum += bp;                            // slot order, identical in every lane
      if (lane == 0) { s_sel_p[wave][r] = bp; s_sel_e[wave][r] = be; }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int r = lane; r < k; r += kWave) {
      const float p = s_sel_p[wave][r];
      a.weights[n * k + r] = a.norm ? p / kept_sum : p;
      a.experts[n * k + r] = s_sel_e[wave][r];
    }
    if (a.w_shared_gate) {
      float z = 0.f;
      if constexpr (kBf16) {
        const uint16_t* xr = static_cast<const uint16_t*>(a.x) + n * D;
        const uint16_t* ws = static_cast<const uint16_t*>(a.w_shared_gate);
        for (int d = lane; d < D; d += kWave) z = fmaf(bf16_to_f32(xr[d]), bf16_to_f32(ws[d]), z);
      } else {
        const float* xr = static_cast<const float*>(a.x) + n * D;
        const float* ws = static_cast<const float*>(a.w_shared_gate);
        for (int d = lane; d < D; d += kWave) z = fmaf(xr[d], ws[d], z);
      }
      z = wave_sum(z);
      if (lane == 0) a.shared_scale[n] = 1.f / (1.f + expf(-z));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int EB>
static void launch_route_eb(const RouteArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.N + kRouteTokens - 1) / kRouteTokens);
  if (a.bf16)
    route_kernel<EB, true><<<grid, kRouteThreads, 0, st>>>(a);
  else
    route_kernel<EB, false><<<grid, kRouteThreads, 0, st>>>(a);
}

void launch_route(const RouteArgs& a, hipStream_t st) {
  const int blocks32 = (a.E + 31) / 32;
  const int eb = (blocks32 + 3) / 4;
  switch (eb) {
    case 1: launch_route_eb<1>(a, st); break;
    case 2: launch_route_eb<2>(a, st); break;
    case 3: launch_route_eb<3>(a, st); break;
    default: launch_route_eb<4>(a, st); break;
  }
}

}  // namespace moe
