// Router kernel: logits = x W_r^T, FP32 softmax over all experts, top-k with the lower index
// winning ties, optional renormalisation, optional shared-expert gate sigmoid(w_s . x).
// ("27. Mixture of experts", section "The router", steps 1-3 and the parity note; section
//  "The shared expert", its equation.)
//
// One workgroup (4 waves) owns a tile of tokens and all E <= 512 experts, so the softmax never
// leaves the workgroup.
//  bf16: 32 tokens per workgroup. k-slices of x and W_r are staged in LDS (16-byte chunks, XOR
//        swizzle); with D % 128 == 0 they stream straight from global memory into four LDS stages,
//        otherwise through registers into two. Wave w computes expert blocks w, w+4, ... with
//        32x32x16 matrix-core steps (bf16 products are exact in fp32, fp32 accumulation). The
//        logits land in LDS unrounded, over the staging buffers.
//        Long batches (N >= 8192, D % 512 == 0, D <= 2048) keep the whole x tile in LDS instead
//        and stream the router weights from L2 (x-stationary kernel, eight waves).
//  fp32: 64 tokens per workgroup, plain FMA dot products.
// Selection: E <= 128 and k <= 8: 16 lanes per token, each sorting 8 candidates, then four rounds
// of pairwise merges of sorted lists. Otherwise each wave walks its tokens; a lane holds experts
// lane, lane+64, ...; k rounds of a wave-wide (p, index) arg-max. Either way ties go to the lower
// index.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteThreads = 256;

// Partial dot product x_row . w over d = g, g + G, ... in 16-byte chunks (G lanes share a row; the
// caller adds the G partials). Four chunks of each operand are loaded before any is used, so a
// lane keeps eight loads in flight instead of one dependent load per element.
template <int G>
__device__ float row_dot_part(const void* x_row, const void* w, int D, bool bf16, int g) {
  const bool vec = ((reinterpret_cast<uintptr_t>(x_row) | reinterpret_cast<uintptr_t>(w)) & 15) == 0;
  float z[4] = {0.f, 0.f, 0.f, 0.f};
  if (bf16 && vec && (D & 7) == 0) {
    const u32x4* xv = static_cast<const u32x4*>(x_row);
    const u32x4* wv = static_cast<const u32x4*>(w);
    const int nc = D >> 3;
    int c = g;
    auto acc8 = [](float zz, u32x4 xa, u32x4 wa) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zz = fmaf(__uint_as_float(xa[i] << 16), __uint_as_float(wa[i] << 16), zz);
        zz = fmaf(__uint_as_float(xa[i] & 0xffff0000u), __uint_as_float(wa[i] & 0xffff0000u), zz);
      }
      return zz;
    };
    for (; c + 3 * G < nc; c += 4 * G) {
      u32x4 xa[4], wa[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xa[u] = xv[c + u * G];
        wa[u] = wv[c + u * G];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) z[u] = acc8(z[u], xa[u], wa[u]);
    }
    for (; c < nc; c += G) z[0] = acc8(z[0], xv[c], wv[c]);
  } else if (!bf16 && vec && (D & 3) == 0) {
    const f32x4* xv = static_cast<const f32x4*>(x_row);
    const f32x4* wv = static_cast<const f32x4*>(w);
    const int nc = D >> 2;
    int c = g;
    for (; c + 3 * G < nc; c += 4 * G) {
      f32x4 xa[4], wa[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xa[u] = xv[c + u * G];
        wa[u] = wv[c + u * G];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[u] = fmaf(xa[u][i], wa[u][i], z[u]);
    }
    for (; c < nc; c += G) {
      const f32x4 xa = xv[c], wa = wv[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[0] = fmaf(xa[i], wa[i], z[0]);
    }
  } else if (bf16) {
    const uint16_t* xr = static_cast<const uint16_t*>(x_row);
    const uint16_t* ws = static_cast<const uint16_t*>(w);
    for (int d = g; d < D; d += G) z[0] = fmaf(bf16_to_f32(xr[d]), bf16_to_f32(ws[d]), z[0]);
  } else {
    const float* xr = static_cast<const float*>(x_row);
    const float* ws = static_cast<const float*>(w);
    for (int d = g; d < D; d += G) z[0] = fmaf(xr[d], ws[d], z[0]);
  }
  return (z[0] + z[1]) + (z[2] + z[3]);
}

__device__ __forceinline__ const void* x_row_of(const RouteArgs& a, int64_t n) {
  return static_cast<const char*>(a.x) + n * a.D * (a.bf16 ? 2 : 4);
}

// Softmax, top-k and outputs for token rows [0, n_rows) of a workgroup whose logits sit in
// s_logit[t * cols + e]. sel_p / sel_e: per-wave scratch of 512 entries each. A lane holds
// experts lane + 64 j, j < 2 EP (E <= 128 EP).
template <int EP>
__device__ void route_select(const RouteArgs& a, const float* s_logit, int cols, int64_t n0, int n_rows,
                             float* sel_p_all, int* sel_e_all, int nw = 4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, D = a.D, k = a.k;
  float* sel_p = sel_p_all + wave * 512;
  int* sel_e = sel_e_all + wave * 512;
  for (int t = wave; t < n_rows; t += nw) {
    const int64_t n = n0 + t;
    constexpr int kPer = 2 * EP;
    float v[kPer];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane + kWave * j;
      v[j] = e < E ? s_logit[t * cols + e] : -INFINITY;
      m = fmaxf(m, v[j]);
    }
    if (a.sigmoid) {                             // selection keys: sigmoid(logit) + bias
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? 1.f / (1.f + expf(-v[j])) + (a.bias ? a.bias[e] : 0.f) : -INFINITY;
      }
    } else {
      m = wave_max_dpp(m);
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? expf(v[j] - m) : 0.f;
        s += v[j];
      }
      s = wave_sum_dpp(s);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? v[j] / s : -INFINITY;    // probabilities; -inf marks "not a candidate"
      }
    }
    if (a.logits) {
      for (int e = lane; e < E; e += kWave) a.logits[n * E + e] = s_logit[t * cols + e];
    }
    float kept_sum = 0.f;
    for (int r = 0; r < k; ++r) {
      float bp = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {          // strict '>' keeps the lowest index of a lane
        if (v[j] > bp) { bp = v[j]; be = lane + kWave * j; }
      }
      wave_argmax_dpp(bp, be);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (lane + kWave * j == be) v[j] = -INFINITY;
      // the weight: the probability, or the unbiased sigmoid score of the picked expert
      const float w = a.sigmoid ? 1.f / (1.f + expf(-s_logit[t * cols + be])) : bp;
      kept_sum += w;                             // slot order, identical in every lane
      if (lane == 0) { sel_p[r] = w; sel_e[r] = be; }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int r = lane; r < k; r += kWave) {
      const float p = sel_p[r];
      a.weights[n * k + r] = a.norm ? p / kept_sum : p;
      a.experts[n * k + r] = sel_e[r];
    }
    if (a.w_shared_gate) {
      float z = row_dot_part<kWave>(x_row_of(a, n), a.w_shared_gate, D, a.bf16, lane);
      z = wave_sum_dpp(z);
      if (lane == 0) a.shared_scale[n] = 1.f / (1.f + expf(-z));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Selection with 16 lanes per token (E <= 128, k <= 8): lane j of a token's group holds experts
// j + 16 i, i < 8, sorts its eight (p, e) pairs, then four xor rounds merge pairs of sorted lists
// (top 8 of the union: elementwise best of one list against the other reversed, a bitonic sequence,
// then a 3-stage bitonic merge). Order: larger p first, equal p -> lower expert index, a total
// order, so every lane of the group ends with the same list. Tokens base + 4 w + g (g = lane / 16)
// of wave w; nw waves share the tile.
__device__ __forceinline__ bool sel_better(float pa, int ea, float pb, int eb) {
  return pa > pb || (pa == pb && ea < eb);
}
__device__ __forceinline__ void sel_ce(float& pa, int& ea, float& pb, int& eb) {   // (a, b) -> (better, worse)
  const bool sw = sel_better(pb, eb, pa, ea);
  const float tp = sw ? pb : pa, up = sw ? pa : pb;
  const int te = sw ? eb : ea, ue = sw ? ea : eb;
  pa = tp; ea = te; pb = up; eb = ue;
}
__device__ __forceinline__ void sel_bitonic_merge8(float* p, int* e) {                // bitonic -> sorted
#pragma unroll
  for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & d) == 0) sel_ce(p[i], e[i], p[i + d], e[i + d]);
}

template <int EP>
__device__ void route_select16(const RouteArgs& a, const float* s_logit, int cols, int64_t n0, int n_rows, int nw) {
  static_assert(EP == 1, "16-lane selection covers E <= 128");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15;
  const int E = a.E, D = a.D, k = a.k;
  for (int base = 0; base < n_rows; base += 4 * nw) {
    const int t = base + 4 * wave + (lane >> 4);
    const bool valid = t < n_rows;
    float p[8];
    int e[8];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = j + 16 * i;
      p[i] = (valid && e[i] < E) ? s_logit[t * cols + e[i]] : -INFINITY;
      m = fmaxf(m, p[i]);
    }
    if (a.sigmoid) {                                               // keys: sigmoid(logit) + bias
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = (valid && e[i] < E) ? 1.f / (1.f + expf(-p[i])) + (a.bias ? a.bias[e[i]] : 0.f) : -INFINITY;
    } else {
      m = fmaxf(m, xor16f<1>(m));
      m = fmaxf(m, xor16f<2>(m));
      m = fmaxf(m, xor16f<4>(m));
      m = fmaxf(m, xor16f<8>(m));
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = e[i] < E ? expf(p[i] - m) : 0.f;
        sum += p[i];
      }
      sum += xor16f<1>(sum);                                        // commutative pairs: same in every lane
      sum += xor16f<2>(sum);
      sum += xor16f<4>(sum);
      sum += xor16f<8>(sum);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = e[i] < E ? p[i] / sum : -INFINITY;  // -inf: never selected
    }
    // sort the lane's eight: bitonic sort (sizes 2, 4, 8)
#pragma unroll
    for (int size = 2; size <= 8; size <<= 1)
#pragma unroll
      for (int d = size >> 1; d >= 1; d >>= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int l = i ^ d;
          if (l > i) {
            if ((i & size) == 0) sel_ce(p[i], e[i], p[l], e[l]);
            else sel_ce(p[l], e[l], p[i], e[i]);
          }
        }
    // merge with the partner lists
    auto merge = [&](auto mc) {
      constexpr int M = decltype(mc)::value;
      float q[8];
      int f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        q[i] = xor16f<M>(p[i]);
        f[i] = xor16<M>(e[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (sel_better(q[7 - i], f[7 - i], p[i], e[i])) { p[i] = q[7 - i]; e[i] = f[7 - i]; }
      sel_bitonic_merge8(p, e);
    };
    merge(std::integral_constant<int, 1>{});
    merge(std::integral_constant<int, 2>{});
    merge(std::integral_constant<int, 4>{});
    merge(std::integral_constant<int, 8>{});
    if (a.sigmoid) {                              // weights: the picked experts' unbiased scores
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < k && valid) p[r] = 1.f / (1.f + expf(-s_logit[t * cols + e[r]]));
    }
    float kept = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < k) kept += p[r];                                       // slot order, same in every lane
    if (valid) {
      const int64_t n = n0 + t;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r == j && r < k) {
          a.weights[n * k + r] = a.norm ? p[r] / kept : p[r];
          a.experts[n * k + r] = e[r];
        }
      if (a.logits) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (j + 16 * i < E) a.logits[n * E + j + 16 * i] = s_logit[t * cols + j + 16 * i];
      }
    }
    if (a.w_shared_gate) {                                         // 16 lanes per token
      float z = 0.f;
      if (valid) z = row_dot_part<16>(x_row_of(a, n0 + t), a.w_shared_gate, D, a.bf16, j);
      z += xor16f<1>(z);
      z += xor16f<2>(z);
      z += xor16f<4>(z);
      z += xor16f<8>(z);
      if (valid && j == 0) a.shared_scale[n0 + t] = 1.f / (1.f + expf(-z));
    }
  }
}

// E <= 128 and k <= 8 take the 16-lane selection, other shapes the per-wave one.
template <int EP>
__device__ void select_tokens(const RouteArgs& a, const float* s_logit, int cols, int64_t n0, int n_rows,
                              float* sel_p, int* sel_e, int nw) {
  if constexpr (EP == 1) {
    if (a.k <= 8) return route_select16<EP>(a, s_logit, cols, n0, n_rows, nw);
  }
  route_select<EP>(a, s_logit, cols, n0, n_rows, sel_p, sel_e, nw);
}

// ---------------------------------------------------------------------------------------------
// bf16: EP = padded experts / 128; wave w owns 32-expert blocks w + 4 b, b < EP.
// ---------------------------------------------------------------------------------------------
constexpr int kRtTok = 32;
constexpr int kRtBK = 64;

// 128-byte rows; chunk c of row r at c ^ ((r >> 1) & 7) (16 rows at one chunk -> 16 distinct slots
// of a 256-byte bank window)
__device__ __forceinline__ int rswz(int row, int chunk) { return row * kRtBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

template <int EP>
__global__ __launch_bounds__(kRouteThreads) void route_bf16_kernel(RouteArgs a) {
  constexpr int EPAD = EP * 128;
  constexpr int XS = kRtTok * kRtBK;             // elements of one x stage
  constexpr int WS = EPAD * kRtBK;               // elements of one W stage
  constexpr int STAGE_BYTES = 2 * (XS + WS) * 2;
  constexpr int LOGIT_BYTES = kRtTok * EPAD * 4;
  constexpr int SEL_BYTES = 4 * 512 * 8;
  static_assert(LOGIT_BYTES + SEL_BYTES <= STAGE_BYTES, "logits and selection scratch alias the stages");
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGE_BYTES / 2];
  uint16_t* sX = smem;                           // [2][XS]
  uint16_t* sW = smem + 2 * XS;                  // [2][WS]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRtTok;
  const int D = a.D, E = a.E;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w = static_cast<const uint16_t*>(a.w_router);

  // loaders: x: one chunk per thread (32 rows x 8 chunks); W: EP*4 chunks per thread
  constexpr int WL = EPAD * 8 / kRouteThreads;
  const int xr = tid >> 3, xc = tid & 7;
  const uint16_t* srcX = x + min<int64_t>(n0 + xr, a.N - 1) * D + xc * 8;
  const uint16_t* srcW[WL];
  int wrow[WL], wch[WL];
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int idx = tid + j * kRouteThreads;
    wrow[j] = idx >> 3;
    wch[j] = idx & 7;
    srcW[j] = w + static_cast<int64_t>(min(wrow[j], E - 1)) * D + wch[j] * 8;
  }
  u32x4 rx, rw[WL];
  auto gload = [&](int kb) {
    rx = (kb + xc * 8 < D) ? *reinterpret_cast<const u32x4*>(srcX + kb) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < WL; ++j)
      rw[j] = (kb + wch[j] * 8 < D && wrow[j] < E) ? *reinterpret_cast<const u32x4*>(srcW[j] + kb) : u32x4{0, 0, 0, 0};
  };
  auto sstore = [&](int buf) {
    *reinterpret_cast<u32x4*>(&sX[buf * XS + rswz(xr, xc)]) = rx;
#pragma unroll
    for (int j = 0; j < WL; ++j) *reinterpret_cast<u32x4*>(&sW[buf * WS + rswz(wrow[j], wch[j])]) = rw[j];
  };

  f32x16 acc[EP];
#pragma unroll
  for (int b = 0; b < EP; ++b) acc[b] = f32x16{};
  const int ksteps = (D + kRtBK - 1) / kRtBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) gload((ks + 1) * kRtBK);
#pragma unroll
    for (int kk = 0; kk < kRtBK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      const u32x4 fa = *reinterpret_cast<const u32x4*>(&sX[buf * XS + rswz(lane & 31, ch)]);
#pragma unroll
      for (int b = 0; b < EP; ++b) {
        if ((wave + 4 * b) * 32 < E) {
          const u32x4 fb = *reinterpret_cast<const u32x4*>(&sW[buf * WS + rswz((wave + 4 * b) * 32 + (lane & 31), ch)]);
          acc[b] = mfma32(fa, fb, acc[b]);
        }
      }
    }
    if (ks + 1 < ksteps) sstore(buf ^ 1);
    __syncthreads();
  }

  float* s_logit = reinterpret_cast<float*>(smem);                         // [kRtTok][EPAD]
  float* s_selp = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + LOGIT_BYTES);
  int* s_sele = reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + LOGIT_BYTES + 4 * 512 * 4);
#pragma unroll
  for (int b = 0; b < EP; ++b) {
    const int col = (wave + 4 * b) * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) s_logit[acc_row(i, lane) * EPAD + col] = acc[b][i];
  }
  __syncthreads();
  const int n_rows = static_cast<int>(min<int64_t>(kRtTok, a.N - n0));
  select_tokens<EP>(a, s_logit, EPAD, n0, n_rows, s_selp, s_sele, 4);
}


// Pipelined variant for D % 128 == 0: 32-wide k-slices go straight from global memory into four LDS
// stages (three in flight). Rows are 64 bytes; chunk c of row r sits at c ^ ((r >> 2) & 3) so the
// 16 lanes the LDS serves together hit 16 distinct 16-byte slots. One DMA instruction = 16 rows.
// Per stage each wave issues 2 EP instructions of W_r rows plus one of x rows (waves 2 and 3 repeat
// waves 0 and 1's x rows into the same place, so every wave issues the same count).
constexpr int kRsK = 32;

template <int EP, bool kPW>
__global__ __launch_bounds__(kRouteThreads) void route_stream_kernel(RouteArgs a) {
  constexpr int EPAD = EP * 128;
  constexpr int XS = kRtTok * kRsK, WS = EPAD * kRsK;    // elements per stage
  constexpr int PER_STAGE = 2 * EP + 1;
  constexpr int LOGIT_BYTES = kRtTok * EPAD * 4;
  constexpr int SEL_BYTES = 4 * 512 * 8;
  static_assert(LOGIT_BYTES + SEL_BYTES <= 4 * WS * 2, "logits and selection scratch alias the W stages");
  __shared__ __attribute__((aligned(1024))) uint16_t sW[4 * WS];   // four W stages, then logits
  __shared__ __attribute__((aligned(1024))) uint16_t sX[4 * XS];
  uint16_t *sW0 = sW, *sW1 = sW + WS, *sW2 = sW + 2 * WS, *sW3 = sW + 3 * WS;
  uint16_t *sX0 = sX, *sX1 = sX + XS, *sX2 = sX + 2 * XS, *sX3 = sX + 3 * XS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRtTok;
  const int D = a.D, E = a.E;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w = static_cast<const uint16_t*>(a.w_router);
  const int lrow = lane >> 2;
  const int lch = (lane & 3) ^ ((lrow >> 2) & 3);
  const int xg = wave & 1;                                  // x DMA group (rows 16 xg .. 16 xg + 15)
  // k-slice of this workgroup: all of D, or D / gridDim.y when the contraction is split
  const int kslice = D / static_cast<int>(gridDim.y);
  const int64_t kbase = static_cast<int64_t>(blockIdx.y) * kslice;
  const uint16_t* srcX = x + min<int64_t>(n0 + xg * 16 + lrow, a.N - 1) * D + kbase + lch * 8;
  const uint16_t* srcW[2 * EP];
#pragma unroll
  for (int q = 0; q < 2 * EP; ++q) {
    if constexpr (kPW) {                                   // 16-row block wave + 4 q: 1 KB per k-block
      const int rb = min(wave + 4 * q, E / 16 - 1);
      srcW[q] = w + (static_cast<int64_t>(rb) * (D / 32) + kbase / 32) * 512 + lane * 8;
    } else {
      const int row = (wave + 4 * q) * 16 + lrow;          // W DMA group wave + 4 q
      srcW[q] = w + static_cast<int64_t>(min(row, E - 1)) * D + kbase + lch * 8;
    }
  }
  auto issue = [&](int ks, uint16_t* sx, uint16_t* sw) {
    const int kb = ks * kRsK;
    dma16(srcX + kb, sx + xg * 512);
#pragma unroll
    for (int q = 0; q < 2 * EP; ++q) dma16(srcW[q] + (kPW ? ks * 512 : kb), sw + (wave + 4 * q) * 512);
  };
  const int ksteps = kslice / kRsK;
  constexpr int W2 = waitcnt_vm(2 * PER_STAGE), W1 = waitcnt_vm(PER_STAGE), W0 = waitcnt_vm(0);
  auto wait_stage = [&](int st) {
    const int ahead = min(2, ksteps - 1 - st);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(W2);
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(W1);
    else __builtin_amdgcn_s_waitcnt(W0);
    lds_barrier();
  };
  // packed weights: a 16-row group's 1 KB holds (row r16, 8-wide k chunk q) at (r16 + 16 q) * 8
  int ko[2], kob[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    ko[kk] = (lane & 31) * kRsK + (((2 * kk + (lane >> 5)) ^ ((lane >> 2) & 3)) << 3);
    kob[kk] = kPW ? ((lane >> 4) & 1) * 512 + (lane & 15) * 8 + (2 * kk + (lane >> 5)) * 128 : ko[kk];
  }
  f32x16 acc[EP];
#pragma unroll
  for (int b = 0; b < EP; ++b) acc[b] = f32x16{};
  auto compute = [&](const uint16_t* sx, const uint16_t* sw) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 fa = *reinterpret_cast<const u32x4*>(&sx[ko[kk]]);
#pragma unroll
      for (int b = 0; b < EP; ++b) {
        if ((wave + 4 * b) * 32 < E) {
          const u32x4 fb = *reinterpret_cast<const u32x4*>(&sw[(wave + 4 * b) * 32 * kRsK + kob[kk]]);
          acc[b] = mfma32(fa, fb, acc[b]);
        }
      }
    }
  };
  issue(0, sX0, sW0);
  issue(1, sX1, sW1);
  issue(2, sX2, sW2);
  for (int ks = 0; ks < ksteps; ks += 4) {
    wait_stage(ks);
    if (ks + 3 < ksteps) issue(ks + 3, sX3, sW3);
    compute(sX0, sW0);
    wait_stage(ks + 1);
    if (ks + 4 < ksteps) issue(ks + 4, sX0, sW0);
    compute(sX1, sW1);
    wait_stage(ks + 2);
    if (ks + 5 < ksteps) issue(ks + 5, sX1, sW1);
    compute(sX2, sW2);
    wait_stage(ks + 3);
    if (ks + 6 < ksteps) issue(ks + 6, sX2, sW2);
    compute(sX3, sW3);
  }
  if (gridDim.y > 1) {
    // split contraction: this slice's partial logits go to partial[blockIdx.y][n][e]
    float* part = a.partial + static_cast<int64_t>(blockIdx.y) * a.N * E;
#pragma unroll
    for (int b = 0; b < EP; ++b) {
      const int col = (wave + 4 * b) * 32 + (lane & 31);
      if (col < E) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t n = n0 + acc_row(i, lane);
          if (n < a.N) part[n * E + col] = acc[b][i];
        }
      }
    }
    return;
  }
  __syncthreads();                                          // all reads of the stages are done
  float* s_logit = reinterpret_cast<float*>(sW);
  float* s_selp = reinterpret_cast<float*>(reinterpret_cast<char*>(sW) + LOGIT_BYTES);
  int* s_sele = reinterpret_cast<int*>(reinterpret_cast<char*>(sW) + LOGIT_BYTES + 4 * 512 * 4);
#pragma unroll
  for (int b = 0; b < EP; ++b) {
    const int col = (wave + 4 * b) * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) s_logit[acc_row(i, lane) * EPAD + col] = acc[b][i];
  }
  __syncthreads();
  const int n_rows = static_cast<int>(min<int64_t>(kRtTok, a.N - n0));
  select_tokens<EP>(a, s_logit, EPAD, n0, n_rows, s_selp, s_sele, 4);
}


// x-stationary variant for long batches (bf16, D % 512 == 0, D <= 2048): the workgroup's 32
// token rows (up to 128 KB) move into LDS once, with 1 KB contiguous DMA instructions, and the
// router weights (shared by every token tile, so L2-resident) stream from global memory straight
// into matrix-core fragments, U k-steps of loads in flight. No partial logits and no second pass.
// Eight waves: wave w takes expert blocks (w % 4) + 4 b over half h = w / 4 of the contraction;
// the halves are added in the order h = 0 + h = 1. LDS: 16-byte chunk c of row r sits at
// c ^ (r & 15), so the 16 rows one ds_read_b128 serves together hit 16 distinct bank slots.
// Long batches: the shared-expert gate of each token of the x tile, from the tile in LDS (chunk c
// of row r at c ^ (r & 15)) and w_s in 16-byte chunks; one wave per token. Called while every wave
// still reads the tile.
__device__ void xs_shared_gate(const RouteArgs& a, const uint16_t* sX, int64_t n0, int n_rows, int nw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, D = a.D, nc = D >> 3;
  const u32x4* ws = static_cast<const u32x4*>(a.w_shared_gate);
  for (int t = wave; t < n_rows; t += nw) {
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = lane; c0 < nc; c0 += 4 * kWave) {
      u32x4 xa[4], wa[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = min(c0 + u * kWave, nc - 1);
        xa[u] = *reinterpret_cast<const u32x4*>(&sX[t * D + ((c ^ (t & 15)) << 3)]);
        wa[u] = ws[c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c0 + u * kWave >= nc) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[u] = fmaf(__uint_as_float(xa[u][i] << 16), __uint_as_float(wa[u][i] << 16), z[u]);
          z[u] = fmaf(__uint_as_float(xa[u][i] & 0xffff0000u), __uint_as_float(wa[u][i] & 0xffff0000u), z[u]);
        }
      }
    }
    const float zz = wave_sum_dpp((z[0] + z[1]) + (z[2] + z[3]));
    if (lane == 0) a.shared_scale[n0 + t] = 1.f / (1.f + expf(-zz));
  }
}

constexpr int kXsMaxD = 2048;
constexpr int kXsThreads = 512;

template <int EP, bool kPW>
__global__ __launch_bounds__(kXsThreads) void route_xs_kernel(RouteArgs a) {
  constexpr int EPAD = EP * 128;
  constexpr int U = EP <= 2 ? 8 : 4;                        // k-steps per load batch
  constexpr int HI_FLOATS = 4 * EP * 16 * 64;               // upper-half accumulators of waves 4..7
  static_assert(HI_FLOATS * 4 <= kRtTok * kXsMaxD * 2, "upper-half sums alias the x tile");
  static_assert(kRtTok * EPAD * 4 + 2 * 8 * 512 * 4 <= kRtTok * kXsMaxD * 2, "logits alias the x tile");
  __shared__ __attribute__((aligned(1024))) uint16_t sX[kRtTok * kXsMaxD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eg = wave & 3, kh = wave >> 2;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRtTok;
  const int D = a.D, E = a.E;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w = static_cast<const uint16_t*>(a.w_router);
  // x tile: instruction i covers row i / IPR, 16-byte chunks 64 (i % IPR) .. + 63 of it
  const int IPR = D / 512;
  for (int i = wave; i < kRtTok * IPR; i += kXsThreads / 64) {
    const int r = i / IPR, q = i - r * IPR;
    const int64_t n = min<int64_t>(n0 + r, a.N - 1);
    dma16(x + n * D + (64 * q + (lane ^ (r & 15))) * 8, sX + r * D + q * 512);
  }
  // weight rows of this wave's blocks; lane: row lane % 32, k-group lane / 32; k from kh * D / 2
  const int ks0 = kh * (D / 32);                            // first 16-wide k-step of this half
  // packed weights: row e's 16-wide k-step s sits in block (e / 16, s / 2) at slot
  // e % 16 + 16 (2 (s % 2) + lane / 32)
  const uint16_t* wp[EP];
#pragma unroll
  for (int b = 0; b < EP; ++b) {
    if constexpr (kPW) {
      const int rb = min((eg + 4 * b) * 2 + ((lane >> 4) & 1), E / 16 - 1);
      wp[b] = w + static_cast<int64_t>(rb) * (D / 32) * 512 + ((lane & 15) + 16 * (lane >> 5)) * 8;
    } else {
      wp[b] = w + static_cast<int64_t>(min((eg + 4 * b) * 32 + (lane & 31), E - 1)) * D + ks0 * 16 + 8 * (lane >> 5);
    }
  }
  u32x4 fb[2][U][EP];
  auto loadw = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = ks0 + k0 + u;
#pragma unroll
      for (int b = 0; b < EP; ++b)
        if ((eg + 4 * b) * 32 < E)
          fb[buf][u][b] = *reinterpret_cast<const u32x4*>(kPW ? wp[b] + (s >> 1) * 512 + (s & 1) * 256 : wp[b] + (k0 + u) * 16);
    }
  };
  f32x16 acc[EP];
#pragma unroll
  for (int b = 0; b < EP; ++b) acc[b] = f32x16{};
  const int arow = (lane & 31) * D;
  auto math = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (2 * (ks0 + k0 + u) + (lane >> 5)) ^ (lane & 15);
      const u32x4 fa = *reinterpret_cast<const u32x4*>(&sX[arow + c * 8]);
#pragma unroll
      for (int b = 0; b < EP; ++b)
        if ((eg + 4 * b) * 32 < E) acc[b] = mfma32(fa, fb[buf][u][b], acc[b]);
    }
  };
  loadw(0, 0);
  __builtin_amdgcn_s_waitcnt(0);                            // the x tile (and the first weights) landed
  __syncthreads();
  const int full = D / 32 / U;                              // batches per half; even: D % 512 == 0, U <= 8
  for (int q = 0; q < full; q += 2) {
    if (q + 1 < full) loadw(1, (q + 1) * U);
    math(0, q * U);
    if (q + 2 < full) loadw(0, (q + 2) * U);
    math(1, (q + 1) * U);
  }
  const int n_rows = static_cast<int>(min<int64_t>(kRtTok, a.N - n0));
  const bool gate_here = a.w_shared_gate && (reinterpret_cast<uintptr_t>(a.w_shared_gate) & 15) == 0;
  if (gate_here) xs_shared_gate(a, sX, n0, n_rows, kXsThreads / 64);
  __syncthreads();                                          // every wave is done reading the x tile
  float* hi = reinterpret_cast<float*>(sX);
  if (kh == 1) {
#pragma unroll
    for (int b = 0; b < EP; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) hi[((eg * EP + b) * 16 + i) * 64 + lane] = acc[b][i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int b = 0; b < EP; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] += hi[((eg * EP + b) * 16 + i) * 64 + lane];
  }
  __syncthreads();                                          // the upper-half sums are consumed
  float* s_logit = reinterpret_cast<float*>(sX);            // [kRtTok][EPAD]
  float* s_selp = s_logit + kRtTok * EPAD;
  int* s_sele = reinterpret_cast<int*>(s_selp + 8 * 512);
  if (kh == 0) {
#pragma unroll
    for (int b = 0; b < EP; ++b) {
      const int col = (eg + 4 * b) * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) s_logit[acc_row(i, lane) * EPAD + col] = acc[b][i];
    }
  }
  __syncthreads();
  RouteArgs sel = a;
  if (gate_here) sel.w_shared_gate = nullptr;               // the gate is done
  select_tokens<EP>(sel, s_logit, EPAD, n0, n_rows, s_selp, s_sele, kXsThreads / 64);
}

// E <= 128: the same x tile with 16x16x32 matrix-core steps. Wave w owns experts 16 w .. + 15
// over the whole contraction and both 16-token halves of the tile; its weight loads are 16 rows x
// 64 bytes, so the lines it reuses over consecutive k-steps (16 x 128 bytes) stay in L1.
template <int U, bool kPW>
__global__ __launch_bounds__(kXsThreads) void route_xs16_kernel(RouteArgs a) {
  constexpr int EPAD = 128;
  static_assert(kRtTok * EPAD * 4 <= kRtTok * kXsMaxD * 2, "logits alias the x tile");
  __shared__ __attribute__((aligned(1024))) uint16_t sX[kRtTok * kXsMaxD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRtTok;
  const int D = a.D, E = a.E;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w = static_cast<const uint16_t*>(a.w_router);
  const int IPR = D / 512;
  for (int i = wave; i < kRtTok * IPR; i += kXsThreads / 64) {
    const int r = i / IPR, q = i - r * IPR;
    const int64_t n = min<int64_t>(n0 + r, a.N - 1);
    dma16(x + n * D + (64 * q + (lane ^ (r & 15))) * 8, sX + r * D + q * 512);
  }
  const bool active = wave * 16 < E;                        // uniform
  // packed weights: block (wave, s) is this wave's 16 rows at k-step s, 1 KB in lane order
  const uint16_t* wp = kPW ? w + static_cast<int64_t>(min(wave, E / 16 - 1)) * (D / 32) * 512 + lane * 8
                           : w + static_cast<int64_t>(min(wave * 16 + (lane & 15), E - 1)) * D + 8 * (lane >> 4);
  u32x4 fb[2][U];
  auto loadw = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (active) fb[buf][u] = *reinterpret_cast<const u32x4*>(wp + (k0 + u) * (kPW ? 512 : 32));
  };
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const int r0 = lane & 15;                                 // token of this lane in each half
  auto math = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (4 * (k0 + u) + (lane >> 4)) ^ r0;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const u32x4 fa = *reinterpret_cast<const u32x4*>(&sX[(tb * 16 + r0) * D + c * 8]);
        if (active) acc[tb] = mfma16(fa, fb[buf][u], acc[tb]);
      }
    }
  };
  loadw(0, 0);
  __builtin_amdgcn_s_waitcnt(0);                            // the x tile (and the first weights) landed
  __syncthreads();
  const int full = D / 32 / U;                              // even: D % 512 == 0, U <= 8
  for (int q = 0; q < full; q += 2) {
    if (q + 1 < full) loadw(1, (q + 1) * U);
    math(0, q * U);
    if (q + 2 < full) loadw(0, (q + 2) * U);
    math(1, (q + 1) * U);
  }
  const int n_rows = static_cast<int>(min<int64_t>(kRtTok, a.N - n0));
  const bool gate_here = a.w_shared_gate && (reinterpret_cast<uintptr_t>(a.w_shared_gate) & 15) == 0;
  if (gate_here) xs_shared_gate(a, sX, n0, n_rows, kXsThreads / 64);
  __syncthreads();                                          // every wave is done reading the x tile
  float* s_logit = reinterpret_cast<float*>(sX);            // [kRtTok][EPAD]
  if (active) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_logit[(tb * 16 + 4 * (lane >> 4) + i) * EPAD + wave * 16 + (lane & 15)] = acc[tb][i];
  }
  __syncthreads();
  RouteArgs sel = a;
  if (gate_here) sel.w_shared_gate = nullptr;               // the gate is done
  route_select16<1>(sel, s_logit, EPAD, n0, n_rows, kXsThreads / 64);
}

// Long bf16 batches with a suitable width take the x-stationary kernel (one workgroup per CU, so
// it wants at least a round of tiles).
static bool route_xs_ok(int64_t N, int D, bool bf16) {
  return bf16 && D % 512 == 0 && D <= kXsMaxD && N >= 8192;
}

// Second pass of a split contraction: logits[n][e] = sum over slices s = 0, 1, ... of
// partial[s][n][e], added in slice order (deterministic), then the same selection as the fused
// path. TOK tokens per workgroup; every thread issues all its loads (up to MS slices of each of
// its entries) before adding anything, so a workgroup's loads are in flight together.
template <int EP, int TOK, int MS>
__global__ __launch_bounds__(kRouteThreads) void route_finish_kernel(RouteArgs a, int n_slices) {
  constexpr int EPAD = EP * 128;
  constexpr int PER = (TOK * EPAD + kRouteThreads - 1) / kRouteThreads;
  __shared__ float s_logit[TOK * EPAD];
  __shared__ float s_selp[4 * 512];
  __shared__ int s_sele[4 * 512];
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * TOK;
  const int E = a.E;
  const int n_rows = static_cast<int>(min<int64_t>(TOK, a.N - n0));
  const int64_t slice_stride = a.N * E;
  float v[PER][MS];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int idx = threadIdx.x + q * kRouteThreads;
    const int t = idx / EPAD, e = idx - t * EPAD;
    const bool ok = t < n_rows && e < E;
    const float* p = a.partial + (n0 + t) * E + e;
#pragma unroll
    for (int sl = 0; sl < MS; ++sl) v[q][sl] = (ok && sl < n_slices) ? p[sl * slice_stride] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int idx = threadIdx.x + q * kRouteThreads;
    const int t = idx / EPAD, e = idx - t * EPAD;
    if (t < TOK) {
      float sum = v[q][0];
#pragma unroll
      for (int sl = 1; sl < MS; ++sl)
        if (sl < n_slices) sum += v[q][sl];
      s_logit[t * EPAD + e] = sum;
    }
  }
  __syncthreads();
  select_tokens<EP>(a, s_logit, EPAD, n0, n_rows, s_selp, s_sele, 4);
}

// ---------------------------------------------------------------------------------------------
// fp32: FMA dot products, 64 tokens per workgroup.
// ---------------------------------------------------------------------------------------------
template <int EP>
__global__ __launch_bounds__(kRouteThreads) void route_f32_kernel(RouteArgs a) {
  constexpr int kTok = 64;
  constexpr int EPAD = EP * 128;
  __shared__ float s_logit[kTok * EPAD];
  __shared__ float s_selp[4 * 512];
  __shared__ int s_sele[4 * 512];
  const int tid = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int D = a.D, E = a.E;
  const float* x = static_cast<const float*>(a.x);
  const float* w = static_cast<const float*>(a.w_router);
  for (int idx = tid; idx < kTok * E; idx += kRouteThreads) {
    const int t = idx / E, e = idx - t * E;
    const int64_t n = min<int64_t>(n0 + t, a.N - 1);
    const f32x4* xv = reinterpret_cast<const f32x4*>(x + n * D);
    const f32x4* wv = reinterpret_cast<const f32x4*>(w + static_cast<int64_t>(e) * D);
    float s = 0.f;
    for (int d = 0; d < D / 4; ++d) {
      const f32x4 u = xv[d], v = wv[d];
      s = fmaf(u[0], v[0], s);
      s = fmaf(u[1], v[1], s);
      s = fmaf(u[2], v[2], s);
      s = fmaf(u[3], v[3], s);
    }
    s_logit[t * EPAD + e] = s;
  }
  __syncthreads();
  const int n_rows = static_cast<int>(min<int64_t>(kTok, a.N - n0));
  select_tokens<EP>(a, s_logit, EPAD, n0, n_rows, s_selp, s_sele, 4);
}

// Slices of the contraction: each workgroup walks D / slices columns in 32-wide stages with three
// stages in flight, so with few token tiles the walk is latency-bound; splitting D over more
// workgroups shortens it. Aim for about 2048 workgroups; each slice keeps >= 128 columns (four
// stages). Needs the partial-logit scratch (slices * N * E fp32).
int route_slices_for(int64_t N, int D, int E, bool bf16) {
  if (!bf16 || D % (4 * kRsK) != 0 || route_xs_ok(N, D, bf16)) return 1;
  const int64_t tiles = (N + kRtTok - 1) / kRtTok;
  int s = 1;
  const int64_t slice_bytes = N * E * 4;         // partial logits of one slice; keep all <= 32 MiB
  while (s * 2 * tiles <= 2048 && (D % (2 * s * 4 * kRsK)) == 0 && 2 * s <= kMaxRouteSlices &&
         2 * s * slice_bytes <= (32ll << 20))
    s *= 2;
  return s;
}

int route_slices(const RouteArgs& a) { return a.partial ? route_slices_for(a.N, a.D, a.E, a.bf16) : 1; }

// Long batches with many experts (the x-stationary range, E > 128): the logits are one dense
// product x W_r^T on the matrix cores (the grouped GEMM's down form with one group: K = D, output
// width E, fp32), written to the scratch and read back by the selection (route_finish_kernel with
// one slice). Each x-stationary workgroup would read all of W_r from L2 (N / 32 times 2 E D bytes);
// 256 x 256 tiles read it N / 256 times and keep the matrix cores fed.
static bool route_gemm_ok(int64_t N, int D, int E, bool bf16) { return route_xs_ok(N, D, bf16) && E > 128; }

int64_t route_scratch_floats(int64_t N, int D, int E, bool bf16) {
  if (route_gemm_ok(N, D, E, bf16)) return N * E;
  const int slices = route_slices_for(N, D, E, bf16);
  return slices > 1 ? slices * N * E : 0;
}

template <int EP, bool kPW>
static void launch_route_bf16(const RouteArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((a.N + kRtTok - 1) / kRtTok);
  const int slices = route_slices(a);
  if (a.partial && route_gemm_ok(a.N, a.D, a.E, a.bf16)) {
    GemmArgs g{};
    g.x = a.x;
    g.w = a.w_router;
    g.out = a.partial;
    g.max_rows = a.N;
    g.G = 1;
    g.D = a.E;                              // output width
    g.I = a.D;                              // contraction
    g.bf16 = true;
    g.packed = kPW;
    launch_down(g, st);
    constexpr int TOK = EP <= 2 ? 16 : 4;
    route_finish_kernel<EP, TOK, 1><<<static_cast<unsigned>((a.N + TOK - 1) / TOK), kRouteThreads, 0, st>>>(a, 1);
    return;
  }
  if (route_xs_ok(a.N, a.D, a.bf16)) {
    if (EP == 1 && a.k <= 8)
      route_xs16_kernel<8, kPW><<<grid, kXsThreads, 0, st>>>(a);
    else
      route_xs_kernel<EP, kPW><<<grid, kXsThreads, 0, st>>>(a);
  } else if (slices > 1) {
    route_stream_kernel<EP, kPW><<<dim3(grid, slices), kRouteThreads, 0, st>>>(a);
    if (slices <= 4 && a.N >= 1024) {       // long batches: few slices, many tokens per workgroup
      constexpr int TOK = EP <= 2 ? 16 : 4;
      route_finish_kernel<EP, TOK, 4><<<static_cast<unsigned>((a.N + TOK - 1) / TOK), kRouteThreads, 0, st>>>(a, slices);
    } else {                                 // short batches: many slices, two tokens per workgroup
      route_finish_kernel<EP, 2, kMaxRouteSlices><<<static_cast<unsigned>((a.N + 1) / 2), kRouteThreads, 0, st>>>(a, slices);
    }
  } else if (a.D % (4 * kRsK) == 0) {
    route_stream_kernel<EP, kPW><<<grid, kRouteThreads, 0, st>>>(a);
  } else if constexpr (!kPW) {              // packed weights always have D % 128 == 0
    route_bf16_kernel<EP><<<grid, kRouteThreads, 0, st>>>(a);
  }
}

template <int EP>
static void launch_route_ep(const RouteArgs& a, hipStream_t st) {
  if (a.bf16) {
    if (a.packed) launch_route_bf16<EP, true>(a, st);
    else launch_route_bf16<EP, false>(a, st);
  } else {
    const unsigned grid = static_cast<unsigned>((a.N + 63) / 64);
    route_f32_kernel<EP><<<grid, kRouteThreads, 0, st>>>(a);
  }
}

void launch_route(const RouteArgs& a, hipStream_t st) {
  switch ((a.E + 127) / 128) {
    case 1: launch_route_ep<1>(a, st); break;
    case 2: launch_route_ep<2>(a, st); break;
    case 3: launch_route_ep<3>(a, st); break;
    default: launch_route_ep<4>(a, st); break;
  }
}

}  // namespace moe
