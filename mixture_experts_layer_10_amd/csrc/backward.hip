// Backward pass of the MoE block ("Qwen3-VL + MoE: train to deploy", section "What a mixture-of-
// experts layer is": router and experts trained through the gated sum). For L = sum(dy * y):
//   experts   z = [a | b] = X_p GU_e^T, h = silu(a) b, dhu = dy[token] Dn_e, dh = w dhu,
//             da = dh b silu'(a), db = dh silu(a), dw = dhu . h (= dy . expert output),
//             dx_rows = [da | db] GU_e, dDn_e = sum_p (w dy)^T h, dGU_e = sum_p [da | db]^T X_p
//   router    dp_sel = (dw - sum_j dw_j w_j) / S (renormalised) or dw, dlogit = p (dp - sum p dp),
//             dW_r = dlogit^T x, dx += dlogit W_r
// The contractions over D, I or E run on the grouped GEMM kernels in their [out, in] form; for bf16
// layers dh and dx read the weights in their stored [K][N] layout (gemm_kstream_kernel for short
// groups, the streaming GEMM's LDS-transpose mode for tall ones), other shapes use transposed weight
// copies. The experts' weight gradients, whose contraction runs over each expert's rows, read those
// rows in place (gemm_wgrad_rows_kernel, bf16 with D and I multiples of 8); the other weight
// gradients use gemm_wgrad_kernel on transposed activation copies whose per-group row ranges are
// padded to multiples of 64 with zeros. For tall groups the SwiGLU backward (h, da, db, dw) runs in
// the epilogue of the recomputed gate_up product (grouped_gemm.hip) and dw_sum_kernel adds its
// per-block partials; otherwise swiglu_bwd_kernel does it from z. This file holds those kernels,
// the transposes and the elementwise steps.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kTT = 64;          // transpose tile

// 16-byte chunks of a row of T (bf16 bits or fp32 bits) <-> its CH elements.
template <typename T> struct Chunk {
  static constexpr int CH = 16 / static_cast<int>(sizeof(T));
  __device__ static void unpack(u32x4 v, T* e) {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      e[i] = sizeof(T) == 2 ? static_cast<T>(v[i >> 1] >> (16 * (i & 1))) : static_cast<T>(v[i]);
  }
  __device__ static u32x4 pack(const T* e) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = sizeof(T) == 2 ? (static_cast<uint32_t>(e[2 * i]) | (static_cast<uint32_t>(e[2 * i + 1]) << 16))
                            : static_cast<uint32_t>(e[i]);
    return v;
  }
};

// out[g][c][r] = in[g][r][c] for r < R, 0 for R <= r < Rp (T = bf16 or fp32 bits). One 64 x 64
// tile per workgroup; rows of 16-byte chunks both ways, staged through LDS with a pad per row.
template <typename T>
__global__ __launch_bounds__(256) void transpose_mat_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                            int R, int C, int Rp) {
  constexpr int CH = Chunk<T>::CH, NC = kTT / CH;
  __shared__ T s[kTT][kTT + 2];
  const int64_t g = blockIdx.z;
  const int r0 = blockIdx.y * kTT, c0 = blockIdx.x * kTT, tid = threadIdx.x;
  const T* src = in + g * R * static_cast<int64_t>(C);
  for (int t = tid; t < kTT * NC; t += 256) {
    const int rr = t / NC, ch = (t % NC) * CH;
    const int r = r0 + rr, c = c0 + ch;
    u32x4 v = {0, 0, 0, 0};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(r) * C + c);
    Chunk<T>::unpack(v, &s[rr][ch]);
  }
  __syncthreads();
  T* dst = out + g * C * static_cast<int64_t>(Rp);
  for (int t = tid; t < kTT * NC; t += 256) {
    const int cc = t / NC, ch = (t % NC) * CH;
    const int c = c0 + cc, r = r0 + ch;
    if (c >= C || r >= Rp) continue;
    T e[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) e[i] = s[ch + i][cc];
    *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(c) * Rp + r) = Chunk<T>::pack(e);
  }
}

void launch_transpose_mat(const void* in, void* out, int64_t G, int R, int C, int Rp, bool f32, hipStream_t st) {
  if (G <= 0 || R <= 0 || C <= 0) return;
  dim3 grid((C + kTT - 1) / kTT, (Rp + kTT - 1) / kTT, static_cast<unsigned>(G));
  if (f32)
    transpose_mat_kernel<uint32_t><<<grid, 256, 0, st>>>(static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out), R, C, Rp);
  else
    transpose_mat_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, C, Rp);
}

// Per-expert row ranges padded to multiples of 64: poff[g] = sum_{g' < g} roundup(counts[g'], 64).
__global__ __launch_bounds__(512) void pad_offsets_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ poff, int G) {
  __shared__ int s_wave[8];
  const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
  const int v = g < G ? (counts[g] + 63) / 64 * 64 : 0;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  if (g < G) poff[g] = before + inc - v;
  if (g == G - 1) poff[G] = before + inc;
}

void launch_pad_offsets(const int32_t* counts, int32_t* poff, int G, hipStream_t st) {
  pad_offsets_kernel<<<1, 512, 0, st>>>(counts, poff, G);
}

// out[m][q] for the padded row space q in [0, qtot): row q of group g (poff[g] <= q < poff[g+1]) is
// sorted row p = off[g] + q - poff[g] if that lies inside the group, else zero. The source row is
// token_of[p] when gathering, the value is scaled by scale[p] when given (rounded to bf16 once).
// With off == nullptr there is one group of n1 rows padded to qtot.
template <typename T>
__global__ __launch_bounds__(256) void transpose_rows_kernel(const T* __restrict__ src, int M,
                                                             const int32_t* __restrict__ gather,
                                                             const float* __restrict__ scale,
                                                             const int32_t* __restrict__ off,
                                                             const int32_t* __restrict__ poff, int G, int n1,
                                                             int64_t qmax, T* __restrict__ out, int64_t ld) {
  constexpr int CH = Chunk<T>::CH, NC = kTT / CH;
  __shared__ T s[kTT][kTT + 2];
  __shared__ int s_src[kTT];
  __shared__ float s_scl[kTT];
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * kTT;
  const int m0 = blockIdx.y * kTT, tid = threadIdx.x;
  const int64_t qtot = off ? poff[G] : qmax;
  if (q0 >= qtot) return;
  if (tid < kTT) {
    const int64_t q = q0 + tid;
    int64_t p = -1;
    if (q < qtot) {
      if (off) {
        int lo = 0, hi = G;                           // poff[lo] <= q < poff[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (poff[mid] <= q) lo = mid; else hi = mid;
        }
        const int64_t r = q - poff[lo];
        if (r < off[lo + 1] - off[lo]) p = off[lo] + r;
      } else if (q < n1) {
        p = q;
      }
    }
    s_src[tid] = p < 0 ? -1 : (gather ? gather[p] : static_cast<int>(p));
    s_scl[tid] = p < 0 ? 0.f : (scale ? scale[p] : 1.f);
  }
  __syncthreads();
  for (int t = tid; t < kTT * NC; t += 256) {
    const int qq = t / NC, ch = (t % NC) * CH;
    const int m = m0 + ch;
    const int srow = s_src[qq];
    u32x4 v = {0, 0, 0, 0};
    if (srow >= 0 && m < M) v = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(srow) * M + m);
    if (scale) {
      const float sc = s_scl[qq];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(T) == 2) {
          const float lo = bf16_to_f32(static_cast<uint16_t>(v[i] & 0xffff)) * sc;
          const float hi = bf16_to_f32(static_cast<uint16_t>(v[i] >> 16)) * sc;
          v[i] = pack_bf16x2(lo, hi);
        } else {
          v[i] = __float_as_uint(__uint_as_float(v[i]) * sc);
        }
      }
    }
    Chunk<T>::unpack(v, &s[qq][ch]);
  }
  __syncthreads();
  for (int t = tid; t < kTT * NC; t += 256) {
    const int mm = t / NC, ch = (t % NC) * CH;
    const int m = m0 + mm;
    const int64_t q = q0 + ch;
    if (m >= M || q >= qtot) continue;
    T e[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) e[i] = s[ch + i][mm];
    *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(m) * ld + q) = Chunk<T>::pack(e);
  }
}

void launch_transpose_rows(const void* src, int M, const int32_t* gather, const float* scale, const int32_t* off,
                           const int32_t* poff, int G, int n1, int64_t qmax, void* out, int64_t ld, bool f32, hipStream_t st) {
  if (qmax <= 0 || M <= 0) return;
  dim3 grid(static_cast<unsigned>((qmax + kTT - 1) / kTT), (M + kTT - 1) / kTT);
  if (f32)
    transpose_rows_kernel<uint32_t><<<grid, 256, 0, st>>>(static_cast<const uint32_t*>(src), M, gather, scale, off, poff, G,
                                                          n1, qmax, static_cast<uint32_t*>(out), ld);
  else
    transpose_rows_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(src), M, gather, scale, off, poff, G,
                                                          n1, qmax, static_cast<uint16_t*>(out), ld);
}

// w_perm[slot_pos[a]] = weights[a], assign_of[slot_pos[a]] = a; ones[a] = 1.
__global__ __launch_bounds__(256) void scatter_assign_kernel(const int32_t* __restrict__ slot_pos, const float* __restrict__ weights,
                                                             float* __restrict__ w_perm, int32_t* __restrict__ assign_of,
                                                             float* __restrict__ ones, int64_t A) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= A) return;
  const int p = slot_pos[a];
  w_perm[p] = weights[a];
  assign_of[p] = static_cast<int32_t>(a);
  ones[a] = 1.f;
}

void launch_scatter_assign(const int32_t* slot_pos, const float* weights, float* w_perm, int32_t* assign_of, float* ones,
                           int64_t A, hipStream_t st) {
  if (A <= 0) return;
  scatter_assign_kernel<<<static_cast<unsigned>((A + 255) / 256), 256, 0, st>>>(slot_pos, weights, w_perm, assign_of, ones, A);
}

// One wave per sorted row p: from z = [a | b] (fp32) and dhu = dy[token] Dn_e (fp32):
//   h = bf16(silu(a) b)                 (the forward's rounding)
//   dw[assign_of[p]] = sum_i dhu_i h_i  (= dy . expert output; index p without assign_of)
//   dh = w dhu, da = dh b silu'(a), db = dh silu(a) -> dab = bf16([da | db])
// Rows at or past *n_rows (when given) are skipped.
// kF32: fp32 layers keep h, da and db in fp32 (no rounding).
template <bool kF32>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ z, const float* __restrict__ dhu,
                                                         const float* __restrict__ w_perm, const int32_t* __restrict__ assign_of,
                                                         const int32_t* __restrict__ n_rows, int64_t A, int I,
                                                         void* __restrict__ h_out, void* __restrict__ dab_out,
                                                         float* __restrict__ dw) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (p >= A || (n_rows && p >= *n_rows)) return;
  const int lane = threadIdx.x & 63;
  const float w = w_perm[p];
  const float* zp = z + p * 2 * I;
  const float* dp = dhu + p * I;
  float dot = 0.f;
  for (int i = lane * 4; i < I; i += 256) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(zp + i);
    const f32x4 bv = *reinterpret_cast<const f32x4*>(zp + I + i);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(dp + i);
    float hh[4], da[4], db[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a = av[t], b = bv[t];
      const float s = 1.0f / (1.0f + __expf(-a));
      hh[t] = kF32 ? a * s * b : bf16_to_f32(f32_to_bf16(a * s * b));
      dot = fmaf(gv[t], hh[t], dot);
      const float dh = w * gv[t];
      da[t] = dh * b * (s * (1.0f + a * (1.0f - s)));
      db[t] = dh * a * s;
    }
    if constexpr (kF32) {
      float* h = static_cast<float*>(h_out);
      float* dab = static_cast<float*>(dab_out);
      *reinterpret_cast<f32x4*>(h + p * I + i) = f32x4{hh[0], hh[1], hh[2], hh[3]};
      *reinterpret_cast<f32x4*>(dab + p * 2 * I + i) = f32x4{da[0], da[1], da[2], da[3]};
      *reinterpret_cast<f32x4*>(dab + p * 2 * I + I + i) = f32x4{db[0], db[1], db[2], db[3]};
    } else {
      uint16_t* h = static_cast<uint16_t*>(h_out);
      uint16_t* dab = static_cast<uint16_t*>(dab_out);
      uint2 hv, dav, dbv;
      hv.x = pack_bf16x2(hh[0], hh[1]);
      hv.y = pack_bf16x2(hh[2], hh[3]);
      dav.x = pack_bf16x2(da[0], da[1]);
      dav.y = pack_bf16x2(da[2], da[3]);
      dbv.x = pack_bf16x2(db[0], db[1]);
      dbv.y = pack_bf16x2(db[2], db[3]);
      *reinterpret_cast<uint2*>(h + p * I + i) = hv;
      *reinterpret_cast<uint2*>(dab + p * 2 * I + i) = dav;
      *reinterpret_cast<uint2*>(dab + p * 2 * I + I + i) = dbv;
    }
  }
  dot = wave_sum(dot);
  if (lane == 0) dw[assign_of ? assign_of[p] : p] = dot;
}

// dw[assign_of[p]] = the sum of row p's per-block partials, in block order (one thread per row).
__global__ __launch_bounds__(256) void dw_sum_kernel(const float* __restrict__ dwp, int nb, const int32_t* __restrict__ assign_of,
                                                     int64_t A, float* __restrict__ dw) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (p >= A) return;
  float s = 0.f;
  for (int c = 0; c < nb; ++c) s += dwp[p * nb + c];
  dw[assign_of ? assign_of[p] : p] = s;
}

void launch_dw_sum(const float* dwp, int nb, const int32_t* assign_of, int64_t A, float* dw, hipStream_t st) {
  if (A <= 0) return;
  dw_sum_kernel<<<static_cast<unsigned>((A + 255) / 256), 256, 0, st>>>(dwp, nb, assign_of, A, dw);
}

void launch_swiglu_bwd(const float* z, const float* dhu, const float* w_perm, const int32_t* assign_of, const int32_t* n_rows,
                       int64_t A, int I, void* h, void* dab, float* dw, bool f32, hipStream_t st) {
  if (A <= 0) return;
  const unsigned grid = static_cast<unsigned>((A + 3) / 4);
  if (f32)
    swiglu_bwd_kernel<true><<<grid, 256, 0, st>>>(z, dhu, w_perm, assign_of, n_rows, A, I, h, dab, dw);
  else
    swiglu_bwd_kernel<false><<<grid, 256, 0, st>>>(z, dhu, w_perm, assign_of, n_rows, A, I, h, dab, dw);
}

// One wave per token: p = softmax(logits) in fp32, the gradient of the kept (renormalised) weights
// back to the logits; dlogit [N, Ep] bf16, zero in the padding columns E <= e < Ep.
template <bool kF32>
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits, const float* __restrict__ weights,
                                                         const int32_t* __restrict__ experts, const float* __restrict__ dw,
                                                         int64_t N, int E, int Ep, int k, int norm,
                                                         void* __restrict__ dlogit) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int lane = threadIdx.x & 63;
  const float* lg = logits + n * E;
  float mx = -INFINITY;
  for (int e = lane; e < E; e += 64) mx = fmaxf(mx, lg[e]);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int e = lane; e < E; e += 64) sum += __expf(lg[e] - mx);
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
  // selected weights' gradients, in slot order (every lane computes the same k-term sums)
  float S = 0.f, dww = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t a = n * k + j;
    S += __expf(lg[experts[a]] - mx) * inv;
    dww += dw[a] * weights[a];
  }
  for (int e = lane; e < Ep; e += 64) {
    float g = 0.f;
    if (e < E) {
      float dp = 0.f, t = 0.f;
      for (int j = 0; j < k; ++j) {
        const int64_t a = n * k + j;
        const float dps = norm ? (dw[a] - dww) / S : dw[a];
        const float pj = __expf(lg[experts[a]] - mx) * inv;
        t += dps * pj;
        if (experts[a] == e) dp = dps;
      }
      const float pe = __expf(lg[e] - mx) * inv;
      g = pe * (dp - t);
    }
    if constexpr (kF32) static_cast<float*>(dlogit)[n * Ep + e] = g;
    else static_cast<uint16_t*>(dlogit)[n * Ep + e] = f32_to_bf16(g);
  }
}

void launch_router_bwd(const float* logits, const float* weights, const int32_t* experts, const float* dw, int64_t N, int E,
                       int Ep, int k, int norm, void* dlogit, bool f32, hipStream_t st) {
  if (N <= 0) return;
  const unsigned grid = static_cast<unsigned>((N + 3) / 4);
  if (f32)
    router_bwd_kernel<true><<<grid, 256, 0, st>>>(logits, weights, experts, dw, N, E, Ep, k, norm, dlogit);
  else
    router_bwd_kernel<false><<<grid, 256, 0, st>>>(logits, weights, experts, dw, N, E, Ep, k, norm, dlogit);
}

// Shared-expert gate g = sigmoid(w_s . x): dz[n] = (dy[n] . s[n]) g (1 - g) in fp32, and the same
// rounded to bf16 in a zero-padded row of qpad entries (the operand of dw_s = sum_n dz[n] x[n]).
template <bool kF32>
__global__ __launch_bounds__(256) void shared_gate_bwd_kernel(const float* __restrict__ sdot, const float* __restrict__ g,
                                                              int64_t N, int64_t qpad, float* __restrict__ dz,
                                                              void* __restrict__ dz_row) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (n >= qpad) return;
  float v = 0.f;
  if (n < N) {
    v = sdot[n] * g[n] * (1.0f - g[n]);
    dz[n] = v;
  }
  if constexpr (kF32) static_cast<float*>(dz_row)[n] = v;
  else static_cast<uint16_t*>(dz_row)[n] = f32_to_bf16(v);
}

void launch_shared_gate_bwd(const float* sdot, const float* g, int64_t N, int64_t qpad, float* dz, void* dz_row, bool f32,
                            hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((qpad + 255) / 256);
  if (f32)
    shared_gate_bwd_kernel<true><<<grid, 256, 0, st>>>(sdot, g, N, qpad, dz, dz_row);
  else
    shared_gate_bwd_kernel<false><<<grid, 256, 0, st>>>(sdot, g, N, qpad, dz, dz_row);
}

// acc[n][d] += add[n][d] (+ dz[n] w_s[d] when dz is given; w_s bf16 or fp32): the shared expert's
// and its gate's input gradients joined to the router's before the final gather.
__global__ __launch_bounds__(256) void add_rows_kernel(float* __restrict__ acc, const float* __restrict__ add,
                                                       const float* __restrict__ dz, const void* __restrict__ ws,
                                                       bool ws_f32, int64_t N, int D) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= N * D) return;
  const int64_t n = i / D;
  const int d = static_cast<int>(i - n * D);
  float v = acc[i] + add[i];
  if (dz) {
    const float w = ws_f32 ? static_cast<const float*>(ws)[d] : bf16_to_f32(static_cast<const uint16_t*>(ws)[d]);
    v = fmaf(dz[n], w, v);
  }
  acc[i] = v;
}

void launch_add_rows(float* acc, const float* add, const float* dz, const void* ws, bool ws_f32, int64_t N, int D,
                     hipStream_t st) {
  const int64_t n = N * D;
  if (n <= 0) return;
  add_rows_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(acc, add, dz, ws, ws_f32, N, D);
}

// ---------------------------------------------------------------------------------------------
// Weight-gradient GEMM: out[g][m][n] = sum_q A[m][q] B[n][q] over q in [poff[g], poff[g+1]) (or
// [0, qtot) for one group), A [M][ld], B [Nn][ld] bf16 with zeros in the padding, out fp32.
// 128 x 128 tiles, four waves of 64 x 64 (2 x 2 blocks of 32 x 32), k step 64 through two LDS
// buffers (register staged), the XOR swizzle of the forward kernels. One workgroup per tile.
// ---------------------------------------------------------------------------------------------
constexpr int kWB = 128, kWK = 64;

__device__ __forceinline__ int wswz(int row, int chunk) { return row * kWK + ((chunk ^ ((row >> 1) & 7)) << 3); }

__global__ __launch_bounds__(256) void gemm_wgrad_kernel(const uint16_t* __restrict__ Am, const uint16_t* __restrict__ Bm,
                                                         int64_t ld, const int32_t* __restrict__ poff, int64_t qtot,
                                                         int M, int Nn, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kWB * kWK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kWB * kWK];
  const int g = blockIdx.z;
  const int m0 = blockIdx.y * kWB, n0 = blockIdx.x * kWB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t q0 = poff ? poff[g] : 0;
  const int64_t q1 = poff ? poff[g + 1] : qtot;
  const int ksteps = static_cast<int>((q1 - q0) / kWK);
  // four 16-byte chunks of A and of B per thread and stage: row (tid + 256 j) / 8, chunk tid % 8
  const uint16_t* srcA[4];
  const uint16_t* srcB[4];
  const int ch = tid & 7;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = (tid + 256 * j) >> 3;
    srcA[j] = Am + static_cast<int64_t>(min(m0 + rr, M - 1)) * ld + q0 + ch * 8;
    srcB[j] = Bm + static_cast<int64_t>(min(n0 + rr, Nn - 1)) * ld + q0 + ch * 8;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  u32x4 ra[4], rb[4];
  auto gload = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = *reinterpret_cast<const u32x4*>(srcA[j] + static_cast<int64_t>(ks) * kWK);
      rb[j] = *reinterpret_cast<const u32x4*>(srcB[j] + static_cast<int64_t>(ks) * kWK);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = (tid + 256 * j) >> 3;
      *reinterpret_cast<u32x4*>(&sA[buf][wswz(rr, ch)]) = ra[j];
      *reinterpret_cast<u32x4*>(&sB[buf][wswz(rr, ch)]) = rb[j];
    }
  };
  if (ksteps > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) gload(ks + 1);
#pragma unroll
    for (int kk = 0; kk < kWK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const u32x4*>(&sA[buf][wswz(wm * 64 + i * 32 + (lane & 31), c)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const u32x4*>(&sB[buf][wswz(wn * 64 + j * 32 + (lane & 31), c)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    }
    if (ks + 1 < ksteps) sstore(buf ^ 1);
    __syncthreads();
  }
  float* og = out + static_cast<int64_t>(g) * M * Nn;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= Nn) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + acc_row(e, lane);
        if (m < M) og[static_cast<int64_t>(m) * Nn + n] = acc[i][j][e];
      }
  }
}

void launch_wgrad(const uint16_t* A, const uint16_t* Bm, int64_t ld, const int32_t* poff, int64_t qtot, int G, int M, int Nn,
                  float* out, hipStream_t st) {
  if (G <= 0 || M <= 0 || Nn <= 0) return;
  dim3 grid((Nn + kWB - 1) / kWB, (M + kWB - 1) / kWB, static_cast<unsigned>(G));
  gemm_wgrad_kernel<<<grid, 256, 0, st>>>(A, Bm, ld, poff, qtot, M, Nn, out);
}

// ---------------------------------------------------------------------------------------------
// Weight-gradient GEMM on the rows in place (no transposed copies): for group g with rows
// p in [off[g], off[g+1]),
//   out[g][m][n] = sum_p bf16(s(p) Am[ra(p)][m]) * Bm[rb(p)][n],
// ra(p) = ga ? ga[p] : p, rb(p) = gb ? gb[p] : p, s(p) = scale ? scale[p] : 1 (the product rounded to
// bf16 once, as the transposed copies round it). Tiles of 256 x 256 (each of a group's rows is
// read once per 256 columns of the other operand: those re-reads, not the matrix cores, bound the
// kernel), eight waves of 128 x 64 (4 x 2 blocks of 32 x 32, each fragment read feeding 1.33
// matrix-core steps); a k-step is 32 rows, staged as [32 rows][256 columns] per operand (32-byte
// chunks swizzled by (2 row) & 7) and read with lds_tr_frag, so the fragments, and the sums in their
// k order, are those of gemm_wgrad_kernel on the zero-padded transposed copies. Two buffers take
// 64 KB. Rows past the group enter as zeros. Per step a thread moves 16 bytes of two A rows and two
// B rows; the row indices and scales of step ks + 1 are loaded during step ks - 1, the rows
// themselves during ks.
// Requires M % 8 == 0 and Nn % 8 == 0 (16-byte row pieces).
// ---------------------------------------------------------------------------------------------
constexpr int kRM = 256, kRN = 256, kRK = 32;   // rows kernel: tile M x N, rows per k-step

template <bool kGA, bool kGB, bool kScale>
__global__ __launch_bounds__(512) void gemm_wgrad_rows_kernel(WgradRowsArgs w) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kRK * kRM];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kRK * kRN];
  const int g = w.order ? w.order[blockIdx.z] : static_cast<int>(blockIdx.z);
  const int m0 = blockIdx.y * kRM, n0 = blockIdx.x * kRN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;                // wave tile: 128 of M x 64 of N
  const int64_t p0 = w.off[g];
  const int64_t cnt = static_cast<int64_t>(w.off[g + 1]) - p0;
  const int ksteps = static_cast<int>((cnt + kRK - 1) / kRK);
  // A and B: rows (tid >> 5) + 16 j (j < 2), 16-byte piece c = tid % 32 of the row's 512 bytes
  const int ca = tid & 31, cb = tid & 31;
  const int colA = min(m0 + ca * 8, w.M - 8), colB = min(n0 + cb * 8, w.Nn - 8);   // pieces past M or Nn: unused
  int soA[2], soB[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = (tid >> 5) + 16 * j;
    soA[j] = q * kRM + ((((ca >> 1) ^ ((2 * q) & 7))) << 4) + (ca & 1) * 8;
    soB[j] = q * kRN + ((((cb >> 1) ^ ((2 * q) & 7))) << 4) + (cb & 1) * 8;
  }
  // Every load is issued unconditionally (rows past the group read the group's last row, and are
  // zeroed by a select before the LDS store): loads guarded per lane compile into branches.
  int ia[2], ib[2];
  bool oka[2], okb[2], oka_st[2], okb_st[2];
  float sc[2], sc_st[2];
  auto gidx = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t q = static_cast<int64_t>(ks) * kRK + (tid >> 5) + 16 * j;
      oka[j] = q < cnt;
      const int64_t p = p0 + min(q, cnt - 1);
      ia[j] = kGA ? w.ga[p] : static_cast<int>(p);
      sc[j] = kScale ? w.scale[p] : 1.f;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t q = static_cast<int64_t>(ks) * kRK + (tid >> 5) + 16 * j;
      okb[j] = q < cnt;
      const int64_t p = p0 + min(q, cnt - 1);
      ib[j] = kGB ? w.gb[p] : static_cast<int>(p);
    }
  };
  u32x4 ra[2], rb[2];
  auto gload = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ra[j] = *reinterpret_cast<const u32x4*>(w.A + static_cast<int64_t>(ia[j]) * w.lda + colA);
      sc_st[j] = sc[j];
      oka_st[j] = oka[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      rb[j] = *reinterpret_cast<const u32x4*>(w.B + static_cast<int64_t>(ib[j]) * w.ldb + colB);
      okb_st[j] = okb[j];
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 v = ra[j];
      if constexpr (kScale) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = pack_bf16x2(bf16_to_f32(static_cast<uint16_t>(v[i] & 0xffff)) * sc_st[j],
                             bf16_to_f32(static_cast<uint16_t>(v[i] >> 16)) * sc_st[j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = oka_st[j] ? v[i] : 0u;
      *reinterpret_cast<u32x4*>(&sA[buf][soA[j]]) = v;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 u = rb[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = okb_st[j] ? u[i] : 0u;
      *reinterpret_cast<u32x4*>(&sB[buf][soB[j]]) = u;
    }
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  if (ksteps > 0) {
    gidx(0);
    gload();
    if (ksteps > 1) gidx(1);
    sstore(0);
    __syncthreads();
  }
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) {
      gload();                                  // rows of step ks + 1 (indices loaded a step ago)
      if (ks + 2 < ksteps) gidx(ks + 2);
    }
#pragma unroll
    for (int kk = 0; kk < kRK / 16; ++kk) {
      u32x4 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds_tr_frag<kRM>(sA[buf], kk, wm * 128 + i * 32, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = lds_tr_frag<kRN>(sB[buf], kk, wn * 64 + j * 32, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    }
    if (ks + 1 < ksteps) sstore(buf ^ 1);
    __syncthreads();
  }
  float* og = w.out + static_cast<int64_t>(g) * w.M * w.Nn;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= w.Nn) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 128 + i * 32 + acc_row(e, lane);
        if (m < w.M) og[static_cast<int64_t>(m) * w.Nn + n] = acc[i][j][e];
      }
  }
}

// Groups ranked by row count, largest first (ties: lower index first). Workgroups start in
// blockIdx order, so with this order the longest sums start first and the short ones fill in
// behind them, instead of a late long group running alone at the end.
__global__ __launch_bounds__(1024) void group_order_kernel(const int32_t* __restrict__ counts, int G,
                                                           int32_t* __restrict__ order) {
  __shared__ int s_c[1024];
  for (int g = threadIdx.x; g < G; g += 1024) s_c[g] = counts[g];
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += 1024) {
    const int c = s_c[g];
    int rank = 0;
    for (int h = 0; h < G; ++h) rank += (s_c[h] > c || (s_c[h] == c && h < g)) ? 1 : 0;
    order[rank] = g;
  }
}

void launch_group_order(const int32_t* counts, int G, int32_t* order, hipStream_t st) {
  if (G <= 0 || G > 1024) return;
  group_order_kernel<<<1, 1024, 0, st>>>(counts, G, order);
}

void launch_wgrad_rows(const WgradRowsArgs& w, int G, hipStream_t st) {
  if (G <= 0 || w.M <= 0 || w.Nn <= 0) return;
  dim3 grid((w.Nn + kRN - 1) / kRN, (w.M + kRM - 1) / kRM, static_cast<unsigned>(G));
  // one compiled copy per combination of gathers and scale (the expert products use (A, scale) for
  // dDn and (B) for dGU)
  const int sel = (w.ga ? 4 : 0) | (w.gb ? 2 : 0) | (w.scale ? 1 : 0);
  switch (sel) {
    case 0: gemm_wgrad_rows_kernel<false, false, false><<<grid, 512, 0, st>>>(w); break;
    case 1: gemm_wgrad_rows_kernel<false, false, true><<<grid, 512, 0, st>>>(w); break;
    case 2: gemm_wgrad_rows_kernel<false, true, false><<<grid, 512, 0, st>>>(w); break;
    case 3: gemm_wgrad_rows_kernel<false, true, true><<<grid, 512, 0, st>>>(w); break;
    case 4: gemm_wgrad_rows_kernel<true, false, false><<<grid, 512, 0, st>>>(w); break;
    case 5: gemm_wgrad_rows_kernel<true, false, true><<<grid, 512, 0, st>>>(w); break;
    case 6: gemm_wgrad_rows_kernel<true, true, false><<<grid, 512, 0, st>>>(w); break;
    default: gemm_wgrad_rows_kernel<true, true, true><<<grid, 512, 0, st>>>(w); break;
  }
}

// fp32 weight gradient (fp32 layers): the same sums with FMAs, one output per thread of a 16 x 16
// tile, 64-wide k-slices through LDS, in q order (deterministic).
__global__ __launch_bounds__(256) void gemm_wgrad_f32_kernel(const float* __restrict__ Am, const float* __restrict__ Bm,
                                                             int64_t ld, const int32_t* __restrict__ poff, int64_t qtot,
                                                             int M, int Nn, float* __restrict__ out) {
  __shared__ float sA[16][kWK + 1];
  __shared__ float sB[16][kWK + 1];
  const int g = blockIdx.z;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 16, tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t q0 = poff ? poff[g] : 0;
  const int64_t q1 = poff ? poff[g + 1] : qtot;
  float acc = 0.f;
  for (int64_t qb = q0; qb < q1; qb += kWK) {
    for (int i = tid; i < 16 * kWK; i += 256) {
      const int r = i / kWK, c = i % kWK;
      sA[r][c] = m0 + r < M ? Am[static_cast<int64_t>(m0 + r) * ld + qb + c] : 0.f;
      sB[r][c] = n0 + r < Nn ? Bm[static_cast<int64_t>(n0 + r) * ld + qb + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kWK; ++c) acc = fmaf(sA[ty][c], sB[tx][c], acc);
    __syncthreads();
  }
  if (m0 + ty < M && n0 + tx < Nn) out[static_cast<int64_t>(g) * M * Nn + static_cast<int64_t>(m0 + ty) * Nn + n0 + tx] = acc;
}

void launch_wgrad_f32(const float* A, const float* Bm, int64_t ld, const int32_t* poff, int64_t qtot, int G, int M, int Nn,
                      float* out, hipStream_t st) {
  if (G <= 0 || M <= 0 || Nn <= 0) return;
  dim3 grid((Nn + 15) / 16, (M + 15) / 16, static_cast<unsigned>(G));
  gemm_wgrad_f32_kernel<<<grid, 256, 0, st>>>(A, Bm, ld, poff, qtot, M, Nn, out);
}

// Split reduction for a single long group (the router's sum over all tokens): slice s covers
// [poff[s], poff[s+1]) of the padded range, poff[s] = min(s * chunk, total); the partial results
// [S][M][Nn] are then added in slice order (deterministic).
__global__ void slice_offsets_kernel(int32_t* __restrict__ poff, int S, int64_t chunk, int64_t total) {
  const int s = threadIdx.x;
  if (s <= S) poff[s] = static_cast<int32_t>(min<int64_t>(s * chunk, total));
}

__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int S, int64_t n, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int s = 0; s < S; ++s) acc += part[s * n + i];
  out[i] = acc;
}

void launch_wgrad_split(const uint16_t* A, const uint16_t* Bm, int64_t ld, int64_t qtot, int M, int Nn, int S,
                        int32_t* poff, float* part, float* out, hipStream_t st) {
  const int64_t chunk = ((qtot + S - 1) / S + kWK - 1) / kWK * kWK;
  slice_offsets_kernel<<<1, 64, 0, st>>>(poff, S, chunk, qtot);
  launch_wgrad(A, Bm, ld, poff, 0, S, M, Nn, part, st);
  const int64_t n = static_cast<int64_t>(M) * Nn;
  sum_slices_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(part, S, n, out);
}


// ---------------------------------------------------------------------------------------------
// Grouped product with the weights read in their stored [K][N] layout, for short groups (the
// backward's dh = dy Dn and dx rows = [da | db] GU when each expert holds a few rows):
//   out[p][n] = sum_k X[row(p)][k] W[g][k][n]   for the rows p of group g, out fp32,
// row(p) = row_index[p] when given. A wave owns 128 columns (two per lane) of one group and walks
// k: one 4-byte weight load per lane and k (a 256-byte run of the weight row), in chunks of 16 k
// with the next chunk's loads in flight during this chunk's products. The group's rows sit in LDS
// in their own layout, so consecutive k pair up in one dword; a byte permute pairs the weights of
// one column for the same two k, and one bf16 dot-product instruction (two products added to an
// fp32 sum) covers them. The loop is compiled once per row count (1..8); a group of more than eight
// rows takes several passes over its weights. No transposed weight copy is needed. K % 32 == 0,
// K <= kKsMaxK.
// ---------------------------------------------------------------------------------------------
constexpr int kKsRows = 8, kKsUnroll = 16;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int R>
__device__ __forceinline__ void kstream_pass(const uint16_t* __restrict__ sX, const uint32_t* __restrict__ wg, bool col_ok,
                                             int K, int NW, float* __restrict__ orow0, int N, int c) {
  float acc[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.f;
  auto load = [&](uint32_t* wv, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kKsUnroll; ++u) wv[u] = __builtin_nontemporal_load(wg + static_cast<int64_t>(k0 + u) * NW);
  };
  auto math = [&](const uint32_t* wv, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kKsUnroll / 8; ++q) {              // eight k at a time
      u32x4 xv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) xv[r] = *reinterpret_cast<const u32x4*>(&sX[r * K + k0 + 8 * q]);
#pragma unroll
      for (int h = 0; h < 4; ++h) {                         // k pair (k0 + 8 q + 2 h, + 1)
        const uint32_t a = wv[8 * q + 2 * h], b = wv[8 * q + 2 * h + 1];
        const uint32_t wc0 = __builtin_amdgcn_perm(b, a, 0x05040100u);   // column c: (W[k][c], W[k+1][c])
        const uint32_t wc1 = __builtin_amdgcn_perm(b, a, 0x07060302u);   // column c + 1
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r][0] = dot2_bf16(xv[r][h], wc0, acc[r][0]);
          acc[r][1] = dot2_bf16(xv[r][h], wc1, acc[r][1]);
        }
      }
    }
  };
  // two chunks of weight rows in registers: the next chunk's loads go out before this chunk's
  // products (past the end they re-read the last chunk, in bounds and unused)
  uint32_t wa[kKsUnroll], wb[kKsUnroll];
  load(wa, 0);
  for (int k0 = 0; k0 < K; k0 += 2 * kKsUnroll) {
    load(wb, min(k0 + kKsUnroll, K - kKsUnroll));
    math(wa, k0);
    load(wa, min(k0 + 2 * kKsUnroll, K - kKsUnroll));
    math(wb, k0 + kKsUnroll);
  }
  if (col_ok) {
#pragma unroll
    for (int r = 0; r < R; ++r) *reinterpret_cast<float2*>(orow0 + static_cast<int64_t>(r) * N + c) = make_float2(acc[r][0], acc[r][1]);
  }
}

__global__ __launch_bounds__(256) void gemm_kstream_kernel(const uint16_t* __restrict__ X, const int32_t* __restrict__ row_index,
                                                           const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
                                                           int K, int N, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[kKsMaxK * kKsRows];
  const int g = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = offsets[g];
  const int rows = offsets[g + 1] - static_cast<int>(r0);
  const int c = (blockIdx.x * 4 + wave) * 128 + 2 * lane;       // this lane's columns c, c + 1
  const bool col_ok = c < N;                                     // N is even
  // lanes past N read column 0 (in bounds) and store nothing
  const uint32_t* wg = reinterpret_cast<const uint32_t*>(W + static_cast<int64_t>(g) * K * N + (col_ok ? c : 0));
  const int NW = N / 2;                                          // weight row stride in 4-byte units
  for (int pass = 0; pass < rows; pass += kKsRows) {
    const int R = min(kKsRows, rows - pass);
    for (int idx = tid; idx < R * (K / 8); idx += 256) {         // rows pass .. pass + R - 1, 16 bytes at a time
      const int r = idx / (K / 8), k8 = idx - r * (K / 8);
      const int64_t p = r0 + pass + r;
      const int64_t src = row_index ? row_index[p] : p;
      *reinterpret_cast<u32x4*>(&sX[r * K + k8 * 8]) = *reinterpret_cast<const u32x4*>(X + src * K + k8 * 8);
    }
    __syncthreads();
    float* orow0 = out + (r0 + pass) * N;
    switch (R) {
      case 1: kstream_pass<1>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      case 2: kstream_pass<2>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      case 3: kstream_pass<3>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      case 4: kstream_pass<4>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      case 5: kstream_pass<5>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      case 6: kstream_pass<6>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      case 7: kstream_pass<7>(sX, wg, col_ok, K, NW, orow0, N, c); break;
      default: kstream_pass<8>(sX, wg, col_ok, K, NW, orow0, N, c); break;
    }
    __syncthreads();                                             // before the next pass restages
  }
}

void launch_kstream(const uint16_t* X, const int32_t* row_index, const int32_t* offsets, int G, const uint16_t* W, int K,
                    int N, float* out, hipStream_t st) {
  if (G <= 0 || K <= 0 || N <= 0) return;
  dim3 grid((N + 511) / 512, static_cast<unsigned>(G));
  gemm_kstream_kernel<<<grid, 256, 0, st>>>(X, row_index, offsets, W, K, N, out);
}

}  // namespace moe
