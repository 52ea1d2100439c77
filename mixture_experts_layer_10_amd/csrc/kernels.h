// Internal launcher interface between the C ABI (moe_abi.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
  const void* x;
  const void* w_router;
  const void* w_shared_gate;  // may be null
  float* logits;              // may be null
  float* weights;
  int32_t* experts;
  float* shared_scale;        // non-null iff w_shared_gate
  float* partial;             // scratch for a split contraction [slices][N][E], or null
  int64_t N;
  int D, E, k;
  int norm;
  bool bf16;
  bool packed;                // w_router in the packed layout ([1, E, D] stack, E % 16 == 0)
  bool sigmoid;               // scores sigmoid(logit) picked by score + bias (else fp32 softmax)
  const float* bias;          // [E] selection bias for sigmoid scores, or null (zeros)
};
constexpr int kMaxRouteSlices = 16;
int route_slices_for(int64_t N, int D, int E, bool bf16);   // slices used when scratch is given
// fp32 scratch the router uses when given a workspace: the split contraction's partial logits, or
// the logits of the dense-product router for long batches with E > 128 (0: none)
int64_t route_scratch_floats(int64_t N, int D, int E, bool bf16);
int route_slices(const RouteArgs& a);
void launch_route(const RouteArgs& a, hipStream_t st);

// Permutation: assignments are processed in chunks of kPermChunk by one workgroup each.
constexpr int kPermChunk = 1024;
struct PermuteArgs {
  const int32_t* experts;   // [A]
  int32_t* block_counts;    // [n_chunks * E] workspace
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E + 1]
  int32_t* token_of;        // [A]
  int32_t* slot_pos;        // [A]; -1 for an assignment dropped by the capacity limit
  int64_t A;
  int E, k;
  int64_t capacity;         // rows kept per expert (>= A: no limit)
};
void launch_permute(const PermuteArgs& a, hipStream_t st);
int64_t permute_chunks(int64_t A);

// x_perm[p] = x[token_of[p]] for p < min(rows, *n_valid) (row_bytes % 16 == 0; n_valid on device).
void launch_gather_rows(const void* x, const int32_t* token_of, const int32_t* n_valid, void* x_perm, int64_t rows,
                        int64_t row_bytes, hipStream_t st);

struct GemmArgs {
  const void* x;          // gate_up: activations; down: h
  const int32_t* row_index;
  const int32_t* offsets; // [G+1] or null (one group of max_rows rows)
  const void* w;          // gate_up [G, 2I, D] or down [G, D, I] (rows), or their packed form
  void* out;              // gate_up: h [rows, I]; down: out [rows, D] fp32
  int64_t max_rows;
  int G;
  int D, I;
  bool bf16;
  bool packed;            // w in the packed layout (bf16, K % 128 == 0, rows % 16 == 0)
  int qbits;              // code kind: 0 bf16 weights; kQInt8 / kQInt4 / kQFp8: a quantised stack
  bool wkn;               // down form, bf16 rows: w stored [G, K, NOUT] (read with LDS transpose loads)
  bool out_f16s;          // down form, bf16: out rows are fp16 values + an int8 exponent per 16 columns
                          // (f16s_row_bytes(NOUT) bytes per row), else fp32 rows
  // gate_up form, bf16 rows, tall groups: the SwiGLU backward in the epilogue when bwd_dab is set.
  // With [a | b] the tile's pre-activations, s = 1 / (1 + exp(-a)) and dh = w[p] dhu:
  // out = h = bf16(a s b), bwd_dab = bf16([dh b s (1 + a (1 - s)) | dh a s]), and
  // bwd_dwp[p][c] = sum of dhu h over columns 32 c .. 32 c + 31 (fp32 partials of dw)
  const float* bwd_dhu;   // [rows, I] fp32
  const float* bwd_w;     // [rows]
  void* bwd_dab;          // [rows, 2I] bf16
  float* bwd_dwp;         // [rows, ceil(I / 32)] fp32
};
// dw[assign_of[p]] = sum over c of dwp[p][c], in column order (p < A)
void launch_dw_sum(const float* dwp, int nb, const int32_t* assign_of, int64_t A, float* dw, hipStream_t st);
void launch_gate_up(const GemmArgs& a, hipStream_t st);
void launch_down(const GemmArgs& a, hipStream_t st);
// whether launch_down takes a.wkn (weights [G, K, NOUT]) for the down form with K = k_in, NOUT = n_out
// over max_rows rows (in G groups when grouped, i.e. with offsets): bf16, tall groups, K % 128 == 0
// and NOUT % 8 == 0
bool wkn_streamable(bool bf16, bool grouped, int64_t max_rows, int G, int k_in, int n_out);
// whether launch_gate_up takes the SwiGLU backward epilogue (bwd_dab set) for a gate_up product of
// width D and I over max_rows rows (row-layout bf16 weights): tall groups, D % 128 == 0, I % 4 == 0
bool bwd_fusable(bool bf16, bool grouped, int64_t max_rows, int G, int D, int I);

// Packed weight layout: a [G, R, K] bf16 matrix (R % 16 == 0, K % 32 == 0) stored as 16 x 32
// fragments, fragment (g, rb, kb) at element ((g * R/16 + rb) * K/32 + kb) * 512, each 1 KB in
// matrix-core lane order (lane l: row rb*16 + l % 16, k = kb*32 + 8 (l / 16) .. + 7).
void launch_pack(const uint16_t* src, uint16_t* dst, int64_t G, int R, int K, hipStream_t st);

// Quantised stack of a [G, R, K] bf16 matrix (R % 16 == 0), codes first, then one fp32 scale per
// row, [G, R], from byte quant_code_bytes(G, R, K, b) on.
// int8 / FP8 (K % 32 == 0): codes in the packed block order, block (g, rb, kb) of 512 bytes at
// ((g * R/16 + rb) * K/32 + kb) * 512, slot l (8 bytes) = row rb*16 + l % 16, columns kb*32 +
// 8 (l / 16) .. + 7.
// int4 (K % 128 == 0): super-blocks of 16 rows x 128 columns, (g, rb, kq) at ((g * R/16 + rb) *
// K/128 + kq) * kQ4Super: 1024 bytes of codes, slot l (16 bytes) = row rb*16 + l % 16, its bytes
// 4 t .. 4 t + 3 the eight codes of columns (4 kq + t) * 32 + 8 (l / 16) .. + 7 (code i as the
// nibble code + 8 in byte i % 4, the high nibble for i >= 4);
// then 64 bytes of group multipliers, byte 1024 + 4 r + t = row rb*16 + r, columns (4 kq + t) * 32
// .. + 31. A weight is code * multiplier * row scale.
constexpr int kQ4Super = 1088;
__host__ __device__ inline int64_t quant_code_bytes(int64_t G, int64_t R, int64_t K, int bits) {
  return bits == 4 ? G * (R / 16) * (K / 128) * kQ4Super : G * R * K * bits / 8;
}
// Code kinds (GemmArgs::qbits and kernel template arguments): bits per code, FP8 marked apart.
constexpr int kQInt8 = 8, kQInt4 = 4, kQFp8 = 9;
__host__ __device__ constexpr int code_bits(int kind) { return kind == kQFp8 ? 8 : kind; }    // 0 for bf16
__host__ __device__ constexpr int code_slot(int kind) { return code_bits(kind); }           // bytes per lane slot
void launch_quantize(const uint16_t* src, uint8_t* dst, int64_t G, int R, int K, int kind, hipStream_t st);

// Expert-output rows in the fp16 form: NOUT fp16 values, then NOUT / 16 int8 exponents (value of
// column c = fp16[c] * 2^exp[c / 16]), padded to 16 bytes. NOUT % 16 == 0.
__host__ __device__ constexpr int64_t f16s_row_bytes(int64_t nout) { return (2 * nout + nout / 16 + 15) / 16 * 16; }

struct CombineArgs {
  const float* out_perm;
  const float* weights;
  const int32_t* slot_pos;
  const float* shared_out;    // may be null
  const float* shared_scale;  // may be null
  void* y;
  int64_t N;
  int D, k;
  bool out_bf16;
  bool in_f16s;               // out_perm and shared_out rows in the fp16 form (f16s_row_bytes(D) bytes)
};
void launch_combine(const CombineArgs& a, hipStream_t st);

// Router load statistics (f, P, balance loss); partial: stats_blocks(N) x E fp32 scratch.
int64_t stats_blocks(int64_t N);
void launch_stats(const float* logits, const int32_t* counts, float* f, float* P, float* loss, float* partial,
                  int64_t N, int E, int k, hipStream_t st);

// Selection-bias nudge: bias[e] -= gamma * sign(counts[e] - A / E).
void launch_bias_update(const int32_t* counts, float* bias, float gamma, int64_t A, int E, hipStream_t st);

// Backward pass helpers (backward.hip). f32: the layer's dtype is fp32 (elements of 4 bytes, no
// rounding of the intermediates); otherwise bf16.
void launch_transpose_mat(const void* in, void* out, int64_t G, int R, int C, int Rp, bool f32, hipStream_t st);
void launch_pad_offsets(const int32_t* counts, int32_t* poff, int G, hipStream_t st);
void launch_transpose_rows(const void* src, int M, const int32_t* gather, const float* scale, const int32_t* off,
                           const int32_t* poff, int G, int n1, int64_t qmax, void* out, int64_t ld, bool f32, hipStream_t st);
void launch_scatter_assign(const int32_t* slot_pos, const float* weights, float* w_perm, int32_t* assign_of, float* ones,
                           int64_t A, hipStream_t st);
void launch_swiglu_bwd(const float* z, const float* dhu, const float* w_perm, const int32_t* assign_of, const int32_t* n_rows,
                       int64_t A, int I, void* h, void* dab, float* dw, bool f32, hipStream_t st);
void launch_shared_gate_bwd(const float* sdot, const float* g, int64_t N, int64_t qpad, float* dz, void* dz_row, bool f32,
                            hipStream_t st);
void launch_add_rows(float* acc, const float* add, const float* dz, const void* ws, bool ws_f32, int64_t N, int D,
                     hipStream_t st);
void launch_router_bwd(const float* logits, const float* weights, const int32_t* experts, const float* dw, int64_t N, int E,
                       int Ep, int k, int norm, void* dlogit, bool f32, hipStream_t st);
void launch_wgrad(const uint16_t* A, const uint16_t* Bm, int64_t ld, const int32_t* poff, int64_t qtot, int G, int M, int Nn,
                  float* out, hipStream_t st);
void launch_wgrad_f32(const float* A, const float* Bm, int64_t ld, const int32_t* poff, int64_t qtot, int G, int M, int Nn,
                      float* out, hipStream_t st);
// Weight gradients from the rows in place: out[g] = sum over the rows p of group g (off) of
// bf16(s(p) A[ra(p)]) (x) B[rb(p)] (outer product, [M, Nn] fp32); ra / rb gather through ga / gb
// when given, s = scale[p] when given. bf16 only; M % 8 == 0, Nn % 8 == 0.
struct WgradRowsArgs {
  const uint16_t* A;
  int64_t lda;
  const int32_t* ga;
  const float* scale;
  const uint16_t* B;
  int64_t ldb;
  const int32_t* gb;
  const int32_t* off;
  const int32_t* order;   // optional: workgroup z computes group order[z] (largest groups first)
  int M, Nn;
  float* out;
};
void launch_wgrad_rows(const WgradRowsArgs& w, int G, hipStream_t st);
// order[0 .. G) = the groups by row count, largest first, ties by index (G <= 1024)
void launch_group_order(const int32_t* counts, int G, int32_t* order, hipStream_t st);
constexpr int kWgradSlices = 16;     // split of a single long reduction (poff: kWgradSlices + 1 entries)
void launch_wgrad_split(const uint16_t* A, const uint16_t* Bm, int64_t ld, int64_t qtot, int M, int Nn, int S,
                        int32_t* poff, float* part, float* out, hipStream_t st);

// Grouped product over short groups with W[g] stored [K][N] (no transposed copy): out[p][n] =
// sum_k X[row(p)][k] W[g][k][n] (bf16 in, fp32 out). K <= kKsMaxK, K % 32 == 0, N even.
constexpr int kKsMaxK = 2048;
void launch_kstream(const uint16_t* X, const int32_t* row_index, const int32_t* offsets, int G, const uint16_t* W, int K,
                    int N, float* out, hipStream_t st);

int device_cu_count();

}  // namespace moe
