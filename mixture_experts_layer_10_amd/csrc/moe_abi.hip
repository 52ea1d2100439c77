// C ABI of the MoE block: host-side validation, workspace carving and kernel launches.
// Every check runs before anything is enqueued; see include/moe.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "kernels.h"

namespace moe {

static thread_local std::string g_last_error;

static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

static int ok() {
  g_last_error.clear();
  return MOE_OK;
}

static int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

static int hip_ok(hipError_t e, const char* what) {
  return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

constexpr int64_t kMaxExperts = 512;

static size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Code kind of a quantised layout (kQInt8, kQInt4, kQFp8), 0 for bf16 / fp32 weights.
static int quant_kind(const moe_config* c) {
  switch (c->weight_layout) {
    case MOE_LAYOUT_Q8: return kQInt8;
    case MOE_LAYOUT_Q4: return kQInt4;
    case MOE_LAYOUT_F8: return kQFp8;
    default: return 0;
  }
}
static int quant_bits(const moe_config* c) { return code_bits(quant_kind(c)); }
// The router's weights are packed (as a [1, E, D] stack) with the experts' when E % 16 == 0.
static bool router_packed(const moe_config* c) { return c->weight_layout != MOE_LAYOUT_ROWS && c->n_experts % 16 == 0; }

// Weight loads are 16 bytes wide (bf16 rows, packed blocks, quantised codes and scales).
static int check_weight_align(const void* p, const char* name) {
  if (reinterpret_cast<uintptr_t>(p) & 15) return fail(MOE_ERR_UNSUPPORTED, "%s at %p is not 16-byte aligned", name, p);
  return MOE_OK;
}

static int validate_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->n_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens = %lld < 0", (long long)c->n_tokens);
  if (c->hidden < 1) return fail(MOE_ERR_INVALID_ARG, "hidden = %lld < 1", (long long)c->hidden);
  if (c->n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts = %lld < 1", (long long)c->n_experts);
  if (c->top_k < 1) return fail(MOE_ERR_INVALID_ARG, "top_k = %lld < 1", (long long)c->top_k);
  if (c->top_k > c->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k = %lld > n_experts = %lld", (long long)c->top_k, (long long)c->n_experts);
  if (c->inter < 1) return fail(MOE_ERR_INVALID_ARG, "inter = %lld < 1", (long long)c->inter);
  if (c->shared_inter < 0) return fail(MOE_ERR_INVALID_ARG, "shared_inter = %lld < 0", (long long)c->shared_inter);
  if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1)
    return fail(MOE_ERR_INVALID_ARG, "norm_topk_prob = %d (must be 0 or 1)", c->norm_topk_prob);
  if (c->weight_layout < MOE_LAYOUT_ROWS || c->weight_layout > MOE_LAYOUT_F8)
    return fail(MOE_ERR_INVALID_ARG, "weight_layout = %d (must be 0 to 4)", c->weight_layout);
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "dtype %d not supported", c->dtype);
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "out_dtype %d not supported", c->out_dtype);
  const int64_t align = c->dtype == MOE_BF16 ? 8 : 4;
  if (c->hidden % align) return fail(MOE_ERR_UNSUPPORTED, "hidden = %lld is not a multiple of %lld", (long long)c->hidden, (long long)align);
  if (c->inter % align) return fail(MOE_ERR_UNSUPPORTED, "inter = %lld is not a multiple of %lld", (long long)c->inter, (long long)align);
  if (c->shared_inter % align)
    return fail(MOE_ERR_UNSUPPORTED, "shared_inter = %lld is not a multiple of %lld", (long long)c->shared_inter, (long long)align);
  if (c->weight_layout != MOE_LAYOUT_ROWS) {
    if (c->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "packed weights need dtype bf16");
    if (c->hidden % 128 || c->inter % 128 || c->shared_inter % 128)
      return fail(MOE_ERR_UNSUPPORTED, "packed weights need hidden, inter and shared_inter multiples of 128");
  }
  if (c->expert_out != MOE_EXPERT_OUT_F32 && c->expert_out != MOE_EXPERT_OUT_F16S)
    return fail(MOE_ERR_INVALID_ARG, "expert_out = %d (must be 0 or 1)", c->expert_out);
  if (c->expert_out == MOE_EXPERT_OUT_F16S) {
    if (c->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "fp16 expert outputs need dtype bf16");
    if (c->hidden % 16) return fail(MOE_ERR_UNSUPPORTED, "fp16 expert outputs need hidden %% 16 == 0 (got %lld)", (long long)c->hidden);
    if (c->weight_layout != MOE_LAYOUT_ROWS && c->weight_layout != MOE_LAYOUT_PACKED)
      return fail(MOE_ERR_UNSUPPORTED, "fp16 expert outputs need row or packed bf16 weights");
  }
  if (c->n_experts > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts = %lld > %lld", (long long)c->n_experts, (long long)kMaxExperts);
  if (c->hidden > (1 << 20) || c->inter > (1 << 20) || c->shared_inter > (1 << 20))
    return fail(MOE_ERR_UNSUPPORTED, "hidden/inter above 2^20");
  if (c->n_tokens > 0 && c->n_tokens * c->top_k > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "n_tokens * top_k = %lld exceeds int32 row indices", (long long)(c->n_tokens * c->top_k));
  return MOE_OK;
}

// Scratch of a split router contraction: slices x N x E fp32 (0 when it runs in one pass).
static size_t route_partial_bytes(const moe_config* c) {
  return static_cast<size_t>(route_scratch_floats(c->n_tokens, static_cast<int>(c->hidden), static_cast<int>(c->n_experts),
                                                  c->dtype == MOE_BF16)) * 4;
}

struct Layout {
  size_t route_partial, weights, experts, shared_scale, counts, offsets, block_counts, token_of, slot_pos, h, out,
      sh_h, sh_out, total;
};

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

static Layout layout_of(const moe_config* c) {
  Layout L{};
  const size_t N = static_cast<size_t>(c->n_tokens), A = N * static_cast<size_t>(c->top_k);
  const size_t E = static_cast<size_t>(c->n_experts), D = static_cast<size_t>(c->hidden);
  const size_t I = static_cast<size_t>(c->inter), Is = static_cast<size_t>(c->shared_inter);
  const size_t eb = elem_bytes(c->dtype);
  size_t at = 0;
  auto take = [&](size_t bytes) { const size_t p = at; at += align256(bytes); return p; };
  L.route_partial = take(route_partial_bytes(c));
  L.block_counts = take(static_cast<size_t>(permute_chunks(static_cast<int64_t>(A))) * E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.weights = take(A * 4);
  L.experts = take(A * 4);
  L.token_of = take(A * 4);
  L.slot_pos = take(A * 4);
  L.shared_scale = take(Is ? N * 4 : 0);
  // expert-output rows: D fp32 values, or the fp16 form's f16s_row_bytes(D)
  const size_t orow = c->expert_out == MOE_EXPERT_OUT_F16S ? static_cast<size_t>(f16s_row_bytes(c->hidden)) : D * 4;
  L.h = take(A * I * eb);
  L.out = take(A * orow);
  L.sh_h = take(Is ? N * Is * eb : 0);
  L.sh_out = take(Is ? N * orow : 0);
  L.total = at;
  return L;
}

static size_t stats_ws_bytes(const moe_config* c) {
  return static_cast<size_t>(stats_blocks(c->n_tokens)) * static_cast<size_t>(c->n_experts) * 4;
}

static size_t permute_ws_bytes(const moe_config* c) {
  const size_t A = static_cast<size_t>(c->n_tokens) * static_cast<size_t>(c->top_k);
  return static_cast<size_t>(permute_chunks(static_cast<int64_t>(A))) * static_cast<size_t>(c->n_experts) * 4;
}

#define MOE_TRY(expr)            \
  do {                           \
    const int _s = (expr);       \
    if (_s != MOE_OK) return _s; \
  } while (0)

static RouteArgs route_args(const moe_config* c, const void* x, const void* w_router, const void* w_shared_gate,
                            float* logits, float* weights, int32_t* experts, float* shared_scale, float* partial,
                            bool sigmoid = false, const float* bias = nullptr) {
  RouteArgs a{};
  a.sigmoid = sigmoid;
  a.bias = bias;
  a.partial = partial;
  a.x = x;
  a.w_router = w_router;
  a.w_shared_gate = w_shared_gate;
  a.logits = logits;
  a.weights = weights;
  a.experts = experts;
  a.shared_scale = shared_scale;
  a.N = c->n_tokens;
  a.D = static_cast<int>(c->hidden);
  a.E = static_cast<int>(c->n_experts);
  a.k = static_cast<int>(c->top_k);
  a.norm = c->norm_topk_prob;
  a.bf16 = c->dtype == MOE_BF16;
  // packed and quantised layouts keep a packed bf16 router when E is a multiple of 16, else rows
  a.packed = router_packed(c);
  return a;
}

static int route_impl(const moe_config* c, const void* x, const void* w_router, const void* w_shared_gate,
                      float* logits, float* weights, int32_t* experts, float* shared_scale, float* partial,
                      hipStream_t st, bool sigmoid = false, const float* bias = nullptr) {
  launch_route(route_args(c, x, w_router, w_shared_gate, logits, weights, experts, shared_scale, partial, sigmoid, bias), st);
  return check_launch("moe_route");
}

static PermuteArgs permute_args(const moe_config* c, const int32_t* experts, int32_t* counts, int32_t* offsets,
                                int32_t* token_of, int32_t* slot_pos, int32_t* block_counts, int64_t capacity = INT64_MAX) {
  PermuteArgs a{};
  a.capacity = capacity;
  a.experts = experts;
  a.block_counts = block_counts;
  a.counts = counts;
  a.offsets = offsets;
  a.token_of = token_of;
  a.slot_pos = slot_pos;
  a.A = c->n_tokens * c->top_k;
  a.E = static_cast<int>(c->n_experts);
  a.k = static_cast<int>(c->top_k);
  return a;
}

static int permute_impl(const moe_config* c, const int32_t* experts, const void* x, int32_t* counts,
                        int32_t* offsets, int32_t* token_of, int32_t* slot_pos, void* x_perm, int32_t* block_counts,
                        hipStream_t st, int64_t capacity = INT64_MAX) {
  const PermuteArgs a = permute_args(c, experts, counts, offsets, token_of, slot_pos, block_counts, capacity);
  launch_permute(a, st);
  if (x_perm)
    launch_gather_rows(x, token_of, offsets + a.E, x_perm, a.A, c->hidden * static_cast<int64_t>(elem_bytes(c->dtype)), st);
  return check_launch("moe_permute");
}

static int ffn_checks(const moe_config* c, int64_t n_groups, int64_t inter, int64_t max_rows, const int32_t* offsets) {
  MOE_TRY(validate_config(c));
  if (n_groups < 1) return fail(MOE_ERR_INVALID_ARG, "n_groups = %lld < 1", (long long)n_groups);
  if (n_groups > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_groups = %lld > %lld", (long long)n_groups, (long long)kMaxExperts);
  if (inter < 1) return fail(MOE_ERR_INVALID_ARG, "inter = %lld < 1", (long long)inter);
  const int64_t align = c->dtype == MOE_BF16 ? 8 : 4;
  if (inter % align) return fail(MOE_ERR_UNSUPPORTED, "inter = %lld is not a multiple of %lld", (long long)inter, (long long)align);
  if (inter > (1 << 20)) return fail(MOE_ERR_UNSUPPORTED, "inter above 2^20");
  if (c->weight_layout != MOE_LAYOUT_ROWS && inter % 128)
    return fail(MOE_ERR_UNSUPPORTED, "packed weights need inter = %lld to be a multiple of 128", (long long)inter);
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "max_rows = %lld < 0", (long long)max_rows);
  if (max_rows > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "max_rows above int32");
  if (!offsets && n_groups != 1) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL with n_groups = %lld", (long long)n_groups);
  return MOE_OK;
}

static GemmArgs gemm_args(const moe_config* c, int64_t n_groups, int64_t inter, int64_t max_rows, const void* x,
                          const int32_t* row_index, const int32_t* offsets, const void* w, void* out) {
  GemmArgs a{};
  a.x = x;
  a.row_index = row_index;
  a.offsets = offsets;
  a.w = w;
  a.out = out;
  a.max_rows = max_rows;
  a.G = static_cast<int>(n_groups);
  a.D = static_cast<int>(c->hidden);
  a.I = static_cast<int>(inter);
  a.bf16 = c->dtype == MOE_BF16;
  a.packed = c->weight_layout != MOE_LAYOUT_ROWS;
  a.qbits = quant_kind(c);
  a.out_f16s = c->expert_out == MOE_EXPERT_OUT_F16S;
  return a;
}

// Expert-output rows are 16-byte vectors in either form.
static int check_out_align(const void* p, const char* name) {
  if (reinterpret_cast<uintptr_t>(p) & 15) return fail(MOE_ERR_UNSUPPORTED, "%s at %p is not 16-byte aligned", name, p);
  return MOE_OK;
}

static int combine_impl(const moe_config* c, const float* out_perm, const float* weights, const int32_t* slot_pos,
                        const float* shared_out, const float* shared_scale, void* y, hipStream_t st) {
  CombineArgs a{};
  a.out_perm = out_perm;
  a.weights = weights;
  a.slot_pos = slot_pos;
  a.shared_out = shared_out;
  a.shared_scale = shared_scale;
  a.y = y;
  a.N = c->n_tokens;
  a.D = static_cast<int>(c->hidden);
  a.k = static_cast<int>(c->top_k);
  a.out_bf16 = c->out_dtype == MOE_BF16;
  a.in_f16s = c->expert_out == MOE_EXPERT_OUT_F16S;
  launch_combine(a, st);
  return check_launch("moe_combine");
}

// Which backward products read their operands in place and which go through transposed copies;
// one decision serves both the workspace layout (no room for copies that are not made) and the
// launches.
//   dh = dy Dn_e and dx rows = [da | db] GU_e (weights used transposed): short groups (a few rows
//   per expert) through launch_kstream, tall groups through the streaming GEMM's [K][N] mode, other
//   shapes through transposed weight copies; likewise the shared expert's two (one group of N rows).
//   The experts' weight gradients read their rows in place for bf16 layers with D and I multiples
//   of 8, else padded transposed copies of the rows.
//   Tall groups (bf16, D % 128 == 0): the SwiGLU backward runs in the epilogue of the recomputed
//   gate_up product (no fp32 pre-activations z in memory), dw from per-block partials.
struct BwdPlan {
  bool short_groups, ks_dh, ks_dx, copy_dn, copy_gu, copy_sdn, copy_sgu, rows_wgrad, fused_swiglu;
};

static BwdPlan bwd_plan_of(const moe_config* c) {
  const int64_t N = c->n_tokens, A = N * c->top_k, E = c->n_experts, D = c->hidden, I = c->inter, Is = c->shared_inter;
  const bool bf = c->dtype == MOE_BF16;
  const int e = static_cast<int>(E), d = static_cast<int>(D), i = static_cast<int>(I), is = static_cast<int>(Is);
  BwdPlan P{};
  P.short_groups = bf && A <= 64LL * E;
  P.ks_dh = P.short_groups && D % 32 == 0 && D <= kKsMaxK;
  P.ks_dx = P.short_groups && (2 * I) % 32 == 0 && 2 * I <= kKsMaxK;
  P.copy_dn = !P.ks_dh && !wkn_streamable(bf, true, A, e, d, i);
  P.copy_gu = !P.ks_dx && !wkn_streamable(bf, true, A, e, 2 * i, d);
  P.copy_sdn = Is > 0 && !wkn_streamable(bf, false, N, 1, d, is);
  P.copy_sgu = Is > 0 && !wkn_streamable(bf, false, N, 1, 2 * is, d);
  P.rows_wgrad = bf && D % 8 == 0 && I % 8 == 0;
  P.fused_swiglu = bwd_fusable(bf, true, A, e, d, i);
  return P;
}

// Backward workspace: routing and permutation state, the recomputed pre-activations, the
// gradients' intermediates, transposed weight copies and the padded transposed activations.
struct BwdLayout {
  size_t route_partial, logits, weights, experts, counts, offsets, block_counts, token_of, slot_pos, w_perm, assign_of,
      ones, dw, poff, gorder, z, dwp, dhu, h, dab, dx_rows, dlogit, dxr, dnT, guT, wrT, doT, xgT, hT, dabT, dlogitT, xT, spoff,
      wr_part, sh_scale, zs, dhus, hs, dabs, sdot, dz, dz_row, dxs, sdnT, sguT, dysT, hsT, dabsT, total;
  int64_t Ep, Qs, Ns;
};

static BwdLayout bwd_layout_of(const moe_config* c) {
  BwdLayout L{};
  const int64_t N = c->n_tokens, A = N * c->top_k, E = c->n_experts, D = c->hidden, I = c->inter, Is = c->shared_inter;
  const int64_t eb = static_cast<int64_t>(elem_bytes(c->dtype));      // layer-dtype intermediates
  L.Ep = (E + 7) / 8 * 8;
  L.Qs = (A + 64 * E + 7) / 8 * 8;
  L.Ns = (N + 63) / 64 * 64;
  size_t at = 0;
  auto take = [&](int64_t bytes) { const size_t p = at; at += align256(static_cast<size_t>(bytes)); return p; };
  L.route_partial = take(static_cast<int64_t>(route_partial_bytes(c)));
  L.logits = take(N * E * 4);
  L.weights = take(A * 4);
  L.experts = take(A * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.block_counts = take(permute_chunks(A) * E * 4);
  L.token_of = take(A * 4);
  L.slot_pos = take(A * 4);
  L.w_perm = take(A * 4);
  L.assign_of = take(A * 4);
  L.ones = take(A * 4);
  L.dw = take(A * 4);
  L.poff = take((E + 1) * 4);
  L.gorder = take(E * 4);
  const BwdPlan P = bwd_plan_of(c);
  L.z = take(P.fused_swiglu ? 0 : A * 2 * I * 4);
  L.dwp = take(P.fused_swiglu ? A * ((I + 31) / 32) * 4 : 0);
  L.dhu = take(A * I * 4);
  L.h = take(A * I * eb);
  L.dab = take(A * 2 * I * eb);
  L.dx_rows = take(A * D * 4);
  L.dlogit = take(N * L.Ep * eb);
  L.dxr = take(N * D * 4);
  L.dnT = take(P.copy_dn ? E * I * D * eb : 0);
  L.guT = take(P.copy_gu ? E * D * 2 * I * eb : 0);
  L.wrT = take(D * L.Ep * eb);
  const int64_t tq = P.rows_wgrad ? 0 : L.Qs;         // padded expert rows of the transposed copies
  L.doT = take(D * tq * eb);
  L.xgT = take(D * tq * eb);
  L.hT = take(I * tq * eb);
  L.dabT = take(2 * I * tq * eb);
  L.dlogitT = take(L.Ep * L.Ns * eb);
  L.xT = take(D * L.Ns * eb);
  L.spoff = take((kWgradSlices + 1) * 4);
  L.wr_part = take(static_cast<int64_t>(kWgradSlices) * std::max(E, 2 * Is) * D * 4);
  // shared expert: one more group over all N tokens
  L.sh_scale = take(Is ? N * 4 : 0);
  L.zs = take(N * 2 * Is * 4);
  L.dhus = take(N * Is * 4);
  L.hs = take(N * Is * eb);
  L.dabs = take(N * 2 * Is * eb);
  L.sdot = take(Is ? N * 4 : 0);
  L.dz = take(Is ? N * 4 : 0);
  L.dz_row = take(Is ? L.Ns * eb : 0);
  L.dxs = take(Is ? N * D * 4 : 0);
  L.sdnT = take(P.copy_sdn ? Is * D * eb : 0);
  L.sguT = take(P.copy_sgu ? D * 2 * Is * eb : 0);
  L.dysT = take(Is ? D * L.Ns * eb : 0);
  L.hsT = take(Is * L.Ns * eb);
  L.dabsT = take(2 * Is * L.Ns * eb);
  L.total = at;
  return L;
}

static int backward_checks(const moe_config* c) {
  MOE_TRY(validate_config(c));
  if (c->weight_layout != MOE_LAYOUT_ROWS) return fail(MOE_ERR_UNSUPPORTED, "the backward pass needs row-layout weights");
  return MOE_OK;
}

// The [out, in] grouped GEMM (fp32 output) on arbitrary operands: out[p] = X[row p] W_g^T, K = k_in.
static GemmArgs nt_args(const void* x, const int32_t* row_index, const int32_t* offsets, int G, int64_t max_rows,
                        const void* w, int n_out, int k_in, void* out, bool bf16) {
  GemmArgs a{};
  a.x = x;
  a.row_index = row_index;
  a.offsets = offsets;
  a.w = w;
  a.out = out;
  a.max_rows = max_rows;
  a.G = G;
  a.D = n_out;      // the down form: NOUT = D, K = I
  a.I = k_in;
  a.bf16 = bf16;
  return a;
}

// The same product with W_g stored [k_in, n_out] (a layer weight in its own layout, used transposed):
// read in place by the streaming kernel's [K][N] mode, or (copy, as BwdPlan decides) through a
// transposed copy in tmp.
static GemmArgs kn_args(const void* x, const int32_t* row_index, const int32_t* offsets, int G, int64_t max_rows,
                        const void* w_kn, bool copy, void* tmp, int n_out, int k_in, void* out, bool bf16, hipStream_t st) {
  GemmArgs a = nt_args(x, row_index, offsets, G, max_rows, w_kn, n_out, k_in, out, bf16);
  a.wkn = !copy;
  if (copy) {
    launch_transpose_mat(w_kn, tmp, G, k_in, n_out, k_in, !bf16, st);
    a.w = tmp;
  }
  return a;
}

// Scratch of moe_forward_noalloc: a fixed device array, so that the call allocates nothing. Each
// device holds its own copy at its own address; the host-side name is only a stand-in, so its
// device address is looked up once per device (with that device current) and kept.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(MOE_ERR_HIP, "moe_forward_noalloc: no current device");
  if (dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "moe_forward_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// A second stream per device for the shared expert, which reads x and its own weights only: it
// runs beside the router, the permutation and the routed products (whose launches leave CUs free:
// the dense-product router fills 64 of them for 8,192 tokens and 512 experts) and is joined before
// the combine. Created on a device's first such call, default priority, never destroyed. The
// mutex keeps each call's fork, side launches and join together, so calls from several host
// threads on one device queue their shared-expert work one after another on the side stream.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
};
static std::mutex g_side_mu[kMaxDevices];
static SideStream g_side[kMaxDevices];

// The device's side stream, or nullptr where none can be made (then the caller stays on its stream).
static SideStream* side_stream_locked(int dev) {
  SideStream& s = g_side[dev];
  if (!s.tried) {
    s.tried = true;
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      s.stream = nullptr;
    }
  }
  return s.stream ? &s : nullptr;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_workspace_bytes(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(validate_config(cfg));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = std::max(layout_of(cfg).total, stats_ws_bytes(cfg));
  return ok();
}

static int route_entry(const moe_config* cfg, const void* x, const void* w_router, const void* w_shared_gate,
                       float* logits, float* weights, int32_t* experts, float* shared_scale, void* ws, size_t ws_bytes,
                       void* stream, bool sigmoid, const float* bias) {
  MOE_TRY(validate_config(cfg));
  if (cfg->n_tokens == 0) return ok();
  if (!x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  if (!w_router) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
  if (!weights) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (!experts) return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
  if ((w_shared_gate == nullptr) != (shared_scale == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "w_shared_gate and shared_scale must be both set or both NULL");
  float* partial = nullptr;
  if (ws) {
    const size_t need = route_partial_bytes(cfg);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
    if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MOE_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
    if (need > 0) partial = static_cast<float*>(ws);
  }
  MOE_TRY(route_impl(cfg, x, w_router, w_shared_gate, logits, weights, experts, shared_scale, partial,
                     static_cast<hipStream_t>(stream), sigmoid, bias));
  return ok();
}

int moe_route(const moe_config* cfg, const void* x, const void* w_router, const void* w_shared_gate, float* logits,
              float* weights, int32_t* experts, float* shared_scale, void* ws, size_t ws_bytes, void* stream) {
  return route_entry(cfg, x, w_router, w_shared_gate, logits, weights, experts, shared_scale, ws, ws_bytes, stream,
                     false, nullptr);
}

int moe_route_sigmoid(const moe_config* cfg, const void* x, const void* w_router, const float* bias, float* logits,
                      float* weights, int32_t* experts, void* ws, size_t ws_bytes, void* stream) {
  return route_entry(cfg, x, w_router, nullptr, logits, weights, experts, nullptr, ws, ws_bytes, stream, true, bias);
}

static int permute_entry(const moe_config* cfg, const int32_t* experts, const void* x, int32_t* counts,
                         int32_t* offsets, int32_t* token_of, int32_t* slot_pos, void* x_perm, void* ws, size_t ws_bytes,
                         void* stream, int64_t capacity) {
  MOE_TRY(validate_config(cfg));
  if (cfg->n_tokens > 0 && !experts) return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
  if (!counts) return fail(MOE_ERR_INVALID_ARG, "counts is NULL");
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if (cfg->n_tokens > 0 && (!token_of || !slot_pos)) return fail(MOE_ERR_INVALID_ARG, "token_of or slot_pos is NULL");
  if ((x == nullptr) != (x_perm == nullptr)) return fail(MOE_ERR_INVALID_ARG, "x and x_perm must be both set or both NULL");
  if (capacity < 0) return fail(MOE_ERR_INVALID_ARG, "capacity = %lld < 0", (long long)capacity);
  const size_t need = permute_ws_bytes(cfg);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  // counts and offsets are defined even for N == 0 (all zero), so the scan always runs.
  MOE_TRY(permute_impl(cfg, experts, x, counts, offsets, token_of, slot_pos, x_perm, static_cast<int32_t*>(ws),
                       static_cast<hipStream_t>(stream), capacity));
  return ok();
}

int moe_permute(const moe_config* cfg, const int32_t* experts, const void* x, int32_t* counts, int32_t* offsets,
                int32_t* token_of, int32_t* slot_pos, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  return permute_entry(cfg, experts, x, counts, offsets, token_of, slot_pos, x_perm, ws, ws_bytes, stream, INT64_MAX);
}

int moe_permute_capped(const moe_config* cfg, int64_t capacity, const int32_t* experts, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* token_of, int32_t* slot_pos, void* x_perm, void* ws, size_t ws_bytes,
                       void* stream) {
  return permute_entry(cfg, experts, x, counts, offsets, token_of, slot_pos, x_perm, ws, ws_bytes, stream, capacity);
}

int moe_expert_gate_up(const moe_config* cfg, int64_t n_groups, int64_t inter, int64_t max_rows, const void* x,
                       const int32_t* row_index, const int32_t* offsets, const void* gate_up, void* h, void* stream) {
  MOE_TRY(ffn_checks(cfg, n_groups, inter, max_rows, offsets));
  if (max_rows == 0) return ok();
  if (!x || !gate_up || !h) return fail(MOE_ERR_INVALID_ARG, "x, gate_up or h is NULL");
  MOE_TRY(check_weight_align(gate_up, "gate_up"));
  launch_gate_up(gemm_args(cfg, n_groups, inter, max_rows, x, row_index, offsets, gate_up, h),
                 static_cast<hipStream_t>(stream));
  MOE_TRY(check_launch("moe_expert_gate_up"));
  return ok();
}

int moe_expert_down(const moe_config* cfg, int64_t n_groups, int64_t inter, int64_t max_rows, const int32_t* offsets,
                    const void* h, const void* down, float* out, void* stream) {
  MOE_TRY(ffn_checks(cfg, n_groups, inter, max_rows, offsets));
  if (max_rows == 0) return ok();
  if (!h || !down || !out) return fail(MOE_ERR_INVALID_ARG, "h, down or out is NULL");
  MOE_TRY(check_weight_align(down, "down"));
  MOE_TRY(check_out_align(out, "out"));
  launch_down(gemm_args(cfg, n_groups, inter, max_rows, h, nullptr, offsets, down, out), static_cast<hipStream_t>(stream));
  MOE_TRY(check_launch("moe_expert_down"));
  return ok();
}

int moe_expert_ffn(const moe_config* cfg, int64_t n_groups, int64_t inter, int64_t max_rows, const void* x,
                   const int32_t* row_index, const int32_t* offsets, const void* gate_up, const void* down, void* h,
                   float* out, void* stream) {
  MOE_TRY(ffn_checks(cfg, n_groups, inter, max_rows, offsets));
  if (max_rows == 0) return ok();
  if (!x || !gate_up || !down || !h || !out) return fail(MOE_ERR_INVALID_ARG, "x, gate_up, down, h or out is NULL");
  MOE_TRY(check_weight_align(gate_up, "gate_up"));
  MOE_TRY(check_weight_align(down, "down"));
  MOE_TRY(check_out_align(out, "out"));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  launch_gate_up(gemm_args(cfg, n_groups, inter, max_rows, x, row_index, offsets, gate_up, h), st);
  MOE_TRY(check_launch("moe_expert_ffn (gate_up)"));
  launch_down(gemm_args(cfg, n_groups, inter, max_rows, h, nullptr, offsets, down, out), st);
  MOE_TRY(check_launch("moe_expert_ffn (down)"));
  return ok();
}

int moe_pack_weights(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols, const void* src, void* dst,
                     void* stream) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "packing needs dtype bf16");
  if (n_groups < 0 || rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "negative size");
  if (rows % 16 || cols % 32)
    return fail(MOE_ERR_UNSUPPORTED, "packing needs rows %% 16 == 0 and cols %% 32 == 0 (got %lld x %lld)",
                (long long)rows, (long long)cols);
  if (rows > (1 << 24) || cols > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "rows/cols above 2^24");
  const int64_t n = n_groups * rows * cols;
  if (n == 0) return ok();
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "src or dst is NULL");
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + 2 * n && d0 < s0 + 2 * n) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
    return fail(MOE_ERR_UNSUPPORTED, "src and dst must be 16-byte aligned");
  launch_pack(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), n_groups, static_cast<int>(rows),
              static_cast<int>(cols), static_cast<hipStream_t>(stream));
  MOE_TRY(check_launch("moe_pack_weights"));
  return ok();
}

static int quant_shape_checks(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (quant_bits(cfg) == 0)
    return fail(MOE_ERR_INVALID_ARG, "weight_layout = %d is not a quantised layout (2, 3 or 4)", cfg->weight_layout);
  if (cfg->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "quantisation needs dtype bf16");
  if (n_groups < 0 || rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "negative size");
  if (rows % 16 || cols % 32)
    return fail(MOE_ERR_UNSUPPORTED, "quantisation needs rows %% 16 == 0 and cols %% 32 == 0 (got %lld x %lld)",
                (long long)rows, (long long)cols);
  if (rows > (1 << 24) || cols > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "rows/cols above 2^24");
  if (quant_kind(cfg) == kQInt4 && cols % 128)
    return fail(MOE_ERR_UNSUPPORTED, "int4 needs cols %% 128 == 0 (got %lld)", (long long)cols);
  return MOE_OK;
}

int moe_quantized_bytes(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols, size_t* bytes) {
  MOE_TRY(quant_shape_checks(cfg, n_groups, rows, cols));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = static_cast<size_t>(quant_code_bytes(n_groups, rows, cols, quant_bits(cfg)) + n_groups * rows * 4);
  return ok();
}

int moe_quantize_weights(const moe_config* cfg, int64_t n_groups, int64_t rows, int64_t cols, const void* src, void* dst,
                         void* stream) {
  MOE_TRY(quant_shape_checks(cfg, n_groups, rows, cols));
  const int64_t n = n_groups * rows * cols;
  if (n == 0) return ok();
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "src or dst is NULL");
  const int bits = quant_bits(cfg);
  const int64_t out_bytes = quant_code_bytes(n_groups, rows, cols, bits) + n_groups * rows * 4;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + out_bytes && d0 < s0 + 2 * n) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
    return fail(MOE_ERR_UNSUPPORTED, "src and dst must be 16-byte aligned");
  launch_quantize(static_cast<const uint16_t*>(src), static_cast<uint8_t*>(dst), n_groups, static_cast<int>(rows),
                  static_cast<int>(cols), quant_kind(cfg), static_cast<hipStream_t>(stream));
  MOE_TRY(check_launch("moe_quantize_weights"));
  return ok();
}

int moe_backward_workspace_bytes(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(backward_checks(cfg));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_layout_of(cfg).total;
  return ok();
}

int moe_backward(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up, const void* down,
                 const void* shared_gate_up, const void* shared_down, const void* w_shared_gate, const void* dy,
                 float* dx, float* dw_router, float* dgate_up, float* ddown, float* dshared_gate_up,
                 float* dshared_down, float* dw_shared_gate, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(backward_checks(cfg));
  if (cfg->n_tokens == 0) return ok();
  if (!x || !w_router || !gate_up || !down || !dy) return fail(MOE_ERR_INVALID_ARG, "x, w_router, gate_up, down or dy is NULL");
  if (!dx || !dw_router || !dgate_up || !ddown) return fail(MOE_ERR_INVALID_ARG, "dx, dw_router, dgate_up or ddown is NULL");
  const bool shared = cfg->shared_inter > 0, gated = shared && w_shared_gate;
  if (shared && (!shared_gate_up || !shared_down || !dshared_gate_up || !dshared_down))
    return fail(MOE_ERR_INVALID_ARG, "shared_inter > 0 needs shared_gate_up, shared_down and their gradients");
  if (!shared && (shared_gate_up || shared_down || w_shared_gate || dshared_gate_up || dshared_down || dw_shared_gate))
    return fail(MOE_ERR_INVALID_ARG, "shared expert tensors given with shared_inter == 0");
  if ((w_shared_gate == nullptr) != (dw_shared_gate == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "w_shared_gate and dw_shared_gate must be both set or both NULL");
  for (const void* p : {x, w_router, gate_up, down, dy, shared_gate_up, shared_down, w_shared_gate})
    if (reinterpret_cast<uintptr_t>(p) & 15) return fail(MOE_ERR_UNSUPPORTED, "inputs must be 16-byte aligned");
  for (const float* p : {dx, dw_router, dgate_up, ddown, dshared_gate_up, dshared_down, dw_shared_gate})
    if (reinterpret_cast<uintptr_t>(p) & 15) return fail(MOE_ERR_UNSUPPORTED, "gradient outputs must be 16-byte aligned");
  const BwdLayout L = bwd_layout_of(cfg);
  if (!ws || ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MOE_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);

  char* base = static_cast<char*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
  auto PV = [&](size_t off) { return static_cast<void*>(base + off); };        // layer-dtype buffers
  const bool f32 = cfg->dtype == MOE_F32, bf = !f32;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t N = cfg->n_tokens, A = N * cfg->top_k;
  const int E = static_cast<int>(cfg->n_experts), D = static_cast<int>(cfg->hidden), I = static_cast<int>(cfg->inter);
  const int Ep = static_cast<int>(L.Ep);
  int32_t* offsets = I32(L.offsets);
  int32_t* token_of = I32(L.token_of);

  // forward pieces: routing (with logits), grouping, pre-activations z = [a | b]
  float* g = gated ? F(L.sh_scale) : nullptr;                 // shared-expert gate sigmoid(w_s . x)
  MOE_TRY(route_impl(cfg, x, w_router, gated ? w_shared_gate : nullptr, F(L.logits), F(L.weights), I32(L.experts), g,
                     route_partial_bytes(cfg) ? F(L.route_partial) : nullptr, st));
  MOE_TRY(permute_impl(cfg, I32(L.experts), nullptr, I32(L.counts), offsets, token_of, I32(L.slot_pos), nullptr,
                       I32(L.block_counts), st));
  launch_scatter_assign(I32(L.slot_pos), F(L.weights), F(L.w_perm), I32(L.assign_of), F(L.ones), A, st);
  launch_pad_offsets(I32(L.counts), I32(L.poff), E, st);
  // The products with transposed weights (dh = dy W_down, dx = [da | db] W_gate_up) read the weights
  // in their stored layout: short groups (a few rows per expert) through launch_kstream, tall groups
  // through the streaming GEMM's [K][N] mode; other shapes through transposed copies (kn_args).
  const BwdPlan P = bwd_plan_of(cfg);
  const bool short_groups = P.short_groups, ks_dh = P.ks_dh, ks_dx = P.ks_dx;
  GemmArgs dh_args{}, dx_args{};
  if (!ks_dh) dh_args = kn_args(dy, token_of, offsets, E, A, down, P.copy_dn, PV(L.dnT), I, D, F(L.dhu), bf, st);
  if (!ks_dx)
    dx_args = kn_args(PV(L.dab), nullptr, offsets, E, A, gate_up, P.copy_gu, PV(L.guT), D, 2 * I, F(L.dx_rows), bf, st);
  launch_transpose_mat(w_router, PV(L.wrT), 1, E, D, Ep, f32, st);               // [D, Ep]
  MOE_TRY(check_launch("moe_backward (setup)"));
  if (!P.fused_swiglu) launch_down(nt_args(x, token_of, offsets, E, A, gate_up, 2 * I, D, F(L.z), bf), st);
  if (ks_dh)
    launch_kstream(static_cast<const uint16_t*>(dy), token_of, offsets, E, static_cast<const uint16_t*>(down), D, I, F(L.dhu), st);
  else
    launch_down(dh_args, st);
  // expert and router gradients of the activations: h, [da | db] and dw = dhu . h
  if (P.fused_swiglu) {
    GemmArgs gu = gemm_args(cfg, E, I, A, x, token_of, offsets, gate_up, PV(L.h));
    gu.bwd_dhu = F(L.dhu);
    gu.bwd_w = F(L.w_perm);
    gu.bwd_dab = PV(L.dab);
    gu.bwd_dwp = F(L.dwp);
    launch_gate_up(gu, st);
    launch_dw_sum(F(L.dwp), static_cast<int>((I + 31) / 32), I32(L.assign_of), A, F(L.dw), st);
  } else {
    launch_swiglu_bwd(F(L.z), F(L.dhu), F(L.w_perm), I32(L.assign_of), offsets + E, A, I, PV(L.h), PV(L.dab), F(L.dw),
                      f32, st);
  }
  MOE_TRY(check_launch("moe_backward (recompute)"));
  launch_router_bwd(F(L.logits), F(L.weights), I32(L.experts), F(L.dw), N, E, Ep, static_cast<int>(cfg->top_k),
                    cfg->norm_topk_prob, PV(L.dlogit), f32, st);
  if (ks_dx)
    launch_kstream(static_cast<const uint16_t*>(PV(L.dab)), nullptr, offsets, E, static_cast<const uint16_t*>(gate_up), 2 * I,
                   D, F(L.dx_rows), st);
  else
    launch_down(dx_args, st);
  launch_down(nt_args(PV(L.dlogit), nullptr, nullptr, 1, N, PV(L.wrT), D, Ep, F(L.dxr), bf), st);
  const int Is = static_cast<int>(cfg->shared_inter);
  if (shared) {
    // the shared expert as one group of all N tokens with row weight g (1 ungated), then its gate
    const GemmArgs dhs_args =
        kn_args(dy, nullptr, nullptr, 1, N, shared_down, P.copy_sdn, PV(L.sdnT), Is, D, F(L.dhus), bf, st);
    const GemmArgs dxs_args =
        kn_args(PV(L.dabs), nullptr, nullptr, 1, N, shared_gate_up, P.copy_sgu, PV(L.sguT), D, 2 * Is, F(L.dxs), bf, st);
    launch_down(nt_args(x, nullptr, nullptr, 1, N, shared_gate_up, 2 * Is, D, F(L.zs), bf), st);
    launch_down(dhs_args, st);
    launch_swiglu_bwd(F(L.zs), F(L.dhus), gated ? g : F(L.ones), nullptr, nullptr, N, Is, PV(L.hs), PV(L.dabs),
                      F(L.sdot), f32, st);
    launch_down(dxs_args, st);
    if (gated) launch_shared_gate_bwd(F(L.sdot), g, N, L.Ns, F(L.dz), PV(L.dz_row), f32, st);
    launch_add_rows(F(L.dxr), F(L.dxs), gated ? F(L.dz) : nullptr, w_shared_gate, f32, N, D, st);
    MOE_TRY(check_launch("moe_backward (shared expert)"));
  }
  moe_config c32 = *cfg;
  c32.out_dtype = MOE_F32;
  c32.expert_out = MOE_EXPERT_OUT_F32;          // dx rows are fp32 whatever form the forward keeps
  MOE_TRY(combine_impl(&c32, F(L.dx_rows), F(L.ones), I32(L.slot_pos), F(L.dxr), nullptr, dx, st));
  // weight gradients over each expert's rows (bf16 with D, I multiples of 8: read in place;
  // otherwise through padded transposes), then over the tokens for W_r
  const int32_t* poff = I32(L.poff);
  const int n1 = static_cast<int>(N);
  const bool rows_wgrad = P.rows_wgrad;
  if (!rows_wgrad) {
    launch_transpose_rows(dy, D, token_of, F(L.w_perm), offsets, poff, E, 0, L.Qs, PV(L.doT), L.Qs, f32, st);
    launch_transpose_rows(x, D, token_of, nullptr, offsets, poff, E, 0, L.Qs, PV(L.xgT), L.Qs, f32, st);
    launch_transpose_rows(PV(L.h), I, nullptr, nullptr, offsets, poff, E, 0, L.Qs, PV(L.hT), L.Qs, f32, st);
    launch_transpose_rows(PV(L.dab), 2 * I, nullptr, nullptr, offsets, poff, E, 0, L.Qs, PV(L.dabT), L.Qs, f32, st);
  }
  launch_transpose_rows(PV(L.dlogit), Ep, nullptr, nullptr, nullptr, nullptr, 1, n1, L.Ns, PV(L.dlogitT), L.Ns, f32, st);
  launch_transpose_rows(x, D, nullptr, nullptr, nullptr, nullptr, 1, n1, L.Ns, PV(L.xT), L.Ns, f32, st);
  MOE_TRY(check_launch("moe_backward (transposes)"));
  // out[g] = A_g B_g^T over the padded rows: matrix cores for bf16, FMAs for fp32 layers; one long
  // group (the sums over all tokens) split in slices on the bf16 path
  auto wgrad = [&](size_t a_off, size_t b_off, int64_t ld, const int32_t* po, int G, int M, int Nn, float* out) {
    if (f32)
      launch_wgrad_f32(F(a_off), F(b_off), ld, po, po ? 0 : ld, G, M, Nn, out, st);
    else if (po)
      launch_wgrad(static_cast<const uint16_t*>(PV(a_off)), static_cast<const uint16_t*>(PV(b_off)), ld, po, 0, G, M, Nn, out, st);
    else
      launch_wgrad_split(static_cast<const uint16_t*>(PV(a_off)), static_cast<const uint16_t*>(PV(b_off)), ld, ld, M, Nn,
                         kWgradSlices, I32(L.spoff), F(L.wr_part), out, st);
  };
  if (rows_wgrad) {
    // dDn_e = sum_p (w dy[token])^T h, dGU_e = sum_p [da | db]^T x[token]
    // tall groups: the longest sums start first (short groups have no long tail to avoid)
    static_assert(kMaxExperts <= 1024, "launch_group_order ranks up to 1024 groups");
    if (!short_groups) launch_group_order(I32(L.counts), static_cast<int>(E), I32(L.gorder), st);
    WgradRowsArgs wd{};
    wd.order = short_groups ? nullptr : I32(L.gorder);
    wd.A = static_cast<const uint16_t*>(dy);
    wd.lda = D;
    wd.ga = token_of;
    wd.scale = F(L.w_perm);
    wd.B = static_cast<const uint16_t*>(PV(L.h));
    wd.ldb = I;
    wd.off = offsets;
    wd.M = D;
    wd.Nn = I;
    wd.out = ddown;
    launch_wgrad_rows(wd, E, st);
    WgradRowsArgs wg{};
    wg.order = wd.order;
    wg.A = static_cast<const uint16_t*>(PV(L.dab));
    wg.lda = 2 * I;
    wg.B = static_cast<const uint16_t*>(x);
    wg.ldb = D;
    wg.gb = token_of;
    wg.off = offsets;
    wg.M = 2 * I;
    wg.Nn = D;
    wg.out = dgate_up;
    launch_wgrad_rows(wg, E, st);
  } else {
    wgrad(L.doT, L.hT, L.Qs, poff, E, D, I, ddown);
    wgrad(L.dabT, L.xgT, L.Qs, poff, E, 2 * I, D, dgate_up);
  }
  wgrad(L.dlogitT, L.xT, L.Ns, nullptr, 1, E, D, dw_router);
  if (shared) {
    launch_transpose_rows(dy, D, nullptr, g, nullptr, nullptr, 1, n1, L.Ns, PV(L.dysT), L.Ns, f32, st);
    launch_transpose_rows(PV(L.hs), Is, nullptr, nullptr, nullptr, nullptr, 1, n1, L.Ns, PV(L.hsT), L.Ns, f32, st);
    launch_transpose_rows(PV(L.dabs), 2 * Is, nullptr, nullptr, nullptr, nullptr, 1, n1, L.Ns, PV(L.dabsT), L.Ns, f32, st);
    wgrad(L.dysT, L.hsT, L.Ns, nullptr, 1, D, Is, dshared_down);
    wgrad(L.dabsT, L.xT, L.Ns, nullptr, 1, 2 * Is, D, dshared_gate_up);
    if (gated) wgrad(L.dz_row, L.xT, L.Ns, nullptr, 1, 1, D, dw_shared_gate);
  }
  MOE_TRY(check_launch("moe_backward (weight gradients)"));
  return ok();
}

int moe_router_stats(const moe_config* cfg, const float* logits, const int32_t* counts, float* f, float* P,
                     float* loss, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (!f || !P || !loss) return fail(MOE_ERR_INVALID_ARG, "f, P or loss is NULL");
  const int64_t N = cfg->n_tokens;
  if (N > 0 && (!logits || !counts)) return fail(MOE_ERR_INVALID_ARG, "logits or counts is NULL");
  const size_t need = stats_ws_bytes(cfg);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0, need);
  launch_stats(logits, counts, f, P, loss, static_cast<float*>(ws), N, static_cast<int>(cfg->n_experts),
               static_cast<int>(cfg->top_k), static_cast<hipStream_t>(stream));
  MOE_TRY(check_launch("moe_router_stats"));
  return ok();
}

int moe_router_bias_update(const moe_config* cfg, const int32_t* counts, float* bias, float gamma, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (!counts || !bias) return fail(MOE_ERR_INVALID_ARG, "counts or bias is NULL");
  if (!(gamma >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "gamma must be >= 0");
  launch_bias_update(counts, bias, gamma, cfg->n_tokens * cfg->top_k, static_cast<int>(cfg->n_experts),
                     static_cast<hipStream_t>(stream));
  MOE_TRY(check_launch("moe_router_bias_update"));
  return ok();
}

int moe_combine(const moe_config* cfg, const float* out_perm, const float* weights, const int32_t* slot_pos,
                const float* shared_out, const float* shared_scale, void* y, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (cfg->n_tokens == 0) return ok();
  if (!out_perm || !weights || !slot_pos || !y) return fail(MOE_ERR_INVALID_ARG, "out_perm, weights, slot_pos or y is NULL");
  if (shared_scale && !shared_out) return fail(MOE_ERR_INVALID_ARG, "shared_scale given without shared_out");
  MOE_TRY(check_out_align(out_perm, "out_perm"));
  if (shared_out) MOE_TRY(check_out_align(shared_out, "shared_out"));
  MOE_TRY(combine_impl(cfg, out_perm, weights, slot_pos, shared_out, shared_scale, y, static_cast<hipStream_t>(stream)));
  return ok();
}

// Argument checks of moe_forward that do not involve the workspace.
static int forward_checks(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up,
                          const void* down, const void* shared_gate_up, const void* shared_down,
                          const void* w_shared_gate, void* y) {
  if (!x || !w_router || !gate_up || !down || !y) return fail(MOE_ERR_INVALID_ARG, "x, w_router, gate_up, down or y is NULL");
  MOE_TRY(check_weight_align(gate_up, "gate_up"));
  MOE_TRY(check_weight_align(down, "down"));
  if (shared_gate_up) MOE_TRY(check_weight_align(shared_gate_up, "shared_gate_up"));
  if (shared_down) MOE_TRY(check_weight_align(shared_down, "shared_down"));
  if (cfg->shared_inter > 0 && (!shared_gate_up || !shared_down))
    return fail(MOE_ERR_INVALID_ARG, "shared_inter > 0 needs shared_gate_up and shared_down");
  if (cfg->shared_inter == 0 && (shared_gate_up || shared_down || w_shared_gate))
    return fail(MOE_ERR_INVALID_ARG, "shared expert tensors given with shared_inter == 0");
  return MOE_OK;
}

// The block on a checked, large-enough, 256-byte aligned workspace.
// fork: the shared expert may run on the device's side stream (not for moe_forward_noalloc, which
// creates nothing).
static int forward_impl(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up, const void* down,
                        const void* shared_gate_up, const void* shared_down, const void* w_shared_gate, void* y,
                        float* weights_out, int32_t* experts_out, void* ws, void* stream, bool fork) {
  const Layout L = layout_of(cfg);
  char* base = static_cast<char*>(ws);
  float* weights = weights_out ? weights_out : reinterpret_cast<float*>(base + L.weights);
  int32_t* experts = experts_out ? experts_out : reinterpret_cast<int32_t*>(base + L.experts);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* token_of = reinterpret_cast<int32_t*>(base + L.token_of);
  int32_t* slot_pos = reinterpret_cast<int32_t*>(base + L.slot_pos);
  float* shared_scale = (cfg->shared_inter && w_shared_gate) ? reinterpret_cast<float*>(base + L.shared_scale) : nullptr;
  void* h = base + L.h;
  float* out = reinterpret_cast<float*>(base + L.out);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t A = cfg->n_tokens * cfg->top_k;

  // the shared expert first: on the side stream where there is one (fork), else ahead on st
  float* sh_out = nullptr;
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock;
  if (cfg->shared_inter > 0) {
    void* sh_h = base + L.sh_h;
    sh_out = reinterpret_cast<float*>(base + L.sh_out);
    hipStream_t ss = st;
    int dev = -1;
    if (fork && hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
      side_lock = std::unique_lock<std::mutex>(g_side_mu[dev]);
      side = side_stream_locked(dev);
      if (side) {
        MOE_TRY(hip_ok(hipEventRecord(side->fork, st), "moe_forward (fork of the shared expert)"));
        MOE_TRY(hip_ok(hipStreamWaitEvent(side->stream, side->fork, 0), "moe_forward (fork of the shared expert)"));
        ss = side->stream;
      }
    }
    launch_gate_up(gemm_args(cfg, 1, cfg->shared_inter, cfg->n_tokens, x, nullptr, nullptr, shared_gate_up, sh_h), ss);
    MOE_TRY(check_launch("moe_forward (shared gate_up)"));
    launch_down(gemm_args(cfg, 1, cfg->shared_inter, cfg->n_tokens, sh_h, nullptr, nullptr, shared_down, sh_out), ss);
    MOE_TRY(check_launch("moe_forward (shared down)"));
    if (side) MOE_TRY(hip_ok(hipEventRecord(side->join, ss), "moe_forward (join of the shared expert)"));
  }

  float* partial = L.route_partial == L.block_counts ? nullptr : reinterpret_cast<float*>(base + L.route_partial);
  MOE_TRY(route_impl(cfg, x, w_router, shared_scale ? w_shared_gate : nullptr, nullptr, weights, experts, shared_scale,
                     route_partial_bytes(cfg) ? partial : nullptr, st));
  MOE_TRY(permute_impl(cfg, experts, nullptr, counts, offsets, token_of, slot_pos, nullptr,
                       reinterpret_cast<int32_t*>(base + L.block_counts), st));
  launch_gate_up(gemm_args(cfg, cfg->n_experts, cfg->inter, A, x, token_of, offsets, gate_up, h), st);
  MOE_TRY(check_launch("moe_forward (gate_up)"));
  launch_down(gemm_args(cfg, cfg->n_experts, cfg->inter, A, h, nullptr, offsets, down, out), st);
  MOE_TRY(check_launch("moe_forward (down)"));
  if (side) MOE_TRY(hip_ok(hipStreamWaitEvent(st, side->join, 0), "moe_forward (join of the shared expert)"));
  MOE_TRY(combine_impl(cfg, out, weights, slot_pos, sh_out, shared_scale, y, st));
  return ok();
}

int moe_forward(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up, const void* down,
                const void* shared_gate_up, const void* shared_down, const void* w_shared_gate, void* y,
                float* weights_out, int32_t* experts_out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (cfg->n_tokens == 0) return ok();
  MOE_TRY(forward_checks(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, y));
  const size_t need = layout_of(cfg).total;
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MOE_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
  return forward_impl(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, y, weights_out,
                      experts_out, ws, stream, true);
}

int moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router, const void* gate_up,
                        const void* down, const void* shared_gate_up, const void* shared_down,
                        const void* w_shared_gate, void* y, float* weights_out, int32_t* experts_out, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (cfg->n_tokens == 0) return ok();
  MOE_TRY(forward_checks(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, y));
  const size_t need = layout_of(cfg).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "moe_forward_noalloc: this layer needs %zu bytes of scratch, above the library's "
                "fixed %zu (use moe_forward with a caller workspace)", need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(&ws));
  return forward_impl(cfg, x, w_router, gate_up, down, shared_gate_up, shared_down, w_shared_gate, y, weights_out,
                      experts_out, ws, stream, false);
}

}  // extern "C"
