// Device helpers shared by the MoE kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16 bits, round to nearest, ties to even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One 32x32x16 bf16 matrix-core step: acc[32x32] += A[32x16] * B[16x32].
// Lane l supplies A row (l % 32) and B column (l % 32), eight consecutive k values each from
// k-group (l / 32); any k order works as long as A and B use the same one.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}

// One 16x16x32 bf16 step: acc[16x16] += A[16x32] * B[32x16]; lane l supplies A row / B column
// (l % 16) with eight k values from k-group (l / 16). Result: element i of lane l holds row
// 4*(l/16) + i, column l % 16.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}

// A 32x32x16 operand from an LDS tile stored k-major: ROW bf16 per k-row, 32-byte chunks placed at
// chunk ^ ((2 row) & 7). Returns what a plain read of the [n][k] layout gives: lane l holds column
// n0 + l % 32 at k = 16 kk + 8 (l / 32) .. + 7. ds_read_b64_tr_b16 hands lane 16 G + 4 a + b (16-lane
// group G) element b of the 8-byte pieces addressed by lanes 16 G + a + 4 t, t = 0..3, so address
// lane 16 G + r points at k-row 16 kk + 8 (G / 2) + r / 4 (+ 4 in the second read) and columns
// n0 + 16 (G % 2) + 4 (r % 4) .. + 3. A half-wave touches four consecutive rows by two chunks; the
// swizzle puts those eight chunks on distinct banks when ROW * 2 bytes is a multiple of 256.
template <int ROW>
__device__ __forceinline__ u32x4 lds_tr_frag(const uint16_t* s, int kk, int n0, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int gq = lane >> 4, rq = lane & 15;
  const int krow = kk * 16 + 8 * (gq >> 1) + (rq >> 2);
  const int ncol = n0 + 16 * (gq & 1) + 4 * (rq & 3);
  u32x2 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = krow + 4 * h;
    const int idx = kr * ROW + (((ncol >> 4) ^ ((2 * kr) & 7)) << 4) + (ncol & 15);
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(s) + idx));
    v[h] = __builtin_bit_cast(u32x2, t);
  }
  return u32x4{v[0][0], v[0][1], v[1][0], v[1][1]};
}

// Accumulator layout of the 32x32 matrix-core result: element i of lane l holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l % 32.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave-wide reductions with DPP row operations (VALU, no LDS traffic): swap neighbours, swap pairs,
// mirror within 8, mirror within 16 -> every lane holds its 16-lane row's result; the four row
// results are then combined from lanes 15, 31, 47, 63 in a fixed order, so the result is the same
// in every lane and deterministic.
#define MOE_DPP(v, ctrl) __builtin_amdgcn_update_dpp(0, (v), (ctrl), 0xF, 0xF, false)
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <typename Op>
__device__ __forceinline__ float wave_reduce_f(float v, Op op) {
  v = op(v, __int_as_float(MOE_DPP(__float_as_int(v), kDppXor1)));
  v = op(v, __int_as_float(MOE_DPP(__float_as_int(v), kDppXor2)));
  v = op(v, __int_as_float(MOE_DPP(__float_as_int(v), kDppHalfMirror)));
  v = op(v, __int_as_float(MOE_DPP(__float_as_int(v), kDppMirror)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  return wave_reduce_f(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return wave_reduce_f(v, [](float a, float b) { return a + b; });
}

// Exchange with lane ^ m inside each 16-lane row (m = 1, 2, 4, 8), in registers: m = 1, 2 are quad
// permutes; m = 4, 8 take the row shifted left (lanes with bit m clear, their partner is above) or
// right (bit set). Only in-row sources are ever selected.
template <int M>
__device__ __forceinline__ int xor16(int v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "row-local exchange");
  if constexpr (M == 1) return MOE_DPP(v, kDppXor1);
  else if constexpr (M == 2) return MOE_DPP(v, kDppXor2);
  else {
    const int up = MOE_DPP(v, 0x100 + M);      // row_shl:M  (lane i <- lane i + M)
    const int dn = MOE_DPP(v, 0x110 + M);      // row_shr:M  (lane i <- lane i - M)
    return (__lane_id() & M) ? dn : up;
  }
}
template <int M>
__device__ __forceinline__ float xor16f(float v) { return __int_as_float(xor16<M>(__float_as_int(v))); }

// Wave-wide arg-max over (p, e) pairs: larger p wins, equal p goes to the lower e.
__device__ __forceinline__ void argmax_step(float& p, int& e, float op, int oe) {
  if (op > p || (op == p && oe < e)) { p = op; e = oe; }
}
__device__ __forceinline__ void wave_argmax_dpp(float& p, int& e) {
  argmax_step(p, e, __int_as_float(MOE_DPP(__float_as_int(p), kDppXor1)), MOE_DPP(e, kDppXor1));
  argmax_step(p, e, __int_as_float(MOE_DPP(__float_as_int(p), kDppXor2)), MOE_DPP(e, kDppXor2));
  argmax_step(p, e, __int_as_float(MOE_DPP(__float_as_int(p), kDppHalfMirror)), MOE_DPP(e, kDppHalfMirror));
  argmax_step(p, e, __int_as_float(MOE_DPP(__float_as_int(p), kDppMirror)), MOE_DPP(e, kDppMirror));
  float bp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 15));
  int be = __builtin_amdgcn_readlane(e, 15);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    argmax_step(bp, be, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 16 * r + 15)),
                __builtin_amdgcn_readlane(e, 16 * r + 15));
  p = bp;
  e = be;
}

// z * sigmoid(z) with the hardware exp and reciprocal (each within a couple of ulp of fp32; the
// result is rounded to bf16 right after, or accumulated in fp32 for fp32 layers).
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's 16 bytes land
// at lds_dst + 16 l, so one instruction fills 1 KB of LDS contiguously; lds_dst must be uniform.
// Issued as inline asm so the compiler inserts no waits for it: callers order it with an explicit
// s_waitcnt vmcnt(n) and a barrier. (Loads return in issue order, so the compiler's own vmcnt
// waits for its loads stay conservative with these in the queue.)
__device__ __forceinline__ void dma16(const void* src, const void* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)lds_dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory");
#endif
}

// dma16 from a uniform base (SGPRs) plus this lane's 32-bit byte offset: one VGPR per source
// instead of a 64-bit address.
__device__ __forceinline__ void dma16_sv(const void* base, uint32_t voff, const void* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)lds_dst));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory");
#endif
}

// The same for 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes land at lds_dst + 4 l, so
// one instruction fills 256 bytes of LDS contiguously.
__device__ __forceinline__ void dma4(const void* src, const void* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)lds_dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(base) : "memory");
#endif
}

// Weight-only quantised codes -> eight bf16 matrix-core inputs, exactly (|code| <= 127 fits bf16's
// 8-bit significand); the row's scale is applied to the fp32 sum afterwards.
// int8: eight signed bytes, code i in byte i; int4: eight signed nibbles, code i in bits 4i..4i+3.
__device__ __forceinline__ u32x4 codes8_to_bf16(u32x2 c) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(static_cast<int32_t>(c[i >> 2] << (24 - 8 * (i & 3))) >> 24);
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}
__device__ __forceinline__ u32x4 codes4_to_bf16(uint32_t c) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(static_cast<int32_t>(c << (28 - 4 * i)) >> 28);
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// int4 words: eight codes k = 0..7 of one row at consecutive columns, code k as the nibble
// code + 8 (0..15) in byte k % 4, low nibble for k < 4, high nibble for k >= 4.
// With their group multiplier m (0..32): code * m exactly as bf16 (an integer of magnitude <= 224).
__device__ __forceinline__ u32x4 codes4m_to_bf16(uint32_t c, uint32_t m) {
  const float fm = static_cast<float>(m), off = -8.f * fm;
  uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
  // opaque to the compiler, so that each code converts with one byte-to-float instruction instead
  // of a 4-bit field extract and a conversion
  asm("" : "+v"(lo), "+v"(hi));
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[k] = fmaf(static_cast<float>((lo >> (8 * k)) & 0xffu), fm, off);
    f[k + 4] = fmaf(static_cast<float>((hi >> (8 * k)) & 0xffu), fm, off);
  }
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}
// The same word as the bf16 values 136 + code (128 + the stored nibble): each 16-bit half is the
// byte 0x43 over a nibble, so one byte permute builds two of them. A product with these weights
// exceeds the one with the codes by 136 times the sum of the other operand.
__device__ __forceinline__ u32x4 codes4_biased_bf16(uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
  constexpr uint32_t kTop = 0x43434343u;
  return u32x4{__builtin_amdgcn_perm(kTop, lo, 0x04010400u), __builtin_amdgcn_perm(kTop, lo, 0x04030402u),
               __builtin_amdgcn_perm(kTop, hi, 0x04010400u), __builtin_amdgcn_perm(kTop, hi, 0x04030402u)};
}

// FP8 (OCP e4m3) codes -> bf16, exactly (3-bit mantissa, exponents 2^-9 .. 2^8 inside bf16's range):
// code i in byte i, converted by the hardware e4m3 -> fp32 instruction two at a time.
__device__ __forceinline__ u32x4 codesf8_to_bf16(u32x2 c) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c[h]), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c[h]), true);
    r[2 * h] = pack_bf16x2(lo[0], lo[1]);
    r[2 * h + 1] = pack_bf16x2(hi[0], hi[1]);
  }
  return r;
}

// fp16 form of expert outputs: the exponent of a 16-column group whose largest magnitude is m:
// floor(log2 m) - 14 (so every value scaled by 2^-exp is below 2^15), at least -128; 0 when m is
// zero or not finite.
__device__ __forceinline__ int f16s_exp(float m) {
  const int be = static_cast<int>((__float_as_uint(m) >> 23) & 0xff);   // m >= 0
  if (m == 0.f || be == 0xff) return 0;
  return max(be - 127 - 14, -128);
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// v * 2^-e rounded to fp16 (nearest, ties to even), two at a time
__device__ __forceinline__ uint32_t pack_f16x2_scaled(float a, float b, int e) {
  const f16x2 v = {static_cast<_Float16>(ldexpf(a, -e)), static_cast<_Float16>(ldexpf(b, -e))};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f16_scaled(float a, int e) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(ldexpf(a, -e)));
}
// the value of an fp16 code (bits) with exponent e, exactly
__device__ __forceinline__ float f16_unscale(uint16_t bits, int e) {
  return ldexpf(static_cast<float>(__builtin_bit_cast(_Float16, bits)), e);
}

// s_waitcnt immediate for vmcnt(n) alone (bits 3:0 and 15:14; expcnt and lgkmcnt at "no wait").
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace moe
