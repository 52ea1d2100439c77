// Weight-only quantisation of expert weights, done once at model load ("Qwen3-VL-MoE" Keras port,
// section "Lower memory": weight-only int8 checkpoints computing in bf16; "27. Mixture of experts",
// section "Dispatch" and stretch exercise 3: experts quantised to 4 bits, router left in bf16).
//
// int8: symmetric absmax per output row, scale = max|w| / 127 in fp32, code = clamp(rint(w / scale),
// -127, 127); an all-zero row gets scale 0 and codes 0. int4: a step per 32-column group written as
// the row's scale s = max|w| / 224 times an integer multiplier mult = min(ceil(max|w_group| / (7 s)),
// 32), code = clamp(rint(w / (s mult)), -7, 7) (codes times multipliers stay exact bf16 integers).
// Every division is an IEEE fp32 division (correctly rounded) and rint ties to even, so codes and
// multipliers are fully determined by the bf16 inputs. FP8 ("Qwen3-VL + MoE: train to deploy", an FP8 copy of the
// model): scale = max|w| / 448, code = the OCP e4m3 byte nearest to clamp(w / scale, -448, 448)
// (the hardware conversion: nearest, ties to even, sign of zero kept).
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per (group, row): lane l takes the 8-column chunks l, l + 64, ... (16-byte loads); the
// row maximum is a wave reduction (exact: max does not depend on order). Chunk c of row r is slot
// (r % 16) + 16 (c % 4) of block (g, r / 16, c / 4).
template <int kKind>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       int64_t rows_total, int R, int K, int64_t code_bytes) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows_total) return;
  const int lane = threadIdx.x & 63;
  static_assert(kKind == kQFp8 || kKind == kQInt8, "int4 has its own kernel");
  constexpr float kQ = kKind == kQFp8 ? 448.f : 127.f;
  const int64_t g = row / R;
  const int r = static_cast<int>(row - g * R);
  const u32x4* w = reinterpret_cast<const u32x4*>(src + row * K);
  const int chunks = K / 8;
  float m = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 v = w[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(bf16_to_f32(static_cast<uint16_t>(v[i >> 1] >> (16 * (i & 1))))));
  }
  m = wave_max(m);
  const float scale = m / kQ;
  const int64_t rb_base = (g * (R / 16) + r / 16) * (K / 32);
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 v = w[c];
    int code[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = bf16_to_f32(static_cast<uint16_t>(v[i >> 1] >> (16 * (i & 1))));
      if constexpr (kKind == kQFp8)
        code[i] = scale > 0.f ? __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(x / scale, -kQ), kQ), 0.f, 0, false) & 0xff : 0;
      else
        code[i] = scale > 0.f ? static_cast<int>(fminf(fmaxf(rintf(x / scale), -kQ), kQ)) : 0;
    }
    const int64_t block = rb_base + c / 4;
    const int slot = (r & 15) + 16 * (c & 3);
    u32x2 out;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      out[h] = static_cast<uint32_t>(code[4 * h] & 0xff) | (static_cast<uint32_t>(code[4 * h + 1] & 0xff) << 8) |
               (static_cast<uint32_t>(code[4 * h + 2] & 0xff) << 16) | (static_cast<uint32_t>(code[4 * h + 3] & 0xff) << 24);
    *reinterpret_cast<u32x2*>(dst + block * 512 + slot * 8) = out;
  }
  if (lane == 0) reinterpret_cast<float*>(dst + code_bytes)[row] = scale;
}

// int4 with group multipliers: one wave per (group, row), lane l takes chunks l, l + 64, ... of 8
// columns; a 32-column group is four consecutive chunks, i.e. four consecutive lanes of one pass,
// which share its maximum by two exchanges. Chunk c of row r goes to super-block (g, r / 16, c / 16),
// slot (r % 16) + 16 (c % 4), bytes 4 t .. 4 t + 3 with t = (c % 16) / 4; the group's multiplier to
// byte 1024 + 4 (r % 16) + t of that super-block.
__global__ __launch_bounds__(256) void quantize_int4_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            int64_t rows_total, int R, int K, int64_t code_bytes) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows_total) return;
  const int lane = threadIdx.x & 63;
  const int64_t g = row / R;
  const int r = static_cast<int>(row - g * R);
  const u32x4* w = reinterpret_cast<const u32x4*>(src + row * K);
  const int chunks = K / 8;                     // a multiple of 16
  float m = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 v = w[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(bf16_to_f32(static_cast<uint16_t>(v[i >> 1] >> (16 * (i & 1))))));
  }
  m = wave_max(m);
  const float s = m / 224.f;
  const float unit = 7.f * s;                   // the span of one multiplier step
  const int64_t sb0 = (g * (R / 16) + r / 16) * (K / 128);
  for (int c = lane; c < chunks; c += 64) {     // the four lanes of a group run the same passes
    const u32x4 v = w[c];
    float x[8];
    float gm = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = bf16_to_f32(static_cast<uint16_t>(v[i >> 1] >> (16 * (i & 1))));
      gm = fmaxf(gm, fabsf(x[i]));
    }
    gm = fmaxf(gm, __shfl_xor(gm, 1));
    gm = fmaxf(gm, __shfl_xor(gm, 2));
    const float mult = unit > 0.f ? fminf(ceilf(gm / unit), 32.f) : 0.f;
    const float step = s * mult;
    uint32_t out = 0;                           // code i as the nibble code + 8: byte i % 4, high nibble for i >= 4
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int code = step > 0.f ? static_cast<int>(fminf(fmaxf(rintf(x[i] / step), -7.f), 7.f)) : 0;
      out |= static_cast<uint32_t>(code + 8) << (8 * (i & 3) + 4 * (i >> 2));
    }
    uint8_t* sb = dst + (sb0 + c / 16) * kQ4Super;
    const int t = (c & 15) >> 2, q8 = c & 3;
    *reinterpret_cast<uint32_t*>(sb + 16 * ((r & 15) + 16 * q8) + 4 * t) = out;
    if (q8 == 0) sb[1024 + 4 * (r & 15) + t] = static_cast<uint8_t>(mult);
  }
  if (lane == 0) reinterpret_cast<float*>(dst + code_bytes)[row] = s;
}

void launch_quantize(const uint16_t* src, uint8_t* dst, int64_t G, int R, int K, int kind, hipStream_t st) {
  const int64_t rows = G * R;
  if (rows <= 0) return;
  const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
  const int64_t cb = quant_code_bytes(G, R, K, code_bits(kind));
  if (kind == kQFp8)
    quantize_kernel<kQFp8><<<grid, 256, 0, st>>>(src, dst, rows, R, K, cb);
  else if (kind == kQInt8)
    quantize_kernel<kQInt8><<<grid, 256, 0, st>>>(src, dst, rows, R, K, cb);
  else
    quantize_int4_kernel<<<grid, 256, 0, st>>>(src, dst, rows, R, K, cb);
}

}  // namespace moe
