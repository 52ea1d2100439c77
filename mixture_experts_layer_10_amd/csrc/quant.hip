// Weight-only quantisation of expert weights, done once at model load ("Qwen3-VL-MoE" Keras port,
// section "Lower memory": weight-only int8 checkpoints computing in bf16; "27. Mixture of experts",
// section "Dispatch" and stretch exercise 3: experts quantised to 4 bits, router left in bf16).
//
// Symmetric absmax per output row: scale = max|w| / Q in fp32, code = clamp(rint(w / scale), -Q, Q)
// with Q = 127 (int8) or 7 (int4); an all-zero row gets scale 0 and codes 0. Both divisions are
// IEEE fp32 divisions (correctly rounded) and rint ties to even, so the integer codes are fully
// determined by the bf16 inputs. FP8 ("Qwen3-VL + MoE: train to deploy", an FP8 copy of the
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
  constexpr float kQ = kKind == kQFp8 ? 448.f : kKind == kQInt8 ? 127.f : 7.f;
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
    if constexpr (code_slot(kKind) == 8) {
      u32x2 out;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        out[h] = static_cast<uint32_t>(code[4 * h] & 0xff) | (static_cast<uint32_t>(code[4 * h + 1] & 0xff) << 8) |
                 (static_cast<uint32_t>(code[4 * h + 2] & 0xff) << 16) | (static_cast<uint32_t>(code[4 * h + 3] & 0xff) << 24);
      *reinterpret_cast<u32x2*>(dst + block * 512 + slot * 8) = out;
    } else {
      uint32_t out = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) out |= static_cast<uint32_t>(code[i] & 0xf) << (4 * i);
      *reinterpret_cast<uint32_t*>(dst + block * 256 + slot * 4) = out;
    }
  }
  if (lane == 0) reinterpret_cast<float*>(dst + code_bytes)[row] = scale;
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
    quantize_kernel<kQInt4><<<grid, 256, 0, st>>>(src, dst, rows, R, K, cb);
}

}  // namespace moe
