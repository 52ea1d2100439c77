// Measured ceilings of the machine, for the benchmark to report beside the published peaks: the
// HBM read rate a plain streaming kernel sustains, and the bf16 matrix-core rate of a loop that
// keeps its operands in registers (no memory or LDS traffic, so it runs at the clock the chip holds
// under matrix-core load). Not part of the MoE library; built as its own small shared library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Read of n16 16-byte vectors, U loads in flight per lane: each workgroup streams one contiguous
// chunk (256 threads x U vectors per step); one word per workgroup is written so the loads are not
// removed. kNT: nontemporal loads.
template <int U, bool kNT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 / gridDim.x) & ~static_cast<int64_t>(256 * U - 1);       // this workgroup's share
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per, hi = lo + per;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i + (U - 1) * 256 < hi; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = kNT ? __builtin_nontemporal_load(&src[i + u * 256]) : src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (blockIdx.x == 0) {                          // the tail past the workgroups' equal shares
    for (int64_t i = per * gridDim.x + threadIdx.x; i < n16; i += 256) {
      const u32x4 v = src[i];
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  __shared__ uint32_t s[256];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= s[t];
    sink[blockIdx.x] = r;
  }
}

// Four independent chains of 32x32x16 bf16 matrix-core steps per wave, iters steps each.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t one = 0x3F80u + static_cast<uint32_t>(lane & 1);   // bf16 1.0 or 1.0078125
  const u32x4 bits = {one | (one << 16), one | (one << 16), one | (one << 16), one | (one << 16)};
  const bf16x8 a = __builtin_bit_cast(bf16x8, bits);
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from src with `grid` workgroups of 256 threads; sink holds grid
// words. Returns 0, or the HIP error of the launch.
// mode: 0 / 1 = 4 / 8 loads in flight per lane, + 2 for nontemporal loads.
int probe_read(const void* src, int64_t bytes, uint32_t* sink, int grid, int mode, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || grid < 1 || mode < 0 || mode > 3) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s16 = static_cast<const u32x4*>(src);
  switch (mode) {
    case 0: read_kernel<4, false><<<grid, 256, 0, st>>>(s16, bytes / 16, sink); break;
    case 1: read_kernel<8, false><<<grid, 256, 0, st>>>(s16, bytes / 16, sink); break;
    case 2: read_kernel<4, true><<<grid, 256, 0, st>>>(s16, bytes / 16, sink); break;
    default: read_kernel<8, true><<<grid, 256, 0, st>>>(s16, bytes / 16, sink); break;
  }
  return static_cast<int>(hipGetLastError());
}

// grid workgroups of four waves, each wave 4 * iters matrix-core steps of 32 x 32 x 16 (32,768
// FLOP each); sink holds 4 * grid floats.
int probe_mfma(float* sink, int iters, int grid, void* stream) {
  if (!sink || iters < 1 || grid < 1) return -1;
  mfma_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return static_cast<int>(hipGetLastError());
}

}
