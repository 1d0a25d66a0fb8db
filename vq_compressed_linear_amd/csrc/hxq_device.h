// Device helpers shared by the libhxq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hxq {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct SidecarView {
  const int32_t* rows;
  const int32_t* cols;
  const float* deltas;
  int64_t nnz;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Byte b of w placed at bits 15:8, `lo` (a lane offset < 256) at bits 7:0, zero above:
// the LDS byte address of entry w.byte[b] in a table with a 256-byte stride per entry.
template <int B>
__device__ __forceinline__ uint32_t byte_addr256(uint32_t w, uint32_t lo) {
  // v_perm_b32: selector bytes 0..3 pick from `lo`, 4..7 from `w`, 0x0c gives 0.
  constexpr uint32_t sel = 0x0c0c0000u | ((4u + B) << 8) | 0x00u;
  return __builtin_amdgcn_perm(w, lo, sel);
}

template <typename T>
__device__ __forceinline__ T lds_load(uint32_t byte_addr, const unsigned char* base) {
  return *reinterpret_cast<const T*>(base + byte_addr);
}

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// First sidecar entry with row >= target, searched by one wave in parallel:
// each round the 64 lanes probe 64 evenly spaced positions of [lo, hi).
// Every lane returns the same value.
__device__ __forceinline__ int64_t wave_lower_bound_rows(const int32_t* rows, int64_t nnz,
                                                         int32_t target) {
  int64_t lo = 0, hi = nnz;
  const int lane = lane_id();
  while (hi - lo > kWave) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int64_t p = lo + lane * step;
    const bool below = (p < hi) && (rows[p] < target);
    const uint64_t mask = __ballot(below);
    const int c = __popcll(mask);
    if (c == 0) return lo;
    const int64_t nlo = lo + (int64_t)(c - 1) * step + 1;
    const int64_t nhi = lo + (int64_t)c * step;
    lo = nlo;
    hi = nhi < hi ? nhi : hi;
  }
  const int64_t p = lo + lane;
  const bool below = (p < hi) && (rows[p] < target);
  return lo + __popcll(__ballot(below));
}

}  // namespace hxq
