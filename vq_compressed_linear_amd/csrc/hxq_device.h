// Device helpers shared by the libhxq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

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

// floor(b * n / parts) for the static split of n items over `parts`
// workgroups (b <= parts): 32-bit arithmetic when the product fits, which is
// every launch plan here (a 64-bit division costs a few hundred scalar cycles
// at kernel start)
__device__ __forceinline__ int split_point(int b, int n, int parts) {
  const uint64_t p = (uint64_t)(uint32_t)b * (uint32_t)n;
  if (p <= 0xffffffffull) return (int)((uint32_t)p / (uint32_t)parts);
  return (int)(p / (uint32_t)parts);
}

// First guess of where row `target` of n rows starts among nnz row-sorted
// sidecar triplets (rows spread evenly); only a search hint.
__device__ __forceinline__ int64_t sidecar_guess(int64_t nnz, int target, int n) {
  return (int64_t)((float)nnz * ((float)target / (float)n));
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

// DPP lane exchange: lanes outside the enabled rows (or reading out of range) get 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes with DPP (no LDS traffic); the total is returned
// wave-uniform (read from lane 63).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xb1>(v);        // quad_perm(1,0,3,2): pairs
  v += dpp_f<0x4e>(v);        // quad_perm(2,3,0,1): quads
  v += dpp_f<0x141>(v);       // row_half_mirror: 8 lanes
  v += dpp_f<0x140>(v);       // row_mirror: every lane holds its 16-lane row sum
  v += dpp_f<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3; lane 63 holds the total
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Integer sum over the 64 lanes (wave-uniform result).
__device__ __forceinline__ int wave_sum_dpp_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return __builtin_amdgcn_readlane(v, 63);
}

// First sidecar entry with row >= target, searched by one wave in parallel:
// each round the 64 lanes probe 64 evenly spaced positions of [lo, hi).
// Every lane returns the same value.  (Probes past the range load a clamped
// position and are masked after the load: a load under a condition would make
// each round wait for every load the wave has in flight.)
__device__ __forceinline__ int64_t wave_lower_bound_rows(const int32_t* rows, int64_t nnz,
                                                         int32_t target) {
  if (nnz <= 0) return 0;
  int64_t lo = 0, hi = nnz;
  const int lane = lane_id();
  while (hi - lo > kWave) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int64_t p = lo + lane * step;
    const int32_t v = rows[p < hi ? p : hi - 1];
    const bool below = (p < hi) & (v < target);
    const uint64_t mask = __ballot(below);
    const int c = __popcll(mask);
    if (c == 0) return lo;
    const int64_t nlo = lo + (int64_t)(c - 1) * step + 1;
    const int64_t nhi = lo + (int64_t)c * step;
    lo = nlo;
    hi = nhi < hi ? nhi : hi;
  }
  // hi > 0 here (nnz > 0, and every round leaves hi >= 1)
  const int64_t p = lo + lane;
  const int32_t v = rows[p < hi ? p : hi - 1];
  const bool below = (p < hi) & (v < target);
  return lo + __popcll(__ballot(below));
}

// The same lower bound, first tried in one round: the wave reads the 1024
// triplet rows around the position a uniform spread would put `target` at
// (`guess`), 16 consecutive ones per lane.  When the answer is strictly inside
// that window it is the number of rows below `target` there; otherwise the
// general search runs.
__device__ __forceinline__ int64_t wave_lower_bound_rows_near(const int32_t* rows, int64_t nnz,
                                                              int32_t target, int64_t guess) {
  constexpr int64_t WIN = 16 * kWave;
  if (nnz <= 0) return 0;
  if (nnz <= WIN) {
    // the whole array fits the window (clamped loads, masked after loading)
    const int lane = lane_id();
    int32_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t p = (int64_t)lane * 16 + j;
      v[j] = rows[p < nnz ? p : nnz - 1];
    }
    int c = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) c += (int)((int64_t)lane * 16 + j < nnz) & (int)(v[j] < target);
    return wave_sum_dpp_i(c);
  }
  int64_t ws = guess - WIN / 2;
  if (ws < 0) ws = 0;
  if (ws > nnz - WIN) ws = nnz - WIN;
  const int lane = lane_id();
  const int4* base = reinterpret_cast<const int4*>(rows + ws + (int64_t)lane * 16);
  int c = 0;
  if (((uintptr_t)(rows + ws) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int4 v = base[q];
      c += (v.x < target) + (v.y < target) + (v.z < target) + (v.w < target);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) c += rows[ws + (int64_t)lane * 16 + j] < target ? 1 : 0;
  }
  const int total = wave_sum_dpp_i(c);
  const bool lo_ok = total > 0 || ws == 0;
  const bool hi_ok = total < WIN || ws + WIN == nnz;
  if (lo_ok && hi_ok) return ws + total;
  return wave_lower_bound_rows(rows, nnz, target);
}

// The same lower bound in two steps, so that the loads can go out long before
// the answer is needed: row_window_load reads the 1024 rows around `guess`
// (clamped to the array), lane l rows l, l + 64, ... of it (each load one
// contiguous 256-byte piece); row_window_lower_bound
// counts the rows below `target` there and falls back to the general search
// when the answer is not strictly inside the window.  Needs nnz > 0.
struct RowWindow {
  int64_t ws;
  int32_t v[16];
};
__device__ __forceinline__ void row_window_load(const int32_t* rows, int64_t nnz, int64_t guess, RowWindow& w) {
  constexpr int64_t WIN = 16 * kWave;
  int64_t ws = guess - WIN / 2;
  if (ws > nnz - WIN) ws = nnz - WIN;
  if (ws < 0) ws = 0;
  w.ws = ws;
  const int64_t p0 = ws + lane_id();
#pragma unroll
  for (int j = 0; j < 16; ++j) w.v[j] = rows[p0 + kWave * j < nnz ? p0 + kWave * j : nnz - 1];
}
__device__ __forceinline__ int64_t row_window_lower_bound(const int32_t* rows, int64_t nnz, int32_t target,
                                                          const RowWindow& w) {
  constexpr int64_t WIN = 16 * kWave;
  const int64_t p0 = w.ws + lane_id();
  int c = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // (the empty asm pins the compare here: hoisted next to the loads, it would
    // make the caller wait for them there)
    int32_t v = w.v[j];
    asm volatile("" : "+v"(v));
    c += (int)(p0 + kWave * j < nnz) & (int)(v < target);
  }
  const int total = wave_sum_dpp_i(c);
  const bool lo_ok = total > 0 || w.ws == 0;
  const bool hi_ok = total < WIN || w.ws + WIN >= nnz;
  if (lo_ok && hi_ok) return w.ws + total;
  return wave_lower_bound_rows(rows, nnz, target);
}

// Asynchronous copies global -> LDS (LDS DMA).  Each active lane moves its 4 or
// 16 bytes; lane i's bytes land at lds_base + i * size.  The LDS base must be
// wave-uniform.  Completion is tracked by the vector-memory counter.
typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ void lds_dma16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void_ptr)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void lds_dma4(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void_ptr)lds_base, 4, 0, 0);
}

// A flag in LDS shared by the waves of one workgroup, read and written as
// LDS accesses (a volatile access through a generic pointer becomes a flat
// access, whose completion is tracked on the vector-memory counter as well,
// so every wait for it would also wait for all loads in flight).
typedef __attribute__((address_space(3))) int lds_int;

__device__ __forceinline__ int lds_flag_load(int* p) {
  return __hip_atomic_load((lds_int*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void lds_flag_store(int* p, int v) {
  __hip_atomic_store((lds_int*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Split form of the window lookup, so its loads can be issued ahead of other
// traffic and resolved later: `issue` reads the 1024 triplet rows around
// `guess` (entry ws + 64 j + lane in load j, so each load instruction covers
// 256 consecutive bytes; positions past the end re-read the last entry, so
// the loads are unconditional); `resolve` counts those below `target` and
// falls back to the general search when the answer is not inside the window.
struct WindowProbe {
  int64_t ws;
  int v[16];
};

__device__ __forceinline__ void window_issue(WindowProbe& w, const int32_t* rows, int64_t nnz, int64_t guess) {
  constexpr int64_t WIN = 16 * kWave;
  int64_t ws = 0;
  if (nnz > WIN) {
    ws = guess - WIN / 2;
    if (ws < 0) ws = 0;
    if (ws > nnz - WIN) ws = nnz - WIN;
  }
  w.ws = ws;
  // wave-uniform base and 32-bit lane offsets, clamped to the last entry
  const int32_t* base = rows + ws;
  const int lim = (int)(nnz - ws < WIN ? nnz - ws : WIN) - 1;
#pragma unroll
  for (int j = 0; j < 16; ++j) w.v[j] = base[min(lane_id() + j * kWave, lim)];
}

__device__ __forceinline__ int64_t window_resolve(const WindowProbe& w, const int32_t* rows, int64_t nnz,
                                                  int32_t target) {
  constexpr int64_t WIN = 16 * kWave;
  const int n = (int)(nnz - w.ws < WIN ? nnz - w.ws : WIN);  // entries in the window
  int c = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // an empty asm that "modifies" the value keeps the compiler from hoisting
    // this comparison (and so the wait for the load) above the caller's
    // barrier, which would stall the issue of loads placed after the probe
    int v = w.v[j];
    asm volatile("" : "+v"(v));
    c += (lane_id() + j * kWave < n && v < target) ? 1 : 0;
  }
  const int64_t total = wave_sum_dpp_i(c);
  const int64_t wend = w.ws + n;
  if ((total > 0 || w.ws == 0) && (w.ws + total < wend || wend == nnz)) return w.ws + total;
  return wave_lower_bound_rows(rows, nnz, target);
}

}  // namespace hxq
