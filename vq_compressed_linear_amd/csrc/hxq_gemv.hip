// fp32-arithmetic HelixLinear kernels: vector-ALU GEMV (u8 and pk12), the
// any-shape fallback and the standalone sidecar add.
//
// The forward is y[m][n] = sum_k (C[idx[n][k]] + S[n][k]) x[m][k] + b[n]
// (model cards, "What is HelixCode?": codebook[indices] @ x with no separate
// decompression; HXQ whitepaper, "Method": sidecar triplets).  The weight is
// never written anywhere: each index is turned into its codebook value in a
// register right before the multiply.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

// ------------------------------------------------------------------ helpers

template <bool XBF>
__device__ __forceinline__ void load_x4(const void* x, int64_t off, float v[4]) {
  if (XBF) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + off);
    v[0] = bf16_to_f32(u.x & 0xffffu);
    v[1] = bf16_to_f32(u.x >> 16);
    v[2] = bf16_to_f32(u.y & 0xffffu);
    v[3] = bf16_to_f32(u.y >> 16);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

template <bool XBF>
__device__ __forceinline__ float load_x1(const void* x, int64_t off) {
  if (XBF) return bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[off]);
  return reinterpret_cast<const float*>(x)[off];
}

__device__ __forceinline__ uint32_t word_of(const uint4& w, int d) {
  return d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w;
}

// Rows [r0, r1) handled by one wave when `rows` rows are spread over
// `waves` waves as evenly as possible (contiguous ranges).
__device__ __forceinline__ void wave_row_range(int64_t rows, int64_t waves, int64_t wave,
                                               int64_t& r0, int64_t& r1) {
  r0 = wave * rows / waves;
  r1 = (wave + 1) * rows / waves;
}

// Adds the sidecar triplets of rows [n0, n0 + R) to the per-lane partial sums.
// `cur` points at the first triplet with row >= n0; it is advanced past the
// triplets of these rows.  Triplets are read 64 at a time, one per lane.
template <int MT, int R, bool XBF>
__device__ __forceinline__ void sidecar_into_partials(const LayerArgs& a, int64_t& cur, int n0,
                                                      int m0, float (&acc)[R][MT]) {
  const int lane = lane_id();
  const int nend = n0 + R;
  while (true) {
    const int64_t e = cur + lane;
    int rr = INT_MAX;
    if (e < a.nnz) rr = a.sc_rows[e];
    const bool in = rr < nend;
    const int cnt = __popcll(__ballot(in));
    if (in) {
      const int cc = a.sc_cols[e];
      const float dd = a.sc_deltas[e];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mm = min(m0 + m, a.M - 1);
        const float t = dd * load_x1<XBF>(a.x, (int64_t)mm * a.K + cc);
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (rr - n0 == r) acc[r][m] += t;
      }
    }
    cur += cnt;
    if (cnt < kWave) break;
  }
}

// Reduces every partial over the wave and stores y for rows [n0, n0 + R) that
// are below `nlim`, and token rows [m0, m0 + MT) below M.
template <int MT, int R>
__device__ __forceinline__ void reduce_store(const LayerArgs& a, float (&acc)[R][MT], int n0,
                                             int64_t nlim, int m0) {
  static_assert(R * MT <= kWave, "one lane per output");
  const int lane = lane_id();
  float out = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float s = wave_sum(acc[r][m]);
      if (lane == r * MT + m) out = s;
    }
  if (lane < R * MT) {
    const int r = lane / MT, m = lane % MT;
    const int64_t n = (int64_t)n0 + r;
    const int mm = m0 + m;
    if (n < nlim && mm < a.M) a.y[(int64_t)mm * a.N + n] = out + (a.bias ? a.bias[n] : 0.f);
  }
}

// ----------------------------------------------------------- u8 VALU GEMV
//
// LDS holds 64 copies of the 256-entry codebook with a 256-byte stride per
// entry: copy j of entry e sits at byte e*256 + 4j.  Lane j reads copy j, so a
// wave's 64 gathers fall in 64 different banks whatever the indices are, and
// the LDS address is one byte-permute of the index word.
//
// Each wave owns a contiguous range of output rows and walks it R rows at a
// time; a lane covers 16 consecutive inputs per step (one 16-byte index load
// per row), the x values it needs are loaded once per step and reused for the
// R rows.

template <int MT, int R, bool XBF>
__global__ __launch_bounds__(256) void gemv_u8_valu(LayerArgs a, int64_t waves_total) {
  __shared__ __align__(16) unsigned char cbs[256 * 256];
  {
    const float* cb = static_cast<const float*>(a.codebook);
    for (int i = threadIdx.x; i < 256 * 16; i += blockDim.x) {
      const float v = cb[i >> 4];
      *reinterpret_cast<float4*>(cbs + (i >> 4) * 256 + (i & 15) * 16) = make_float4(v, v, v, v);
    }
  }
  __syncthreads();

  const int lane = lane_id();
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  int64_t rw0, rw1;
  wave_row_range(a.N, waves_total, wave, rw0, rw1);
  if (rw0 >= rw1) return;
  const int K = a.K;
  const int kchunks = K >> 4;

  for (int64_t m0l = (int64_t)blockIdx.y * MT; m0l < a.M; m0l += (int64_t)gridDim.y * MT) {
    const int m0 = (int)m0l;
    int64_t cur = 0;
    if (a.nnz > 0) cur = wave_lower_bound_rows(a.sc_rows, a.nnz, (int32_t)rw0);
    for (int64_t n0 = rw0; n0 < rw1; n0 += R) {
      float acc[R][MT];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

      for (int kc = lane; kc < kchunks; kc += kWave) {
        uint4 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (n0 + r < rw1)
            w[r] = *reinterpret_cast<const uint4*>(a.indices + (n0 + r) * (int64_t)K + (int64_t)kc * 16);
          else
            w[r] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float xv[MT][4];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int mm = min(m0 + m, a.M - 1);
            load_x4<XBF>(a.x, (int64_t)mm * K + (int64_t)kc * 16 + d * 4, xv[m]);
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t wd = word_of(w[r], d);
            const float c0 = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
            const float c1 = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
            const float c2 = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
            const float c3 = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              float s = acc[r][m];
              s = fmaf(c0, xv[m][0], s);
              s = fmaf(c1, xv[m][1], s);
              s = fmaf(c2, xv[m][2], s);
              s = fmaf(c3, xv[m][3], s);
              acc[r][m] = s;
            }
          }
        }
      }
      if (a.nnz > 0) sidecar_into_partials<MT, R, XBF>(a, cur, (int)n0, m0, acc);
      reduce_store<MT, R>(a, acc, (int)n0, rw1, m0);
    }
  }
}

// ---------------------------------------------------------- pk12 VALU GEMV
//
// LDS holds the 4096 codebook pairs (32 KB, 8 bytes per entry).  A lane covers
// 16 consecutive inputs per step: 12 index bytes = four 3-byte groups = eight
// 12-bit indices, each selecting the pair of weights (2j, 2j+1).

template <int MT, int R, bool XBF>
__global__ __launch_bounds__(256) void gemv_pk12_valu(LayerArgs a, int64_t waves_total) {
  __shared__ __align__(16) unsigned char cbs[4096 * 8];
  {
    const float4* cb = static_cast<const float4*>(a.codebook);
    for (int i = threadIdx.x; i < 4096 / 2; i += blockDim.x)
      reinterpret_cast<float4*>(cbs)[i] = cb[i];
  }
  __syncthreads();

  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  int64_t rw0, rw1;
  wave_row_range(a.N, waves_total, wave, rw0, rw1);
  if (rw0 >= rw1) return;
  const int K = a.K;
  const int kchunks = K >> 4;
  const int64_t row_bytes = (int64_t)3 * (K >> 2);

  for (int64_t m0l = (int64_t)blockIdx.y * MT; m0l < a.M; m0l += (int64_t)gridDim.y * MT) {
    const int m0 = (int)m0l;
    int64_t cur = 0;
    if (a.nnz > 0) cur = wave_lower_bound_rows(a.sc_rows, a.nnz, (int32_t)rw0);
    for (int64_t n0 = rw0; n0 < rw1; n0 += R) {
      float acc[R][MT];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

      for (int kc = lane; kc < kchunks; kc += kWave) {
        uint32_t g[R][4];  // the four 24-bit groups of each row (upper bits unused)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint3 u = make_uint3(0, 0, 0);
          if (n0 + r < rw1)
            u = *reinterpret_cast<const uint3*>(a.indices + (n0 + r) * row_bytes + (int64_t)kc * 12);
          g[r][0] = u.x;
          g[r][1] = __builtin_amdgcn_alignbit(u.y, u.x, 24);
          g[r][2] = __builtin_amdgcn_alignbit(u.z, u.y, 16);
          g[r][3] = u.z >> 8;
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float xv[MT][4];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int mm = min(m0 + m, a.M - 1);
            load_x4<XBF>(a.x, (int64_t)mm * K + (int64_t)kc * 16 + d * 4, xv[m]);
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t v = g[r][d];
            const float2 ca = lds_load<float2>((v << 3) & 0x7ff8u, cbs);
            const float2 cb = lds_load<float2>((v >> 9) & 0x7ff8u, cbs);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              float s = acc[r][m];
              s = fmaf(ca.x, xv[m][0], s);
              s = fmaf(ca.y, xv[m][1], s);
              s = fmaf(cb.x, xv[m][2], s);
              s = fmaf(cb.y, xv[m][3], s);
              acc[r][m] = s;
            }
          }
        }
      }
      if (a.nnz > 0) sidecar_into_partials<MT, R, XBF>(a, cur, (int)n0, m0, acc);
      reduce_store<MT, R>(a, acc, (int)n0, rw1, m0);
    }
  }
}

// ------------------------------------------------------------------ generic
//
// One wave per output row, any K and alignment, both formats.  Lanes stride
// over the inputs one weight at a time; four token rows per pass.

template <bool PK12, bool XBF>
__global__ __launch_bounds__(256) void generic_fwd(LayerArgs a) {
  const int lane = lane_id();
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.N) return;
  const int K = a.K;
  int64_t lo = 0, hi = 0;
  if (a.nnz > 0) {
    lo = wave_lower_bound_rows(a.sc_rows, a.nnz, (int32_t)n);
    hi = wave_lower_bound_rows(a.sc_rows, a.nnz, (int32_t)(n + 1));
  }
  const int64_t row_bytes = PK12 ? (int64_t)3 * ((K + 3) / 4) : (int64_t)K;
  const uint8_t* irow = a.indices + n * row_bytes;
  const float* cb = static_cast<const float*>(a.codebook);
  for (int m0 = 0; m0 < a.M; m0 += 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = lane; k < K; k += kWave) {
      float w;
      if (PK12) {
        const int j = k >> 1, t = j >> 1;
        const uint32_t v = (uint32_t)irow[3 * t] | ((uint32_t)irow[3 * t + 1] << 8) |
                           ((uint32_t)irow[3 * t + 2] << 16);
        const uint32_t e = (j & 1) ? (v >> 12) : (v & 0xfffu);
        w = cb[2 * e + (k & 1)];
      } else {
        w = cb[irow[k]];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mm = min(m0 + i, a.M - 1);
        acc[i] = fmaf(w, load_x1<XBF>(a.x, (int64_t)mm * K + k), acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (m0 + i >= a.M) break;
      float sc = 0.f;
      for (int64_t e = lo + lane; e < hi; e += kWave)
        sc = fmaf(a.sc_deltas[e], load_x1<XBF>(a.x, (int64_t)(m0 + i) * K + a.sc_cols[e]), sc);
      const float s = wave_sum(acc[i]) + wave_sum(sc);
      if (lane == 0) a.y[(int64_t)(m0 + i) * a.N + n] = s + (a.bias ? a.bias[n] : 0.f);
    }
  }
}

// ------------------------------------------------------------- sidecar add
//
// y[m][r] += sum of d * x[m][c] over the triplets of row r.  The thread that
// holds the first triplet of a row sums the whole run in triplet order, so
// every output element has exactly one writer.

template <bool XBF>
__global__ __launch_bounds__(256) void sidecar_add_kernel(LayerArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.nnz) return;
  const int r = a.sc_rows[e];
  if (e > 0 && a.sc_rows[e - 1] == r) return;
  for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
    float s = 0.f;
    for (int64_t f = e; f < a.nnz && a.sc_rows[f] == r; ++f)
      s = fmaf(a.sc_deltas[f], load_x1<XBF>(a.x, m * a.K + a.sc_cols[f]), s);
    a.y[m * a.N + r] += s;
  }
}

// ---------------------------------------------------------------- launchers

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

bool gemv_fast_path_ok(const LayerArgs& a, bool pk12) {
  if (a.K % 16 != 0) return false;
  const uintptr_t ia = reinterpret_cast<uintptr_t>(a.indices);
  const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
  if (xa % 16 != 0) return false;
  if (pk12) return ia % 4 == 0 && reinterpret_cast<uintptr_t>(a.codebook) % 16 == 0;
  return ia % 16 == 0;
}

template <int MT, int R>
static hipError_t launch_valu_mt(const LayerArgs& a, bool pk12, hipStream_t stream) {
  const int cus = device_cu_count();
  const int wgs_per_cu = pk12 ? 4 : 2;  // LDS: 32 KB (pk12) or 64 KB (u8) per workgroup
  const int64_t row_groups = ((int64_t)a.N + R - 1) / R;
  int64_t blocks = (row_groups + 3) / 4;
  const int64_t cap = (int64_t)cus * wgs_per_cu;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  int64_t mchunks = ((int64_t)a.M + MT - 1) / MT;
  if (mchunks > 65535) mchunks = 65535;
  const dim3 grid((unsigned)blocks, (unsigned)mchunks);
  const int64_t waves = blocks * 4;
  if (pk12) {
    if (a.x_bf16)
      hipLaunchKernelGGL((gemv_pk12_valu<MT, R, true>), grid, dim3(256), 0, stream, a, waves);
    else
      hipLaunchKernelGGL((gemv_pk12_valu<MT, R, false>), grid, dim3(256), 0, stream, a, waves);
  } else {
    if (a.x_bf16)
      hipLaunchKernelGGL((gemv_u8_valu<MT, R, true>), grid, dim3(256), 0, stream, a, waves);
    else
      hipLaunchKernelGGL((gemv_u8_valu<MT, R, false>), grid, dim3(256), 0, stream, a, waves);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_valu(const LayerArgs& a, bool pk12, hipStream_t stream) {
  if (a.M == 1) return launch_valu_mt<1, 4>(a, pk12, stream);
  if (a.M == 2) return launch_valu_mt<2, 4>(a, pk12, stream);
  if (a.M <= 4) return launch_valu_mt<4, 4>(a, pk12, stream);
  if (a.M <= 8) return launch_valu_mt<8, 2>(a, pk12, stream);
  return launch_valu_mt<16, 1>(a, pk12, stream);
}

hipError_t launch_generic(const LayerArgs& a, bool pk12, hipStream_t stream) {
  const int64_t blocks = ((int64_t)a.N + 3) / 4;
  const dim3 grid((unsigned)blocks);
  if (pk12) {
    if (a.x_bf16)
      hipLaunchKernelGGL((generic_fwd<true, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((generic_fwd<true, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.x_bf16)
      hipLaunchKernelGGL((generic_fwd<false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((generic_fwd<false, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_sidecar_add(const LayerArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.nnz + 255) / 256;
  int64_t gy = a.M;
  if (gy > 65535) gy = 65535;
  const dim3 grid((unsigned)blocks, (unsigned)gy);
  if (a.x_bf16)
    hipLaunchKernelGGL((sidecar_add_kernel<true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((sidecar_add_kernel<false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hxq
