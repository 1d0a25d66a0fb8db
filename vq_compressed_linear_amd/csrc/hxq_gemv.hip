// fp32-arithmetic HelixLinear kernels: vector-ALU GEMV (u8 and pk12), the
// any-shape fallback and the standalone sidecar add.
//
// The forward is y[m][n] = sum_k (C[idx[n][k]] + S[n][k]) x[m][k] + b[n]
// (model cards, "What is HelixCode?": codebook[indices] @ x with no separate
// decompression; HXQ whitepaper, "Method": sidecar triplets).  The weight is
// never written anywhere: each index is turned into its codebook value in a
// register right before the multiply.

#include <atomic>

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

// ------------------------------------------------------------------ helpers

template <bool XBF>
__device__ __forceinline__ float4 load_x4(const void* x, int64_t off) {
  if (XBF) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + off);
    return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffffu),
                       bf16_to_f32(u.y >> 16));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
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

// ------------------------------------------------------------- VALU GEMV
//
// One kernel template for both formats.
//
// u8: LDS holds 64 copies of the 256-entry codebook with a 256-byte stride per
// entry: copy j of entry e sits at byte e*256 + 4j.  Lane j reads copy j, so a
// wave's 64 gathers fall in 64 different banks whatever the indices are, and
// the LDS address of index byte b is one byte-permute of the index word.
// pk12: LDS holds the 4096 codebook pairs (32 KB, 8 bytes per entry); one
// 8-byte gather yields the two weights (2j, 2j+1) of a 12-bit index.
//
// Each wave owns a contiguous range of output rows and walks it in groups of R
// rows.  A group is cut along K into slices of 64 lanes x CPL chunks, a chunk
// being 16 consecutive inputs of one row (16 index bytes for u8, 12 for pk12).
// The (group, slice) items are software-pipelined: the index and x loads of the
// next item are in flight while the current one is gathered and multiplied.
// The wave's sidecar triplets are read 64 at a time into registers (one per
// lane) with the x values they need, and added to the lane partials of their
// row before the group's wave reduction.

template <bool PK12, int R, int CPL, int MT, bool XBF>
struct Item {
  uint32_t w[R][CPL][PK12 ? 3 : 4];
  float x[MT][CPL][16];
};

template <bool PK12, int R, int CPL, int MT, bool XBF>
__device__ __forceinline__ void load_item(Item<PK12, R, CPL, MT, XBF>& it, const LayerArgs& a,
                                          int64_t n0, int64_t rw1, int s, int m0, int lane,
                                          int64_t row_bytes) {
  const int kchunks = a.K >> 4;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int kc = (s * CPL + c) * kWave + lane;
    const bool kin = kc < kchunks;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool in = kin && (n0 + r < rw1);
      const uint8_t* p = a.indices + (n0 + r) * row_bytes;
      if (PK12) {
        uint3 u = make_uint3(0, 0, 0);
        if (in) u = *reinterpret_cast<const uint3*>(p + (int64_t)kc * 12);
        it.w[r][c][0] = u.x;
        it.w[r][c][1] = u.y;
        it.w[r][c][2] = u.z;
      } else {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (in) u = *reinterpret_cast<const uint4*>(p + (int64_t)kc * 16);
        it.w[r][c][0] = u.x;
        it.w[r][c][1] = u.y;
        it.w[r][c][2] = u.z;
        it.w[r][c][3] = u.w;
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = min(m0 + m, a.M - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kin) v = load_x4<XBF>(a.x, (int64_t)mm * a.K + (int64_t)kc * 16 + q * 4);
        it.x[m][c][4 * q + 0] = v.x;
        it.x[m][c][4 * q + 1] = v.y;
        it.x[m][c][4 * q + 2] = v.z;
        it.x[m][c][4 * q + 3] = v.w;
      }
    }
  }
}

template <bool PK12, int R, int CPL, int MT, bool XBF>
__device__ __forceinline__ void compute_item(const Item<PK12, R, CPL, MT, XBF>& it,
                                             float (&acc)[R][MT], const unsigned char* cbs,
                                             uint32_t lane4) {
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float wv[16];
      if (PK12) {
        const uint32_t g[4] = {it.w[r][c][0], __builtin_amdgcn_alignbit(it.w[r][c][1], it.w[r][c][0], 24),
                               __builtin_amdgcn_alignbit(it.w[r][c][2], it.w[r][c][1], 16),
                               it.w[r][c][2] >> 8};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float2 ca = lds_load<float2>((g[d] << 3) & 0x7ff8u, cbs);
          const float2 cb = lds_load<float2>((g[d] >> 9) & 0x7ff8u, cbs);
          wv[4 * d + 0] = ca.x;
          wv[4 * d + 1] = ca.y;
          wv[4 * d + 2] = cb.x;
          wv[4 * d + 3] = cb.y;
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = it.w[r][c][d];
          wv[4 * d + 0] = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
          wv[4 * d + 1] = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
          wv[4 * d + 2] = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
          wv[4 * d + 3] = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float s = acc[r][m];
#pragma unroll
        for (int j = 0; j < 16; ++j) s = fmaf(wv[j], it.x[m][c][j], s);
        acc[r][m] = s;
      }
    }
}

// Sidecar state of a wave.  The triplets of the wave's rows are found and
// read in the background while the index stream runs: a one-round window
// lookup is issued before the first index loads, the triplets [b0, b0 + 64)
// (one per lane: row, column, delta) after the first item, and the x values
// at their columns only when a flush needs them.
template <int MT>
struct Side {
  int64_t ws;    // window start of the lookup
  int4 wp[4];    // the 16 triplet rows this lane read in the window
  int64_t b0;    // first triplet of the batch held in registers
  int row;       // INT_MAX when the lane holds no triplet of this wave
  int col;
  float d;
  float xv[MT];
  int phase;     // 0 none, 1 window issued, 2 triplets loaded, 3 x loaded
};

constexpr int64_t kWin = 16 * kWave;  // triplet rows read by the window lookup

template <int MT>
__device__ __forceinline__ void side_issue_window(Side<MT>& sd, const LayerArgs& a, int64_t rw0, int lane) {
  int64_t ws = 0;
  if (a.nnz > kWin) {
    ws = (int64_t)((double)a.nnz * (double)rw0 / (double)a.N) - kWin / 2;
    ws &= ~(int64_t)3;  // 16-byte aligned start when the array is
    if (ws < 0) ws = 0;
    if (ws > a.nnz - kWin) ws = a.nnz - kWin;
  }
  sd.ws = ws;
  const int64_t p0 = ws + (int64_t)lane * 16;
  const bool vec = ((reinterpret_cast<uintptr_t>(a.sc_rows + ws) & 15) == 0) && ws + kWin <= a.nnz;
  if (vec) {
    const int4* b = reinterpret_cast<const int4*>(a.sc_rows + p0);
#pragma unroll
    for (int q = 0; q < 4; ++q) sd.wp[q] = b[q];
  } else {
    int v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (p0 + j < a.nnz) ? a.sc_rows[p0 + j] : INT_MAX;
#pragma unroll
    for (int q = 0; q < 4; ++q) sd.wp[q] = make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
  sd.phase = 1;
}

template <int MT>
__device__ __forceinline__ void side_load_triplets(Side<MT>& sd, const LayerArgs& a, int64_t b0, int64_t rw1,
                                                   int lane) {
  sd.b0 = b0;
  const int64_t e = b0 + lane;
  int r = INT_MAX, c = 0;
  float d = 0.f;
  if (e < a.nnz) {
    r = a.sc_rows[e];
    c = a.sc_cols[e];
    d = a.sc_deltas[e];
  }
  const bool in = r < rw1;
  sd.row = in ? r : INT_MAX;
  sd.col = c;
  sd.d = in ? d : 0.f;
  sd.phase = 2;
}

template <int MT>
__device__ __forceinline__ void side_resolve(Side<MT>& sd, const LayerArgs& a, int64_t rw0, int64_t rw1,
                                             int lane) {
  const int32_t t = (int32_t)rw0;
  int c = 0;
  const int64_t p0 = sd.ws + (int64_t)lane * 16;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int4 v = sd.wp[q];
    c += (p0 + 4 * q + 0 < a.nnz && v.x < t) + (p0 + 4 * q + 1 < a.nnz && v.y < t) +
         (p0 + 4 * q + 2 < a.nnz && v.z < t) + (p0 + 4 * q + 3 < a.nnz && v.w < t);
  }
  const int64_t total = wave_sum_dpp_i(c);
  const int64_t wend = sd.ws + kWin < a.nnz ? sd.ws + kWin : a.nnz;
  int64_t b0;
  if ((total > 0 || sd.ws == 0) && (sd.ws + total < wend || wend == a.nnz))
    b0 = sd.ws + total;
  else
    b0 = wave_lower_bound_rows(a.sc_rows, a.nnz, t);
  side_load_triplets(sd, a, b0, rw1, lane);
}

template <int MT, bool XBF>
__device__ __forceinline__ void side_load_x(Side<MT>& sd, const LayerArgs& a, int m0) {
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = min(m0 + m, a.M - 1);
    sd.xv[m] = sd.row != INT_MAX ? load_x1<XBF>(a.x, (int64_t)mm * a.K + sd.col) : 0.f;
  }
  sd.phase = 3;
}

template <bool PK12, int R, int CPL, int MT, bool XBF, int D>
__global__ __launch_bounds__(256, 2) void gemv_valu(LayerArgs a, int64_t waves_total) {
  constexpr int CB_BYTES = PK12 ? 4096 * 8 : 256 * 256;
  constexpr int STASH_ROWS = 64;  // rows of results a wave holds before the sidecar pass
  static_assert(STASH_ROWS % R == 0, "groups tile the stash");
  __shared__ __align__(16) unsigned char cbs[CB_BYTES];
  __shared__ float stash_all[4][STASH_ROWS * MT];
  using It = Item<PK12, R, CPL, MT, XBF>;

  const int lane = lane_id();
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  float* stash = stash_all[threadIdx.x >> 6];
  int64_t rw0, rw1;
  wave_row_range(a.N, waves_total, wave, rw0, rw1);
  const int64_t row_bytes = PK12 ? (int64_t)3 * (a.K >> 2) : (int64_t)a.K;
  const int slices = (a.K / 16 + CPL * kWave - 1) / (CPL * kWave);
  const int64_t groups = (rw1 - rw0 + R - 1) / R;
  const int64_t items = groups * slices;
  const bool has_side = a.nnz > 0 && items > 0;

  // Codebook staging: this thread's share of the values is loaded first so
  // that writing the LDS copies waits on those loads only.
  constexpr int CB_LOADS = PK12 ? 8 : 16;
  float4 cbv4[PK12 ? CB_LOADS : 1];
  float cbv1[PK12 ? 1 : CB_LOADS];
  if (PK12) {
    const float4* cb = static_cast<const float4*>(a.codebook);
#pragma unroll
    for (int j = 0; j < CB_LOADS; ++j) cbv4[j] = cb[threadIdx.x + 256 * j];
  } else {
    const float* cb = static_cast<const float*>(a.codebook);
#pragma unroll
    for (int j = 0; j < CB_LOADS; ++j) cbv1[j] = cb[(threadIdx.x >> 4) + 16 * j];
  }

  It buf[D];
  Side<MT> sd;
  sd.phase = 0;
  sd.row = INT_MAX;
  auto item_n0 = [&](int64_t i) { return rw0 + (i / slices) * R; };
  auto start_chunk = [&](int m0) {
    if (has_side) side_issue_window(sd, a, rw0, lane);
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
      if (u < items) load_item(buf[u], a, item_n0(u), rw1, (int)(u % slices), m0, lane, row_bytes);
  };
  start_chunk(blockIdx.y * MT);
#pragma unroll
  for (int j = 0; j < CB_LOADS; ++j) {
    if (PK12) {
      reinterpret_cast<float4*>(cbs)[threadIdx.x + 256 * j] = cbv4[j];
    } else {
      const float v = cbv1[j];
      *reinterpret_cast<float4*>(cbs + ((threadIdx.x >> 4) + 16 * j) * 256 + (threadIdx.x & 15) * 16) =
          make_float4(v, v, v, v);
    }
  }
  __syncthreads();

  for (int64_t m0l = (int64_t)blockIdx.y * MT; m0l < a.M; m0l += (int64_t)gridDim.y * MT) {
    const int m0 = (int)m0l;
    if (m0l != (int64_t)blockIdx.y * MT) start_chunk(m0);
    if (items == 0) continue;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
    int64_t s0 = rw0;  // first row held in the stash

    // Sidecar for the stash rows [s0, s1), then the stash goes to y.
    auto flush = [&](int64_t s1) {
      if (has_side) {
        if (sd.phase == 1) side_resolve(sd, a, rw0, rw1, lane);
        if (sd.phase == 2) side_load_x<MT, XBF>(sd, a, m0);
        while (true) {
          // the triplets of these rows, in order, each added by the lane holding it
          uint64_t mask = __ballot(sd.row >= s0 && sd.row < s1);
          while (mask) {
            const int e = __builtin_ctzll(mask);
            mask &= mask - 1;
            if (lane == e) {
              float* slot = stash + (int64_t)(sd.row - s0) * MT;
#pragma unroll
              for (int m = 0; m < MT; ++m) slot[m] = fmaf(sd.d, sd.xv[m], slot[m]);
            }
          }
          const int last = __builtin_amdgcn_readlane(sd.row, 63);
          if (last == INT_MAX || last >= s1) break;
          side_load_triplets(sd, a, sd.b0 + kWave, rw1, lane);
          side_load_x<MT, XBF>(sd, a, m0);
        }
      }
      const int cnt = (int)(s1 - s0) * MT;
      for (int idx = lane; idx < cnt; idx += kWave) {
        const int r = idx / MT, m = idx % MT;
        if (m0 + m < a.M) a.y[(int64_t)(m0 + m) * a.N + s0 + r] = stash[idx];
      }
      s0 = s1;
    };

    auto finish_group = [&](int64_t n0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float t = wave_sum_dpp(acc[r][m]);
          const int64_t n = n0 + r;
          if (lane == r * MT + m && n < rw1)
            stash[(n - s0) * MT + m] = t + (a.bias ? a.bias[n] : 0.f);
          acc[r][m] = 0.f;
        }
      const int64_t n1 = n0 + R < rw1 ? n0 + R : rw1;
      if (n1 == rw1 || n1 - s0 == STASH_ROWS) flush(n1);
    };

    for (int64_t base = 0; base < items; base += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t i = base + u;
        if (i >= items) break;
        const int64_t j = i + D - 1;
        if (j < items) load_item(buf[(u + D - 1) % D], a, item_n0(j), rw1, (int)(j % slices), m0, lane, row_bytes);
        compute_item(buf[u], acc, cbs, lane4);
        if (sd.phase == 1) side_resolve(sd, a, rw0, rw1, lane);
        if ((i % slices) == slices - 1) finish_group(item_n0(i));
      }
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

// Compute units of the current device, queried once per device and kept
// (zero in the table means not yet queried).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < kMaxDevices;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  if (slot) cached[dev].store(cus, std::memory_order_relaxed);
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

template <bool PK12, int R, int CPL, int MT, int D>
static hipError_t launch_valu_cfg(const LayerArgs& a, hipStream_t stream, int64_t blocks) {
  int64_t mchunks = ((int64_t)a.M + MT - 1) / MT;
  if (mchunks > 65535) mchunks = 65535;
  const dim3 grid((unsigned)blocks, (unsigned)mchunks);
  const int64_t waves = blocks * 4;
  if (a.x_bf16)
    hipLaunchKernelGGL((gemv_valu<PK12, R, CPL, MT, true, D>), grid, dim3(256), 0, stream, a, waves);
  else
    hipLaunchKernelGGL((gemv_valu<PK12, R, CPL, MT, false, D>), grid, dim3(256), 0, stream, a, waves);
  return hipGetLastError();
}

// Tiling by token count and by how many rows each wave gets: short row
// ranges take one row per group with wider K slices so a wave still has a few
// kilobytes of index loads in flight.
template <bool PK12>
static hipError_t launch_valu_fmt(const LayerArgs& a, hipStream_t stream) {
  const int cus = device_cu_count();
  const int64_t cap = (int64_t)cus * 2;  // two 256-thread workgroups per CU
  int64_t blocks = ((int64_t)a.N + 3) / 4;  // at least one row per wave
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const double rows_per_wave = (double)a.N / (double)(blocks * 4);
  if (a.M == 1) {
    if (rows_per_wave >= 3.0) return launch_valu_cfg<PK12, 4, 1, 1, 3>(a, stream, blocks);
    return launch_valu_cfg<PK12, 1, 2, 1, 3>(a, stream, blocks);
  }
  if (a.M == 2) return launch_valu_cfg<PK12, 2, 1, 2, 3>(a, stream, blocks);
  return launch_valu_cfg<PK12, 2, 1, 4, 2>(a, stream, blocks);  // token chunks of 4
}

hipError_t launch_gemv_valu(const LayerArgs& a, bool pk12, hipStream_t stream) {
  // one token: the decode kernel; 2 to 8 the 4x4-block matrix-core GEMV
  // (2 to 4 tokens: 50 us for the Qwen decode step against 56-72 us on the
  // decode kernel), up to 4 tokens where that does not take the layer the
  // decode kernel; then the 16x16 matrix-core GEMV, past 64 tokens in
  // launches of 64; where that does not fit either, token groups through the
  // decode kernel, then the vector kernels
  DecodeSeg sg = {a.codebook, a.indices, a.sc_rows, a.sc_cols, a.sc_deltas, a.nnz, a.bias, a.y, a.N, 0, 0, 0.f};
  hipError_t err = hipSuccess;
  if (a.M >= 2 && a.M <= 8 && gemv_mfma4_ok(a, pk12)) {
    const GemvSeg gs = {static_cast<const float*>(a.codebook), a.indices, a.sc_rows, a.sc_cols, a.sc_deltas, a.nnz,
                        a.bias, a.y, a.N, 0};
    if (gemv_mfma4_group_fits(&gs, 1)) return launch_gemv_mfma4_grouped(&gs, 1, pk12, a.x, a.x_bf16, a.M, a.K, stream);
  }
  if (a.M <= 4 && launch_decode(&sg, 1, pk12, a.x, a.x_bf16, a.M, a.K, stream, err)) return err;
  if (gemv_mfma_takes(a, pk12)) return launch_gemv_mfma_tokens(a, pk12, stream);
  if (a.M > 4 && a.M <= kChunkMaxM && launch_decode_chunked(&sg, 1, pk12, a.x, a.x_bf16, a.M, a.K, stream, err))
    return err;
  return pk12 ? launch_valu_fmt<true>(a, stream) : launch_valu_fmt<false>(a, stream);
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

// ------------------------------------------------------------ stream read
// Reference for the attainable read bandwidth: reads `bytes` of `src` once,
// 16 bytes per lane per request, each wave a contiguous stretch with eight
// requests in flight, and folds what it read into one word per workgroup
// (so no load can be dropped): the XOR of all sink words is the XOR of all
// 32-bit words of the buffer.  Same grid shape as the decode kernel.  NT:
// non-temporal loads (the form the streaming kernels use past the L2s'
// capacity).

namespace hxq {

template <bool NT>
__global__ __launch_bounds__(512) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                           uint32_t* __restrict__ sink) {
  // the grid sweeps the buffer in order: each round every thread requests P
  // pieces, round r of the grid covering one contiguous window of
  // P * threads pieces (faster than one stretch per wave: the requests in
  // flight stay close together).  The next round's requests go out before
  // this round's data is folded, so 2 P pieces per thread are in flight
  // across the round boundary.
  constexpr int P = 4;
  const int lane = threadIdx.x & 63;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  auto request = [&](int64_t i0, u32x4 (&v)[P], uint32_t (&keep)[P]) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t i = i0 + p * nthr + t;
      keep[p] = i < n16 ? 0xffffffffu : 0u;  // a thread past the end re-reads a valid piece and drops it
      const u32x4* q = src + (i < n16 ? i : n16 - 1);
      v[p] = NT ? __builtin_nontemporal_load(q) : *q;
    }
  };
  auto fold = [&](const u32x4 (&v)[P], const uint32_t (&keep)[P]) {
#pragma unroll
    for (int p = 0; p < P; ++p) acc ^= (v[p].x ^ v[p].y ^ v[p].z ^ v[p].w) & keep[p];
  };
  // two register sets in turn (no copies, so no wait for data still in
  // flight); requests past the end read valid pieces that are dropped
  u32x4 va[P], vb[P];
  uint32_t ka[P], kb[P];
  const int64_t R = P * nthr;
  const int64_t rounds = (n16 + R - 1) / R;
  request(0, va, ka);
  for (int64_t r = 0; r < rounds; r += 2) {
    // (scheduling barriers keep each fold below the next round's requests)
    request((r + 1) * R, vb, kb);
    __builtin_amdgcn_sched_barrier(0);
    fold(va, ka);
    request((r + 2) * R, va, ka);
    __builtin_amdgcn_sched_barrier(0);
    fold(vb, kb);
  }
  // fold across the wave; each wave stores its own word (no barrier and no
  // atomics, so the waves retire independently, as in a plain read)
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if (lane == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int sink_words, bool nt,
                              hipStream_t stream) {
  // one workgroup per 8 sink words (a word per wave; the caller picks the
  // grid), no more than the buffer's pieces need
  int64_t grid = sink_words / 8;
  const int64_t need = (bytes / 16 + 511) / 512;
  if (grid > need) grid = need;
  if (grid > 65535) grid = 65535;
  if (grid < 1) grid = 1;
  if (nt)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)grid), dim3(512), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)grid), dim3(512), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace hxq
