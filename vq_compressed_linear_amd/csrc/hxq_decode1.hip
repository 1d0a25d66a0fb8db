// Decode GEMV for one token row (K % 16 == 0, K <= 12288), u8 and pk12, one
// or several layers per launch: the lean variant of the decode kernel.
//
// y[n] = sum_k (C[idx[n][k]] + S[n][k]) x[k] + b[n]  (model cards, "What is
// HelixCode?"; HXQ whitepaper, "Method" and "2D vector quantization"; the
// inference paragraph: gather + sidecar + matmul, no dense weight formed).
//
// A workgroup (one per CU) owns a contiguous run of rows of one layer; wave w
// takes rows w, w + 8, ... of the run, a whole row at a time: lane l holds the
// weights k = 16 (64 c + l) .. + 15 of chunk c (16 index bytes u8, 12 bytes =
// 8 pairs pk12) and the matching x, read once from LDS into registers when
// K <= 4096, else read from LDS chunk by chunk (x zero-padded to whole
// chunks; index loads past the row end re-read its last piece).  Per
// row: the codebook gather (LDS, 64 copies per entry for u8 so every lane has
// its own bank; the 4096 pairs for pk12), fp32 FMAs into four partial sums,
// a DPP reduction, one LDS word.  Index bytes are loaded three rows ahead;
// nothing is claimed or counted at run time, so the loop issues few scalar
// instructions and the waves of all CUs sweep the index rows together.
// Epilogue: one thread per row adds its sidecar terms delta * x[c] in stored
// order (x from LDS) and the bias.  Deterministic.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace dc1 {
constexpr int THREADS = 512, WAVES = THREADS / 64;
constexpr int RMAX = 96;      // rows per workgroup
constexpr int SCAP = 512;     // sidecar triplets per epilogue pass
constexpr int KMAX = 12288;
constexpr int OFF_X = 0;                    // x as fp32, KMAX, in lane order (xoff)
constexpr int OFF_PART = OFF_X + KMAX * 4;  // row sums
constexpr int OFF_TV = OFF_PART + RMAX * 4; // sidecar terms of a pass
constexpr int OFF_MISC = OFF_TV + SCAP * 4; // lo, hi (int64), row ranges
constexpr int LDS_DYN = OFF_MISC + 16 + 2 * RMAX * 4;
}  // namespace dc1

// Where x[k] sits in LDS (floats): element e of 16-byte piece h of lane l's
// chunk c (k = 16 (64 c + l) + 4 h + e) at ((4 c + h) 64 + l) 4 + e, so the
// lanes' reads of piece h are consecutive 16-byte pieces (no bank conflicts).
__device__ __forceinline__ int xoff(int k) {
  return ((((k >> 10) << 2) + ((k >> 2) & 3)) * 64 + ((k >> 4) & 63)) * 4 + (k & 3);
}

// CH: chunks of 16 weights per lane and row (K <= 1024 CH); XL: x read from
// LDS per chunk (else held in registers, K == 1024 CH); ONE: no wave has more
// than one row (the launch plan's rows per workgroup <= 8), so a wave requests
// its row alone instead of a ring of three; NT: index bytes loaded
// non-temporally (launches that stream more than the L2s hold)
template <bool PK12, bool XBF, int CH, bool XL, bool ONE, bool NT>
__global__ __launch_bounds__(dc1::THREADS, 1) void decode1_gemv(GemvMArgs ga) {
  using namespace dc1;
  __shared__ __align__(16) unsigned char cbs[PK12 ? 4096 * 8 : 256 * 256];
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem + OFF_X);
  float* part = reinterpret_cast<float*>(smem + OFF_PART);
  float* tv = reinterpret_cast<float*>(smem + OFF_TV);
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + OFF_MISC);
  int* rsb = reinterpret_cast<int*>(smem + OFF_MISC + 16);
  int* rse = rsb + RMAX;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int G = gridDim.x, bx = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int bb = (bx < full) ? (bx % 8) * per + bx / 8 : bx;  // each XCD a contiguous run of rows
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < ga.nseg && bb >= ga.wg0[i]) si = i;
  const GemvSeg& a = ga.seg[si];
  const int Gl = (si + 1 < ga.nseg ? ga.wg0[si + 1] : G) - ga.wg0[si];
  const int b = bb - ga.wg0[si];
  const int N = a.N, K = ga.K;
  const int r0 = split_point(b, N, Gl), r1 = split_point(b + 1, N, Gl);
  const int nrow = r1 - r0;
  const int nj = nrow > wave ? (nrow - wave + WAVES - 1) / WAVES : 0;  // this wave's rows
  constexpr int CB = PK12 ? 12 : 16;                                   // index bytes per chunk
  const int64_t row_bytes = (int64_t)K / 16 * CB;

  // ---- prologue.  Requests in the order they are waited for: the bias (used
  // last, but one small load), the codebook and x (the barrier waits for
  // their LDS copies), the sidecar window (waves 0 and 1), then the index
  // bytes of the wave's first rows.
  float bias_v = 0.f;
  if (a.bias) bias_v = a.bias[min(r0 + tid, N - 1)];
  constexpr int CBV = PK12 ? 4096 * 8 / 16 / THREADS : 1;
  u32x4 cbv[CBV];
  float cv = 0.f;
  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) cbv[i] = reinterpret_cast<const u32x4*>(a.codebook)[tid + i * THREADS];
  } else {
    cv = a.codebook[tid & 255];
  }
  // x: 16-byte pieces, thread t the pieces t, t + 512, ... (clamped: a thread
  // past the end loads and stores the last piece again, so neither the load
  // nor the store sits under a condition); one copy per workgroup in LDS
  constexpr int XE = XBF ? 8 : 4;  // elements per piece
  constexpr int XPT = (CH * 1024 / XE + THREADS - 1) / THREADS;
  const int xpieces = K / XE;
  u32x4 xv[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) xv[i] = reinterpret_cast<const u32x4*>(ga.x)[min(tid + THREADS * i, xpieces - 1)];
  const bool srch = a.nnz > 0 && wave < 2 && nrow > 0;
  const int target = wave == 0 ? r0 : r1;
  RowWindow win;
  if (srch) row_window_load(a.sc_rows, a.nnz, sidecar_guess(a.nnz, target, N), win);

  // ---- index bytes of the wave's row j (past its last row: a valid stand-in, unused)
  typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
  const int kch = K / 16;  // chunks of 16 in a row
  auto load_row = [&](int j, u32x4 (&iq)[CH]) {
    const int row = min(r0 + wave + WAVES * min(j, max(nj - 1, 0)), N - 1);
    const uint8_t* p = a.indices + (int64_t)row * row_bytes;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = XL ? min(64 * c + lane, kch - 1) : 64 * c + lane;
      if (PK12) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(p + CB * cc);
        iq[c] = u32x4{v[0], v[1], v[2], 0u};
      } else {
        iq[c] = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + CB * cc))
                   : *reinterpret_cast<const u32x4*>(p + CB * cc);
      }
    }
  };
  u32x4 IQ[ONE ? 1 : 3][CH];
  load_row(0, IQ[0]);
  if constexpr (!ONE) {
    load_row(1, IQ[1]);
    load_row(2, IQ[2]);
  }
  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) reinterpret_cast<u32x4*>(cbs)[tid + i * THREADS] = cbv[i];
  } else {
    const int e = tid & 255, h = tid >> 8;
    const float4 v4 = make_float4(cv, cv, cv, cv);
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<float4*>(cbs + e * 256 + (((8 * h + q + e) & 15) << 4)) = v4;
  }
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int q = min(tid + THREADS * i, xpieces - 1);
    if (XBF) {
      const u32x4 w = xv[i];
      *reinterpret_cast<float4*>(xs + xoff(8 * q)) = make_float4(
          __uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
          __uint_as_float(w[1] & 0xffff0000u));
      *reinterpret_cast<float4*>(xs + xoff(8 * q + 4)) = make_float4(
          __uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u), __uint_as_float(w[3] << 16),
          __uint_as_float(w[3] & 0xffff0000u));
    } else {
      *reinterpret_cast<u32x4*>(xs + xoff(4 * q)) = xv[i];
    }
  }
  if (XL)  // zeros from K up to whole chunks of every lane
    for (int k = K + 4 * tid; k < 1024 * CH; k += 4 * THREADS)
      *reinterpret_cast<float4*>(xs + xoff(k)) = make_float4(0.f, 0.f, 0.f, 0.f);
  asm volatile("" ::: "memory");  // the lookup (and its wait) stays below the loads
  if (tid < RMAX) rsb[tid] = rse[tid] = 0;  // the first sidecar pass's row ranges
  if (srch) {
    const int64_t v = row_window_lower_bound(a.sc_rows, a.nnz, target, win);
    if (lane == 0) lohi[wave] = v;
  }
  __syncthreads();

  // the lane's x: k = 16 (64 c + lane) + i
  constexpr int XRC = XL ? 1 : CH;
  float xr[XRC][16];
  auto read_x = [&](int c, float (&d)[16]) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 v = *reinterpret_cast<const float4*>(xs + ((4 * c + h) * 64 + lane) * 4);
      d[4 * h] = v.x, d[4 * h + 1] = v.y, d[4 * h + 2] = v.z, d[4 * h + 3] = v.w;
    }
  };
  if (!XL)
#pragma unroll
    for (int c = 0; c < XRC; ++c) read_x(c, xr[c]);
  // the block's triplet range and the first epilogue pass's triplets
  int64_t lo = 0, hi = 0;
  if (a.nnz > 0 && nrow > 0) {
    lo = lohi[0];
    hi = lohi[1];
  }
  int tc = 0, tr = 0, trp = 0, trn = 0;
  float tdl = 0.f;
  if (lo < hi && tid < SCAP) {
    const int cnt = (int)min<int64_t>(SCAP, hi - lo);
    const int64_t ee = lo + min(tid, cnt - 1);
    tc = a.sc_cols[ee];
    tdl = a.sc_deltas[ee];
    tr = a.sc_rows[ee];
    trp = a.sc_rows[ee > 0 ? ee - 1 : 0];
    trn = a.sc_rows[ee + 1 < a.nnz ? ee + 1 : ee];
  }

  // ---- one row: four partial sums (weights 4 d + e go to sum e), then the wave sum
  auto row = [&](auto r_c, int j) {
    constexpr int R = decltype(r_c)::value;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float xl[16];
      if (XL) read_x(c, xl);
      const float(&xc)[16] = XL ? xl : xr[XL ? 0 : c];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float w[4];
        if (PK12) {
          const u32x4 v4 = IQ[R][c];
          const uint32_t v = d == 0 ? (v4[0] & 0xffffffu)
                           : d == 1 ? (__builtin_amdgcn_alignbit(v4[1], v4[0], 24) & 0xffffffu)
                           : d == 2 ? (__builtin_amdgcn_alignbit(v4[2], v4[1], 16) & 0xffffffu)
                                    : (v4[2] >> 8);
          const float2 p0 = lds_load<float2>((v & 0xfffu) << 3, cbs);
          const float2 p1 = lds_load<float2>((v >> 12) << 3, cbs);
          w[0] = p0.x, w[1] = p0.y, w[2] = p1.x, w[3] = p1.y;
        } else {
          const uint32_t wd = IQ[R][c][d];
          w[0] = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
          w[1] = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
          w[2] = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
          w[3] = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = fmaf(w[e], xc[4 * d + e], s[e]);
      }
    }
    const float t = wave_sum_dpp((s[0] + s[1]) + (s[2] + s[3]));
    if (lane == 0) part[wave + WAVES * j] = t;
    if constexpr (!ONE) load_row(j + 3, IQ[R]);
  };
  if constexpr (ONE) {
    if (nj > 0) row(std::integral_constant<int, 0>{}, 0);
  } else {
    int j = 0;
    for (; j + 2 < nj; j += 3) {
      row(std::integral_constant<int, 0>{}, j);
      row(std::integral_constant<int, 1>{}, j + 1);
      row(std::integral_constant<int, 2>{}, j + 2);
    }
    if (j < nj) row(std::integral_constant<int, 0>{}, j);
    if (j + 1 < nj) row(std::integral_constant<int, 1>{}, j + 1);
  }
  // the first sidecar pass's terms (x from LDS; the triplets arrived during
  // the rows), before the barrier, so the epilogue only adds them
  const int cnt0 = (int)min<int64_t>(SCAP, hi - lo);
  if (lo < hi && tid < cnt0) {
    tv[tid] = tdl * xs[xoff(tc)];
    if (tid == 0 || trp != tr) rsb[tr - r0] = tid;
    if (tid == cnt0 - 1 || trn != tr) rse[tr - r0] = tid + 1;
  }
  __syncthreads();

  // ---- epilogue: thread r -> row r0 + r
  float out = tid < nrow ? part[tid] : 0.f;
  if (tid < nrow)
    for (int e = rsb[tid]; e < rse[tid]; ++e) out += tv[e];
  for (int64_t e0 = lo + SCAP; e0 < hi; e0 += SCAP) {  // more triplets than one pass takes
    const int cnt = (int)min<int64_t>(SCAP, hi - e0);
    __syncthreads();
    if (tid < RMAX) rsb[tid] = rse[tid] = 0;
    __syncthreads();
    if (tid < SCAP) {
      const int64_t ee = e0 + min(tid, cnt - 1);
      tc = a.sc_cols[ee];
      tdl = a.sc_deltas[ee];
      tr = a.sc_rows[ee];
      trp = a.sc_rows[ee > 0 ? ee - 1 : 0];
      trn = a.sc_rows[ee + 1 < a.nnz ? ee + 1 : ee];
      if (tid < cnt) {
        tv[tid] = tdl * xs[xoff(tc)];
        if (tid == 0 || trp != tr) rsb[tr - r0] = tid;
        if (tid == cnt - 1 || trn != tr) rse[tr - r0] = tid + 1;
      }
    }
    __syncthreads();
    if (tid < nrow)
      for (int e = rsb[tid]; e < rse[tid]; ++e) out += tv[e];
  }
  if (tid < nrow) a.y[r0 + tid] = out + bias_v;
}

bool decode1_ok(const DecodeSeg& s, bool pk12, bool xbf, int M, int K, const void* x) {
  if (M != 1 || K < 16 || K > dc1::KMAX || K % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(s.indices) % (pk12 ? 4 : 16) != 0) return false;
  if (pk12 && reinterpret_cast<uintptr_t>(s.codebook) % 16 != 0) return false;
  (void)xbf;
  return reinterpret_cast<uintptr_t>(x) % 16 == 0;
}

bool decode1_takes(const DecodeSeg& s, bool pk12, bool xbf, int M, int K, const void* x) {
  return decode1_ok(s, pk12, xbf, M, K, x) && (int64_t)s.N <= (int64_t)device_cu_count() * dc1::RMAX;
}

// Workgroups per layer in proportion to its rows, one per CU at most, each
// owning at most RMAX rows; false when that does not fit.
static bool decode1_plan(GemvMArgs& g, int& grid) {
  using namespace dc1;
  const int cus = device_cu_count();
  int64_t rows = 0;
  for (int i = 0; i < g.nseg; ++i) rows += g.seg[i].N;
  const int64_t want = rows < cus ? rows : cus;
  int alloc[kMaxSegments];
  int64_t tot = 0;
  for (int i = 0; i < g.nseg; ++i) {
    const int64_t need = (g.seg[i].N + RMAX - 1) / RMAX;
    int64_t share = want * g.seg[i].N / rows;
    if (share < need) share = need;
    if (share < 1) share = 1;
    if (share > g.seg[i].N) share = g.seg[i].N;
    alloc[i] = (int)share;
    tot += share;
  }
  if (tot > cus) return false;
  grid = 0;
  for (int i = 0; i < g.nseg; ++i) {
    g.wg0[i] = grid;
    grid += alloc[i];
  }
  for (int i = g.nseg; i < kMaxSegments; ++i) {
    g.wg0[i] = INT_MAX;
    g.seg[i] = g.seg[0];
  }
  return true;
}

template <bool PK12, bool XBF, int CH, bool XL, bool ONE, bool NT>
static hipError_t launch_decode1_o(const GemvMArgs& g, int grid, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&decode1_gemv<PK12, XBF, CH, XL, ONE, NT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, dc1::LDS_DYN);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((decode1_gemv<PK12, XBF, CH, XL, ONE, NT>), dim3((unsigned)grid), dim3(dc1::THREADS),
                     dc1::LDS_DYN, stream, g);
  return hipGetLastError();
}

// one: at most one row per wave (no ring); lng: non-temporal index loads
// (ring instance only: no ring-less launch streams that much)
template <bool PK12, bool XBF, int CH, bool XL>
static hipError_t launch_decode1_x(const GemvMArgs& g, int grid, bool one, bool lng, hipStream_t stream) {
  if (one) return launch_decode1_o<PK12, XBF, CH, XL, true, false>(g, grid, stream);
  return lng ? launch_decode1_o<PK12, XBF, CH, XL, false, true>(g, grid, stream)
             : launch_decode1_o<PK12, XBF, CH, XL, false, false>(g, grid, stream);
}

// K a multiple of 1024 up to 4096: x in registers; otherwise x from LDS with
// the smallest instantiated chunk count that covers K
template <bool PK12, bool XBF>
static hipError_t launch_decode1_k(const GemvMArgs& g, int grid, bool one, bool lng, hipStream_t stream) {
  if (g.K % 1024 == 0 && g.K <= 4096) {
    switch (g.K / 1024) {
      case 1: return launch_decode1_x<PK12, XBF, 1, false>(g, grid, one, lng, stream);
      case 2: return launch_decode1_x<PK12, XBF, 2, false>(g, grid, one, lng, stream);
      case 3: return launch_decode1_x<PK12, XBF, 3, false>(g, grid, one, lng, stream);
      default: return launch_decode1_x<PK12, XBF, 4, false>(g, grid, one, lng, stream);
    }
  }
  const int ch = (g.K + 1023) / 1024;
  if (ch <= 2) return launch_decode1_x<PK12, XBF, 2, true>(g, grid, one, lng, stream);
  if (ch <= 4) return launch_decode1_x<PK12, XBF, 4, true>(g, grid, one, lng, stream);
  if (ch <= 6) return launch_decode1_x<PK12, XBF, 6, true>(g, grid, one, lng, stream);
  if (ch <= 8) return launch_decode1_x<PK12, XBF, 8, true>(g, grid, one, lng, stream);
  if (ch <= 11) return launch_decode1_x<PK12, XBF, 11, true>(g, grid, one, lng, stream);
  return launch_decode1_x<PK12, XBF, 12, true>(g, grid, one, lng, stream);
}

bool launch_decode1(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                    hipStream_t stream, hipError_t& err) {
  if (nseg < 1 || nseg > kMaxSegments) return false;
  for (int i = 0; i < nseg; ++i)
    if (!decode1_ok(segs[i], pk12, xbf, M, K, x)) return false;
  GemvMArgs g;
  g.x = x;
  g.M = M;
  g.K = K;
  g.nseg = nseg;
  for (int i = 0; i < nseg; ++i)
    g.seg[i] = {static_cast<const float*>(segs[i].codebook), segs[i].indices, segs[i].sc_rows, segs[i].sc_cols,
                segs[i].sc_deltas, segs[i].nnz, segs[i].bias, segs[i].y, segs[i].N, segs[i].N};
  int grid = 0;
  if (!decode1_plan(g, grid)) return false;
  // the most rows any workgroup owns: at most one per wave takes the ring-less instance
  int most = 0;
  for (int i = 0; i < nseg; ++i) {
    const int wgs = (i + 1 < nseg ? g.wg0[i + 1] : grid) - g.wg0[i];
    const int r = (g.seg[i].N + wgs - 1) / wgs;
    if (r > most) most = r;
  }
  const bool one = most <= dc1::WAVES;
  // non-temporal index loads past the L2s' capacity (Qwen decode step: gate|up
  // 12.6 -> 11.8-12.1 us, the four launches 35.3 -> 31.7 us)
  int64_t ib = 0;
  for (int i = 0; i < nseg; ++i) ib += index_bytes(segs[i].N, K, pk12);
  const bool lng = ib > kStreamPastCacheBytes;
  if (pk12)
    err = xbf ? launch_decode1_k<true, true>(g, grid, one, lng, stream) : launch_decode1_k<true, false>(g, grid, one, lng, stream);
  else
    err = xbf ? launch_decode1_k<false, true>(g, grid, one, lng, stream)
              : launch_decode1_k<false, false>(g, grid, one, lng, stream);
  return true;
}

}  // namespace hxq
