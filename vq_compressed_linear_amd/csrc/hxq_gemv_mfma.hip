// Matrix-core HelixLinear GEMV for up to 64 tokens (used from 5, and below
// that where the decode kernel does not fit), u8 and pk12, fp32 or bf16 x.
//
// y[m][n] = sum_k (W[n][k] + S[n][k]) x[m][k] + b[n], W the codebook value of
// the weight's index (u8) or component k % 2 of its pair's entry (pk12), with
// fp32 products
// and fp32 sums: the codebook values (fp32) and x (fp32, or bf16 upcast
// exactly) go into v_mfma_f32_16x16x4_f32, so the arithmetic is the fp32
// arithmetic of the vector paths, in another summation order.  (The model
// cards' "codebook[indices] @ x" with no dense weight; the HXQ whitepaper's
// inference paragraph: gather + sidecar + matmul.)
//
// At a handful of tokens the vector kernel spends M fused multiply-adds per
// gathered weight and becomes ALU-bound; here one gather feeds a 16-token
// matrix-core step, and the index stream stays the bottleneck up to M = 16.
//
// Work split: a workgroup owns whole fragments of 16 rows (at most FMAX) and
// all of K.  Tokens come in TG groups of 16 (one group up to 16 tokens, two
// up to 32, four up to 64); the eight waves are TG teams of 8 / TG, and wave
// c of a team takes the 64-deep chunk c of every slice (512 / TG deep) for
// the team's tokens, so every index byte is fetched by TG waves (the repeats
// hit the caches).  Lane (g, l16) holds the indices of row l16,
// k = 16 g .. 16 g + 15 of its chunk (16 bytes u8, 12 bytes = 8 pairs pk12);
// matrix-core step s sums k = 16 g + s
// over g, with x read as the B operand for the same k.  x is staged per slice
// in LDS (double-buffered, one barrier per slice) from registers loaded three
// slices ahead.  A team's partial
// tiles are added in wave order at the end; sidecar terms delta * x are added
// after them in stored order, then the bias.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace gmv {
constexpr int THREADS = 512, WAVES = THREADS / 64;
constexpr int KC = 64;                 // k per wave chunk: 16 index bytes per lane
constexpr int FMAX = 4;                // 16-row fragments per workgroup
constexpr int XSL = 16 * KC * WAVES * 4;  // one fp32 x slice (tokens x k): 32 KB
constexpr int TV = 8192;               // sidecar terms (triplets x staged tokens) per epilogue pass
constexpr int OFF_MISC = 2 * XSL;      // lo, hi (int64), row ranges
constexpr int LDS_DYN = OFF_MISC + 16 + 2 * FMAX * 16 * 4;
static_assert(WAVES * FMAX * 64 * 16 + TV * 4 <= 2 * XSL, "partials and sidecar terms fit the x buffers");
}  // namespace gmv

// FN: fragments per workgroup (the launch's largest; a workgroup may own one
// fewer); MX: x rows staged per slice (8, 16, 32 or 64, at least M)
template <bool PK12, bool XBF, int FN, int MX>
__global__ __launch_bounds__(gmv::THREADS, 1) void gemv_mfma(GemvMArgs ga) {
  using namespace gmv;
  constexpr int TG = MX > 16 ? MX / 16 : 1;  // token groups of 16
  constexpr int WPG = WAVES / TG;            // waves per team
  constexpr int KS = KC * WPG;               // k per slice: one chunk per wave of a team
  constexpr int MXR = 16 * TG;               // token slots of the result tile
  constexpr int SCAP = TV / MXR;             // sidecar triplets per epilogue pass
  static_assert(MX * KS * 4 <= XSL, "x slice fits its buffer");
  // u8: fp32 codebook, 64 copies per entry; pk12: the 4096 fp32 pairs
  __shared__ __align__(16) unsigned char cbs[PK12 ? 4096 * 8 : 256 * 256];
  extern __shared__ __align__(16) unsigned char smem[];
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + OFF_MISC);
  int* rsb = reinterpret_cast<int*>(smem + OFF_MISC + 16);  // per row of the block: first, end term
  int* rse = rsb + FMAX * 16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int team = wave / WPG, cw = wave % WPG;  // token group, chunk in the slice
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int G = gridDim.x, bx = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int bb = (bx < full) ? (bx % 8) * per + bx / 8 : bx;  // each XCD a contiguous run of rows
  // the layer: workgroups wg0[i] .. wg0[i + 1] - 1 belong to layer i
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < ga.nseg && bb >= ga.wg0[i]) si = i;
  const GemvSeg& a = ga.seg[si];
  const int Gl = (si + 1 < ga.nseg ? ga.wg0[si + 1] : G) - ga.wg0[si];
  const int b = bb - ga.wg0[si];
  const int M = ga.M, N = a.N, K = ga.K;
  const int f0 = split_point(b, a.nfrag, Gl), f1 = split_point(b + 1, a.nfrag, Gl);
  const int F = f1 - f0;  // FN - 1 .. FN, uniform
  const int r0 = f0 * 16, r1 = min(f1 * 16, N);
  const int nsl = (K + KS - 1) / KS;

  // ---- index bytes of (slice s, fragment f): row of fragment f, this wave's chunk
  const uint8_t* irow[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int row = min((f0 + min(f, max(F - 1, 0))) * 16 + l16, N - 1);
    irow[f] = PK12 ? a.indices + (int64_t)row * (K / 4 * 3) + 12 * g : a.indices + (int64_t)row * K + 16 * g;
  }
  typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
  auto load_iq = [&](int s, u32x4* d) {
    const int k0 = min(s * KS + cw * KC, K - KC);  // chunks past K read a valid one, unused
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if (PK12) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(irow[f] + k0 / 4 * 3);
        d[f] = u32x4{v[0], v[1], v[2], 0u};
      } else {
        d[f] = *reinterpret_cast<const u32x4*>(irow[f] + k0);
      }
    }
  };
  // ---- x slice: piece p = tid + 512 i covers token p / (KS / 4), k = 4 (p % (KS / 4))
  // .. + 3 of the slice; token t = 16 q + t16 is stored at
  // ((q * KS / 16 + k / 16) * 16 + t16) * 64 + (k % 16) * 4.  With MX = 8, rows 8 .. 15
  // of the LDS slice are never written: they only reach result columns that are not
  // stored.
  constexpr int XPT = MX * KS / 4 / THREADS;  // 4-wide pieces per thread
  constexpr int PR = KS / 4;                  // pieces per token row
  static_assert(XPT * THREADS == MX * PR, "pieces cover the slice");
  auto load_x = [&](int s, u32x4* XR) {
    const int sc = min(s, nsl - 1);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int p = tid + THREADS * i, t = p / PR, kq = p % PR;
      const int k = min(sc * KS + 4 * kq, K - 4);
      const int tm = min(t, M - 1);
      // (no zeroing: tokens past M repeat row M - 1 into result columns that are
      // never stored, and k past K only reaches chunks whose steps are skipped;
      // a select on the loaded value would become a branch around the load)
      if (XBF) {
        const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(ga.x) + (int64_t)tm * K + k);
        XR[i] = u32x4{h.x << 16, h.x & 0xffff0000u, h.y << 16, h.y & 0xffff0000u};
      } else {
        XR[i] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(ga.x) + (int64_t)tm * K + k);
      }
    }
  };
  auto store_x = [&](int s, const u32x4* XR) {
    unsigned char* buf = smem + (s & 1) * XSL;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int p = tid + THREADS * i, t = p / PR, kq = p % PR;
      *reinterpret_cast<u32x4*>(buf + ((((t >> 4) * (KS / 16) + (kq >> 2)) * 16 + (t & 15)) << 6) +
                                ((kq & 3) << 4)) = XR[i];
    }
  };

  // x and index bytes of slice j live in register set j % 3, loaded three
  // slices ahead (a slice's own work is short next to a memory round trip)
  // (x of slice 0 and the codebook first: their LDS stores wait for them, and
  // loads complete in order)
  // sidecar: waves 0 and 1 look up the first triplet of rows r0 and r1; their
  // window loads go out before everything else, so the answer does not wait
  // for the prefetch behind it
  const bool srch = a.nnz > 0 && wave < 2 && F > 0;  // uniform
  const int target = wave == 0 ? r0 : r1;
  RowWindow win;
  if (srch) row_window_load(a.sc_rows, a.nnz, sidecar_guess(a.nnz, target, N), win);
  u32x4 IQ[3][FN], XR[3][XPT];
  load_x(0, XR[0]);
  constexpr int CBV = PK12 ? 4096 * 8 / 16 / THREADS : 1;  // 16-byte codebook pieces per thread
  u32x4 cbv[CBV];
  float cv = 0.f;
  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) cbv[i] = reinterpret_cast<const u32x4*>(a.codebook)[tid + i * THREADS];
  } else {
    cv = a.codebook[tid & 255];
  }
  load_iq(0, IQ[0]);
  load_iq(1, IQ[1]);
  load_iq(2, IQ[2]);
  load_x(1, XR[1]);
  load_x(2, XR[2]);

  // ---- codebook.  u8: entry e, copy j at byte e * 256 + 4 j; threads t, t + 256 write
  // half each.  pk12: the table as stored, entry e at byte 8 e.
  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) reinterpret_cast<u32x4*>(cbs)[tid + i * THREADS] = cbv[i];
  } else {
    const int e = tid & 255, h = tid >> 8;
    const float4 v4 = make_float4(cv, cv, cv, cv);
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<float4*>(cbs + e * 256 + (((8 * h + q + e) & 15) << 4)) = v4;
  }
  // ---- sidecar: the block's triplet range [lo, hi) (kept below the prefetch: a
  // compiler barrier stops the lookup, and its wait, from being hoisted above it)
  asm volatile("" ::: "memory");
  if (srch) {
    const int64_t v = row_window_lower_bound(a.sc_rows, a.nnz, target, win);
    if (lane == 0) lohi[wave] = v;
  }
  store_x(0, XR[0]);
  load_x(3, XR[0]);
  __syncthreads();

  // the block's triplet range, and the triplets of the first epilogue pass,
  // requested now: they are older than every load the slices wait for
  int64_t lo = 0, hi = 0;
  if (a.nnz > 0 && F > 0) {
    lo = lohi[0];
    hi = lohi[1];
  }
  const int te = tid % SCAP, tq = tid / SCAP;  // epilogue: triplet, token group
  int tc = 0, tr = 0, trp = 0, trn = 0;
  float tdl = 0.f;
  if (lo < hi && tid < SCAP * TG) {
    const int cnt = (int)min<int64_t>(SCAP, hi - lo);
    const int64_t ee = lo + min(te, cnt - 1);
    tc = a.sc_cols[ee];
    tdl = a.sc_deltas[ee];
    tr = a.sc_rows[ee];
    trp = a.sc_rows[ee > 0 ? ee - 1 : 0];
    trn = a.sc_rows[ee + 1 < a.nnz ? ee + 1 : ee];
  }

  f32x4 acc[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one slice: x(s) in buffer s & 1, its index bytes in IQ[s % 3]; stores
  // x(s + 1), loads x(s + 4) and the index bytes of slice s + 3
  auto slice = [&](auto r_c, int s) {
    constexpr int R = decltype(r_c)::value;  // s % 3
    u32x4* iq = IQ[R];
    store_x(s + 1, XR[(R + 1) % 3]);
    load_x(s + 4, XR[(R + 1) % 3]);
    const bool live = s * KS + cw * KC < K;  // uniform
    const unsigned char* xb = smem + (s & 1) * XSL + (((team * (KS / 16) + 4 * cw + g) * 16 + l16) << 6);
    const u32x4 xq0 = *reinterpret_cast<const u32x4*>(xb);
    const u32x4 xq1 = *reinterpret_cast<const u32x4*>(xb + 16);
    const u32x4 xq2 = *reinterpret_cast<const u32x4*>(xb + 32);
    const u32x4 xq3 = *reinterpret_cast<const u32x4*>(xb + 48);
    const u32x4 xq[4] = {xq0, xq1, xq2, xq3};
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if (f < F && live) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float w0, w1, w2, w3;
          if (PK12) {
            // pair group d: 24 bits at byte 3 d of the lane's 12, indices (a, b) =
            // (v & 0xfff, v >> 12) for weights 4 d, 4 d + 1 and 4 d + 2, 4 d + 3
            const uint32_t v = d == 0 ? (iq[f][0] & 0xffffffu)
                             : d == 1 ? (__builtin_amdgcn_alignbit(iq[f][1], iq[f][0], 24) & 0xffffffu)
                             : d == 2 ? (__builtin_amdgcn_alignbit(iq[f][2], iq[f][1], 16) & 0xffffffu)
                                      : (iq[f][2] >> 8);
            const float2 p0 = lds_load<float2>((v & 0xfffu) << 3, cbs);
            const float2 p1 = lds_load<float2>((v >> 12) << 3, cbs);
            w0 = p0.x, w1 = p0.y, w2 = p1.x, w3 = p1.y;
          } else {
            const uint32_t wd = iq[f][d];
            w0 = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
            w1 = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
            w2 = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
            w3 = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
          }
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(w0, __uint_as_float(xq[d][0]), acc[f], 0, 0, 0);
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(w1, __uint_as_float(xq[d][1]), acc[f], 0, 0, 0);
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(w2, __uint_as_float(xq[d][2]), acc[f], 0, 0, 0);
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(w3, __uint_as_float(xq[d][3]), acc[f], 0, 0, 0);
        }
      }
    }
    load_iq(s + 3, iq);
    __syncthreads();
  };
  int s = 0;
  for (; s + 2 < nsl; s += 3) {
    slice(std::integral_constant<int, 0>{}, s);
    slice(std::integral_constant<int, 1>{}, s + 1);
    slice(std::integral_constant<int, 2>{}, s + 2);
  }
  if (s < nsl) slice(std::integral_constant<int, 0>{}, s);
  if (s + 1 < nsl) slice(std::integral_constant<int, 1>{}, s + 1);

  // ---- partial tiles, each team's in wave order; lane (g, l16), register r of
  // fragment f: row 16 f + 4 g + r of the block, token 16 team + l16
  f32x4* part = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int f = 0; f < FN; ++f)
    if (f < F) part[(wave * FMAX + f) * 64 + lane] = acc[f];
  const int nrow = r1 - r0;
  __syncthreads();
  // thread o -> token o / (16 FMAX), block row o % (16 FMAX): consecutive threads store
  // consecutive outputs
  constexpr int OPT = FMAX * 16 * MXR / THREADS;
  float out[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + THREADS * i, t = o / (16 * FMAX), j = o % (16 * FMAX);
    float v = 0.f;
    if (j < 16 * F) {
      const int f = j >> 4, jr = j & 15, ln = (t & 15) + 16 * (jr >> 2), w0 = (t >> 4) * WPG;
#pragma unroll
      for (int w = 0; w < WPG; ++w) v += part[((w0 + w) * FMAX + f) * 64 + ln][jr & 3];
    }
    out[i] = v;
  }
  // ---- sidecar terms delta * x[t][c], each output's in stored order, SCAP triplets a pass
  float* tv = reinterpret_cast<float*>(smem + WAVES * FMAX * 64 * 16);
  for (int64_t e0 = lo; e0 < hi; e0 += SCAP) {
    const int cnt = (int)min<int64_t>(SCAP, hi - e0);
    __syncthreads();
    for (int i = tid; i < 16 * FMAX; i += THREADS) rsb[i] = rse[i] = 0;
    __syncthreads();
    // thread e + SCAP q takes triplet e for tokens 16 q .. 16 q + 15; all loads of a
    // pass are issued together (the first pass's triplets are already here)
    if (tid < SCAP * TG) {
      const int e = te, q = tq;
      if (e0 != lo) {
        const int64_t ee = e0 + min(e, cnt - 1);
        tc = a.sc_cols[ee];
        tdl = a.sc_deltas[ee];
        tr = a.sc_rows[ee];
        trp = a.sc_rows[ee > 0 ? ee - 1 : 0];
        trn = a.sc_rows[ee + 1 < a.nnz ? ee + 1 : ee];
      }
      const int c = tc, r = tr, rp = trp, rn = trn;
      const float dl = tdl;
      float xv[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int tm = min(16 * q + t, M - 1);
        xv[t] = XBF ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(ga.x)[(int64_t)tm * K + c] << 16)
                    : static_cast<const float*>(ga.x)[(int64_t)tm * K + c];
      }
      if (e < cnt) {
#pragma unroll
        for (int t = 0; t < 16; ++t) tv[e * MXR + 16 * q + t] = dl * xv[t];
        if (q == 0 && (e == 0 || rp != r)) rsb[r - r0] = e;
        if (q == 0 && (e == cnt - 1 || rn != r)) rse[r - r0] = e + 1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int o = tid + THREADS * i, t = o / (16 * FMAX), j = o % (16 * FMAX);
      if (j < nrow)
        for (int e = rsb[j]; e < rse[j]; ++e) out[i] += tv[e * MXR + t];
    }
  }
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + THREADS * i, t = o / (16 * FMAX), j = o % (16 * FMAX);
    if (t < M && j < nrow) {
      const int n = r0 + j;
      a.y[(int64_t)t * N + n] = out[i] + (a.bias ? a.bias[n] : 0.f);
    }
  }
}

bool gemv_mfma_ok(const LayerArgs& a, bool pk12) {
  if (a.M < 1 || a.M > kGemvMfmaMaxM || a.K < gmv::KC || a.K % gmv::KC != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.indices) % (pk12 ? 4 : 16) != 0) return false;
  if (pk12 && reinterpret_cast<uintptr_t>(a.codebook) % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.x) % (a.x_bf16 ? 8 : 16) != 0) return false;
  return true;
}

template <bool PK12, bool XBF, int FN, int MX>
static hipError_t launch_gemv_mfma_x(const GemvMArgs& g, int grid, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_mfma<PK12, XBF, FN, MX>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, gmv::LDS_DYN);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemv_mfma<PK12, XBF, FN, MX>), dim3((unsigned)grid), dim3(gmv::THREADS), gmv::LDS_DYN, stream, g);
  return hipGetLastError();
}

template <bool PK12, bool XBF, int MX>
static hipError_t launch_gemv_mfma_f(const GemvMArgs& g, int fn, int grid, hipStream_t stream) {
  switch (fn) {
    case 1: return launch_gemv_mfma_x<PK12, XBF, 1, MX>(g, grid, stream);
    case 2: return launch_gemv_mfma_x<PK12, XBF, 2, MX>(g, grid, stream);
    case 3: return launch_gemv_mfma_x<PK12, XBF, 3, MX>(g, grid, stream);
    default: return launch_gemv_mfma_x<PK12, XBF, 4, MX>(g, grid, stream);
  }
}

template <bool PK12>
static hipError_t launch_gemv_mfma_p(const GemvMArgs& g, bool xbf, int fn, int grid, hipStream_t stream) {
  if (xbf) {
    if (g.M <= 8) return launch_gemv_mfma_f<PK12, true, 8>(g, fn, grid, stream);
    if (g.M <= 16) return launch_gemv_mfma_f<PK12, true, 16>(g, fn, grid, stream);
    if (g.M <= 32) return launch_gemv_mfma_f<PK12, true, 32>(g, fn, grid, stream);
    return launch_gemv_mfma_f<PK12, true, 64>(g, fn, grid, stream);
  }
  if (g.M <= 8) return launch_gemv_mfma_f<PK12, false, 8>(g, fn, grid, stream);
  if (g.M <= 16) return launch_gemv_mfma_f<PK12, false, 16>(g, fn, grid, stream);
  if (g.M <= 32) return launch_gemv_mfma_f<PK12, false, 32>(g, fn, grid, stream);
  return launch_gemv_mfma_f<PK12, false, 64>(g, fn, grid, stream);
}

// Workgroups per layer in proportion to its 16-row fragments, each layer at
// least ceil(fragments / FMAX); false when the launch would need more
// fragments per workgroup than the kernel takes.
static bool gemv_mfma_plan(GemvMArgs& g, int& grid, int& fn) {
  using namespace gmv;
  const int cus = device_cu_count();
  int64_t frags = 0;
  for (int i = 0; i < g.nseg; ++i) frags += g.seg[i].nfrag;
  int64_t want = frags < cus ? frags : cus;
  int alloc[kMaxSegments];
  int64_t tot = 0;
  for (int i = 0; i < g.nseg; ++i) {
    const int64_t need = (g.seg[i].nfrag + FMAX - 1) / FMAX;
    int64_t share = want * g.seg[i].nfrag / frags;
    if (share < need) share = need;
    if (share < 1) share = 1;
    if (share > g.seg[i].nfrag) share = g.seg[i].nfrag;
    alloc[i] = (int)share;
    tot += share;
  }
  if (tot > INT_MAX / 2) return false;
  grid = 0;
  fn = 1;
  for (int i = 0; i < g.nseg; ++i) {
    g.wg0[i] = grid;
    grid += alloc[i];
    const int f = (g.seg[i].nfrag + alloc[i] - 1) / alloc[i];
    if (f > fn) fn = f;
  }
  for (int i = g.nseg; i < kMaxSegments; ++i) {
    g.wg0[i] = INT_MAX;
    g.seg[i] = g.seg[0];
  }
  return fn <= FMAX;
}

hipError_t launch_gemv_mfma_grouped(const GemvSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M,
                                    int K, hipStream_t stream) {
  if (nseg < 1 || nseg > kMaxSegments) return hipErrorInvalidValue;
  GemvMArgs g;
  g.x = x;
  g.M = M;
  g.K = K;
  g.nseg = nseg;
  for (int i = 0; i < nseg; ++i) {
    g.seg[i] = segs[i];
    g.seg[i].nfrag = (segs[i].N + 15) / 16;
  }
  int grid = 0, fn = 1;
  if (!gemv_mfma_plan(g, grid, fn)) return hipErrorInvalidValue;
  return pk12 ? launch_gemv_mfma_p<true>(g, xbf, fn, grid, stream) : launch_gemv_mfma_p<false>(g, xbf, fn, grid, stream);
}

bool gemv_mfma_group_fits(const GemvSeg* segs, int nseg) {
  if (nseg < 1 || nseg > kMaxSegments) return false;
  GemvMArgs g;
  g.nseg = nseg;
  for (int i = 0; i < nseg; ++i) {
    g.seg[i] = segs[i];
    g.seg[i].nfrag = (segs[i].N + 15) / 16;
  }
  int grid = 0, fn = 1;
  // one workgroup per CU at most: otherwise separate launches run better
  return gemv_mfma_plan(g, grid, fn) && grid <= device_cu_count();
}

hipError_t launch_gemv_mfma(const LayerArgs& a, bool pk12, hipStream_t stream) {
  const GemvSeg sg = {static_cast<const float*>(a.codebook), a.indices, a.sc_rows, a.sc_cols, a.sc_deltas, a.nnz,
                      a.bias, a.y, a.N, 0};
  return launch_gemv_mfma_grouped(&sg, 1, pk12, a.x, a.x_bf16, a.M, a.K, stream);
}

bool gemv_mfma_takes(const LayerArgs& a, bool pk12) {
  LayerArgs c = a;
  c.M = min(a.M, kGemvMfmaMaxM);
  return a.M >= 1 && gemv_mfma_ok(c, pk12);
}

hipError_t launch_gemv_mfma_tokens(const LayerArgs& a, bool pk12, hipStream_t stream) {
  if (a.M <= kGemvMfmaMaxM) return launch_gemv_mfma(a, pk12, stream);
  // launches of 64 tokens on offset x and y rows; the offsets are multiples of
  // 64 rows of K % 64 == 0 elements, so x stays aligned
  LayerArgs c = a;
  const size_t xrow = (size_t)a.K * (a.x_bf16 ? 2 : 4);
  for (int m0 = 0; m0 < a.M; m0 += kGemvMfmaMaxM) {
    c.M = min(kGemvMfmaMaxM, a.M - m0);
    c.x = static_cast<const unsigned char*>(a.x) + (size_t)m0 * xrow;
    c.y = a.y + (size_t)m0 * a.N;
    const hipError_t err = launch_gemv_mfma(c, pk12, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace hxq
