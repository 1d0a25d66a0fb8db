// Matrix-core HelixLinear GEMV for 5 to 8 tokens on 4x4 fp32 blocks, u8 and
// pk12, fp32 or bf16 x, one or several layers per launch.
//
// y[m][n] = sum_k (W[n][k] + S[n][k]) x[m][k] + b[n], W the codebook value of
// the weight's index (u8) or component k % 2 of its pair's entry (pk12), with
// fp32 products and fp32 sums (model cards, "What is HelixCode?"; HXQ
// whitepaper, "Method" and "2D vector quantization"; inference paragraph:
// gather + sidecar + matmul, with no dense weight formed).
//
// v_mfma_f32_4x4x1_16b_f32 computes 16 independent 4 x 4 outer products: lane
// 4 b + t gives row t of block b's A column and column t of its B row, and
// receives block b's results for column t (register r = row r).  Here block b
// is a 16-deep stretch of k: a unit of work is 4 output rows (a fragment) x
// 256 k (a chunk), lane (b, i) holds the 16 index bytes of row i at
// k = 16 b .. 16 b + 15 of the chunk (12 bytes = 8 pairs for pk12), and step s
// multiplies the weights at k = 16 b + s by x at the same k for 4 tokens.  The
// 16 blocks' partial sums are added across lanes once per fragment.  With 5
// to 8 tokens every product the unit computes is used (a 16-column tile would
// waste half), and 4-row fragments spread any layer over all CUs.
//
// A workgroup (one per CU) owns a run of F fragments of one layer; wave w takes
// the chunks w, w + 8, ... of K for every fragment, in groups of FG fragments
// (one accumulator set).  x goes straight from global memory (L2) into the B
// operand registers, so the main loop has no LDS staging and no barrier; index
// bytes and x are loaded three (group, chunk) steps ahead.  Each wave's sums
// per (row, token) go to LDS; the epilogue adds them in wave order, then the
// sidecar terms delta * x in stored order, then the bias.  Deterministic.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace gm4 {
constexpr int THREADS = 512, WAVES = THREADS / 64;
constexpr int KC = 256;     // k per chunk: 16 blocks x 16
constexpr int FMAX = 24;    // fragments per workgroup
constexpr int MXR = 8;      // token slots of the result
constexpr int TV = 4096;    // sidecar terms (triplets x token slots) per epilogue pass
constexpr int SCAP = TV / MXR;
constexpr int XSW = 2 * 4 * 1024;                        // per wave: x of one chunk, 8 fp32 token rows
constexpr int OFF_XST = 0;                               // [wave] x staging (wave-private)
constexpr int OFF_TV = 0;                                // epilogue sidecar terms (over the staging)
constexpr int OFF_PART = OFF_XST + WAVES * XSW;          // [wave][fragment][token][row] fp32
constexpr int OFF_MISC = OFF_PART + WAVES * FMAX * MXR * 4 * 4;  // lo, hi (int64), row ranges
constexpr int LDS_DYN = OFF_MISC + 16 + 2 * FMAX * 4 * 4;
static_assert(SCAP <= THREADS, "one triplet per thread in a pass");
static_assert(TV * 4 <= WAVES * XSW, "sidecar terms fit the staging area");
}  // namespace gm4

// The 16 blocks' sums of one 4x4x1 result (v = rows 0..3 of the lane's
// column): lane l returns the total over blocks of row l / 16 for column l % 4
// (lanes with l % 16 >= 4 hold copies).  Within each 16-lane row the blocks
// l, l + 4, l + 8, l + 12 are added by rotation; the four row sums of the four
// values are then added by the gfx950 row swaps, two values per swap.
template <int CTRL>
__device__ __forceinline__ float ror_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float reduce_blocks(f32x4 v) {
  float s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = ror_add<0x124>(ror_add<0x128>(v[r]));  // row_ror:8, row_ror:4
  // rows (s0.r0 + s0.r1, s1.r0 + s1.r1, s0.r2 + s0.r3, s1.r2 + s1.r3)
  const auto p01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[0]), __float_as_uint(s[1]), false, false);
  const auto p23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[2]), __float_as_uint(s[3]), false, false);
  const float h01 = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
  const float h23 = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
  // row q: the total of value q
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(h01), __float_as_uint(h23), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// TG: groups of 4 tokens (1 up to 4 tokens, 2 up to 8); FG: fragments per
// accumulator group (1 to 4, no more than a workgroup owns); X1: K <= 2048,
// so a wave has at most one chunk and loads its x once; NT: index bytes
// loaded non-temporally (launches that stream more than the L2s hold)
template <bool PK12, bool XBF, int TG, int FG, bool X1, bool NT>
__global__ __launch_bounds__(gm4::THREADS, 1) void gemv_mfma4(GemvMArgs ga) {
  using namespace gm4;
  // u8: fp32 codebook, 64 copies per entry (copy j at byte e * 256 + 4 j);
  // pk12: the 4096 fp32 pairs
  __shared__ __align__(16) unsigned char cbs[PK12 ? 4096 * 8 : 256 * 256];
  extern __shared__ __align__(16) unsigned char smem[];
  float* part = reinterpret_cast<float*>(smem + OFF_PART);
  unsigned char* xst = smem + OFF_XST;  // this wave's staging: + wave * XSW
  float* tv = reinterpret_cast<float*>(smem + OFF_TV);
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + OFF_MISC);
  int* rsb = reinterpret_cast<int*>(smem + OFF_MISC + 16);  // per row of the block: first, end term
  int* rse = rsb + FMAX * 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lb = lane >> 2, lt = lane & 3;  // block (16-deep k stretch), row / token in the block
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
  const int M = ga.M, N = a.N, K = ga.K;
  const int f0 = split_point(b, a.nfrag, Gl), f1 = split_point(b + 1, a.nfrag, Gl);
  const int F = f1 - f0;
  const int r0 = f0 * 4, r1 = min(f1 * 4, N);
  const int ngrp = (F + FG - 1) / FG;
  const int nch = K / KC;
  const int nchw = nch > wave ? (nch - wave + WAVES - 1) / WAVES : 0;  // this wave's chunks
  const int T = ngrp * nchw;                                           // its (group, chunk) steps
  const int64_t row_bytes = PK12 ? (int64_t)(K / 4) * 3 : (int64_t)K;

  // sidecar: waves 0 and 1 look up the first triplet of rows r0 and r1, their
  // window loads issued before everything else
  const bool srch = a.nnz > 0 && wave < 2 && F > 0;  // uniform
  const int target = wave == 0 ? r0 : r1;
  RowWindow win;
  if (srch) row_window_load(a.sc_rows, a.nnz, sidecar_guess(a.nnz, target, N), win);

  // ---- step t = (group t / nchw, chunk wave + 8 (t % nchw)): index bytes of
  // the group's FG fragments and x of the chunk for the TG token groups.  x is
  // loaded in whole rows (load h of token group u: token 4 u + h fp32, or
  // tokens 4 u + 2 h, + 1 bf16, 16 bytes a lane, so each load is one
  // contiguous piece) and reaches the operand layout through the wave's LDS
  // staging area.
  typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
  constexpr int XW = XBF ? 2 : 4;  // 16-byte loads of x per lane and token group
  // (steps past the end, also for a wave without chunks, load a valid
  // stand-in that is not used: the loads stay unconditional, so the waits
  // before the first barrier cover only what they need)
  const int nw = max(nchw, 1);
  auto load_iq = [&](int t, u32x4 (&iq)[FG]) {
    const int tc = max(min(t, T - 1), 0);
    const int g = tc / nw, q = tc - g * nw;
    const int k0 = min(wave + WAVES * q, nch - 1) * KC + 16 * lb;
#pragma unroll
    for (int f = 0; f < FG; ++f) {
      const int row = min(r0 + 4 * min(g * FG + f, max(F - 1, 0)) + lt, N - 1);
      const uint8_t* p = a.indices + (int64_t)row * row_bytes;
      if (PK12) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(p + k0 / 4 * 3);
        iq[f] = u32x4{v[0], v[1], v[2], 0u};
      } else {
        iq[f] = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + k0))
                   : *reinterpret_cast<const u32x4*>(p + k0);
      }
    }
  };
  auto load_x = [&](int t, u32x4 (&xr)[TG][XW]) {
    const int tc = max(min(t, T - 1), 0);
    const int q = tc % nw;
    const int kc = min(wave + WAVES * q, nch - 1) * KC;
#pragma unroll
    for (int u = 0; u < TG; ++u)
#pragma unroll
      for (int h = 0; h < XW; ++h) {
        // tokens past M repeat row M - 1 (their results are not stored)
        if (XBF) {
          const int tm = min(4 * u + 2 * h + (lane >> 5), M - 1);
          xr[u][h] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(ga.x) + (int64_t)tm * K + kc +
                                                     8 * (lane & 31));
        } else {
          const int tm = min(4 * u + h, M - 1);
          xr[u][h] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(ga.x) + (int64_t)tm * K + kc + 4 * lane);
        }
      }
  };

  // x: with X1 one set for the whole launch, else one per step in flight
  u32x4 IQ[3][FG], XR[X1 ? 1 : 3][TG][XW];
  load_iq(0, IQ[0]);
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
  load_iq(1, IQ[1]);
  if (!X1) load_x(1, XR[X1 ? 0 : 1]);
  load_iq(2, IQ[2]);
  if (!X1) load_x(2, XR[X1 ? 0 : 2]);
  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) reinterpret_cast<u32x4*>(cbs)[tid + i * THREADS] = cbv[i];
  } else {
    const int e = tid & 255, h = tid >> 8;
    const float4 v4 = make_float4(cv, cv, cv, cv);
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<float4*>(cbs + e * 256 + (((8 * h + q + e) & 15) << 4)) = v4;
  }
  // the lookup stays below the prefetch (a compiler barrier keeps it, and its
  // wait, from being hoisted above)
  asm volatile("" ::: "memory");
  if (srch) {
    const int64_t v = row_window_lower_bound(a.sc_rows, a.nnz, target, win);
    if (lane == 0) lohi[wave] = v;
  }
  __syncthreads();

  // the block's triplet range, and the first epilogue pass's triplets,
  // requested now (older than every load the steps wait for)
  int64_t lo = 0, hi = 0;
  if (a.nnz > 0 && F > 0) {
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

  // x through the wave's staging area: token row r of group u at (u * 4 + r)
  // KB (fp32) or (u * 4 + r) / 2 KB (bf16), 16-byte piece p of a row at
  // 16 (p ^ r) (a lane's operand reads then fall in distinct banks); lane
  // (b, j) reads token 4 u + j, k = 16 b .. 16 b + 15 of the chunk
  unsigned char* xw = xst + wave * XSW;
  auto stage_x = [&](const u32x4 (&xr)[TG][XW], float (&xf)[TG][16]) {
#pragma unroll
    for (int u = 0; u < TG; ++u)
#pragma unroll
      for (int h = 0; h < XW; ++h) {
        if (XBF) {
          const int r = 2 * h + (lane >> 5), p = lane & 31;
          *reinterpret_cast<u32x4*>(xw + (4 * u + r) * 512 + 16 * (p ^ r)) = xr[u][h];
        } else {
          *reinterpret_cast<u32x4*>(xw + (4 * u + h) * 1024 + 16 * (lane ^ h)) = xr[u][h];
        }
      }
#pragma unroll
    for (int u = 0; u < TG; ++u)
#pragma unroll
      for (int h = 0; h < XW; ++h) {
        const int p = XW * lb + h;
        const u32x4 v = *reinterpret_cast<const u32x4*>(xw + (4 * u + lt) * (XBF ? 512 : 1024) + 16 * (p ^ lt));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (XBF) {
            xf[u][8 * h + 2 * e] = __uint_as_float(v[e] << 16);
            xf[u][8 * h + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
          } else {
            xf[u][4 * h + e] = __uint_as_float(v[e]);
          }
        }
      }
  };
  float x1[TG][16];
  if (X1) stage_x(XR[0], x1);
  else {
#pragma unroll
    for (int u = 0; u < TG; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) x1[u][e] = 0.f;
  }

  f32x4 acc[FG][TG];
#pragma unroll
  for (int f = 0; f < FG; ++f)
#pragma unroll
    for (int u = 0; u < TG; ++u) acc[f][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one step: products of IQ[R] and XR[R], then (last chunk of a group) the
  // group's sums to LDS, then the loads of step t + 3 into set R
  auto step = [&](auto r_c, int t) {
    constexpr int R = decltype(r_c)::value;
    const int g = t / nchw, q = t - g * nchw;
    float xs[TG][16];
    if (!X1) stage_x(XR[X1 ? 0 : R], xs);
    const float(&xf)[TG][16] = X1 ? x1 : xs;
    // codebook values of pair group d (weights 4 d .. 4 d + 3) of each fragment
    auto gather = [&](int d, float (&w)[FG][4]) {
#pragma unroll
      for (int f = 0; f < FG; ++f) {
        if (PK12) {
          // pair group d: 24 bits at byte 3 d of the lane's 12, pair indices
          // (v & 0xfff, v >> 12) for weights 4 d, 4 d + 1 and 4 d + 2, 4 d + 3
          const u32x4 v4 = IQ[R][f];
          const uint32_t v = d == 0 ? (v4[0] & 0xffffffu)
                           : d == 1 ? (__builtin_amdgcn_alignbit(v4[1], v4[0], 24) & 0xffffffu)
                           : d == 2 ? (__builtin_amdgcn_alignbit(v4[2], v4[1], 16) & 0xffffffu)
                                    : (v4[2] >> 8);
          const float2 p0 = lds_load<float2>((v & 0xfffu) << 3, cbs);
          const float2 p1 = lds_load<float2>((v >> 12) << 3, cbs);
          w[f][0] = p0.x, w[f][1] = p0.y, w[f][2] = p1.x, w[f][3] = p1.y;
        } else {
          const uint32_t wd = IQ[R][f][d];
          w[f][0] = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
          w[f][1] = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
          w[f][2] = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
          w[f][3] = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
        }
      }
    };
    // the gathers of pair group d + 1 go out before the products of group d
    // (scheduling barriers keep that order), so their latency hides behind
    // the matrix ops
    float wb[2][FG][4];
    gather(0, wb[0]);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (d < 3) gather(d + 1, wb[(d + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int f = 0; f < FG; ++f)
#pragma unroll
          for (int u = 0; u < TG; ++u)
            acc[f][u] = __builtin_amdgcn_mfma_f32_4x4x1f32(wb[d & 1][f][e], xf[u][4 * d + e], acc[f][u], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (q == nchw - 1) {  // uniform: the group's last chunk
#pragma unroll
      for (int f = 0; f < FG; ++f) {
        const int fi = g * FG + f;
#pragma unroll
        for (int u = 0; u < TG; ++u) {
          // lane 16 r + t holds row r of fragment fi for token 4 u + t
          const float sv = reduce_blocks(acc[f][u]);
          if (fi < F && (lane & 12) == 0) part[((wave * FMAX + fi) * MXR + 4 * u + (lane & 3)) * 4 + (lane >> 4)] = sv;
          acc[f][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    load_iq(t + 3, IQ[R]);
    if (!X1) load_x(t + 3, XR[X1 ? 0 : R]);
  };
  int t = 0;
  for (; t + 2 < T; t += 3) {
    step(std::integral_constant<int, 0>{}, t);
    step(std::integral_constant<int, 1>{}, t + 1);
    step(std::integral_constant<int, 2>{}, t + 2);
  }
  if (t < T) step(std::integral_constant<int, 0>{}, t);
  if (t + 1 < T) step(std::integral_constant<int, 1>{}, t + 1);
  // x at the first epilogue pass's sidecar columns, requested before the
  // partial sums are added (its triplets arrived long ago)
  float xv[MXR];
  if (lo < hi && tid < SCAP) {
#pragma unroll
    for (int u = 0; u < MXR; ++u) {
      const int tm = min(u, M - 1);
      xv[u] = XBF ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(ga.x)[(int64_t)tm * K + tc] << 16)
                  : static_cast<const float*>(ga.x)[(int64_t)tm * K + tc];
    }
  }
  __syncthreads();

  // ---- epilogue: thread o -> token o / (4 FMAX), block row o % (4 FMAX)
  const int nrow = r1 - r0;
  const int wlim = min(WAVES, nch);  // waves that computed
  constexpr int OPT = (FMAX * 4 * MXR + THREADS - 1) / THREADS;
  float out[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + THREADS * i, tk = o / (4 * FMAX), j = o % (4 * FMAX);
    float v = 0.f;
    if (tk < MXR && j < nrow) {
      for (int w = 0; w < wlim; ++w) v += part[((w * FMAX + (j >> 2)) * MXR + tk) * 4 + (j & 3)];
    }
    out[i] = v;
  }
  // sidecar terms delta * x[t][c], each output's in stored order, SCAP triplets a pass
  for (int64_t e0 = lo; e0 < hi; e0 += SCAP) {
    const int cnt = (int)min<int64_t>(SCAP, hi - e0);
    __syncthreads();
    for (int i = tid; i < 4 * FMAX; i += THREADS) rsb[i] = rse[i] = 0;
    __syncthreads();
    if (tid < SCAP) {
      if (e0 != lo) {
        const int64_t ee = e0 + min(tid, cnt - 1);
        tc = a.sc_cols[ee];
        tdl = a.sc_deltas[ee];
        tr = a.sc_rows[ee];
        trp = a.sc_rows[ee > 0 ? ee - 1 : 0];
        trn = a.sc_rows[ee + 1 < a.nnz ? ee + 1 : ee];
      }
      if (e0 != lo) {
#pragma unroll
        for (int u = 0; u < MXR; ++u) {
          const int tm = min(u, M - 1);
          xv[u] = XBF ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(ga.x)[(int64_t)tm * K + tc] << 16)
                      : static_cast<const float*>(ga.x)[(int64_t)tm * K + tc];
        }
      }
      if (tid < cnt) {
#pragma unroll
        for (int u = 0; u < MXR; ++u) tv[tid * MXR + u] = tdl * xv[u];
        if (tid == 0 || trp != tr) rsb[tr - r0] = tid;
        if (tid == cnt - 1 || trn != tr) rse[tr - r0] = tid + 1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int o = tid + THREADS * i, tk = o / (4 * FMAX), j = o % (4 * FMAX);
      if (tk < MXR && j < nrow)
        for (int e = rsb[j]; e < rse[j]; ++e) out[i] += tv[e * MXR + tk];
    }
  }
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + THREADS * i, tk = o / (4 * FMAX), j = o % (4 * FMAX);
    if (tk < M && tk < MXR && j < nrow) {
      const int n = r0 + j;
      a.y[(int64_t)tk * N + n] = out[i] + (a.bias ? a.bias[n] : 0.f);
    }
  }
}

bool gemv_mfma4_ok(const LayerArgs& a, bool pk12) {
  if (a.M < 1 || a.M > gm4::MXR || a.K < gm4::KC || a.K % gm4::KC != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.indices) % (pk12 ? 4 : 16) != 0) return false;
  if (pk12 && reinterpret_cast<uintptr_t>(a.codebook) % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.x) % 16 != 0) return false;
  return true;
}

// Workgroups per layer in proportion to its 4-row fragments (each layer at
// least ceil(fragments / FMAX)), one per CU at most; false when that does not
// fit.
static bool gemv_mfma4_plan(GemvMArgs& g, int& grid, int& fmax) {
  using namespace gm4;
  const int cus = device_cu_count();
  int64_t frags = 0;
  for (int i = 0; i < g.nseg; ++i) frags += g.seg[i].nfrag;
  const int64_t want = frags < cus ? frags : cus;
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
  if (tot > cus) return false;
  grid = 0;
  fmax = 1;
  for (int i = 0; i < g.nseg; ++i) {
    g.wg0[i] = grid;
    grid += alloc[i];
    const int f = (int)((g.seg[i].nfrag + alloc[i] - 1) / alloc[i]);  // most fragments of a workgroup
    if (f > fmax) fmax = f;
  }
  for (int i = g.nseg; i < kMaxSegments; ++i) {
    g.wg0[i] = INT_MAX;
    g.seg[i] = g.seg[0];
  }
  return true;
}

static bool gemv_mfma4_args(const GemvSeg* segs, int nseg, GemvMArgs& g) {
  if (nseg < 1 || nseg > kMaxSegments) return false;
  g.nseg = nseg;
  for (int i = 0; i < nseg; ++i) {
    g.seg[i] = segs[i];
    g.seg[i].nfrag = (segs[i].N + 3) / 4;
  }
  return true;
}

bool gemv_mfma4_group_fits(const GemvSeg* segs, int nseg) {
  GemvMArgs g;
  int grid = 0, fmax = 1;
  return gemv_mfma4_args(segs, nseg, g) && gemv_mfma4_plan(g, grid, fmax);
}

template <bool PK12, bool XBF, int TG, int FG, bool X1, bool NT>
static hipError_t launch_gemv_mfma4_x(const GemvMArgs& g, int grid, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemv_mfma4<PK12, XBF, TG, FG, X1, NT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, gm4::LDS_DYN);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemv_mfma4<PK12, XBF, TG, FG, X1, NT>), dim3((unsigned)grid), dim3(gm4::THREADS),
                     gm4::LDS_DYN, stream, g);
  return hipGetLastError();
}

// Non-temporal index loads for launches that stream more than the L2s hold
// (Qwen decode step at 8 tokens 62.5 -> 59.5 us, at 4 tokens 50.1 -> 47.9 us).
template <bool PK12, bool XBF, int TG, int FG>
static hipError_t launch_gemv_mfma4_k(const GemvMArgs& g, int grid, hipStream_t stream) {
  const bool x1 = g.K <= gm4::KC * gm4::WAVES;
  int64_t ib = 0;
  for (int i = 0; i < g.nseg; ++i) ib += index_bytes(g.seg[i].N, g.K, PK12);
  if (ib > kStreamPastCacheBytes)
    return x1 ? launch_gemv_mfma4_x<PK12, XBF, TG, FG, true, true>(g, grid, stream)
              : launch_gemv_mfma4_x<PK12, XBF, TG, FG, false, true>(g, grid, stream);
  return x1 ? launch_gemv_mfma4_x<PK12, XBF, TG, FG, true, false>(g, grid, stream)
            : launch_gemv_mfma4_x<PK12, XBF, TG, FG, false, false>(g, grid, stream);
}

template <bool PK12, bool XBF, int TG>
static hipError_t launch_gemv_mfma4_f(const GemvMArgs& g, int fmax, int grid, hipStream_t stream) {
  // the group size that pads the busiest workgroup's fragments least (the
  // larger on ties)
  int fg = 4;
  for (int c = 3; c >= 1; --c)
    if ((fmax + c - 1) / c * c < (fmax + fg - 1) / fg * fg) fg = c;
  if (fg == 1) return launch_gemv_mfma4_k<PK12, XBF, TG, 1>(g, grid, stream);
  if (fg == 2) return launch_gemv_mfma4_k<PK12, XBF, TG, 2>(g, grid, stream);
  if (fg == 3) return launch_gemv_mfma4_k<PK12, XBF, TG, 3>(g, grid, stream);
  return launch_gemv_mfma4_k<PK12, XBF, TG, 4>(g, grid, stream);
}

template <bool PK12>
static hipError_t launch_gemv_mfma4_p(const GemvMArgs& g, bool xbf, int fmax, int grid, hipStream_t stream) {
  if (xbf)
    return g.M <= 4 ? launch_gemv_mfma4_f<PK12, true, 1>(g, fmax, grid, stream)
                    : launch_gemv_mfma4_f<PK12, true, 2>(g, fmax, grid, stream);
  return g.M <= 4 ? launch_gemv_mfma4_f<PK12, false, 1>(g, fmax, grid, stream)
                  : launch_gemv_mfma4_f<PK12, false, 2>(g, fmax, grid, stream);
}

hipError_t launch_gemv_mfma4_grouped(const GemvSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M,
                                     int K, hipStream_t stream) {
  GemvMArgs g;
  if (!gemv_mfma4_args(segs, nseg, g)) return hipErrorInvalidValue;
  g.x = x;
  g.M = M;
  g.K = K;
  int grid = 0, fmax = 1;
  if (!gemv_mfma4_plan(g, grid, fmax)) return hipErrorInvalidValue;
  return pk12 ? launch_gemv_mfma4_p<true>(g, xbf, fmax, grid, stream)
              : launch_gemv_mfma4_p<false>(g, xbf, fmax, grid, stream);
}

}  // namespace hxq
