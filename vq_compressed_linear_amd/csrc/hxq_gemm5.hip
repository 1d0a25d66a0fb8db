// bf16 matrix-core HelixLinear GEMM with 256-token x 256-output tiles
// (prefill shapes), u8 and pk12 formats.
//
// y[m][n] = sum_k x[m][k] * Wq[n][k] + b[n], with Wq[n][k] the bf16 rounding
// (nearest, ties to even) of the fp32 value C[idx[n][k]] + S[n][k] (the
// codebook entry plus every sidecar delta at (n, k), added in fp32 in stored
// order).  The model cards ("What is HelixCode?") describe the layer as
// codebook[indices] @ x with no decompression step; the HXQ whitepaper's
// inference paragraph adds the sidecar to the gathered weights before the
// matmul, which is what the operand rounding does here.  The dense weight
// only ever exists as a 32-deep k-stage of the tile's rows in LDS.
//
// Four waves, one per SIMD, each owning 128 tokens x 128 outputs (2 x 2 over
// the tile; 16 accumulator tiles of 32 x 32, v_mfma_f32_32x32x16_bf16, in
// the accumulation registers).  Per 32-deep stage a CU reads the operands
// from LDS once per wave (64 KB), gathers 8192 codebook entries (each weight
// once, shared by the tile's 256 tokens) and stores 16 KB of weight tile and
// 16 KB of x.  Measured with probes on the target: a matrix op takes 33
// clocks, and the gathers, not the operand bytes, are the LDS cost that
// competes with the matrix ops; the u8 codebook therefore sits in LDS as 64
// copies, lane l reading copy l (one bank per lane: 5-8% faster than 32
// copies, where lanes l and l + 32 share a bank).  With one wave per SIMD
// every stall of the wave also stalls its matrix core, so the stage is
// ordered by hand.
//
// Pipeline of stage s (one barrier per stage; the operands of s were read
// during stage s - 1):
//   - the 32 matrix ops of stage s;
//   - between them: reads of stage s + 1's operands into the second register
//     set, gathers and packing of W(s + 2) (from index bytes requested two
//     stages ago) into the weight buffer W(s) used (its reads ended with
//     stage s - 1), its sidecar patches, the store of x(s + 2) (registers
//     requested two stages ago) into x(s)'s slot likewise, and the requests
//     for x and index bytes of stage s + 4.  Two weight buffers and two x
//     slots suffice.
// All global loads are ordinary loads the compiler waits for.
//
// Sidecar triplets become patches before the main loop (for each distinct
// (row, col) of the tile the bf16 of C[idx] + deltas and its byte position in
// the stage's weight tile), binned by (stage, wave building the row).  A tile
// with more triplets than the patch area, or K > 12288, builds plain codebook
// weights and adds x * (bf16(C[idx] + deltas) - bf16(C[idx])) per distinct
// (row, col) in fp32 in its epilogue: the same products, summed in another
// order.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace gemm5 {
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int THREADS = 256, WAVES = 4;
constexpr int XR = 2;          // x stages in LDS
constexpr int WR = 2;          // weight-tile stages in LDS
constexpr int MAXST = 384;     // stages on the patch path: K <= 12288
constexpr int CAP = 4096;      // patches per tile
constexpr int XS = BM * BK * 2;  // bytes of one x stage (16 blocks of 16 tokens)
constexpr int WT = BN * BK * 2;  // bytes of one weight stage (8 row blocks x 2 sub-steps)
template <bool PK12>
struct Lay {
  static constexpr int CB = PK12 ? 4096 * 4 : 256 * 256;
  static constexpr int MAXBINS = MAXST * WAVES;
  static constexpr int OFF_CBF = 0;
  static constexpr int OFF_W = OFF_CBF + (PK12 ? 0 : 1024);
  static constexpr int OFF_X = OFF_W + WR * WT;
  static constexpr int OFF_BINS = OFF_X + XR * XS;
  static constexpr int OFF_PATCH = OFF_BINS + ((MAXBINS + 8) * 2 + 15) / 16 * 16;
  static constexpr int OFF_MISC = OFF_PATCH + CAP * 4;
  static constexpr int LDS = OFF_MISC + 16 + 4 * WAVES;
  static_assert(CAP <= WR * WT, "head flags overlay the weight tiles");
  static_assert(4096 + (MAXBINS + 4) * 4 <= WR * WT, "bin counters overlay the weight tiles after the head flags");
  static_assert(MAXBINS % THREADS == 0, "bin prefix split");
  static_assert(CB + LDS <= 160 * 1024, "LDS");
};
struct Ops {
  bf16x8 a[2][4];  // weights: sub-step, row block
  bf16x8 b[2][4];  // x: sub-step, token group
};
}  // namespace gemm5

template <bool PK12>
__global__ __launch_bounds__(256, 1) void gemm5_bf16(GemmArgs ga) {
  using namespace gemm5;
  using Ly = Lay<PK12>;
  constexpr int UB = PK12 ? 12 : 16;  // index bytes of a 16-weight unit
  constexpr int IS = PK12 ? 24 : 32;  // index bytes per row and stage
  typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
  __shared__ __align__(16) unsigned char cbs[Ly::CB];
  extern __shared__ __align__(16) unsigned char smem[];
  float* cbf = reinterpret_cast<float*>(smem + Ly::OFF_CBF);
  uint16_t* bins = reinterpret_cast<uint16_t*>(smem + Ly::OFF_BINS);
  uint32_t* patch = reinterpret_cast<uint32_t*>(smem + Ly::OFF_PATCH);
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + Ly::OFF_MISC);
  int* wsum = reinterpret_cast<int*>(smem + Ly::OFF_MISC + 16);
  unsigned char* wbuf = smem + Ly::OFF_W;
  unsigned char* xbuf = smem + Ly::OFF_X;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;

  const int G = gridDim.x, bx = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int L = (bx < full) ? (bx % 8) * per + bx / 8 : bx;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < ga.nseg && L >= ga.seg[i].tile0) si = i;
  const GemmSeg& sg = ga.seg[si];
  const int M = ga.M, N = sg.N, K = ga.K;
  int tl = L - sg.tile0;
  // a split launch (one layer): run `split` of the tile's k stages
  int split = 0;
  if (ga.S > 1) {
    const int tiles = ga.tiles_m * ((N + BN - 1) / BN);
    split = tl / tiles;
    tl -= split * tiles;
  }
  const int m0 = (tl % ga.tiles_m) * BM, n0 = (tl / ga.tiles_m) * BN;
  const int kb = split * ga.sst;                // the run's first stage
  const int nk = min(K / BK - kb, ga.sst);      // and its stages
  const int64_t row_bytes = PK12 ? (int64_t)(K / 4) * 3 : (int64_t)K;

  // x piece j of this wave: block 4 wave + j (16 tokens), lane i: token
  // m0 + 16 (4 wave + j) + i % 16, k = 32 stage + 8 (i / 16) + [0, 8), kept at
  // byte 16 i of the block
  const unsigned char* xb = static_cast<const unsigned char*>(ga.x);
  const unsigned char* xsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    xsrc[j] = xb + (int64_t)min(m0 + 16 * (4 * wave + j) + (lane & 15), M - 1) * (K * 2) + 16 * (lane >> 4) +
              kb * (BK * 2);
  auto load_x = [&](int st, u32x4 (&v)[4]) {
    const int sc = min(st, nk - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const u32x4*>(xsrc[j] + sc * (BK * 2));
  };
  auto store_x = [&](int st, const u32x4 (&v)[4]) {
    unsigned char* d = xbuf + (st % XR) * XS + (4 * wave) * 1024 + 16 * lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(d + 1024 * j) = v[j];
  };
  // index bytes: this wave builds rows 64 wave + 32 rb + l32 (rb = 0, 1), k-half h
  const uint8_t* isrc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
    isrc[rb] = sg.indices + (int64_t)min(n0 + 64 * wave + 32 * rb + l32, N - 1) * row_bytes + UB * h + kb * IS;
  auto load_i = [&](int st, u32x4 (&q)[2]) {
    const int sc = min(st, nk - 1);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (PK12) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(isrc[rb] + sc * IS);
        q[rb] = u32x4{v[0], v[1], v[2], 0u};
      } else {
        q[rb] = *reinterpret_cast<const u32x4*>(isrc[rb] + sc * IS);
      }
    }
  };
  // first requests: the sidecar search (a chain of dependent loads heads the
  // set-up), then x and index bytes of stages 0 and 1; stages 2 and 3 after
  // the set-up, so the chain does not queue behind them
  if (sg.nnz > 0 && wave < 2) {
    const int target = wave == 0 ? n0 : min(n0 + BN, N);
    const int64_t guess = (int64_t)((double)sg.nnz * (double)target / (double)N);
    const int64_t v = wave_lower_bound_rows_near(sg.sc_rows, sg.nnz, target, guess);
    if (lane == 0) lohi[wave] = v;
  }
  u32x4 xp0[4], xp1[4], xs0[4], xs1[4], ip0[2], ip1[2], iq0[2], iq1[2];
  load_i(0, ip0);
  load_x(0, xp0);
  load_i(1, ip1);
  load_x(1, xp1);

  // ---- codebook.  u8: 64 copies per entry (entry e, copy c at byte 256 e + 4 c),
  // lane l reads copy l; pk12:
  // each component rounded to nearest even on its own
  if (PK12) {
#pragma unroll
    for (int i = 0; i < 4096 / THREADS; ++i) {
      const int e = tid + THREADS * i;
      const float2 c = reinterpret_cast<const float2*>(sg.codebook)[e];
      reinterpret_cast<uint32_t*>(cbs)[e] = f32_to_bf16_rne(c.x) | (f32_to_bf16_rne(c.y) << 16);
    }
  } else {
    const int e = tid;
    const float cv = sg.codebook[e];
    const float vb = __uint_as_float(f32_to_bf16_rne(cv) << 16);
    const float4 v4 = make_float4(vb, vb, vb, vb);
#pragma unroll
    for (int q = 0; q < 16; ++q) *reinterpret_cast<float4*>(cbs + e * 256 + (((q + e) & 15) << 4)) = v4;
    cbf[e] = cv;
  }

  // ---- sidecar: the tile's triplet range [lo, hi)
  const bool long_k = nk > MAXST;
  const int nbins = nk * WAVES;
  int* cnt32 = reinterpret_cast<int*>(wbuf + 4096);  // after the head flags; the weight buffers are first written after the set-up
  if (!long_k)
    for (int i = tid; i <= nbins; i += THREADS) cnt32[i] = 0;
  __syncthreads();
  int64_t lo = 0, hi = 0;
  if (sg.nnz > 0) {
    lo = lohi[0];
    hi = lohi[1];
  }
  const int64_t cnt = hi - lo;
  const bool walk = long_k || cnt > CAP;  // uniform

  if (!walk && cnt > 0) {
    // patches: bf16 of C[idx] + deltas per distinct (row, col) and its byte
    // position in the stage's weight tile, binned by (stage, wave building the row)
    constexpr int QMAX = CAP / THREADS;
    unsigned char* hflag = wbuf;  // the weight buffers are first written after the set-up
    int tr[QMAX], tc[QMAX];
    bool head[QMAX], inr[QMAX];  // inr: in this run's stages
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int64_t e = lo + tid + (int64_t)THREADS * q;
      const int64_t ec = e < hi ? e : lo;
      const int64_t ep = ec > lo ? ec - 1 : lo;
      tr[q] = sg.sc_rows[ec];
      tc[q] = sg.sc_cols[ec];
      const int pr = sg.sc_rows[ep], pc = sg.sc_cols[ep];
      head[q] = e < hi && (e == lo || pr != tr[q] || pc != tc[q]);
      inr[q] = (unsigned)(tc[q] / BK - kb) < (unsigned)nk;
      if (e < hi) hflag[e - lo] = head[q] ? 1 : 0;
      if (head[q] && inr[q]) atomicAdd(&cnt32[1 + (tc[q] / BK - kb) * WAVES + ((tr[q] - n0) >> 6)], 1);
    }
    __syncthreads();
    {
      constexpr int PT = Ly::MAXBINS / THREADS;
      int c4[PT];
      int tot = 0;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int b = PT * tid + i;
        c4[i] = b < nbins ? cnt32[1 + b] : 0;
        tot += c4[i];
      }
      int inc = tot;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d);
        if (lane >= d) inc += o;
      }
      if (lane == 63) wsum[wave] = inc;
      __syncthreads();
      int base = inc - tot;
      for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int b = PT * tid + i;
        if (b < nbins) {
          cnt32[1 + b] = base;
          bins[b] = (uint16_t)base;
        }
        base += c4[i];
      }
      if (tid == THREADS - 1) bins[nbins] = (uint16_t)base;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      if (!head[q] || !inr[q]) continue;
      const int64_t e = lo + tid + (int64_t)THREADS * q;
      float v = sg.sc_deltas[e];
      if (PK12) {
        const uint8_t* pb = sg.indices + (int64_t)tr[q] * row_bytes + (tc[q] >> 2) * 3;
        const uint32_t g24 = (uint32_t)pb[0] | ((uint32_t)pb[1] << 8) | ((uint32_t)pb[2] << 16);
        const uint32_t pi = ((tc[q] >> 1) & 1) ? (g24 >> 12) : (g24 & 0xfffu);
        v = sg.codebook[2 * pi + (tc[q] & 1)] + v;
      } else {
        v = cbf[sg.indices[(int64_t)tr[q] * K + tc[q]]] + v;
      }
      for (int64_t e2 = e + 1; e2 < hi && !hflag[e2 - lo]; ++e2) v += sg.sc_deltas[e2];
      // byte position of (row nl, column kl) in a stage's tile: block
      // (nl / 32, sub-step kl / 16), lane half (kl / 8) % 2, element kl % 8
      const int nl = tr[q] - n0, kl = tc[q] % BK;
      const uint32_t pos = (uint32_t)(((nl >> 5) * 2 + (kl >> 4)) * 1024 + ((((kl >> 3) & 1) * 32 + (nl & 31)) * 16) +
                                      (kl & 7) * 2);
      patch[atomicAdd(&cnt32[1 + (tc[q] / BK - kb) * WAVES + (nl >> 6)], 1)] = pos | (f32_to_bf16_rne(v) << 16);
    }
  } else if (!walk) {
    for (int i = tid; i <= nbins; i += THREADS) bins[i] = 0;
  }
  int* rsb = reinterpret_cast<int*>(patch);
  int* rse = rsb + BN;
  if (walk) {
    for (int i = tid; i < BN; i += THREADS) rsb[i] = rse[i] = 0;
    __syncthreads();
    for (int64_t e = lo + tid; e < hi; e += THREADS) {
      const int r = sg.sc_rows[e];
      if (e == lo || sg.sc_rows[e - 1] != r) rsb[r - n0] = (int)(e - lo);
      if (e == hi - 1 || sg.sc_rows[e + 1] != r) rse[r - n0] = (int)(e - lo + 1);
    }
  }
  __syncthreads();

  // ---- building: lane (h, l32) turns the 16 (12) index bytes of row
  // 32 RB + l32, k = 16 h + [0, 16) (RB = 2 wave + rb) into 8 operand words:
  // block (RB, sub-step h) at bytes 16 l32 (k + [0, 8)) and 512 + 16 l32
  const uint32_t lane4 = (uint32_t)lane << 2;
  auto wofs = [&](int rb) { return (2 * (2 * wave + rb) + h) * 1024 + l32 * 16; };
  auto build = [&](const u32x4 iq, unsigned char* wt, int rb) {
    uint32_t w[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (PK12) {
        const uint32_t v = d == 0 ? (iq[0] & 0xffffffu)
                         : d == 1 ? (__builtin_amdgcn_alignbit(iq[1], iq[0], 24) & 0xffffffu)
                         : d == 2 ? (__builtin_amdgcn_alignbit(iq[2], iq[1], 16) & 0xffffffu)
                                  : (iq[2] >> 8);
        w[2 * d] = lds_load<uint32_t>((v & 0xfffu) << 2, cbs);
        w[2 * d + 1] = lds_load<uint32_t>((v >> 12) << 2, cbs);
      } else {
        const uint32_t wd = iq[d];
        const uint32_t f0 = lds_load<uint32_t>(byte_addr256<0>(wd, lane4), cbs);
        const uint32_t f1 = lds_load<uint32_t>(byte_addr256<1>(wd, lane4), cbs);
        const uint32_t f2 = lds_load<uint32_t>(byte_addr256<2>(wd, lane4), cbs);
        const uint32_t f3 = lds_load<uint32_t>(byte_addr256<3>(wd, lane4), cbs);
        w[2 * d] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        w[2 * d + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
      }
    }
    const int o = wofs(rb);
    *reinterpret_cast<u32x4*>(wt + o) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(wt + o + 512) = u32x4{w[4], w[5], w[6], w[7]};
  };
  auto patch_stage = [&](int st, unsigned char* wt) {
    const int b = st * WAVES + wave;
    const int q0 = bins[b], q1 = bins[b + 1];
    for (int q = q0 + lane; q < q1; q += 64) {
      const uint32_t p = patch[q];
      *reinterpret_cast<uint16_t*>(wt + (p & 0xffffu)) = (uint16_t)(p >> 16);
    }
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[g][f][r] = 0.f;

  // operand reads: weights of row block 4 wn + f, sub-step s at
  // (2 (4 wn + f) + s) KB + 16 lane; x of tokens 128 wm + 32 g + l32, sub-step
  // s: block 8 wm + 2 g + l32 / 16, byte 16 ((2 s + h) 16 + l32 % 16)
  const int aoff = (8 * wn) * 1024 + lane * 16;
  const int boff = (8 * wm + (l32 >> 4)) * 1024 + (h * 16 + (l32 & 15)) * 16;
  auto read_ops = [&](int st, Ops& o) {
    const unsigned char* wt = wbuf + (st % WR) * WT;
    const unsigned char* xt = xbuf + (st % XR) * XS;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int f = 0; f < 4; ++f) o.a[sub][f] = *reinterpret_cast<const bf16x8*>(wt + aoff + (2 * f + sub) * 1024);
#pragma unroll
      for (int g = 0; g < 4; ++g) o.b[sub][g] = *reinterpret_cast<const bf16x8*>(xt + boff + g * 2048 + sub * 512);
    }
  };

  load_i(2, iq0);
  load_x(2, xs0);
  load_i(3, iq1);
  load_x(3, xs1);
  // W(0), W(1), x(0), x(1) into LDS.  Tiles on the walk path (more
  // triplets than patches, or K past the bins) build plain codebook weights
  // here and add their sidecar terms in the epilogue.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    build(ip0[rb], wbuf, rb);
    build(ip1[rb], wbuf + WT, rb);
  }
  if (!walk) {
    patch_stage(0, wbuf);
    if (nk > 1) patch_stage(1, wbuf + WT);
  }
  store_x(0, xp0);
  store_x(1, xp1);
  __syncthreads();
  {
    Ops oa, ob;
    read_ops(0, oa);
    // stage s: read the operands of s + 1 and multiply those of s; build
    // W(s + 2) and store x(s + 2) (both requested two stages ago); request
    // x and index bytes of s + 4
    // one wave per SIMD, so the stage is ordered by hand (each unit fenced
    // off from the scheduler), with the LDS work spread evenly over its 32
    // matrix ops: sub-step 0's ops each followed by two codebook gathers for
    // W(s + 2), every other one by a weight-operand read for stage s + 1;
    // sub-step 1's ops by the x-operand reads for s + 1, the store of x(s + 2)
    // and, once the gathers have long arrived, the packing and stores of
    // W(s + 2) and its sidecar patches (bins read a stage ahead, entries
    // early in the stage).  x and index bytes of s + 4 are requested once
    // their registers are free.
    auto stage = [&](int s, Ops& cur, Ops& nxt, u32x4 (&xr)[4], u32x4 (&ir)[2], int& pb0, int& pb1) {
      unsigned char* wt2 = wbuf + ((s + 2) % WR) * WT;
      const unsigned char* wn1 = wbuf + ((s + 1) % WR) * WT;
      const unsigned char* xn1 = xbuf + ((s + 1) % XR) * XS;
      uint32_t gw[2][16];
      auto mm = [&](int sub, int i) {
        const int f = i >> 2, g = i & 3;
        acc[g][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[sub][f], cur.b[sub][g], acc[g][f], 0, 0, 0);
      };
      // gathers of unit (rb, d): u8 four words of k 4 d + [0, 4), pk12 two pair words
      auto gather = [&](int rb, int d, int half) {
        const u32x4 iq = ir[rb];
        if (PK12) {
          const uint32_t v = d == 0 ? (iq[0] & 0xffffffu)
                           : d == 1 ? (__builtin_amdgcn_alignbit(iq[1], iq[0], 24) & 0xffffffu)
                           : d == 2 ? (__builtin_amdgcn_alignbit(iq[2], iq[1], 16) & 0xffffffu)
                                    : (iq[2] >> 8);
          if (half == 0) gw[rb][2 * d] = lds_load<uint32_t>((v & 0xfffu) << 2, cbs);
          else gw[rb][2 * d + 1] = lds_load<uint32_t>((v >> 12) << 2, cbs);
        } else {
          const uint32_t wd = iq[d];
          if (half == 0) {
            gw[rb][4 * d] = lds_load<uint32_t>(byte_addr256<0>(wd, lane4), cbs);
            gw[rb][4 * d + 1] = lds_load<uint32_t>(byte_addr256<1>(wd, lane4), cbs);
          } else {
            gw[rb][4 * d + 2] = lds_load<uint32_t>(byte_addr256<2>(wd, lane4), cbs);
            gw[rb][4 * d + 3] = lds_load<uint32_t>(byte_addr256<3>(wd, lane4), cbs);
          }
        }
      };
      auto opread = [&](int j) {  // j = 0..15: 8 weight reads then 8 x reads
        const int sub = (j >> 2) & 1, q = j & 3;
        if (j < 8) nxt.a[sub][q] = *reinterpret_cast<const bf16x8*>(wn1 + aoff + (2 * q + sub) * 1024);
        else nxt.b[sub][q] = *reinterpret_cast<const bf16x8*>(xn1 + boff + q * 2048 + sub * 512);
      };
      auto pack_store = [&](int rb, int hw) {  // words 4 hw + [0, 4) of row block rb
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * hw + e;
          if (PK12) w[e] = gw[rb][k];
          else w[e] = __builtin_amdgcn_perm(gw[rb][2 * k + 1], gw[rb][2 * k], 0x07060302u);
        }
        *reinterpret_cast<u32x4*>(wt2 + wofs(rb) + 512 * hw) = u32x4{w[0], w[1], w[2], w[3]};
      };
      unsigned char* xd = xbuf + ((s + 2) % XR) * XS + (4 * wave) * 1024 + 16 * lane;
      // this stage's patch range (bins of W(s + 2), read during stage s - 1)
      const bool pt = !walk && s + 2 < nk;  // uniform
      const int q0 = __builtin_amdgcn_readfirstlane(pb0), q1 = __builtin_amdgcn_readfirstlane(pb1);
      uint32_t pe = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mm(0, i);
        gather(i >> 3, (i >> 1) & 3, i & 1);
        if (i & 1) opread(i >> 1);
        if (i == 2 && pt && q0 + lane < q1) pe = patch[q0 + lane];
        if (i == 4 && !walk) {  // bins of W(s + 3), used next stage (past the end: unused)
          const int b = min(s + 3, nk) * WAVES + wave;
          pb0 = bins[b];
          pb1 = bins[min(b + 1, nbins)];
        }
        if (i == 15) load_i(s + 4, ir);  // after the last gather that reads ir
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mm(1, i);
        if (!(i & 1)) opread(8 + (i >> 1));
        if (i == 1 || i == 3 || i == 5 || i == 7) *reinterpret_cast<u32x4*>(xd + 1024 * (i >> 1)) = xr[i >> 1];
        if (i == 8) load_x(s + 4, xr);
        if (i & 1 && i >= 9) pack_store((i - 9) >> 2, ((i - 9) >> 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (pt && q0 + lane < q1) *reinterpret_cast<uint16_t*>(wt2 + (pe & 0xffffu)) = (uint16_t)(pe >> 16);
      if (pt && q1 - q0 > 64) {
        for (int q = q0 + 64 + lane; q < q1; q += 64) {
          const uint32_t p = patch[q];
          *reinterpret_cast<uint16_t*>(wt2 + (p & 0xffffu)) = (uint16_t)(p >> 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // patch bins of W(2), for stage 0
    int pb0 = 0, pb1 = 0;
    if (!walk) {
      const int b = min(2, nk) * WAVES + wave;
      pb0 = bins[b];
      pb1 = bins[min(b + 1, nbins)];
    }
    int s = 0;
    for (; s + 1 < nk; s += 2) {
      stage(s, oa, ob, xs0, iq0, pb0, pb1);
      stage(s + 1, ob, oa, xs1, iq1, pb0, pb1);
    }
    if (s < nk) stage(s, oa, ob, xs0, iq0, pb0, pb1);
  }

  // ---- epilogue: per token group, each wave turns its 32 tokens x 128
  // outputs into rows in a 16 KB LDS region of its own and stores 512-byte
  // row pieces (chunk c of row t at 16 ((c ^ t) % 32))
  {
    constexpr int RS = 32 * 128 * 4;
    constexpr int CBW = Ly::CB / RS;
    static_assert(Ly::LDS >= (WAVES - CBW) * RS, "epilogue regions fit");
    unsigned char* reg = wave < CBW ? cbs + wave * RS : smem + (wave - CBW) * RS;
    const bool vec_ok = (N & 3) == 0;
    float bv[4][4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 32 * (4 * wn + f) + 8 * q + 4 * h + r;
          bv[f][q][r] = (sg.bias && n < N && split == 0) ? sg.bias[n] : 0.f;  // once per output
        }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 8 * f + 2 * q + h;
          *reinterpret_cast<float4*>(reg + l32 * 512 + ((c ^ l32) & 31) * 16) =
              make_float4(acc[g][f][4 * q] + bv[f][q][0], acc[g][f][4 * q + 1] + bv[f][q][1],
                          acc[g][f][4 * q + 2] + bv[f][q][2], acc[g][f][4 * q + 3] + bv[f][q][3]);
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int n = n0 + 128 * wn + 4 * l32;  // this lane's 4 outputs of each row
      float4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 2 * i + h;
        v[i] = *reinterpret_cast<const float4*>(reg + t * 512 + ((l32 ^ t) & 31) * 16);
      }
      if (walk && split == 0) {
        // the sidecar of the lane's outputs (all of k, in the first run): for each distinct (row, col),
        // x times (bf16(C[idx] + deltas) - bf16(C[idx])), both bf16 values exact in fp32
        const uint16_t* xh = static_cast<const uint16_t*>(ga.x);
        const int mb = m0 + 128 * wm + 32 * g + h;
        for (int j = 0; j < 4; ++j) {
          const int nn = n + j;
          if (nn >= N) break;
          const int64_t e1 = lo + rse[nn - n0];
          for (int64_t e = lo + rsb[nn - n0]; e < e1; ++e) {
            const int c = sg.sc_cols[e];
            float cv;
            if (PK12) {
              const uint8_t* pb = sg.indices + (int64_t)nn * row_bytes + (c >> 2) * 3;
              const uint32_t g24 = (uint32_t)pb[0] | ((uint32_t)pb[1] << 8) | ((uint32_t)pb[2] << 16);
              const uint32_t pi = ((c >> 1) & 1) ? (g24 >> 12) : (g24 & 0xfffu);
              cv = sg.codebook[2 * pi + (c & 1)];
            } else {
              cv = sg.codebook[sg.indices[(int64_t)nn * K + c]];
            }
            float w = cv + sg.sc_deltas[e];
            while (e + 1 < e1 && sg.sc_cols[e + 1] == c) {
              ++e;
              w += sg.sc_deltas[e];
            }
            const float d = __uint_as_float(f32_to_bf16_rne(w) << 16) - __uint_as_float(f32_to_bf16_rne(cv) << 16);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int m = min(mb + 2 * i, M - 1);
              const float xv = __uint_as_float((uint32_t)xh[(int64_t)m * K + c] << 16);
              if (j == 0) v[i].x += xv * d;
              else if (j == 1) v[i].y += xv * d;
              else if (j == 2) v[i].z += xv * d;
              else v[i].w += xv * d;
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 2 * i + h;
        const int m = m0 + 128 * wm + 32 * g + t;
        if (m >= M || n >= N) continue;
        float* yp = (ga.S > 1 ? ga.ws + (int64_t)split * ga.slot_stride : sg.y) + (int64_t)m * N + n;
        if (vec_ok) {
          if (ga.S > 1)  // a run's partial sum, read back by the reduction right after: keep it in the cache
            *reinterpret_cast<float4*>(yp) = v[i];
          else  // y: written once, not read again by this launch
            __builtin_nontemporal_store(f32x4{v[i].x, v[i].y, v[i].z, v[i].w}, reinterpret_cast<f32x4*>(yp));
        } else {
          yp[0] = v[i].x;
          if (n + 1 < N) yp[1] = v[i].y;
          if (n + 2 < N) yp[2] = v[i].z;
          if (n + 3 < N) yp[3] = v[i].w;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

template <bool PK12>
static hipError_t launch_gemm5(GemmArgs& ga, hipStream_t stream, int grid = 0) {
  using Ly = gemm5::Lay<PK12>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm5_bf16<PK12>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, Ly::LDS);
  if (attr != hipSuccess) return attr;
  int64_t tiles = 0;
  for (int i = 0; i < ga.nseg; ++i) {
    ga.seg[i].tile0 = (int)tiles;
    tiles += (int64_t)ga.tiles_m * ((ga.seg[i].N + gemm5::BN - 1) / gemm5::BN);
    if (tiles > INT_MAX) return hipErrorInvalidValue;
  }
  if (grid > 0) tiles = grid;
  hipLaunchKernelGGL((gemm5_bf16<PK12>), dim3((unsigned)tiles), dim3(gemm5::THREADS), Ly::LDS, stream, ga);
  return hipGetLastError();
}

bool gemm5_path_ok(const LayerArgs& a, bool pk12) {
  if (!a.x_bf16 || a.K % gemm5::BK != 0 || a.K < gemm5::BK) return false;
  if (reinterpret_cast<uintptr_t>(a.indices) % (pk12 ? 4 : 16) != 0) return false;
  if (pk12 && reinterpret_cast<uintptr_t>(a.codebook) % 8 != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.x) % 16 != 0) return false;
  const int64_t tiles = (((int64_t)a.M + gemm5::BM - 1) / gemm5::BM) * (((int64_t)a.N + 127) / 128);
  return tiles <= INT_MAX;
}

int64_t gemm5_tiles(const GemmSeg* segs, int nseg, int M) {
  int64_t t = 0;
  const int64_t tm = ((int64_t)M + gemm5::BM - 1) / gemm5::BM;
  for (int i = 0; i < nseg; ++i) t += tm * ((segs[i].N + gemm5::BN - 1) / gemm5::BN);
  return t;
}

hipError_t launch_gemm5_grouped(const GemmSeg* segs, int nseg, bool pk12, const void* x, int M, int K,
                                hipStream_t stream) {
  if (nseg < 1 || nseg > kMaxSegments) return hipErrorInvalidValue;
  GemmArgs ga;
  ga.x = x;
  ga.M = M;
  ga.K = K;
  ga.tiles_m = (M + gemm5::BM - 1) / gemm5::BM;
  ga.nseg = nseg;
  for (int i = 0; i < nseg; ++i) ga.seg[i] = segs[i];
  for (int i = nseg; i < kMaxSegments; ++i) ga.seg[i] = segs[0];
  ga.S = 1;
  ga.sst = K / gemm5::BK;
  ga.ws = nullptr;
  ga.slot_stride = 0;
  return pk12 ? launch_gemm5<true>(ga, stream) : launch_gemm5<false>(ga, stream);
}

// Layers of at least 128 stages (K >= 4096: shorter ones spend more on
// their partial sums' traffic than the split gains; o at 2048 tokens 45 ->
// 67 us in two runs), in runs of at least MINST stages, about one workgroup
// per CU, at most MAXST stages each (the patch bins), at most 64 runs.
Gemm5Split gemm5_split_plan(int M, int N, int K) {
  constexpr int MINST = 24;
  Gemm5Split p = {1, K / gemm5::BK, 0};
  const int64_t tiles = (int64_t)((M + gemm5::BM - 1) / gemm5::BM) * ((N + gemm5::BN - 1) / gemm5::BN);
  const int nk = K / gemm5::BK;
  if (nk < 128) return p;
  int64_t S = (device_cu_count() + tiles - 1) / tiles;
  if (S > nk / MINST) S = nk / MINST;
  if (S > 64) S = 64;
  const int smin = (nk + gemm5::MAXST - 1) / gemm5::MAXST;
  if (S < 2 || S < smin) return p;
  p.sst = (int)((nk + S - 1) / S);
  p.S = (nk + p.sst - 1) / p.sst;
  p.bytes = p.S > 1 ? (int64_t)p.S * M * N * 4 : 0;
  if (p.S < 2) p = {1, nk, 0};
  return p;
}

hipError_t launch_gemm5_split(const GemmSeg& sg, bool pk12, const void* x, int M, int K, float* ws, int64_t ws_bytes,
                              hipStream_t stream) {
  const Gemm5Split p = gemm5_split_plan(M, sg.N, K);
  if (p.S < 2 || ws == nullptr || ws_bytes < p.bytes) return hipErrorInvalidValue;
  GemmArgs ga;
  ga.x = x;
  ga.M = M;
  ga.K = K;
  ga.tiles_m = (M + gemm5::BM - 1) / gemm5::BM;
  ga.nseg = 1;
  for (int i = 0; i < kMaxSegments; ++i) ga.seg[i] = sg;
  ga.S = p.S;
  ga.sst = p.sst;
  ga.ws = ws;
  ga.slot_stride = (int64_t)M * sg.N;
  const int64_t tiles = (int64_t)ga.tiles_m * ((sg.N + gemm5::BN - 1) / gemm5::BN);
  if (tiles * p.S > INT_MAX) return hipErrorInvalidValue;
  // the launcher counts one run's tiles; the grid covers all runs
  hipError_t e = pk12 ? launch_gemm5<true>(ga, stream, (int)(tiles * p.S))
                      : launch_gemm5<false>(ga, stream, (int)(tiles * p.S));
  if (e != hipSuccess) return e;
  return launch_bwdx_reduce(ws, sg.y, (int64_t)M * sg.N, p.S, stream);
}

}  // namespace hxq
