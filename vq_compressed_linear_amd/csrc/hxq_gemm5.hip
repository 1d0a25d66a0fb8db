// bf16 matrix-core HelixLinear GEMM with 256-token tiles and LDS operand
// staging by DMA (prefill shapes), u8 and pk12 formats.
//
// y[m][n] = sum_k x[m][k] * Wq[n][k] + b[n], with Wq[n][k] the bf16 rounding
// (nearest, ties to even) of the fp32 value C[idx[n][k]] + S[n][k] (the
// codebook entry plus every sidecar delta at (n, k), added in fp32 in stored
// order).  The model cards ("What is HelixCode?") describe the layer as
// codebook[indices] @ x with no decompression step; the HXQ whitepaper's
// inference paragraph adds the sidecar to the gathered weights before the
// matmul, which is what the operand rounding does here.  The dense weight
// only ever exists as one 32-deep k-stage of the tile's rows in LDS.
//
// Per CU and 32-deep stage of a 256 x 256 tile (gfx950 numbers measured with
// probes on the target):
//   - matrix cores: 1024 clocks per SIMD (v_mfma_f32_32x32x16_bf16);
//   - codebook gathers: one per weight, shared by the 256 tokens: 8192 lanes
//     at about 32 lanes per clock (a 32-copy table is as fast as 64 copies);
//   - LDS reads of the weight operands: each wave reads its 128 outputs'
//     tile, 64 KB, at about 180 bytes per clock;
//   - global bytes: 16 KB of x and 8 KB of index bytes, which at 1-2 us of
//     loaded latency must be requested two to three stages ahead.  They are
//     copied into LDS rings by 16-byte DMA (global_load_lds), which needs no
//     registers; each DMA instruction reads 16 rows x 64 contiguous bytes of
//     x (whole 64-byte sectors).
//
// Waves: four along the tokens (64 each) times WN along the outputs (32 NF
// each); 2 x NF accumulator tiles of 32 x 32 per wave.  k order inside a
// stage: sub-step s and lane half h take k = 16 s + 8 h + [0, 8) for both
// operands (the matrix cores' own order).
//
// Pipeline (stage s, one barrier per stage):
//   - every wave requests x(s + 2) (its share of the 16 token blocks) and the
//     index bytes of its own 32 weight rows for stage s + 3;
//   - waits until its own index bytes of stage s + 1 have landed (no other
//     wave reads them), dequantises W(s + 1) into the other weight buffer and
//     applies its sidecar patches of that stage (same wave, so after its own
//     stores in LDS order);
//   - multiplies x(s) by W(s);
//   - waits until its x(s + 1) requests have landed, barrier.
// The request counts per stage are fixed (clamped stage indices past the
// end), so each wait is a constant count of outstanding requests.  The
// compiler does not see these requests (inline asm): it emits no waits for
// them, and the loop issues no other global loads.
//
// Sidecar triplets are turned into patches before the main loop (for each
// distinct (row, col) of the tile, the bf16 of C[idx] + deltas and its byte
// position in the stage's weight tile), binned by (stage, wave).  A tile with
// more triplets than the patch area, or K > 12288, patches its weights while
// dequantising instead (each lane walks its row's triplets in global memory:
// slower, same values).

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace gemm5 {
constexpr int BM = 256;       // tokens per tile
constexpr int BK = 32;        // k per stage
constexpr int WM = 4;         // waves along the tokens, 64 tokens each
constexpr int XR = 3;         // x stages in LDS
constexpr int IR = 3;         // index-byte stages in LDS
constexpr int MAXST = 384;    // stages on the patch path: K <= 12288
constexpr int CAP = 4096;     // patches per tile
constexpr int XS = BM * BK * 2;  // bytes of one x stage (16 blocks of 1 KB)

template <int WN, int NF, bool PK12>
struct Lay {
  static constexpr int THREADS = 256 * WN;
  static constexpr int WAVES = 4 * WN;
  static constexpr int BN = 32 * NF * WN;
  static constexpr int WT = BN * BK * 2;                 // bytes of one stage's weight tile
  static constexpr int UB = PK12 ? 12 : 16;              // index bytes of a 16-weight unit
  static constexpr int IW = 64 * 16;                     // LDS bytes per wave and stage (32 rows; a
                                                         // 12-byte DMA lane also takes a 16-byte slot)
  static constexpr int XPW = 16 / WAVES;                 // x blocks each wave requests per stage
  static constexpr int CB = PK12 ? 4096 * 4 : 256 * 128;  // static LDS (address 0)
  static constexpr int MAXBINS = MAXST * WAVES;          // bins (stage, wave)
  static constexpr int OFF_CBF = 0;                      // dynamic LDS; u8: the fp32 codebook
  static constexpr int OFF_W = OFF_CBF + (PK12 ? 0 : 1024);
  static constexpr int OFF_X = OFF_W + 2 * WT;
  static constexpr int OFF_I = OFF_X + XR * XS;
  static constexpr int OFF_BINS = OFF_I + IR * WAVES * IW;  // uint16 bin starts
  static constexpr int OFF_PATCH = OFF_BINS + ((MAXBINS + 8) * 2 + 15) / 16 * 16;
  static constexpr int OFF_MISC = OFF_PATCH + CAP * 4;
  static constexpr int LDS = OFF_MISC + 16 + 4 * WAVES;
  static_assert(BN == 32 * WAVES, "one 32-row block of the weight tile per wave");
  static_assert(XPW * WAVES == 16, "x blocks split evenly over the waves");
  static_assert(CAP <= 2 * WT, "head flags overlay the weight tiles");
  static_assert((MAXBINS + 4) * 4 <= XS, "bin counters overlay the third x stage");
  static_assert(MAXBINS % THREADS == 0, "bin prefix split");
  static_assert(CB + LDS <= 160 * 1024, "LDS");
};

// 16-byte (or 12-byte) copy global -> LDS: lane i's bytes land at lds + i * 16
// (a 12-byte copy also uses 16-byte slots, as probed on the target).  The LDS
// address is wave-uniform; m0 is restored.
template <int BYTES>
__device__ __forceinline__ void dma(const void* g, uint32_t lds) {
  uint32_t save;
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
}  // namespace gemm5

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int WN, int NF, bool PK12>
__global__ __launch_bounds__(256 * WN, 1) void gemm5_bf16(GemmArgs ga) {
  using namespace gemm5;
  using Ly = Lay<WN, NF, PK12>;
  constexpr int THREADS = Ly::THREADS, WAVES = Ly::WAVES, BN = Ly::BN, WT = Ly::WT;
  constexpr int UB = Ly::UB, IW = Ly::IW, XPW = Ly::XPW;
  constexpr int IS = PK12 ? 24 : 32;  // index bytes per row and stage
  // u8: entry e, copy c (c < 32) at byte 128 e + 4 c, bf16 in the upper half;
  // pk12: entry e at byte 4 e, bf16 of component 0 (even k) in the low half.
  // A static array sits at LDS address 0: a gather address is index arithmetic only
  __shared__ __align__(16) unsigned char cbs[Ly::CB];
  extern __shared__ __align__(16) unsigned char smem[];
  float* cbf = reinterpret_cast<float*>(smem + Ly::OFF_CBF);
  uint16_t* bins = reinterpret_cast<uint16_t*>(smem + Ly::OFF_BINS);  // bin b = stage * WAVES + wave
  uint32_t* patch = reinterpret_cast<uint32_t*>(smem + Ly::OFF_PATCH);
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + Ly::OFF_MISC);
  int* wsum = reinterpret_cast<int*>(smem + Ly::OFF_MISC + 16);
  unsigned char* wbuf = smem + Ly::OFF_W;
  const uint32_t lds_x = lds_addr(smem + Ly::OFF_X);
  const uint32_t lds_i = lds_addr(smem + Ly::OFF_I);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int h = lane >> 5, l32 = lane & 31;

  // ---- the tile: each XCD takes a contiguous run of tiles; segments own
  // consecutive tile ranges, tokens fastest within a segment
  const int G = gridDim.x, bx = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int L = (bx < full) ? (bx % 8) * per + bx / 8 : bx;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < ga.nseg && L >= ga.seg[i].tile0) si = i;
  const GemmSeg& sg = ga.seg[si];
  const int M = ga.M, N = sg.N, K = ga.K;
  const int tl = L - sg.tile0;
  const int m0 = (tl % ga.tiles_m) * BM, n0 = (tl / ga.tiles_m) * BN;
  const int nk = K / BK;
  const int64_t row_bytes = PK12 ? (int64_t)(K / 4) * 3 : (int64_t)K;

  // ---- DMA sources.  x block b (16 tokens, one stage) lane i: token
  // m0 + 16 b + i % 16, k = stage * 32 + 8 (i / 16) + [0, 8), landing at
  // byte 16 i of the block.  This wave requests blocks XPW * wave + j.
  const unsigned char* xb = static_cast<const unsigned char*>(ga.x);
  const unsigned char* xsrc[XPW];
#pragma unroll
  for (int j = 0; j < XPW; ++j)
    xsrc[j] = xb + (int64_t)min(m0 + 16 * (XPW * wave + j) + (lane & 15), M - 1) * (K * 2) + 16 * (lane >> 4);
  // index bytes: this wave's rows 32 wave + [0, 32); lane i takes row
  // 32 wave + i % 32 and k-half i / 32 of the stage, landing at byte 16 i
  const int nl_own = 32 * wave + l32;
  const uint8_t* isrc = sg.indices + (int64_t)min(n0 + nl_own, N - 1) * row_bytes + UB * h;
  auto req_x = [&](int st) {
    const int sc = min(st, nk - 1);
    const uint32_t dst = lds_x + (uint32_t)((st % XR) * XS) + (uint32_t)(XPW * wave) * 1024u;
#pragma unroll
    for (int j = 0; j < XPW; ++j) dma<16>(xsrc[j] + sc * (BK * 2), dst + 1024u * j);
  };
  auto req_i = [&](int st) {
    const int sc = min(st, nk - 1);
    dma<UB>(isrc + sc * IS, lds_i + (uint32_t)(((st % IR) * WAVES + wave) * IW));
  };
  // first requests, in the order the loop's waits count them:
  // [idx(0)], [x(0), idx(1)], [x(1), idx(2)]
  req_i(0);
  req_x(0);
  req_i(1);
  req_x(1);
  req_i(2);

  // ---- codebook.  u8: 32 copies per entry (the LDS serves 32 lanes of a
  // 4-byte gather per clock, so lane l reads copy l % 32 conflict-free); the
  // fp32 values too.  pk12: each component rounded to nearest even on its own
  if (PK12) {
#pragma unroll
    for (int i = 0; i < 4096 / THREADS; ++i) {
      const int e = tid + THREADS * i;
      const float2 c = reinterpret_cast<const float2*>(sg.codebook)[e];
      reinterpret_cast<uint32_t*>(cbs)[e] = f32_to_bf16_rne(c.x) | (f32_to_bf16_rne(c.y) << 16);
    }
  } else {
    constexpr int TPE = THREADS / 256, PER = 8 / TPE;  // threads per entry, 16-byte stores each
    const int e = tid & 255, part = tid >> 8;
    const float cv = sg.codebook[e];
    const float vb = __uint_as_float(f32_to_bf16_rne(cv) << 16);
    const float4 v4 = make_float4(vb, vb, vb, vb);
#pragma unroll
    for (int q = 0; q < PER; ++q)
      *reinterpret_cast<float4*>(cbs + e * 128 + (((PER * part + q + e) & 7) << 4)) = v4;
    if (part == 0) cbf[e] = cv;
  }

  // ---- sidecar: the tile's triplet range [lo, hi)
  const bool long_k = nk > MAXST;
  const int nbins = nk * WAVES;
  int* cnt32 = reinterpret_cast<int*>(smem + Ly::OFF_X + 2 * XS);  // counters (third x stage, free until stage 0)
  if (!long_k)
    for (int i = tid; i <= nbins; i += THREADS) cnt32[i] = 0;
  if (sg.nnz > 0 && wave < 2) {
    const int target = wave == 0 ? n0 : min(n0 + BN, N);
    const int64_t guess = (int64_t)((double)sg.nnz * (double)target / (double)N);
    const int64_t v = wave_lower_bound_rows_near(sg.sc_rows, sg.nnz, target, guess);
    if (lane == 0) lohi[wave] = v;
  }
  __syncthreads();
  int64_t lo = 0, hi = 0;
  if (sg.nnz > 0) {
    lo = lohi[0];
    hi = lohi[1];
  }
  const int64_t cnt = hi - lo;
  const bool walk = long_k || cnt > CAP;  // uniform

  if (!walk && cnt > 0) {
    // patches: the bf16 of C[idx] + deltas for each distinct (row, col) of the
    // tile and its byte position in the stage's weight tile, sorted by
    // (stage, wave that dequantises the row: row block nl / 32 is wave nl / 32)
    constexpr int QMAX = CAP / THREADS;
    unsigned char* hflag = wbuf;  // head flags (the weight buffers are first written after the set-up)
    int tr[QMAX], tc[QMAX];
    bool head[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int64_t e = lo + tid + (int64_t)THREADS * q;
      const int64_t ec = e < hi ? e : lo;
      const int64_t ep = ec > lo ? ec - 1 : lo;
      tr[q] = sg.sc_rows[ec];
      tc[q] = sg.sc_cols[ec];
      const int pr = sg.sc_rows[ep], pc = sg.sc_cols[ep];
      head[q] = e < hi && (e == lo || pr != tr[q] || pc != tc[q]);
      if (e < hi) hflag[e - lo] = head[q] ? 1 : 0;
      if (head[q]) atomicAdd(&cnt32[1 + (tc[q] / BK) * WAVES + ((tr[q] - n0) >> 5)], 1);
    }
    __syncthreads();
    // exclusive prefix over the counts cnt32[1 .. nbins]
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
          bins[b] = (uint16_t)base;  // start of bin b
        }
        base += c4[i];
      }
      if (tid == THREADS - 1) bins[nbins] = (uint16_t)base;
    }
    __syncthreads();
    // place (cnt32[1 + b] advances through bin b)
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      if (!head[q]) continue;
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
      patch[atomicAdd(&cnt32[1 + (tc[q] / BK) * WAVES + (nl >> 5)], 1)] = pos | (f32_to_bf16_rne(v) << 16);
    }
  } else if (!walk) {
    for (int i = tid; i <= nbins; i += THREADS) bins[i] = 0;
  }
  // walk path: triplet range of every tile row (overlays the patch area)
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

  // ---- dequantisation of this wave's 32 rows of one stage: lane (h, l32)
  // takes row 32 wave + l32, k = 16 h + [0, 16) (sub-step h) from its 16 (12)
  // index bytes; operand words of lane half 0 (k + [0, 8)) and 1 (k + [8, 16))
  // go to block (wave, h) at bytes 16 l32 and 16 (32 + l32)
  const uint32_t lanec = (uint32_t)(lane & 31) << 2;
  const int wofs = (wave * 2 + h) * 1024 + l32 * 16;
  auto read_idx = [&](int st) {
    const unsigned char* src = smem + Ly::OFF_I + ((st % IR) * WAVES + wave) * IW + 16 * lane;
    if (PK12) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(src);  // 4-byte aligned
      return u32x4{p[0], p[1], p[2], 0u};
    }
    return *reinterpret_cast<const u32x4*>(src);
  };
  auto build = [&](const u32x4 iq, unsigned char* wt) {
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
        const uint32_t f0 = lds_load<uint32_t>(((wd << 7) & 0x7f80u) | lanec, cbs);
        const uint32_t f1 = lds_load<uint32_t>(((wd >> 1) & 0x7f80u) | lanec, cbs);
        const uint32_t f2 = lds_load<uint32_t>(((wd >> 9) & 0x7f80u) | lanec, cbs);
        const uint32_t f3 = lds_load<uint32_t>(((wd >> 17) & 0x7f80u) | lanec, cbs);
        w[2 * d] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        w[2 * d + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
      }
    }
    *reinterpret_cast<u32x4*>(wt + wofs) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(wt + wofs + 512) = u32x4{w[4], w[5], w[6], w[7]};
  };
  // this wave's patches of stage st, after its own stores of that tile
  auto patch_stage = [&](int st, unsigned char* wt) {
    const int b = st * WAVES + wave;
    const int q0 = bins[b], q1 = bins[b + 1];
    for (int q = q0 + lane; q < q1; q += 64) {
      const uint32_t p = patch[q];
      *reinterpret_cast<uint16_t*>(wt + (p & 0xffffu)) = (uint16_t)(p >> 16);
    }
  };
  // walk path: a cursor over the lane's row's triplets (columns of the other
  // half of each stage are skipped)
  int64_t scur = 0, send = 0;
  int snc = INT_MAX;
  auto walk_init = [&]() {
    scur = lo + rsb[nl_own];
    send = lo + rse[nl_own];
    snc = scur < send ? sg.sc_cols[scur] : INT_MAX;
  };
  auto walk_stage = [&](int st, const u32x4 iq, unsigned char* wt) {
    const int c0 = st * BK + 16 * h, c1 = c0 + 16;
    while (snc < c1) {
      const int c = snc;
      if (c >= c0) {
        const int p = c - c0;  // column within the lane's 16
        float v = sg.sc_deltas[scur];
        if (PK12) {
          const int d = p >> 2;
          const uint32_t g24 = d == 0 ? (iq[0] & 0xffffffu)
                             : d == 1 ? (__builtin_amdgcn_alignbit(iq[1], iq[0], 24) & 0xffffffu)
                             : d == 2 ? (__builtin_amdgcn_alignbit(iq[2], iq[1], 16) & 0xffffffu)
                                      : (iq[2] >> 8);
          const uint32_t pi = ((p >> 1) & 1) ? (g24 >> 12) : (g24 & 0xfffu);
          v = sg.codebook[2 * pi + (p & 1)] + v;
        } else {
          v = cbf[(iq[p >> 2] >> ((p & 3) * 8)) & 0xffu] + v;
        }
        while (scur + 1 < send && sg.sc_cols[scur + 1] == c) {
          ++scur;
          v += sg.sc_deltas[scur];
        }
        *reinterpret_cast<uint16_t*>(wt + wofs + (p >> 3) * 512 + (p & 7) * 2) = (uint16_t)f32_to_bf16_rne(v);
      }
      ++scur;
      snc = scur < send ? sg.sc_cols[scur] : INT_MAX;
    }
  };

  f32x16 acc[2][NF];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[g][f][r] = 0.f;

  // operand reads: A (weights) of block f, sub-step s at (2 (wn NF + f) + s) KB + 16 lane;
  // B (x) of token group g, sub-step s: block 4 wm + 2 g + l32 / 16, byte
  // 16 ((2 s + h) 16 + l32 % 16)
  const int aoff = (wn * NF * 2) * 1024 + lane * 16;
  const int boff = (4 * wm + (l32 >> 4)) * 1024 + (h * 16 + (l32 & 15)) * 16;

  auto run = [&](auto walk_c) {
    constexpr bool WALK = decltype(walk_c)::value;
    if (WALK) walk_init();
    // W(0): its index bytes were requested first ([idx(0)], then 2 x (XPW + 1) requests)
    vm_wait<2 * XPW + 2>();
    {
      const u32x4 iq = read_idx(0);
      build(iq, wbuf);
      if (WALK) walk_stage(0, iq, wbuf);
      else patch_stage(0, wbuf);
    }
    vm_wait<XPW + 2>();  // x(0) landed
    __syncthreads();

    for (int s = 0; s < nk; ++s) {
      const unsigned char* wcur = wbuf + (s & 1) * WT;
      unsigned char* wnext = wbuf + ((s + 1) & 1) * WT;
      const unsigned char* xcur = smem + Ly::OFF_X + (s % XR) * XS;
      req_x(s + 2);
      req_i(s + 3);
      // this wave's index bytes of stage s + 1 (requested two stages ago)
      vm_wait<2 * XPW + 2>();
      // multiply x(s) by W(s) and dequantise W(s + 1) (past the last stage: a
      // copy of the last stage's bytes into the idle buffer, never read) in one
      // scheduling region: the stage's operand reads go out first, then the
      // gathers, spread between the matrix ops
      bf16x8 aop[2][NF], bop[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
          bop[sub][g] = *reinterpret_cast<const bf16x8*>(xcur + boff + g * 2048 + sub * 512);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          aop[sub][f] = *reinterpret_cast<const bf16x8*>(wcur + aoff + (2 * f + sub) * 1024);
      }
      const u32x4 iq = read_idx(s + 1);
      build(iq, wnext);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int g = 0; g < 2; ++g)
            acc[g][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[sub][f], bop[sub][g], acc[g][f], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (NF + 2) + 1, 0);
#pragma unroll
      for (int i = 0; i < 2 * NF * 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
      // sidecar of W(s + 1): after this wave's own stores of it
      if (s + 1 < nk) {
        if (WALK) walk_stage(s + 1, iq, wnext);
        else patch_stage(s + 1, wnext);
      }
      vm_wait<XPW + 2>();  // this wave's x(s + 1) landed
      __syncthreads();
    }
    vm_wait<0>();  // no copy into LDS may outlive the workgroup
  };
  if (walk) run(std::true_type{});
  else run(std::false_type{});

  // ---- epilogue.  Tile (g, f), register r holds output 32 (wn NF + f) + 8 (r / 4) + 4 h + r % 4
  // of token 64 wm + 32 g + l32.  Written straight out, each store instruction
  // would put 32 bytes into each of 32 rows; instead each wave turns its 32
  // tokens x 32 NF outputs of one token group into rows in a 16 KB LDS region
  // of its own (the codebook and the rings are dead by now) and stores whole
  // 512-byte row pieces.  Chunk c (4 outputs) of row t sits at 16 ((c ^ t) % 32)
  // so both the stores into LDS and the row reads spread over the banks.
  {
    constexpr int RS = 32 * 32 * NF * 4;     // bytes of one wave's region
    constexpr int CBW = Ly::CB / RS;         // regions inside the codebook area
    static_assert(NF == 4, "32 chunks of 4 outputs per row");
    static_assert(Ly::LDS >= (WAVES - CBW) * RS, "epilogue regions fit");
    unsigned char* reg = wave < CBW ? cbs + wave * RS : smem + (wave - CBW) * RS;
    const bool vec_ok = (N & 3) == 0;
    float bv[NF][4][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 32 * (wn * NF + f) + 8 * q + 4 * h + r;
          bv[f][q][r] = (sg.bias && n < N) ? sg.bias[n] : 0.f;
        }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 8 * f + 2 * q + h;
          *reinterpret_cast<float4*>(reg + l32 * 512 + ((c ^ l32) & 31) * 16) =
              make_float4(acc[g][f][4 * q] + bv[f][q][0], acc[g][f][4 * q + 1] + bv[f][q][1],
                          acc[g][f][4 * q + 2] + bv[f][q][2], acc[g][f][4 * q + 3] + bv[f][q][3]);
        }
      // the rows are read by other lanes of this wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int n = n0 + 32 * NF * wn + 4 * l32;  // this lane's 4 outputs of each row
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 2 * i + h;
        const float4 v = *reinterpret_cast<const float4*>(reg + t * 512 + ((l32 ^ t) & 31) * 16);
        const int m = m0 + 64 * wm + 32 * g + t;
        if (m >= M || n >= N) continue;
        float* yp = sg.y + (int64_t)m * N + n;
        if (vec_ok) {
          *reinterpret_cast<float4*>(yp) = v;
        } else {
          yp[0] = v.x;
          if (n + 1 < N) yp[1] = v.y;
          if (n + 2 < N) yp[2] = v.z;
          if (n + 3 < N) yp[3] = v.w;
        }
      }
      // the region is written again for the next token group
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

template <int WN, int NF, bool PK12>
static hipError_t launch_gemm5(GemmArgs& ga, hipStream_t stream) {
  using Ly = gemm5::Lay<WN, NF, PK12>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm5_bf16<WN, NF, PK12>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, Ly::LDS);
  if (attr != hipSuccess) return attr;
  int64_t tiles = 0;
  for (int i = 0; i < ga.nseg; ++i) {
    ga.seg[i].tile0 = (int)tiles;
    tiles += (int64_t)ga.tiles_m * ((ga.seg[i].N + Ly::BN - 1) / Ly::BN);
    if (tiles > INT_MAX) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((gemm5_bf16<WN, NF, PK12>), dim3((unsigned)tiles), dim3(Ly::THREADS), Ly::LDS, stream, ga);
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
  using Ly = gemm5::Lay<2, 4, false>;
  int64_t t = 0;
  const int64_t tm = ((int64_t)M + gemm5::BM - 1) / gemm5::BM;
  for (int i = 0; i < nseg; ++i) t += tm * ((segs[i].N + Ly::BN - 1) / Ly::BN);
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
  return pk12 ? launch_gemm5<2, 4, true>(ga, stream) : launch_gemm5<2, 4, false>(ga, stream);
}

}  // namespace hxq
