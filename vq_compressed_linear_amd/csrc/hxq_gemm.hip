// bf16 matrix-core HelixLinear GEMM for the u8 format (prefill shapes).
//
// y[m][n] = sum_k x[m][k] * Wq[n][k] + b[n], with Wq[n][k] the bf16 rounding
// (nearest, ties to even) of the fp32 value C[idx[n][k]] + S[n][k].  The
// product runs on CDNA4 bf16 MFMA (16x16x32) with fp32 accumulation.  The
// weight exists only as a 128 x 32 bf16 tile in LDS for the k-step that uses
// it (the model cards' "codebook[indices] @ x" with no decompression pass; the
// HXQ whitepaper's inference paragraph adds the sidecar to the gathered
// weights before the matmul, which is where it is added here too, in fp32).
//
// Workgroup tile 128 (tokens) x 128 (outputs), k-step 32, 4 waves in 2 x 2,
// each wave 64 x 64 = 4 x 4 MFMA tiles.  Per k-step every thread loads 32
// bytes of x and 16 index bytes into registers one step ahead, then stores x
// and the gathered weights into LDS.  Gathers read a 64-copy bf16 codebook
// (copy j of entry e at byte e*256 + 4j, value in the upper 16 bits) so each
// lane reads its own bank.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace gemm {
constexpr int BM = 128, BN = 128, BK = 32, THREADS = 256;
constexpr int ROW = BK * 2 + 16;                  // bytes per LDS tile row (+16 pad)
constexpr int LDS_CB = 0;                         // 256 entries x 256 B
constexpr int LDS_CBF = LDS_CB + 256 * 256;       // fp32 codebook, 1 KB
constexpr int LDS_XS = LDS_CBF + 1024;            // x tile, BM rows
constexpr int LDS_WS = LDS_XS + BM * ROW;         // weight tile, BN rows
constexpr int LDS_RS = LDS_WS + BN * ROW;         // sidecar row ranges: 2 x BN int32
constexpr int LDS_LOHI = LDS_RS + 2 * BN * 4;     // 2 int64
constexpr int LDS_TOTAL = LDS_LOHI + 16;
}  // namespace gemm

__global__ __launch_bounds__(256) void gemm_u8_bf16(LayerArgs a, int tiles_m) {
  using namespace gemm;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.M, N = a.N, K = a.K;

  // Workgroups are dealt to the 8 XCDs round-robin; renumber so that each XCD
  // gets a contiguous run of tiles (consecutive tiles share a weight column).
  const int G = gridDim.x, b = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int L = (b < full) ? (b % 8) * per + b / 8 : b;
  const int tm = L % tiles_m, tn = L / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- stage the codebook: 64 bf16 copies + one fp32 copy
  {
    const float* cb = static_cast<const float*>(a.codebook);
    for (int i = tid; i < 256 * 16; i += THREADS) {
      const float v = cb[i >> 4];
      const float vb = __uint_as_float(f32_to_bf16_rne(v) << 16);
      *reinterpret_cast<float4*>(smem + LDS_CB + (i >> 4) * 256 + (i & 15) * 16) =
          make_float4(vb, vb, vb, vb);
    }
    reinterpret_cast<float*>(smem + LDS_CBF)[tid] = cb[tid];
  }
  // ---- sidecar: triplet range of every tile row
  int* rs_begin = reinterpret_cast<int*>(smem + LDS_RS);
  int* rs_end = rs_begin + BN;
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + LDS_LOHI);
  if (tid < BN) {
    rs_begin[tid] = 0;
    rs_end[tid] = 0;
  }
  if (a.nnz > 0 && wave == 0) {
    const int64_t lo = wave_lower_bound_rows(a.sc_rows, a.nnz, n0);
    const int64_t hi = wave_lower_bound_rows(a.sc_rows, a.nnz, min(n0 + BN, N));
    if (lane == 0) {
      lohi[0] = lo;
      lohi[1] = hi;
    }
  }
  __syncthreads();
  int64_t sc_lo = 0;
  if (a.nnz > 0) {
    sc_lo = lohi[0];
    const int64_t hi = lohi[1];
    for (int64_t e = sc_lo + tid; e < hi; e += THREADS) {
      const int r = a.sc_rows[e];
      if (e == sc_lo || a.sc_rows[e - 1] != r) rs_begin[r - n0] = (int)(e - sc_lo);
      if (e == hi - 1 || a.sc_rows[e + 1] != r) rs_end[r - n0] = (int)(e - sc_lo + 1);
    }
  }
  __syncthreads();

  // ---- per-thread load assignment
  const int xr = tid >> 1, xh = tid & 1;   // x tile: row xr, bytes 32*xh .. +31
  const int wr = tid >> 1, wh = tid & 1;   // weight tile: row wr, k 16*wh .. +15
  const uint16_t* xrow =
      static_cast<const uint16_t*>(a.x) + (int64_t)min(m0 + xr, M - 1) * K + xh * 16;
  const uint8_t* irow = a.indices + (int64_t)min(n0 + wr, N - 1) * K + wh * 16;
  int64_t sc_cur = 0, sc_end = 0;
  int sc_nc = INT_MAX;
  if (a.nnz > 0) {
    sc_cur = sc_lo + rs_begin[wr];
    sc_end = sc_lo + rs_end[wr];
    if (sc_cur < sc_end) sc_nc = a.sc_cols[sc_cur];
  }
  const uint32_t lane4 = (uint32_t)lane << 2;
  const float* cbf = reinterpret_cast<const float*>(smem + LDS_CBF);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  uint4 xa = make_uint4(0, 0, 0, 0), xb = xa, wi = xa;
  if (nk > 0) {
    xa = *reinterpret_cast<const uint4*>(xrow);
    xb = *reinterpret_cast<const uint4*>(xrow + 8);
    wi = *reinterpret_cast<const uint4*>(irow);
  }
  const int wm = wave & 1, wn = wave >> 1;

  for (int ks = 0; ks < nk; ++ks) {
    const int k0 = ks * BK;
    // x -> LDS
    *reinterpret_cast<uint4*>(smem + LDS_XS + xr * ROW + xh * 32) = xa;
    *reinterpret_cast<uint4*>(smem + LDS_XS + xr * ROW + xh * 32 + 16) = xb;
    // indices -> bf16 weights -> LDS
    {
      uint32_t pk[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t wd = d == 0 ? wi.x : d == 1 ? wi.y : d == 2 ? wi.z : wi.w;
        const uint32_t f0 = lds_load<uint32_t>(byte_addr256<0>(wd, lane4), smem + LDS_CB);
        const uint32_t f1 = lds_load<uint32_t>(byte_addr256<1>(wd, lane4), smem + LDS_CB);
        const uint32_t f2 = lds_load<uint32_t>(byte_addr256<2>(wd, lane4), smem + LDS_CB);
        const uint32_t f3 = lds_load<uint32_t>(byte_addr256<3>(wd, lane4), smem + LDS_CB);
        pk[2 * d] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        pk[2 * d + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
      }
      unsigned char* dst = smem + LDS_WS + wr * ROW + wh * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      // sidecar triplets that fall in this thread's 16 columns: C + deltas in
      // fp32 (triplet order), rounded once to bf16.
      const int c0 = k0 + wh * 16, c1 = c0 + 16;
      while (sc_nc < c1) {
        const int c = sc_nc;
        if (c >= c0) {
          const int p = c - c0;
          const uint32_t word = p < 4 ? wi.x : p < 8 ? wi.y : p < 12 ? wi.z : wi.w;
          float v = cbf[(word >> ((p & 3) * 8)) & 0xffu] + a.sc_deltas[sc_cur];
          while (sc_cur + 1 < sc_end && a.sc_cols[sc_cur + 1] == c) {
            ++sc_cur;
            v += a.sc_deltas[sc_cur];
          }
          *reinterpret_cast<uint16_t*>(dst + p * 2) = (uint16_t)f32_to_bf16_rne(v);
        }
        ++sc_cur;
        sc_nc = sc_cur < sc_end ? a.sc_cols[sc_cur] : INT_MAX;
      }
    }
    __syncthreads();
    if (ks + 1 < nk) {
      xa = *reinterpret_cast<const uint4*>(xrow + k0 + BK);
      xb = *reinterpret_cast<const uint4*>(xrow + k0 + BK + 8);
      wi = *reinterpret_cast<const uint4*>(irow + k0 + BK);
    }
    bf16x8 af[4], bw[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      af[f] = *reinterpret_cast<const bf16x8*>(smem + LDS_XS + (wm * 64 + f * 16 + (lane & 15)) * ROW +
                                               (lane >> 4) * 16);
      bw[f] = *reinterpret_cast<const bf16x8*>(smem + LDS_WS + (wn * 64 + f * 16 + (lane & 15)) * ROW +
                                               (lane >> 4) * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  // ---- epilogue: lane l, register r of tile (i, j) holds row 4*(l/16)+r, column l%16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + (lane & 15);
    if (n >= N) continue;
    const float bn = a.bias ? a.bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (m < M) a.y[(int64_t)m * N + n] = acc[i][j][r] + bn;
      }
  }
}

bool gemm_path_ok(const LayerArgs& a) {
  if (!a.x_bf16 || a.K % gemm::BK != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.indices) % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.x) % 16 != 0) return false;
  const int64_t tiles = (((int64_t)a.M + gemm::BM - 1) / gemm::BM) * (((int64_t)a.N + gemm::BN - 1) / gemm::BN);
  return tiles <= INT_MAX;
}

hipError_t launch_gemm_bf16(const LayerArgs& a, hipStream_t stream) {
  // once per process (a function-local static is initialised exactly once,
  // also under concurrent first calls)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_u8_bf16),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, gemm::LDS_TOTAL);
  if (attr != hipSuccess) return attr;
  const int tiles_m = (a.M + gemm::BM - 1) / gemm::BM;
  const int tiles_n = (a.N + gemm::BN - 1) / gemm::BN;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  hipLaunchKernelGGL(gemm_u8_bf16, grid, dim3(gemm::THREADS), gemm::LDS_TOTAL, stream, a, tiles_m);
  return hipGetLastError();
}



// ---------------------------------------------------------------- pipelined GEMM
//
// The same product and rounding as above, arranged so that the matrix cores
// are not left waiting.
//   - Workgroup tile 128 tokens x (128 * FN) outputs.  Eight waves (two per
//     SIMD, so one can issue while the other waits) sit side by side along the
//     outputs; each owns 16 * FN outputs for all 128 tokens (8 x FN MFMA
//     tiles of fp32 accumulators, in ordinary VGPRs: at two waves per SIMD a
//     wave has 256 registers in all).  FN is 2, or 1 when 128-output tiles
//     need no more rounds over the CUs.
//   - A k-stage is 64 deep.  x reaches the MFMAs through a ring of four LDS
//     tiles; stages go in pairs with one barrier per pair, and the x of a
//     stage is loaded into registers two stages before it is stored.  A tile
//     is kept in operand order: 1 KB block (i, u) holds the 16 bytes lane
//     (g, l16) reads for token block i and sub-step u at position
//     16 g + (l16 ^ (2 g + u)), so every eight lanes of an operand read cover
//     one 128-byte segment (128-bit reads of rows 128 bytes apart run at half
//     rate), while the eight pieces a row's global load brings land in eight
//     different bank groups.
//   - Each lane turns its own 16 index bytes per fragment into bf16 operands
//     with codebook gathers from LDS, one stage ahead of the MFMAs that use
//     them; index bytes are loaded two stages ahead.  No weight tile is
//     written and no gather is repeated by another wave.  Lane group g
//     (lane / 16) covers k = 16 g + 8 u + [0, 8) in MFMA sub-step u, for A and
//     B alike, so the sum over k is unchanged.
//   - Sidecar triplets are turned into patches before the main loop: for each
//     distinct (row, col) of the tile, the bf16 of fp32 C[idx] + deltas
//     (triplet order), binned by (stage, wave) in LDS.  A wave reads the
//     patches of the next stage while its MFMAs run and overwrites the operand
//     halves they name.  A tile with more triplets than the patch area holds,
//     or a very long K, walks its sidecar rows from global memory instead
//     (slower, same values).

namespace gemm3 {
constexpr int THREADS = 512, WAVES = THREADS / 64, BM = 128, BK = 64, FM = BM / 16;
constexpr int ATILE = BM * BK * 2;     // 16 KB: 16 operand blocks of 1 KB
constexpr int RING = 4;                // x tiles in LDS
constexpr int MAXBINS = 2048;          // 8 bins per stage: K <= 16384 on the patch path
constexpr int QMAX = 8;                // triplets per thread on the patch path
constexpr int CAP = QMAX * THREADS;    // patches per tile
constexpr int PRE = 8;                 // patches a wave reads ahead per stage
constexpr int OFF_CBF = RING * ATILE;
constexpr int OFF_BINS = OFF_CBF + 1024;
constexpr int OFF_PATCH = OFF_BINS + (MAXBINS + 4) * 4;
constexpr int XPT = ATILE / 16 / THREADS;  // 16-byte x pieces per thread per stage
static_assert(XPT * THREADS * 16 == ATILE, "the x stores cover the tile");
constexpr int OFF_MISC = OFF_PATCH + (CAP + PRE) * 4;
constexpr int LDS_DYN = OFF_MISC + 64;
static_assert(2 * 256 * 4 <= CAP * 4, "walk-path row ranges overlay the patch area");
static_assert(MAXBINS % THREADS == 0, "bin prefix: whole bins per thread");
static_assert(CAP <= ATILE, "head flags overlay an x tile");
}  // namespace gemm3

// PK12: 2D-VQ layers (HXQ whitepaper, "2D vector quantization"): 12-bit pair
// indices, three bytes per two pairs, the 4096-pair codebook as bf16 pairs in
// LDS (one gather gives the operand word of two k-adjacent weights)
template <int FN, bool PK12>
__global__ __launch_bounds__(gemm3::THREADS, 1) void gemm3_bf16(GemmArgs ga) {
  using namespace gemm3;
  constexpr int BN = 16 * WAVES * FN;
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  // operands of one stage in one vector: fragment j at words 8 j .. 8 j + 7,
  // the first four for sub-step 0, the last four for sub-step 1
  typedef uint32_t vecB __attribute__((ext_vector_type(8 * FN)));
  // u8: 64 copies per entry, bf16 in the upper half; pk12: entry e at byte 4 e,
  // bf16 of component 0 (even k) in the low half, component 1 in the high half
  __shared__ __align__(16) unsigned char cbs[PK12 ? 4096 * 4 : 256 * 256];
  extern __shared__ __align__(16) unsigned char smem[];
  float* cbf = reinterpret_cast<float*>(smem + OFF_CBF);
  int* bins = reinterpret_cast<int*>(smem + OFF_BINS);  // bin b spans patch[bins[b] .. bins[b + 1])
  uint32_t* patch = reinterpret_cast<uint32_t*>(smem + OFF_PATCH);
  int64_t* lohi = reinterpret_cast<int64_t*>(smem + OFF_MISC);
  int* wsum = reinterpret_cast<int*>(smem + OFF_MISC + 16);  // one per wave
  unsigned char* hflag = smem + 2 * ATILE;  // head flags of the tile's triplets (prologue only)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, bx = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int L = (bx < full) ? (bx % 8) * per + bx / 8 : bx;  // each XCD a contiguous run of tiles
  // the layer this tile belongs to: segments own consecutive tile ranges
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < ga.nseg && L >= ga.seg[i].tile0) si = i;
  const GemmSeg& sg = ga.seg[si];
  LayerArgs a;
  a.codebook = sg.codebook;
  a.indices = sg.indices;
  a.sc_rows = sg.sc_rows;
  a.sc_cols = sg.sc_cols;
  a.sc_deltas = sg.sc_deltas;
  a.nnz = sg.nnz;
  a.x = ga.x;
  a.x_bf16 = true;
  a.bias = sg.bias;
  a.y = sg.y;
  a.M = ga.M;
  a.N = sg.N;
  a.K = ga.K;
  const int M = a.M, N = a.N, K = a.K;
  const int tiles_m = ga.tiles_m;
  const int tm = (L - sg.tile0) % tiles_m, tn = (L - sg.tile0) / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = K / BK;
  const int g = lane >> 4, l16 = lane & 15;
  const int nw = wave * 16 * FN;  // the wave's first output within the tile
  const uint32_t lane4 = (uint32_t)lane << 2;

  // ---- operand addresses
  // x piece p = tid + 512 i: tile row r = p / 8, 16-byte piece c = p % 8, stored at
  // block (r / 16, c % 2), position 16 (c / 2) + ((r % 16) ^ c)
  const unsigned char* xb = static_cast<const unsigned char*>(a.x);
  uint32_t xoff[XPT];
  int xst[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int p = tid + THREADS * i, r = p >> 3, c = p & 7;
    xoff[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)(K * 2) + c * 16;
    xst[i] = ((r >> 4) * 2 + (c & 1)) * 1024 + (((c >> 1) * 16 + ((r & 15) ^ c)) << 4);
  }
  // index bytes of fragment j: output n0 + nw + 16 j + l16, k = 16 g .. 16 g + 15 of the stage
  // (u8: 16 bytes; pk12: 12 bytes, the 8 pairs (k, k + 1) of those 16 k)
  constexpr int IB = PK12 ? 12 : 16;
  const int64_t row_bytes = PK12 ? (int64_t)(K / 4) * 3 : (int64_t)K;
  const uint8_t* irow[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) irow[j] = a.indices + (int64_t)min(n0 + nw + 16 * j + l16, N - 1) * row_bytes + IB * g;
  // A operand of token block i, sub-step u: block 2 i + u
  const int aoff0 = (g * 16 + (l16 ^ (2 * g))) * 16, aoff1 = 1024 + (g * 16 + (l16 ^ (2 * g + 1))) * 16;

  u32x4 XA[XPT], XB[XPT], IQ[FN];
  auto load_x = [&](int st, u32x4* d) {
    const uint32_t kx = (uint32_t)min(st, nk - 1) * (BK * 2);
#pragma unroll
    for (int i = 0; i < XPT; ++i) d[i] = *reinterpret_cast<const u32x4*>(xb + xoff[i] + kx);
  };
  auto store_x = [&](int st, const u32x4* d) {
    unsigned char* t = smem + (st & (RING - 1)) * ATILE;
#pragma unroll
    for (int i = 0; i < XPT; ++i) *reinterpret_cast<u32x4*>(t + xst[i]) = d[i];
  };
  typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
  auto load_iq = [&](int st, u32x4* d) {
    const int kn = min(st, nk - 1) * (BK / 16 * IB);  // index bytes per stage and row
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (PK12) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(irow[j] + kn);
        d[j] = u32x4{v[0], v[1], v[2], 0u};
      } else {
        d[j] = *reinterpret_cast<const u32x4*>(irow[j] + kn);
      }
    }
  };
  load_x(0, XA);
  load_x(1, XB);
  load_iq(0, IQ);

  // ---- codebook.  u8: threads t and t + 256 stage half of entry t's 64 bf16
  // copies each (pieces rotated against bank conflicts); fp32 values too.
  // pk12: thread t packs pairs t, t + 512, ... (each component rounded to
  // nearest even on its own)
  if (PK12) {
#pragma unroll
    for (int i = 0; i < 4096 / THREADS; ++i) {
      const int e = tid + THREADS * i;
      const float2 c = reinterpret_cast<const float2*>(a.codebook)[e];
      reinterpret_cast<uint32_t*>(cbs)[e] = f32_to_bf16_rne(c.x) | (f32_to_bf16_rne(c.y) << 16);
    }
  } else {
    const int e = tid & 255, h = tid >> 8;
    const float cv = static_cast<const float*>(a.codebook)[e];
    const float vb = __uint_as_float(f32_to_bf16_rne(cv) << 16);
    const float4 v4 = make_float4(vb, vb, vb, vb);
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<float4*>(cbs + e * 256 + (((8 * h + q + e) & 15) << 4)) = v4;
    if (h == 0) cbf[e] = cv;
  }
  // ---- sidecar: the tile's triplet range [lo, hi)
  const int nbins = nk * WAVES;
  const bool long_k = nbins > MAXBINS;
  if (!long_k)
    for (int i = tid; i <= nbins; i += THREADS) bins[i] = 0;
  if (a.nnz > 0 && wave < 2) {
    const int target = wave == 0 ? n0 : min(n0 + BN, N);
    const int64_t guess = (int64_t)((double)a.nnz * (double)target / (double)N);
    const int64_t v = wave_lower_bound_rows_near(a.sc_rows, a.nnz, target, guess);
    if (lane == 0) lohi[wave] = v;
  }
  __syncthreads();
  int64_t lo = 0, hi = 0;
  if (a.nnz > 0) {
    lo = lohi[0];
    hi = lohi[1];
  }
  const int64_t cnt = hi - lo;
  const bool walk = long_k || cnt > CAP;  // uniform

  if (!walk && cnt > 0) {
    // patches: thread t takes triplets lo + t + 256 q
    int tr[QMAX], tc[QMAX], pr[QMAX], pc[QMAX];
    float td[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int64_t e = lo + tid + (int64_t)THREADS * q;
      const int64_t ec = e < hi ? e : lo;
      const int64_t ep = ec > lo ? ec - 1 : lo;
      tr[q] = a.sc_rows[ec];
      tc[q] = a.sc_cols[ec];
      pr[q] = a.sc_rows[ep];
      pc[q] = a.sc_cols[ep];
      td[q] = a.sc_deltas[ec];
    }
    uint32_t tb[QMAX];
    bool head[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int64_t e = lo + tid + (int64_t)THREADS * q;
      head[q] = e < hi && (e == lo || pr[q] != tr[q] || pc[q] != tc[q]);
      if (PK12) {
        // the 24-bit group holding the pair of column tc (the pair is tc / 2)
        const uint8_t* pb = a.indices + (int64_t)tr[q] * row_bytes + (tc[q] >> 2) * 3;
        tb[q] = (uint32_t)pb[0] | ((uint32_t)pb[1] << 8) | ((uint32_t)pb[2] << 16);
      } else {
        tb[q] = a.indices[(int64_t)tr[q] * K + tc[q]];
      }
      if (e < hi) hflag[e - lo] = head[q] ? 1 : 0;
      if (head[q]) atomicAdd(&bins[1 + (tc[q] / BK) * WAVES + (tr[q] - n0) / (16 * FN)], 1);
    }
    __syncthreads();
    // exclusive prefix over the counts in bins[1 ..]: thread t owns PT of them
    {
      constexpr int PT = MAXBINS / THREADS;
      int c4[PT];
      int tot = 0;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        c4[i] = PT * tid + i < nbins ? bins[1 + PT * tid + i] : 0;
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
        if (PT * tid + i < nbins) bins[1 + PT * tid + i] = base;
        base += c4[i];
      }
    }
    __syncthreads();
    // place; afterwards bins[1 + b] is the end of bin b, i.e. the start of bin b + 1
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      if (!head[q]) continue;
      const int64_t e = lo + tid + (int64_t)THREADS * q;
      float v = td[q];
      if (PK12) {
        const uint32_t pi = ((tc[q] >> 1) & 1) ? (tb[q] >> 12) : (tb[q] & 0xfffu);
        v += static_cast<const float*>(a.codebook)[2 * pi + (tc[q] & 1)];
      } else {
        v += cbf[tb[q]];
      }
      for (int64_t e2 = e + 1; e2 < hi && !hflag[e2 - lo]; ++e2) v += a.sc_deltas[e2];
      // patch word: lane (bits 0-5), column in the lane's 16 (bits 6-9), fragment (10-11), bf16 (16-31)
      const int rl = tr[q] - n0, cl = tc[q] % BK;
      const uint32_t w = (uint32_t)(rl % 16 + 16 * (cl / 16)) | ((uint32_t)(cl % 16) << 6) |
                         ((uint32_t)((rl / 16) % FN) << 10) | (f32_to_bf16_rne(v) << 16);
      patch[atomicAdd(&bins[1 + (tc[q] / BK) * WAVES + rl / (16 * FN)], 1)] = w;
    }
  }
  // walk path: triplet range of every tile row (overlays the patch area)
  int* rsb = reinterpret_cast<int*>(patch);
  int* rse = rsb + BN;
  if (walk) {
    for (int i = tid; i < BN; i += THREADS) rsb[i] = rse[i] = 0;
    __syncthreads();
    for (int64_t e = lo + tid; e < hi; e += THREADS) {
      const int r = a.sc_rows[e];
      if (e == lo || a.sc_rows[e - 1] != r) rsb[r - n0] = (int)(e - lo);
      if (e == hi - 1 || a.sc_rows[e + 1] != r) rse[r - n0] = (int)(e - lo + 1);
    }
  }
  __syncthreads();

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operands of one stage from its index bytes: u8 16 gathers and 8 packs per
  // fragment; pk12 8 gathers (24-bit group d holds pairs 2 d, 2 d + 1 as
  // v & 0xfff, v >> 12; operand word e is the pair of k = 2 e, 2 e + 1)
  auto build = [&](const u32x4* iq, vecB& out) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (PK12) {
          const uint32_t v = d == 0 ? (iq[j][0] & 0xffffffu)
                           : d == 1 ? (__builtin_amdgcn_alignbit(iq[j][1], iq[j][0], 24) & 0xffffffu)
                           : d == 2 ? (__builtin_amdgcn_alignbit(iq[j][2], iq[j][1], 16) & 0xffffffu)
                                    : (iq[j][2] >> 8);
          out[8 * j + 2 * d] = lds_load<uint32_t>((v & 0xfffu) << 2, cbs);
          out[8 * j + 2 * d + 1] = lds_load<uint32_t>((v >> 12) << 2, cbs);
          continue;
        }
        const uint32_t wd = iq[j][d];
        const uint32_t f0 = lds_load<uint32_t>(byte_addr256<0>(wd, lane4), cbs);
        const uint32_t f1 = lds_load<uint32_t>(byte_addr256<1>(wd, lane4), cbs);
        const uint32_t f2 = lds_load<uint32_t>(byte_addr256<2>(wd, lane4), cbs);
        const uint32_t f3 = lds_load<uint32_t>(byte_addr256<3>(wd, lane4), cbs);
        out[8 * j + 2 * d] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        out[8 * j + 2 * d + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
      }
  };
  // patches: the bin of (stage st, this wave) and its first PRE words, read early
  struct PatchPre {
    int q0, q1;
    uint32_t w[PRE];
  };
  auto patch_read = [&](int st, PatchPre& pp) {
    const int b = min(st, nk - 1) * WAVES + wave;
    pp.q0 = bins[b];
    pp.q1 = st < nk ? bins[b + 1] : pp.q0;
#pragma unroll
    for (int t = 0; t < PRE; ++t) pp.w[t] = patch[pp.q0 + t];
  };
  auto patch_one = [&](uint32_t ent, vecB& v) {
    const uint32_t keep = (ent & 64u) ? 0x0000ffffu : 0xffff0000u;
    const uint32_t put = ((ent >> 16) * 0x10001u) & ~keep;
    const bool mine = lane == (int)(ent & 63u);
    if constexpr (FN == 1) {
      // one fragment: the compiler selects among the eight words (faster here
      // than without the fragment test, as measured)
      const uint32_t e = (ent >> 7) & 7u;
      const uint32_t old = v[e];
      v[e] = (mine && ((ent >> 10) & 3u) == 0u) ? ((old & keep) | put) : old;
    } else {
      // uniform (fragment, word): one indexed register read and write
      const uint32_t at = ((ent >> 10) & 3u) * 8u + ((ent >> 7) & 7u);
      const uint32_t old = v[at];
      v[at] = mine ? ((old & keep) | put) : old;
    }
  };
  auto patch_apply = [&](const PatchPre& pp, vecB& v) {
    const int q0 = __builtin_amdgcn_readfirstlane(pp.q0);
    const int n = __builtin_amdgcn_readfirstlane(pp.q1) - q0;
    if (n <= 0) return;
#pragma unroll
    for (int t = 0; t < PRE; ++t)
      if (t < n) patch_one(__builtin_amdgcn_readfirstlane(pp.w[t]), v);
    for (int q = PRE; q < n; ++q) patch_one(__builtin_amdgcn_readfirstlane(patch[q0 + q]), v);
  };
  // walk path: per-lane cursors over the sidecar row of each fragment
  int64_t scur[FN], send[FN];
  int snc[FN];
  auto walk_init = [&]() {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rl = nw + 16 * j + l16;
      scur[j] = lo + rsb[rl];
      send[j] = lo + rse[rl];
      snc[j] = scur[j] < send[j] ? a.sc_cols[scur[j]] : INT_MAX;
    }
  };
  auto walk_stage = [&](int st, const u32x4* iq, vecB& v) {
    if (st >= nk) return;
    const int c0 = st * BK + 16 * g, c1 = c0 + 16;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      while (snc[j] < c1) {
        const int c = snc[j];
        if (c >= c0) {
          const int p = c - c0;
          float val = a.sc_deltas[scur[j]];
          if (PK12) {
            // pair p / 2 of the lane's 8: group p / 4 of the 12 bytes
            const int d = p >> 2;
            const uint32_t v = d == 0 ? (iq[j][0] & 0xffffffu)
                             : d == 1 ? (__builtin_amdgcn_alignbit(iq[j][1], iq[j][0], 24) & 0xffffffu)
                             : d == 2 ? (__builtin_amdgcn_alignbit(iq[j][2], iq[j][1], 16) & 0xffffffu)
                                      : (iq[j][2] >> 8);
            const uint32_t pi = ((p >> 1) & 1) ? (v >> 12) : (v & 0xfffu);
            val += static_cast<const float*>(a.codebook)[2 * pi + (p & 1)];
          } else {
            const uint32_t word = iq[j][p >> 2];
            val += cbf[(word >> ((p & 3) * 8)) & 0xffu];
          }
          while (scur[j] + 1 < send[j] && a.sc_cols[scur[j] + 1] == c) {
            ++scur[j];
            val += a.sc_deltas[scur[j]];
          }
          const uint32_t h = f32_to_bf16_rne(val);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e == (p >> 1)) {
              const uint32_t old = v[8 * j + e];
              v[8 * j + e] = (p & 1) ? ((old & 0xffffu) | (h << 16)) : ((old & 0xffff0000u) | h);
            }
        }
        ++scur[j];
        snc[j] = scur[j] < send[j] ? a.sc_cols[scur[j]] : INT_MAX;
      }
    }
  };

  vecB B0, B1;
  auto run = [&](auto walk_c) {
    constexpr bool WALK = decltype(walk_c)::value;
    if (WALK) walk_init();
    // x(0), x(1) into the ring, operands of stage 0 into B0
    store_x(0, XA);
    store_x(1, XB);
    load_x(2, XA);
    load_x(3, XB);
    build(IQ, B0);
    if (WALK) {
      walk_stage(0, IQ, B0);
    } else {
      PatchPre pp;
      patch_read(0, pp);
      patch_apply(pp, B0);
    }
    load_iq(1, IQ);
    __syncthreads();

    // stage s: x(s) in ring slot s % 4, operands of s in B[s & 1]; the index
    // bytes of s + 1 in IQ (loaded a stage ago).  The first stage of a pair
    // stores x(s + 2), x(s + 3) (loaded two stages ago) and loads x(s + 4),
    // x(s + 5).
    auto stage = [&](auto par_c, int s, bool top, bool bar) {
      constexpr int P = decltype(par_c)::value;
      vecB& Bc = P ? B1 : B0;
      vecB& Bn = P ? B0 : B1;
      const unsigned char* abuf = smem + (s & (RING - 1)) * ATILE;
      if (top) {
        store_x(s + 2, XA);
        load_x(s + 4, XA);
        store_x(s + 3, XB);
        load_x(s + 5, XB);
      }
      PatchPre pp;
      if (!WALK) patch_read(s + 1, pp);
      build(IQ, Bn);
      if (!WALK) load_iq(s + 2, IQ);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const bf16x8 aop = *reinterpret_cast<const bf16x8*>(abuf + (u ? aoff1 : aoff0) + i * 2048);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const u32x4 bw = u32x4{Bc[8 * j + 4 * u], Bc[8 * j + 4 * u + 1], Bc[8 * j + 4 * u + 2],
                                   Bc[8 * j + 4 * u + 3]};
            // weights as the A operand, x as B: the result tile is y transposed,
            // so each lane ends up with four consecutive outputs of one token
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bw), aop, acc[i][j], 0, 0, 0);
          }
        }
      if (WALK) {
        walk_stage(s + 1, IQ, Bn);
        load_iq(s + 2, IQ);
      } else {
        patch_apply(pp, Bn);
      }
      if (bar) __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nk; s += 2) {
      stage(std::integral_constant<int, 0>{}, s, true, false);
      stage(std::integral_constant<int, 1>{}, s + 1, false, true);
    }
    if (s < nk) stage(std::integral_constant<int, 0>{}, s, true, false);
  };
  if (walk) run(std::true_type{});
  else run(std::false_type{});

  // ---- epilogue: lane l, register r of tile (i, j): output 16 j + 4 (l / 16) + r, token 16 i + l % 16
  const bool vec_ok = (N & 3) == 0;
  const bool bias_vec = vec_ok && a.bias && (reinterpret_cast<uintptr_t>(a.bias) & 15) == 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + nw + 16 * j + 4 * g;
    if (n >= N) continue;
    float bv[4];
    if (bias_vec) {
      const float4 b4 = *reinterpret_cast<const float4*>(a.bias + n);
      bv[0] = b4.x, bv[1] = b4.y, bv[2] = b4.z, bv[3] = b4.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = (a.bias && n + r < N) ? a.bias[n + r] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + 16 * i + l16;
      if (m >= M) continue;
      float* yp = a.y + (int64_t)m * N + n;
      if (vec_ok) {
        __builtin_nontemporal_store(
            f32x4{acc[i][j][0] + bv[0], acc[i][j][1] + bv[1], acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]},
            reinterpret_cast<f32x4*>(yp));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) yp[r] = acc[i][j][r] + bv[r];
      }
    }
  }
}

template <int FN, bool PK12>
static hipError_t launch_gemm3(GemmArgs& ga, hipStream_t stream) {
  using namespace gemm3;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm3_bf16<FN, PK12>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_DYN);
  if (attr != hipSuccess) return attr;
  int64_t tiles = 0;
  for (int i = 0; i < ga.nseg; ++i) {
    ga.seg[i].tile0 = (int)tiles;
    tiles += (int64_t)ga.tiles_m * ((ga.seg[i].N + 16 * WAVES * FN - 1) / (16 * WAVES * FN));
    if (tiles > INT_MAX) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((gemm3_bf16<FN, PK12>), dim3((unsigned)tiles), dim3(THREADS), LDS_DYN, stream, ga);
  return hipGetLastError();
}

bool gemm2_path_ok(const LayerArgs& a, bool pk12) {
  if (!a.x_bf16 || a.K % gemm3::BK != 0 || a.K < gemm3::BK) return false;
  if (reinterpret_cast<uintptr_t>(a.indices) % (pk12 ? 4 : 16) != 0) return false;
  if (pk12 && reinterpret_cast<uintptr_t>(a.codebook) % 8 != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.x) % 16 != 0) return false;
  const int64_t tiles = (((int64_t)a.M + gemm3::BM - 1) / gemm3::BM) * (((int64_t)a.N + 127) / 128);
  if (tiles > INT_MAX) return false;
  // x offsets are 32-bit
  return (int64_t)a.M * a.K * 2 < ((int64_t)1 << 32);
}

// Output tile width by rounds of tiles over the CUs: a 128-output tile takes
// about as long as a 256-output one (the per-stage LDS work of a wave is the
// same), so 256 outputs unless 128 needs no more rounds.
hipError_t launch_gemm_grouped(const GemmSeg* segs, int nseg, bool pk12, const void* x, int M, int K,
                               hipStream_t stream) {
  if (nseg < 1 || nseg > kMaxSegments) return hipErrorInvalidValue;
  GemmArgs ga;
  ga.x = x;
  ga.M = M;
  ga.K = K;
  ga.tiles_m = (M + gemm3::BM - 1) / gemm3::BM;
  ga.nseg = nseg;
  int64_t wide = 0, narrow = 0;
  for (int i = 0; i < nseg; ++i) {
    ga.seg[i] = segs[i];
    wide += (int64_t)ga.tiles_m * ((segs[i].N + 255) / 256);
    narrow += (int64_t)ga.tiles_m * ((segs[i].N + 127) / 128);
  }
  for (int i = nseg; i < kMaxSegments; ++i) ga.seg[i] = segs[0];
  const int64_t cus = device_cu_count();
  const bool use_wide = (wide + cus - 1) / cus < (narrow + cus - 1) / cus;
  if (pk12) return use_wide ? launch_gemm3<2, true>(ga, stream) : launch_gemm3<1, true>(ga, stream);
  return use_wide ? launch_gemm3<2, false>(ga, stream) : launch_gemm3<1, false>(ga, stream);
}

hipError_t launch_gemm2_bf16(const LayerArgs& a, bool pk12, hipStream_t stream) {
  const GemmSeg sg = {static_cast<const float*>(a.codebook), a.indices, a.sc_rows, a.sc_cols, a.sc_deltas,
                      a.nnz, a.bias, a.y, a.N, 0};
  return launch_gemm_grouped(&sg, 1, pk12, a.x, a.M, a.K, stream);
}

}  // namespace hxq
