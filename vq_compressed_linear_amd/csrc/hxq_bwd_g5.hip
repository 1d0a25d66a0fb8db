// Input gradient dx = dy W on bf16 matrix cores with 256-token x 256-column
// tiles (u8 format, bf16 dy, training-size batches).
//
//     dx[m][k] = sum_n dy[m][n] * Wq[n][k],   Wq = bf16(C[idx] + S)
//
// (model cards, "Good to Know": LoRA trains through frozen HelixLinear
// layers, which needs this product; W as in "What is HelixCode?" and the HXQ
// whitepaper's "Method").  The weight value is the codebook value plus any
// sidecar deltas at that position, added in fp32 in stored order and rounded
// once to bf16 (nearest, ties to even): the value the forward GEMM uses.
// fp32 accumulation.
//
// The structure of the forward's 256 x 256 tile kernel with the roles of the
// weight's two axes exchanged: the tile is 256 tokens x 256 columns of dx and
// the contraction runs over the layer's rows n, 32 per stage.  Four waves,
// one per SIMD, each 128 tokens x 128 columns (v_mfma_f32_32x32x16_bf16, 16
// accumulator tiles in the accumulation registers).  Each stage's weight
// tile (32 rows x 256 columns) is built once per workgroup in LDS and shared
// by the tile's 256 tokens; the matrix cores want it contraction-major (8
// consecutive rows of one column per 16-byte operand piece), so the builder
// transposes on the way: lane l of wave w loads 4 index bytes (columns
// 4 l .. + 3) of each of the rows 8 w .. + 7, gathers their 32 bf16 values
// from the 64-copy codebook and packs, per column, its 8 rows into one
// 16-byte piece (4 byte permutes, one store).  Per stage and lane that is
// the forward's count of gathers, permutes and stores.  The pieces of a
// column block sit at rows XOR-swizzled so that both the builders' stores
// (consecutive lanes four columns apart) and the operand reads are free of
// bank conflicts.  dy is staged like the forward's x (its rows are
// contraction-major already).
//
// Sidecar: the patch words of the binning kernel (hxq_bwd_mfma.hip: per
// 32-row step and 128-column bin, each word the bf16 of C + deltas of one
// distinct (row, col) and its place in the step) are read for the tile's
// two bins one stage ahead of use and written over the built weights by the
// wave that built their row.
//
// Row splits (to fill the GPU when the tiles are few) store into workspace
// slots that the reduction kernel sums in split order.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace bg5 {
constexpr int BM = 256, BN = 256, BK = 32;  // tokens, columns, rows per stage
constexpr int THREADS = 256, WAVES = 4;
constexpr int XR = 2, WR = 2;               // dy slots and weight buffers in LDS
constexpr int MAXST = 512;                  // stages per split (bin starts kept in LDS)
constexpr int XS = BM * BK * 2;             // bytes of one dy stage
constexpr int WT = BN * BK * 2;             // bytes of one weight stage
constexpr int CB = 256 * 256;               // 64 bf16 copies per codebook entry
constexpr int OFF_W = 0;
constexpr int OFF_X = OFF_W + WR * WT;
constexpr int OFF_BS = OFF_X + XR * XS;     // per stage: word range of the tile's two bins
constexpr int LDS = OFF_BS + MAXST * 3 * 4;
static_assert(CB + LDS <= 160 * 1024, "LDS");
constexpr int RS = 32 * 128 * 4;            // epilogue region of a wave
static_assert(CB >= WAVES * RS, "epilogue regions fit the codebook area");
struct Ops {
  bf16x8 a[2][4];  // weights: sub-step, column block
  bf16x8 b[2][4];  // dy: sub-step, token group
};
// the place of row r (0..31) of column block b among the block's 32 pieces
__host__ __device__ constexpr int swz(int r, int b) { return r ^ ((r >> 3) & 3) ^ ((b & 1) << 3); }
}  // namespace bg5

__global__ __launch_bounds__(256, 1) void bwdx_g5(BwdG5Args a) {
  using namespace bg5;
  __shared__ __align__(16) unsigned char cbs[CB];
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* wbuf = smem + OFF_W;
  unsigned char* xbuf = smem + OFF_X;
  int* bsl = reinterpret_cast<int*>(smem + OFF_BS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;

  // consecutive workgroups of a launch go round the eight XCDs: give each
  // XCD a contiguous run of tiles (tokens fastest), so the tiles sharing
  // index bytes share its L2
  const int G = gridDim.x, bx = blockIdx.x;
  const int per = G / 8, full = per * 8;
  const int L = (bx < full) ? (bx % 8) * per + bx / 8 : bx;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < a.nseg && L >= a.seg[i].wg0) si = i;
  const BwdG5Seg& sg = a.seg[si];
  const int tiles = a.tiles_m * a.tiles_k;
  const int Ls = L - sg.wg0;
  const int s = Ls / tiles, tl = Ls - s * tiles;
  const int m0 = (tl % a.tiles_m) * BM, k0 = (tl / a.tiles_m) * BN;
  const int M = a.M, N = sg.N, K = a.K;
  const int n_lo = s * sg.R;
  const int nst = (min(N, n_lo + sg.R) - n_lo) / BK;  // N and R are multiples of 32

  // dy piece j of this wave: block 4 wave + j (16 tokens), lane i: token
  // m0 + 16 (4 wave + j) + i % 16, rows n_lo + 32 stage + 8 (i / 16) + [0, 8)
  const unsigned char* dyb = reinterpret_cast<const unsigned char*>(sg.dy);
  const unsigned char* xsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    xsrc[j] = dyb + ((int64_t)min(m0 + 16 * (4 * wave + j) + (lane & 15), M - 1) * N + n_lo) * 2 + 16 * (lane >> 4);
  auto load_x = [&](int st, u32x4 (&v)[4]) {
    const int sc = min(st, nst - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const u32x4*>(xsrc[j] + sc * (BK * 2));
  };
  auto store_x = [&](int st, const u32x4 (&v)[4]) {
    unsigned char* d = xbuf + (st % XR) * XS + (4 * wave) * 1024 + 16 * lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(d + 1024 * j) = v[j];
  };
  // index bytes: rows n_lo + 32 stage + 8 wave + j (j < 8), columns 4 lane .. + 3
  // of the tile (past K: the row's last four, never stored)
  const uint8_t* isrc = sg.indices + (int64_t)(n_lo + 8 * wave) * K + min(k0 + 4 * lane, K - 4);
  auto load_i = [&](int st, uint32_t (&q)[8]) {
    const int sc = min(st, nst - 1);
    const uint8_t* p = isrc + (int64_t)(sc * BK) * K;
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = *reinterpret_cast<const uint32_t*>(p + (int64_t)j * K);
  };
  uint32_t ip0[8], ip1[8], iq0[8], iq1[8];
  u32x4 xp0[4], xp1[4], xs0[4], xs1[4];
  load_i(0, ip0);
  load_x(0, xp0);
  load_i(1, ip1);
  load_x(1, xp1);

  // ---- codebook: 64 bf16 copies per entry (entry e, copy c at byte 256 e +
  // 4 c, the value in the upper half), lane l reads copy l
  {
    const int e = tid;
    const float vb = __uint_as_float(f32_to_bf16_rne(sg.codebook[e]) << 16);
    const float4 v4 = make_float4(vb, vb, vb, vb);
#pragma unroll
    for (int q = 0; q < 16; ++q) *reinterpret_cast<float4*>(cbs + e * 256 + (((q + e) & 15) << 4)) = v4;
  }
  // ---- the word ranges of the tile's two sidecar bins per stage: [bs0, bs1)
  // columns k0 .. + 127, [bs1, bs2) the next 128
  const bool side = sg.CT > 0;
  {
    const int step0 = n_lo / BK, b0 = k0 / 128;
    for (int i = tid; i < nst * 3; i += THREADS) {
      const int st = i / 3, c = i - 3 * st;
      bsl[i] = side ? sg.binstart[(int64_t)(step0 + st) * (sg.CT + 1) + min(b0 + c, sg.CT)] : 0;
    }
  }
  load_i(2, iq0);
  load_x(2, xs0);
  load_i(3, iq1);
  load_x(3, xs1);
  __syncthreads();

  // ---- building: lane l of wave w turns the 4 index bytes of each of its 8
  // rows into 4 pieces, one per column 4 l + c: piece (column block b =
  // l / 8, sub-step w / 2, half w % 2, row 4 (l % 8) + c), rows 8 w .. + 7
  // in order
  const uint32_t lane4 = (uint32_t)lane << 2;
  int wofs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int b = lane >> 3, r = 4 * (lane & 7) + c;
    wofs[c] = ((b * 2 + (wave >> 1)) * 64 + (wave & 1) * 32 + swz(r, b)) * 16;
  }
  auto pack = [&](const uint32_t (&g)[8][4], int c) {
    return u32x4{__builtin_amdgcn_perm(g[1][c], g[0][c], 0x07060302u), __builtin_amdgcn_perm(g[3][c], g[2][c], 0x07060302u),
                 __builtin_amdgcn_perm(g[5][c], g[4][c], 0x07060302u), __builtin_amdgcn_perm(g[7][c], g[6][c], 0x07060302u)};
  };
  auto build = [&](const uint32_t (&iq)[8], unsigned char* wt) {
    uint32_t g[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g[j][0] = lds_load<uint32_t>(byte_addr256<0>(iq[j], lane4), cbs);
      g[j][1] = lds_load<uint32_t>(byte_addr256<1>(iq[j], lane4), cbs);
      g[j][2] = lds_load<uint32_t>(byte_addr256<2>(iq[j], lane4), cbs);
      g[j][3] = lds_load<uint32_t>(byte_addr256<3>(iq[j], lane4), cbs);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(wt + wofs[c]) = pack(g, c);
  };
  // a patch word's byte in the weight tile (kl: its column in the tile), or
  // -1 when another wave built its row
  auto patch_pos = [&](uint32_t wd, int kl_hi) {
    const int lf = (int)(wd & 63u);
    const int jj = 8 * (lf >> 4) + 2 * (int)((wd >> 9) & 3u) + (int)((wd >> 11) & 1u);
    const int kl = kl_hi + 8 * (lf & 15) + (int)((wd >> 6) & 7u);
    const int b = kl >> 5;
    const int pos = ((b * 2 + (jj >> 4)) * 64 + ((jj >> 3) & 1) * 32 + swz(kl & 31, b)) * 16 + (jj & 7) * 2;
    return (lf >> 4) == wave ? pos : -1;
  };
  auto patch_range = [&](int q0, int q1, int q2, unsigned char* wt) {  // every word of [q0, q2)
    for (int q = q0 + lane; q < q2; q += 64) {
      const uint32_t wd = sg.bpat[q];
      const int p = patch_pos(wd, q >= q1 ? 128 : 0);
      if (p >= 0) *reinterpret_cast<uint16_t*>(wt + p) = (uint16_t)(wd >> 16);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[g][f][r] = 0.f;

  // operand reads: weights of column block 4 wn + f, sub-step s: lane
  // (h, l32) reads piece 32 h + swz(l32, f) of block (2 (4 wn + f) + s); dy
  // of tokens 128 wm + 32 g + l32 as the forward's x
  const int aoff0 = (8 * wn) * 1024 + (32 * h + swz(l32, 0)) * 16;
  const int aoff1 = (8 * wn) * 1024 + (32 * h + swz(l32, 1)) * 16;
  const int boff = (8 * wm + (l32 >> 4)) * 1024 + (h * 16 + (l32 & 15)) * 16;
  auto read_ops = [&](int st, Ops& o) {
    const unsigned char* wt = wbuf + (st % WR) * WT;
    const unsigned char* xt = xbuf + (st % XR) * XS;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
        o.a[sub][f] = *reinterpret_cast<const bf16x8*>(wt + ((f & 1) ? aoff1 : aoff0) + (2 * f + sub) * 1024);
#pragma unroll
      for (int g = 0; g < 4; ++g) o.b[sub][g] = *reinterpret_cast<const bf16x8*>(xt + boff + g * 2048 + sub * 512);
    }
  };

  // W(0), W(1) with their patches, dy(0), dy(1) into LDS
  build(ip0, wbuf);
  build(ip1, wbuf + WT);
  if (side) {
    patch_range(bsl[0], bsl[1], bsl[2], wbuf);
    if (nst > 1) patch_range(bsl[3], bsl[4], bsl[5], wbuf + WT);
  }
  store_x(0, xp0);
  store_x(1, xp1);
  __syncthreads();
  {
    Ops oa, ob;
    read_ops(0, oa);
    // stage s, ordered by hand as in the forward kernel: sub-step 0's 16
    // matrix ops each followed by two gathers for W(s + 2) (row i / 2,
    // columns 2 (i % 2) + [0, 2)), every other one by a weight-operand read
    // for s + 1; sub-step 1's by the dy-operand reads, the store of dy(s + 2)
    // and the packing and stores of W(s + 2).  Its patch words are requested
    // at the start of the stage (their range read from LDS a stage before)
    // and written after the stores.  dy and index bytes of s + 4 are
    // requested once their registers are free.
    auto stage = [&](int s, Ops& cur, Ops& nxt, u32x4 (&xr)[4], uint32_t (&ir)[8], int& pq0, int& pq1,
                     int& pq2) {
      unsigned char* wt2 = wbuf + ((s + 2) % WR) * WT;
      const unsigned char* wn1 = wbuf + ((s + 1) % WR) * WT;
      const unsigned char* xn1 = xbuf + ((s + 1) % XR) * XS;
      uint32_t gw[8][4];
      auto mm = [&](int sub, int i) {
        const int f = i >> 2, g = i & 3;
        acc[g][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[sub][f], cur.b[sub][g], acc[g][f], 0, 0, 0);
      };
      auto gather = [&](int i) {
        const int j = i >> 1, c = 2 * (i & 1);
        if (c == 0) {
          gw[j][0] = lds_load<uint32_t>(byte_addr256<0>(ir[j], lane4), cbs);
          gw[j][1] = lds_load<uint32_t>(byte_addr256<1>(ir[j], lane4), cbs);
        } else {
          gw[j][2] = lds_load<uint32_t>(byte_addr256<2>(ir[j], lane4), cbs);
          gw[j][3] = lds_load<uint32_t>(byte_addr256<3>(ir[j], lane4), cbs);
        }
      };
      auto opread = [&](int j) {  // j = 0..15: 8 weight reads then 8 dy reads
        const int sub = (j >> 2) & 1, q = j & 3;
        if (j < 8)
          nxt.a[sub][q] = *reinterpret_cast<const bf16x8*>(wn1 + ((q & 1) ? aoff1 : aoff0) + (2 * q + sub) * 1024);
        else
          nxt.b[sub][q] = *reinterpret_cast<const bf16x8*>(xn1 + boff + q * 2048 + sub * 512);
      };
      unsigned char* xd = xbuf + ((s + 2) % XR) * XS + (4 * wave) * 1024 + 16 * lane;
      const bool pt = side && s + 2 < nst;  // uniform
      const int q0 = __builtin_amdgcn_readfirstlane(pq0), q1 = __builtin_amdgcn_readfirstlane(pq1),
                q2 = __builtin_amdgcn_readfirstlane(pq2);
      uint32_t pe = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mm(0, i);
        gather(i);
        if (i & 1) opread(i >> 1);
        // (unconditional, so that the compiler's counter waits stay exact;
        // clamped: an empty last bin starts at nnz, and without a sidecar
        // the ranges are 0 and bpat a stand-in word)
        if (i == 0) pe = sg.bpat[max(min(q0 + lane, sg.nnz - 1), 0)];
        if (i == 4) {  // word ranges of W(s + 3), used next stage (past the end: unused)
          const int b = 3 * min(s + 3, nst - 1);
          pq0 = bsl[b];
          pq1 = bsl[b + 1];
          pq2 = bsl[b + 2];
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
        if ((i & 1) && i >= 9) *reinterpret_cast<u32x4*>(wt2 + wofs[(i - 9) >> 1]) = pack(gw, (i - 9) >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (pt && q0 + lane < q2) {
        const int p = patch_pos(pe, q0 + lane >= q1 ? 128 : 0);
        if (p >= 0) *reinterpret_cast<uint16_t*>(wt2 + p) = (uint16_t)(pe >> 16);
      }
      if (pt && q2 - q0 > 64) {
        // rare: the words past the first 64, one at a time through the scalar
        // unit (a vector load in a loop here would make the compiler's
        // counter waits after it cover every load in flight), each waited
        // for in its own asm block
        for (int q = q0 + 64; q < q2; ++q) {
          const uint32_t* wp = sg.bpat + q;
          uint32_t wd;
          asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(wd) : "s"(wp) : "memory");
          const int p = patch_pos(wd, q >= q1 ? 128 : 0);
          if (lane == 0 && p >= 0) *reinterpret_cast<uint16_t*>(wt2 + p) = (uint16_t)(wd >> 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // word ranges of W(2), for stage 0
    int pq0 = 0, pq1 = 0, pq2 = 0;
    {
      const int b = 3 * min(2, nst - 1);
      pq0 = bsl[b];
      pq1 = bsl[b + 1];
      pq2 = bsl[b + 2];
    }
    int s2 = 0;
    for (; s2 + 1 < nst; s2 += 2) {
      stage(s2, oa, ob, xs0, iq0, pq0, pq1, pq2);
      stage(s2 + 1, ob, oa, xs1, iq1, pq0, pq1, pq2);
    }
    if (s2 < nst) stage(s2, oa, ob, xs0, iq0, pq0, pq1, pq2);
  }

  // ---- epilogue: per token group, each wave turns its 32 tokens x 128
  // columns into rows in a 16 KB LDS region of its own (the codebook area)
  // and stores 512-byte row pieces (chunk c of row t at 16 ((c ^ t) % 32))
  {
    unsigned char* reg = cbs + wave * RS;
    float* out = a.out + (int64_t)(sg.slot0 + s) * a.slot_stride;
    const bool split_out = a.slot_stride != 0;  // slots summed afterwards, else dx itself
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 8 * f + 2 * q + h;
          *reinterpret_cast<float4*>(reg + l32 * 512 + ((c ^ l32) & 31) * 16) =
              make_float4(acc[g][f][4 * q], acc[g][f][4 * q + 1], acc[g][f][4 * q + 2], acc[g][f][4 * q + 3]);
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int k = k0 + 128 * wn + 4 * l32;  // this lane's 4 columns of each row
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 2 * i + h;
        const int m = m0 + 128 * wm + 32 * g + t;
        const float4 v = *reinterpret_cast<const float4*>(reg + t * 512 + ((l32 ^ t) & 31) * 16);
        if (m < M && k < K) {
          float* op = out + (int64_t)m * K + k;
          if (split_out)  // a partial sum the reduction reads back soon: keep it in the cache
            *reinterpret_cast<float4*>(op) = v;
          else
            __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(op));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// The shapes and pointers this kernel takes: u8, bf16 dy, whole 32-row
// steps and 128-column bins, K <= 16384; dy and dx 16-byte and indices
// 4-byte aligned.
bool bwdx_g5_ok(const BwdArgs& a, bool pk12) {
  if (pk12 || !a.dy_bf16 || a.M < 1 || a.N < bg5::BK || a.K < 128) return false;
  if (a.N % bg5::BK != 0 || a.K % 128 != 0 || a.K > 16384) return false;
  if ((int64_t)a.N > (int64_t)64 * bg5::MAXST * bg5::BK) return false;  // at most 64 splits
  const uintptr_t ip = reinterpret_cast<uintptr_t>(a.indices), dp = reinterpret_cast<uintptr_t>(a.dy);
  const uintptr_t xp = reinterpret_cast<uintptr_t>(a.dx);
  return dp % 16 == 0 && xp % 16 == 0 && ip % 4 == 0;
}

// Row splits: enough workgroups for about one per CU, at least 8 stages per
// split, at most MAXST.
BwdMPlan bwdx_g5_plan(int M, int N, int K, int64_t nnz) {
  BwdMPlan p;
  p.ctw = (K + bg5::BN - 1) / bg5::BN;
  p.mtiles = (M + bg5::BM - 1) / bg5::BM;
  const int64_t tiles = (int64_t)p.ctw * p.mtiles;
  const int nsteps = N / bg5::BK;
  int64_t S = (device_cu_count() + tiles - 1) / tiles;
  const int64_t smax = nsteps / 8 > 0 ? nsteps / 8 : 1;
  if (S > smax) S = smax;
  if (S > 64) S = 64;
  const int64_t smin = (nsteps + bg5::MAXST - 1) / bg5::MAXST;
  if (S < smin) S = smin;
  if (S < 1) S = 1;
  const int spp = (nsteps + (int)S - 1) / (int)S;
  p.R = spp * bg5::BK;
  p.S = (nsteps + spp - 1) / spp;
  p.CT = nnz > 0 ? K / 128 : 0;
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  p.split_bytes = p.S > 1 ? al((int64_t)p.S * M * K * 4) : 0;
  p.bin_bytes = nnz > 0 ? al((int64_t)nsteps * (p.CT + 1) * 4) + al(nnz * 4) : 0;
  return p;
}

static hipError_t launch_g5(const BwdG5Args& g, int64_t blocks, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwdx_g5),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, bg5::LDS);
  if (attr != hipSuccess) return attr;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwdx_g5, dim3((unsigned)blocks), dim3(bg5::THREADS), bg5::LDS, stream, g);
  return hipGetLastError();
}

// A layer's segment: its bins into `bins` first when it has a sidecar
// (without one the kernel reads a stand-in word: its first index bytes).
static hipError_t g5_segment(const BwdArgs& a, int R, int CT, unsigned char* bins, BwdG5Seg& sg,
                             hipStream_t stream) {
  sg.codebook = a.codebook;
  sg.indices = a.indices;
  sg.dy = static_cast<const uint16_t*>(a.dy);
  sg.N = a.N;
  sg.R = R;
  sg.CT = a.nnz > 0 ? CT : 0;
  sg.nnz = a.nnz > 0 ? (int)a.nnz : 1;
  sg.binstart = nullptr;
  sg.bpat = reinterpret_cast<const uint32_t*>(a.indices);
  if (a.nnz > 0) {
    const int nsteps = a.N / bg5::BK;
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    int* binstart = reinterpret_cast<int*>(bins);
    uint32_t* bpat = reinterpret_cast<uint32_t*>(bins + al((int64_t)nsteps * (CT + 1) * 4));
    const hipError_t e = launch_bwdx_bin(a, false, CT, binstart, bpat, stream);
    if (e != hipSuccess) return e;
    sg.binstart = binstart;
    sg.bpat = bpat;
  }
  return hipSuccess;
}

// As launch_bwdx_mfma: sidecar binning, the product, the sum of the splits
// (a.slots set: the splits go to slots a.slot0 .. + S - 1, not summed).
hipError_t launch_bwdx_g5(const BwdArgs& a, hipStream_t stream) {
  const BwdMPlan p = bwdx_g5_plan(a.M, a.N, a.K, a.nnz);
  const bool grouped = a.slots != nullptr;
  const int64_t split_bytes = grouped ? 0 : p.split_bytes;
  if (a.ws_bytes < split_bytes + p.bin_bytes || (split_bytes + p.bin_bytes > 0 && a.ws == nullptr))
    return hipErrorInvalidValue;
  unsigned char* w = reinterpret_cast<unsigned char*>(a.ws);
  BwdG5Args g = {};
  g.out = grouped ? a.slots + (int64_t)a.slot0 * a.M * a.K : p.S > 1 ? reinterpret_cast<float*>(w) : a.dx;
  g.slot_stride = (grouped || p.S > 1) ? (int64_t)a.M * a.K : 0;
  g.M = a.M;
  g.K = a.K;
  g.tiles_m = p.mtiles;
  g.tiles_k = p.ctw;
  g.nseg = 1;
  hipError_t e = g5_segment(a, p.R, a.K / 128, w + split_bytes, g.seg[0], stream);
  if (e != hipSuccess) return e;
  g.seg[0].wg0 = 0;
  g.seg[0].slot0 = 0;
  e = launch_g5(g, (int64_t)p.ctw * p.mtiles * p.S, stream);
  if (e != hipSuccess || p.S == 1 || grouped) return e;
  return launch_bwdx_reduce(g.out, a.dx, (int64_t)a.M * a.K, p.S, stream);
}

BwdG5Group bwdx_g5_group_plan(int M, int K, const int* Ns, const int64_t* nnzs, int n) {
  BwdG5Group g = {};
  const int64_t tiles = (int64_t)((M + bg5::BM - 1) / bg5::BM) * ((K + bg5::BN - 1) / bg5::BN);
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += Ns[i] / bg5::BK;
  int64_t target = (device_cu_count() + tiles - 1) / tiles;
  if (target > 64) target = 64;
  int64_t R = (total + target - 1) / target;  // stages per run
  if (R < 8) R = 8;
  if (R > bg5::MAXST) R = bg5::MAXST;
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  for (int i = 0; i < n; ++i) {
    const int steps = Ns[i] / bg5::BK;
    int S = (int)((steps + R / 2) / R);
    if (S < 1) S = 1;
    const int smin = (steps + bg5::MAXST - 1) / bg5::MAXST;
    if (S < smin) S = smin;
    const int spp = (steps + S - 1) / S;
    g.S[i] = (steps + spp - 1) / spp;
    g.R[i] = spp * bg5::BK;
    g.slots += g.S[i];
    g.bins[i] = nnzs[i] > 0 ? al((int64_t)steps * (K / 128 + 1) * 4) + al(nnzs[i] * 4) : 0;
    g.bin_total += g.bins[i];
  }
  return g;
}

hipError_t launch_bwdx_g5_grouped(const BwdArgs* ls, int n, float* slots, unsigned char* bins, hipStream_t stream) {
  if (n < 1 || n > kMaxSegments) return hipErrorInvalidValue;
  int Ns[kMaxSegments];
  int64_t nnzs[kMaxSegments];
  for (int i = 0; i < n; ++i) {
    Ns[i] = ls[i].N;
    nnzs[i] = ls[i].nnz;
  }
  const int M = ls[0].M, K = ls[0].K;
  const BwdG5Group p = bwdx_g5_group_plan(M, K, Ns, nnzs, n);
  BwdG5Args g = {};
  g.out = slots;
  g.slot_stride = (int64_t)M * K;
  g.M = M;
  g.K = K;
  g.tiles_m = (M + bg5::BM - 1) / bg5::BM;
  g.tiles_k = (K + bg5::BN - 1) / bg5::BN;
  g.nseg = n;
  const int64_t tiles = (int64_t)g.tiles_m * g.tiles_k;
  int64_t wg = 0;
  int slot = 0;
  for (int i = 0; i < n; ++i) {
    const hipError_t e = g5_segment(ls[i], p.R[i], K / 128, bins, g.seg[i], stream);
    if (e != hipSuccess) return e;
    bins += p.bins[i];
    if (wg > INT_MAX) return hipErrorInvalidConfiguration;
    g.seg[i].wg0 = (int)wg;
    g.seg[i].slot0 = slot;
    wg += tiles * p.S[i];
    slot += p.S[i];
  }
  for (int i = n; i < kMaxSegments; ++i) g.seg[i] = g.seg[0];
  return launch_g5(g, wg, stream);
}

}  // namespace hxq
