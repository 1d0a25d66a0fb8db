// Decode GEMV for one to four token rows, u8 and pk12, one or several layers
// per launch.
//
// y[m][n] = sum_k (C[idx[n][k]] + S[n][k]) x[m][k] + b[n]  (model cards, "What
// is HelixCode?"; HXQ whitepaper, "Method", sidecar outlier correction).  The
// weight is never formed: each index becomes its codebook value in a register
// right before the multiply.  A launch may carry several layers that read the
// same x (the HXQ whitepaper keeps one codebook per tensor, so each layer
// brings its own codebook, indices, sidecar, bias and output).
//
// One 512-thread workgroup per CU owns a contiguous range of output rows of
// one layer.  Its LDS holds, for the whole launch:
//   - the codebook: u8 as 64 copies with a 256-byte stride per entry (copy j
//     of entry e at byte e*256 + 4j, so lane j only ever touches bank j), pk12
//     as the 4096 pairs (8 bytes each);
//   - the token rows of x, zero-padded to whole K slices;
//   - one partial sum per (row, K slice, token), the block's sidecar triplets
//     and per-row ranges into them.
// Work unit = one row x one K slice (64 lanes x CPL chunks of 16 inputs),
// numbered row-major.  Waves take units from a counter in LDS, D-1 ahead of
// the one they compute, so waves that are served faster take more; a wave's x
// slice stays in registers and is re-read from LDS only when the slice
// changes, and the codebook gather is the only per-weight LDS access.
//
// Everything a block needs besides the index stream (codebook, x, bias, the
// first sidecar probe) is requested before the first barrier, together with
// the first D-1 index units of each wave, so the block pays one memory round
// trip before it streams.  Wave 7 then resolves the block's sidecar range and
// stages its triplets while the others stream, and joins the stream after.
// After the second barrier one thread per row adds its partials in slice
// order, its sidecar terms in stored order and the bias, and writes y: the
// per-row arithmetic does not depend on which wave computed what, so results
// are bit-identical from run to run.
//
// Every wave executes the prologue, and a CU issues about one vector and one
// scalar instruction per cycle over all its waves: hence 8 waves with deep
// rings rather than 16 shallow ones, and no divisions or 64-bit index
// arithmetic per wave where a precomputed value or a 32-bit offset will do.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace dec {

constexpr int THREADS = 512;
constexpr int WAVES = THREADS / kWave;
constexpr int SW = WAVES - 1;        // streaming waves 0 .. SW-1
constexpr int HELPER = WAVES - 1;    // the sidecar wave
constexpr int SIDE_CAP = 512;        // triplets staged per pass
constexpr int LDS_LIMIT = 160 * 1024;
// s_waitcnt immediate (gfx9 layout: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]) that waits for LDS and scalar memory only
constexpr int kLgkmOnly = 0xc07f;

struct Lay {
  int xs, part, scol, sdl, rs, re, misc, total;
};

__host__ __device__ inline int a16(int v) { return (v + 15) & ~15; }

// Dynamic LDS layout.  kp: padded row length of x in elements; xb: bytes per
// x element; rows_cap: most rows any block owns; S: K slices.
__host__ __device__ inline Lay layout(int MT, int xb, int kp, int rows_cap, int S) {
  Lay L;
  L.xs = 0;
  L.part = a16(MT * kp * xb);
  L.scol = L.part + a16(rows_cap * S * MT * 4);
  L.sdl = L.scol + SIDE_CAP * 4;
  L.rs = L.sdl + SIDE_CAP * 4;
  L.re = L.rs + a16(rows_cap * 4);
  L.misc = L.re + a16(rows_cap * 4);  // [0] staged triplet count, [1] unit counter, [4..5] int64 first triplet
  L.total = L.misc + 32;
  return L;
}

}  // namespace dec

template <bool PK12, int CPL>
struct UnitBuf {
  uint32_t w[CPL][PK12 ? 3 : 4];
};

// Index loads of one unit: chunk (s * CPL + c) * 64 + lane of the row at
// `rowp` (wave-uniform).  Chunks past the row's end re-read its last chunk
// (their x is zero), so the loads are unconditional and the compiler's wait
// counts stay exact.
template <bool PK12, int CPL>
__device__ __forceinline__ void load_unit(UnitBuf<PK12, CPL>& u, const uint8_t* rowp, int s, int lane,
                                          int kchunks) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint32_t kc = (uint32_t)min((s * CPL + c) * kWave + lane, kchunks - 1);
    const uint8_t* p = rowp + kc * (PK12 ? 12u : 16u);
    if (PK12) {
      const uint3 v = *reinterpret_cast<const uint3*>(p);
      u.w[c][0] = v.x;
      u.w[c][1] = v.y;
      u.w[c][2] = v.z;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      u.w[c][0] = v.x;
      u.w[c][1] = v.y;
      u.w[c][2] = v.z;
      u.w[c][3] = v.w;
    }
  }
}

// x in LDS, chunk-interleaved so that the 64 lanes of a wave (consecutive
// chunks of 16 inputs) read consecutive 16-byte pieces: a chunk is XP pieces
// of 16 bytes (XP = 4 for fp32, 2 for bf16), and piece j of chunk kc of token
// row m sits at piece index (m * XP + j) * kcp + kc, kcp = chunks per padded
// row.  Pieces past K are zero.
template <bool XBF>
__host__ __device__ constexpr int x_pieces_per_chunk() {
  return XBF ? 2 : 4;
}

template <bool XBF>
__device__ __forceinline__ int x_piece_slot(int m, int piece, int kcp) {
  constexpr int XP = x_pieces_per_chunk<XBF>();
  return (m * XP + piece % XP) * kcp + piece / XP;
}

template <bool XBF>
__device__ __forceinline__ float x_elem(const unsigned char* xs, int m, int k, int kcp) {
  constexpr int PER = XBF ? 8 : 4;  // elements per piece
  const int off = x_piece_slot<XBF>(m, k / PER, kcp) * 16 + (k % PER) * (XBF ? 2 : 4);
  return XBF ? bf16_to_f32(*reinterpret_cast<const uint16_t*>(xs + off)) : *reinterpret_cast<const float*>(xs + off);
}

// The lane's inputs of slice s (CPL chunks of 16) for each token row, widened
// to fp32.
template <int MT, int CPL, bool XBF>
__device__ __forceinline__ void load_x_slice(float (&xr)[MT][CPL][16], const unsigned char* xs, int kcp, int s,
                                             int lane) {
  constexpr int XP = x_pieces_per_chunk<XBF>();
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int kc = (s * CPL + c) * kWave + lane;
#pragma unroll
      for (int jp = 0; jp < XP; ++jp) {
        const u32x4 v = reinterpret_cast<const u32x4*>(xs)[(m * XP + jp) * kcp + kc];
        if (XBF) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            xr[m][c][8 * jp + 2 * t] = bf16_to_f32(v[t] & 0xffffu);
            xr[m][c][8 * jp + 2 * t + 1] = bf16_to_f32(v[t] >> 16);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) xr[m][c][4 * jp + t] = __uint_as_float(v[t]);
        }
      }
    }
}

// acc[m] += sum over the unit's 16 * CPL weights of w * x[m].
template <bool PK12, int CPL, int MT>
__device__ __forceinline__ void compute_unit(const UnitBuf<PK12, CPL>& u, const float (&xr)[MT][CPL][16],
                                             float (&acc)[MT], const unsigned char* cbs, uint32_t lane4) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float wv[16];
    if (PK12) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // the d-th 3-byte group of the 12 loaded bytes: two 12-bit pair indices
        const uint32_t g = d == 0   ? u.w[c][0]
                           : d == 1 ? __builtin_amdgcn_alignbit(u.w[c][1], u.w[c][0], 24)
                           : d == 2 ? __builtin_amdgcn_alignbit(u.w[c][2], u.w[c][1], 16)
                                    : u.w[c][2] >> 8;
        const float2 ca = lds_load<float2>((g << 3) & 0x7ff8u, cbs);
        const float2 cb = lds_load<float2>((g >> 9) & 0x7ff8u, cbs);
        wv[4 * d + 0] = ca.x;
        wv[4 * d + 1] = ca.y;
        wv[4 * d + 2] = cb.x;
        wv[4 * d + 3] = cb.y;
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t wd = u.w[c][d];
        wv[4 * d + 0] = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
        wv[4 * d + 1] = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
        wv[4 * d + 2] = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
        wv[4 * d + 3] = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float a = acc[m];
#pragma unroll
      for (int j = 0; j < 16; ++j) a = fmaf(wv[j], xr[m][c][j], a);
      acc[m] = a;
    }
  }
}

// Lane 63 receives the sum over the 64 lanes (DPP only; other lanes hold
// partial sums).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f<0xb1>(v);
  v += dpp_f<0x4e>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  v += dpp_f<0x142, 0xa>(v);
  v += dpp_f<0x143, 0xc>(v);
  return v;
}

template <bool PK12, int CPL, int MT, bool XBF, int D, int XPR>
__global__ __launch_bounds__(dec::THREADS, 1) void decode_gemv(DecodeArgs a) {
  using namespace dec;
  // static array: its LDS address is a constant, so each gather's address is
  // the byte permute alone
  __shared__ __align__(16) unsigned char cbs[PK12 ? 4096 * 8 : 256 * 256];
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lane4 = (uint32_t)lane << 2;

  // Launch constants: requested together and waited for once (the empty asm
  // uses them all, so the compiler cannot defer each load to its first use
  // and wait for it there).
  const int G = a.grid;
  int wg0[kMaxSegments];
#pragma unroll
  for (int i = 0; i < kMaxSegments; ++i) wg0[i] = a.wg0[i];
  const int M = a.M, K = a.K, S = a.S, rows_cap = a.rows_cap;
  const void* xg = a.x;
  asm volatile("" ::"s"(G), "s"(wg0[1]), "s"(wg0[2]), "s"(wg0[3]), "s"(wg0[4]), "s"(wg0[5]), "s"(wg0[6]),
               "s"(wg0[7]), "s"(M), "s"(K), "s"(S), "s"(rows_cap), "s"(xg));
  // Blocks are dealt to the 8 XCDs round-robin; renumber them so that each
  // XCD takes a contiguous run of rows (its L2 then holds one region of the
  // sidecar arrays instead of eight).
  const int b = (G & 7) == 0 ? (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  // The layer, found without branches, then its descriptor in one request.
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i) si += b >= wg0[i] ? 1 : 0;
  const DecodeSeg sg = a.seg[si];
  asm volatile("" ::"s"(sg.codebook), "s"(sg.indices), "s"(sg.sc_rows), "s"(sg.sc_cols), "s"(sg.sc_deltas),
               "s"(sg.nnz), "s"(sg.bias), "s"(sg.y), "s"(sg.N), "s"(sg.rows_q), "s"(sg.rows_r),
               "s"(sg.side_per_row));
  int w0i = 0;
#pragma unroll
  for (int i = 0; i < kMaxSegments; ++i) w0i = i == si ? wg0[i] : w0i;
  const int j = b - w0i;
  const int r0 = j * sg.rows_q + (j < sg.rows_r ? j : sg.rows_r);
  const int r1 = r0 + sg.rows_q + (j < sg.rows_r ? 1 : 0);
  const int nrows = r1 - r0;

  const int kchunks = K >> 4;
  const int kp = S * CPL * kWave * 16;
  constexpr int XB = XBF ? 2 : 4;
  constexpr int CB = PK12 ? 12 : 16;  // index bytes per chunk of 16 weights
  const int64_t row_bytes = PK12 ? (int64_t)3 * (K >> 2) : (int64_t)K;
  const Lay Lo = layout(MT, XB, kp, rows_cap, S);
  unsigned char* xs = smem + Lo.xs;
  float* part = reinterpret_cast<float*>(smem + Lo.part);
  int* scol = reinterpret_cast<int*>(smem + Lo.scol);
  float* sdl = reinterpret_cast<float*>(smem + Lo.sdl);
  int* rs = reinterpret_cast<int*>(smem + Lo.rs);
  int* re = reinterpret_cast<int*>(smem + Lo.re);
  int* misc = reinterpret_cast<int*>(smem + Lo.misc);
  const bool has_side = sg.nnz > 0;
  const bool helper = wave == HELPER;
  const int mrows = M < MT ? M : MT;

  // Unit u = (row u / S, slice u % S), numbered row-major, so consecutive
  // units are consecutive pieces of one row in memory.  Before
  // the first barrier wave w requests its P0 "static" units w + SW * q; after
  // it every wave (the helper once its sidecar work is done) claims further
  // units from a counter in LDS, so waves that are served faster take more.
  const int units = nrows * S;
  const float inv_s = 1.0f / (float)S;
  auto row_of = [&](int u) {  // u / S; exact since u < 2^22 and S < 2^10
    return __builtin_amdgcn_readfirstlane((int)(((float)u + 0.5f) * inv_s));
  };
  const uint8_t* rows_base = sg.indices + (int64_t)r0 * row_bytes;
  // Lane byte offsets of the chunks of one K slice (the slice of the units
  // being requested); chunks past the row's end re-read its last chunk, whose
  // inputs are zero.  A request past the end of the wave's run re-reads a
  // unit of the first row with these offsets.
  uint32_t loff[CPL];
  auto set_loff = [&](int s) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) loff[c] = (uint32_t)min((s * CPL + c) * kWave + lane, kchunks - 1) * CB;
  };
  auto load_unit = [&](UnitBuf<PK12, CPL>& u, const uint8_t* rowp) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint8_t* p = rowp + loff[c];
      if (PK12) {
        const uint3 v = *reinterpret_cast<const uint3*>(p);
        u.w[c][0] = v.x;
        u.w[c][1] = v.y;
        u.w[c][2] = v.z;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        u.w[c][0] = v.x;
        u.w[c][1] = v.y;
        u.w[c][2] = v.z;
        u.w[c][3] = v.w;
      }
    }
  };

  // the ring: slot q holds unit us[q] * nrows + ur[q] when us[q] >= 0
  UnitBuf<PK12, CPL> ring[D];
  int us[D], ur[D];
#pragma unroll
  for (int q = 0; q < D; ++q) us[q] = -1, ur[q] = 0;
  int ls = -1;  // slice of loff
  auto request = [&](int q, int u) {
    // loads unit u (or, past the last unit, a valid stand-in) into slot q
    const bool real = u < units;
    const int r = real ? row_of(u) : 0;
    const int sl = real ? u - r * S : (ls < 0 ? 0 : ls);
    if (sl != ls) {
      ls = sl;
      set_loff(sl);
    }
    load_unit(ring[q], rows_base + (int64_t)r * row_bytes);
    us[q] = real ? sl : -1;
    ur[q] = r;
  };
  constexpr int P0 = D > 3 ? 2 : D - 1;  // units per wave requested before the first barrier
  // ---- prologue.  The first data every wave waits for is its first index
  // units, so those are requested first (the helper requests its sidecar
  // probe instead), then the codebook and x pieces for the LDS copies, which
  // land right behind them.  The helper runs at raised issue priority
  // throughout: it is the youngest wave on its SIMD and would otherwise only
  // issue when the streaming waves stall.
  WindowProbe w0, w1;
  if (helper) {
    __builtin_amdgcn_s_setprio(3);
    if (has_side) {
      window_issue(w0, sg.sc_rows, sg.nnz, (int64_t)((float)r0 * sg.side_per_row));
      window_issue(w1, sg.sc_rows, sg.nnz, (int64_t)((float)r1 * sg.side_per_row));
    }
  } else {
#pragma unroll
    for (int q = 0; q < P0; ++q) request(q, wave + SW * q);
  }
  constexpr int CBV = PK12 ? 4096 * 8 / 16 / THREADS : 1;  // 16-byte codebook pieces per thread
  u32x4 cbv[CBV];
  float cb1 = 0.f;
  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) cbv[i] = static_cast<const u32x4*>(sg.codebook)[tid + i * THREADS];
  } else {
    cb1 = static_cast<const float*>(sg.codebook)[wave * 32 + (lane >> 1)];
  }
  // x: XPR 16-byte pieces of each padded row per thread; reads clamped into
  // the row, pieces past the data stored as zero
  const int row_pieces = kp * XB / 16;
  const int real_pieces = K * XB / 16;
  u32x4 xv[MT][XPR];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < XPR; ++i) {
      const int q = min(tid + i * THREADS, real_pieces - 1);
      const int mm = m < M ? m : M - 1;
      if (i * THREADS < row_pieces)  // block-uniform
        xv[m][i] = static_cast<const u32x4*>(xg)[(int64_t)mm * real_pieces + q];
    }
  const float bias_v = (sg.bias != nullptr && tid < nrows) ? sg.bias[r0 + tid] : 0.f;
  __builtin_amdgcn_sched_barrier(0);

  if (PK12) {
#pragma unroll
    for (int i = 0; i < CBV; ++i) reinterpret_cast<u32x4*>(cbs)[tid + i * THREADS] = cbv[i];
  } else {
    // entry e, copy c at byte e * 256 + 4 c; each lane stores 8 of the 16
    // four-copy slots of its entry, rotated so one store spreads over the banks
    const int e = wave * 32 + (lane >> 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = ((lane & 1) * 8 + i + (lane >> 1)) & 15;
      *reinterpret_cast<float4*>(cbs + e * 256 + slot * 16) = make_float4(cb1, cb1, cb1, cb1);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < XPR; ++i) {
      const int q = tid + i * THREADS;
      if (i * THREADS < row_pieces && q < row_pieces)
        reinterpret_cast<u32x4*>(xs)[x_piece_slot<XBF>(m, q, kp / 16)] =
            (m < M && q < real_pieces) ? xv[m][i] : u32x4{0, 0, 0, 0};
    }
  if (tid < nrows) {
    rs[tid] = 0;
    re[tid] = 0;
  }
  if (tid == 0) misc[1] = SW * P0;  // next unit to claim
  __syncthreads();

  if (helper) {
    // ---- the block's sidecar triplets [s_lo, s_hi): the first SIDE_CAP into LDS
    int64_t s_lo = 0, s_hi = 0;
    if (has_side) {
      s_lo = window_resolve(w0, sg.sc_rows, sg.nnz, r0);
      s_hi = window_resolve(w1, sg.sc_rows, sg.nnz, r1);
      const int cnt = (int)(s_hi - s_lo > SIDE_CAP ? SIDE_CAP : s_hi - s_lo);
      constexpr int NB = SIDE_CAP / kWave;
      int tr[NB], tc[NB];
      float td[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        if (q * kWave < cnt) {
          const int i = q * kWave + lane;
          const int64_t e = s_lo + (i < cnt ? i : 0);
          tr[q] = sg.sc_rows[e];
          tc[q] = sg.sc_cols[e];
          td[q] = sg.sc_deltas[e];
        }
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int i = q * kWave + lane;
        if (q * kWave < cnt && i < cnt) {
          scol[i] = tc[q];
          sdl[i] = td[q];
        }
      }
      // run boundaries: the neighbours' rows come from registers by lane
      // shuffles (reading the other lanes' LDS stores would need a wave-level
      // fence to be ordered after them)
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        if (q * kWave < cnt) {  // uniform
          const int r = tr[q];
          const int up = __shfl_up(r, 1, kWave);    // lane - 1 (lane 0: its own)
          const int dn = __shfl_down(r, 1, kWave);  // lane + 1 (lane 63: its own)
          // the last row of the previous 64 and the first of the next
          const int prevq = q > 0 ? __shfl(tr[q > 0 ? q - 1 : 0], kWave - 1, kWave) : 0;
          const bool more = q + 1 < NB && (q + 1) * kWave < cnt;
          const int nextq = more ? __shfl(tr[q + 1 < NB ? q + 1 : q], 0, kWave) : 0;
          const int i = q * kWave + lane;
          if (i < cnt) {
            const int prev = lane == 0 ? prevq : up;
            const int next = lane == kWave - 1 ? nextq : dn;
            if (i == 0 || prev != r) rs[r - r0] = i;
            if (i + 1 == cnt || next != r) re[r - r0] = i + 1;
          }
        }
      }
    }
    if (lane == 0) {
      misc[0] = (int)(s_hi - s_lo);
      reinterpret_cast<int64_t*>(misc)[2] = s_lo;
    }
    __builtin_amdgcn_s_setprio(0);
  }
  {
    // ---- streaming (the helper joins with an empty ring): D-1 units ahead;
    // each unit's sums are reduced across the wave and lane 63 writes the
    // (row, slice) partial
    int* ctr = misc + 1;
    auto claim = [&]() {
      int u = 0;
      if (lane == 0) u = __hip_atomic_fetch_add((lds_int*)ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return __builtin_amdgcn_readfirstlane(u);
    };
    // fill the ring to D-1 units (the helper's is still empty)
#pragma unroll
    for (int q = 0; q < D - 1; ++q)
      if (q >= P0 || helper) request(q, claim());
    float xr[MT][CPL][16];
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    int x_s = -1;
    int live = 0;  // real units in the ring
#pragma unroll
    for (int q = 0; q < D - 1; ++q) live += us[q] >= 0 ? 1 : 0;
    while (live > 0) {
#pragma unroll
      for (int q = 0; q < D; ++q) {
        const int qn = (q + D - 1) % D;
        request(qn, claim());
        live += us[qn] >= 0 ? 1 : 0;
        if (us[q] >= 0) {
          if (us[q] != x_s) {
            x_s = us[q];
            load_x_slice<MT, CPL, XBF>(xr, xs, kp / 16, x_s, lane);
          }
          compute_unit<PK12, CPL, MT>(ring[q], xr, acc, cbs, lane4);
          float t[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            t[m] = wave_sum_to_lane63(acc[m]);
            acc[m] = 0.f;
          }
          if (lane == kWave - 1) {
            float* dst = part + (ur[q] * S + us[q]) * MT;
#pragma unroll
            for (int m = 0; m < MT; ++m) dst[m] = t[m];
          }
          us[q] = -1;
          live -= 1;
        }
      }
    }
  }
  __syncthreads();

  // ---- one thread per row: partials in slice order, sidecar terms in order, bias
  float out[MT];
  if (tid < nrows) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = 0.f;
      for (int s = 0; s < S; ++s) v += part[(tid * S + s) * MT + m];
      out[m] = v;
    }
  }
  auto add_side = [&]() {
    if (tid < nrows) {
      for (int i = rs[tid]; i < re[tid]; ++i) {
        const float d = sdl[i];
        const int c = scol[i];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float xv1 = x_elem<XBF>(xs, m, c, kp / 16);
          out[m] = fmaf(d, xv1, out[m]);
        }
      }
    }
  };
  add_side();
  const int s_cnt = misc[0];
  if (has_side && s_cnt > SIDE_CAP) {
    // more triplets than one staging pass holds: the rest in further passes,
    // each row's terms still in stored order
    const int64_t s_lo = reinterpret_cast<const int64_t*>(misc)[2];
    const int64_t s_hi = s_lo + s_cnt;
    for (int64_t e0 = s_lo + SIDE_CAP; e0 < s_hi; e0 += SIDE_CAP) {
      __syncthreads();
      if (tid < nrows) {
        rs[tid] = 0;
        re[tid] = 0;
      }
      __syncthreads();
      const int64_t e = e0 + tid;
      const int64_t e_end = e0 + SIDE_CAP < s_hi ? e0 + SIDE_CAP : s_hi;
      if (tid < SIDE_CAP && e < e_end) {
        const int r = sg.sc_rows[e];
        scol[tid] = sg.sc_cols[e];
        sdl[tid] = sg.sc_deltas[e];
        if (e == e0 || sg.sc_rows[e - 1] != r) rs[r - r0] = tid;
        if (e + 1 == e_end || sg.sc_rows[e + 1] != r) re[r - r0] = tid + 1;
      }
      __syncthreads();
      add_side();
    }
  }
  if (tid < nrows) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < mrows) sg.y[(int64_t)m * sg.N + r0 + tid] = out[m] + bias_v;
  }
}

// ------------------------------------------------------------------ launch

namespace {

template <bool PK12, int CPL, int MT, bool XBF, int D, int XPR>
hipError_t launch_cfg(const DecodeArgs& a, int grid, int lds, hipStream_t stream) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_gemv<PK12, CPL, MT, XBF, D, XPR>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, dec::LDS_LIMIT - (PK12 ? 4096 * 8 : 256 * 256));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((decode_gemv<PK12, CPL, MT, XBF, D, XPR>), dim3((unsigned)grid), dim3(dec::THREADS), lds, stream,
                     a);
  return hipGetLastError();
}

template <bool PK12, int CPL, int MT, int D, int XPR>
hipError_t launch_xdt(const DecodeArgs& a, bool xbf, int grid, int lds, hipStream_t stream) {
  return xbf ? launch_cfg<PK12, CPL, MT, true, D, XPR>(a, grid, lds, stream)
             : launch_cfg<PK12, CPL, MT, false, D, XPR>(a, grid, lds, stream);
}

// Tile shapes by token rows: CPL chunks per lane per unit, ring depth D, and
// XPR 16-byte x pieces per thread and token row (the longest padded x row a
// launch takes is XPR * THREADS * 16 bytes).
constexpr int kCpl[4] = {2, 1, 1, 4};
constexpr int kDepth[4] = {6, 8, 6, 4};
constexpr int kXpr[4] = {6, 11, 2, 6};

struct Plan {
  int MT, ti, CPL, S, rows_cap, lds, grid;
};

// Chooses the tile shape and deals the CUs to the layers in proportion to
// their index bytes.  Returns false when the call does not fit this kernel.
bool plan(const DecodeSeg* segs, int nseg, bool pk12, bool xbf, int M, int K, int cus, DecodeArgs& a,
          Plan& p) {
  if (M < 1 || M > 4 || K < 16 || nseg < 1 || nseg > kMaxSegments) return false;
  p.MT = M == 1 ? 1 : M == 2 ? 2 : 4;
  const int ti = p.MT == 1 ? (K > 4096 ? 3 : 0) : p.MT == 2 ? 1 : 2;
  p.ti = ti;
  p.CPL = kCpl[ti];
  const int kchunks = K / 16;
  p.S = (kchunks + p.CPL * kWave - 1) / (p.CPL * kWave);
  const int kp = p.S * p.CPL * kWave * 16;
  const int xb = xbf ? 2 : 4;
  if ((int64_t)kp * xb / 16 > (int64_t)kXpr[ti] * dec::THREADS) return false;
  const int64_t row_bytes = pk12 ? 3 * (int64_t)(K / 4) : K;
  double total = 0;
  for (int i = 0; i < nseg; ++i) total += (double)segs[i].N * row_bytes;
  // workgroups per layer: proportional to its index bytes, at least one and
  // enough for one thread per row in the epilogue, in total the CU count
  // when that is possible (one workgroup fits a CU; more would queue)
  int64_t w[kMaxSegments];
  double frac[kMaxSegments];
  int64_t used = 0;
  for (int i = 0; i < nseg; ++i) {
    const int64_t N = segs[i].N;
    const double share = (double)cus * (double)N * (double)row_bytes / total;
    int64_t wi = (int64_t)share;
    const int64_t need = (N + dec::THREADS - 1) / dec::THREADS;
    if (wi < need) wi = need;
    if (wi < 1) wi = 1;
    if (wi > N) wi = N;
    w[i] = wi;
    frac[i] = share - (double)wi;
    used += wi;
  }
  while (used < cus) {  // hand out the rest by largest remaining share
    int best = -1;
    for (int i = 0; i < nseg; ++i)
      if (w[i] < segs[i].N && (best < 0 || frac[i] > frac[best])) best = i;
    if (best < 0) break;
    w[best] += 1;
    frac[best] -= 1.0;
    used += 1;
  }
  if (used > INT_MAX / 2) return false;
  int wg = 0, rows_cap = 1;
  for (int i = 0; i < nseg; ++i) {
    const int64_t N = segs[i].N;
    a.seg[i] = segs[i];
    a.seg[i].rows_q = (int)(N / w[i]);
    a.seg[i].rows_r = (int)(N % w[i]);
    a.seg[i].side_per_row = (float)((double)segs[i].nnz / (double)N);
    a.wg0[i] = wg;
    wg += (int)w[i];
    const int rc = (int)((N + w[i] - 1) / w[i]);
    if (rc > rows_cap) rows_cap = rc;
  }
  for (int i = nseg; i < kMaxSegments; ++i) {
    a.seg[i] = a.seg[0];
    a.wg0[i] = INT_MAX;
  }
  a.grid = wg;
  a.M = M;
  a.K = K;
  a.S = p.S;
  a.rows_cap = rows_cap;
  p.rows_cap = rows_cap;
  p.grid = wg;
  const int cb = pk12 ? 4096 * 8 : 256 * 256;
  const int64_t lds = dec::layout(p.MT, xb, kp, rows_cap, p.S).total;
  if (lds + cb > dec::LDS_LIMIT) return false;
  p.lds = (int)lds;
  return true;
}

}  // namespace

static bool launch_decode_plan(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                               hipStream_t stream, hipError_t& err);

// One token row with K <= 4096 goes to the lean kernel (hxq_decode1.hip)
// layer by layer as a single-layer call would: one launch when every layer
// takes it and they fit together, else one launch per layer.
bool launch_decode(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                   hipStream_t stream, hipError_t& err) {
  if (M == 1 && nseg >= 1 && nseg <= kMaxSegments) {
    int n1 = 0;
    for (int i = 0; i < nseg; ++i) n1 += decode1_takes(segs[i], pk12, xbf, M, K, x) ? 1 : 0;
    if (n1 == nseg) {
      if (launch_decode1(segs, nseg, pk12, x, xbf, M, K, stream, err)) return true;
      for (int i = 0; i < nseg; ++i) {
        if (!launch_decode1(&segs[i], 1, pk12, x, xbf, M, K, stream, err)) return false;
        if (err != hipSuccess) return true;
      }
      return true;
    }
    if (n1 > 0) {
      // mixed: every layer on its own kernel, checked before anything is launched
      DecodeArgs a;
      Plan p;
      for (int i = 0; i < nseg; ++i)
        if (!decode1_takes(segs[i], pk12, xbf, M, K, x) && !plan(&segs[i], 1, pk12, xbf, M, K, device_cu_count(), a, p))
          return false;
      for (int i = 0; i < nseg; ++i) {
        const bool ok = decode1_takes(segs[i], pk12, xbf, M, K, x)
                            ? launch_decode1(&segs[i], 1, pk12, x, xbf, M, K, stream, err)
                            : launch_decode_plan(&segs[i], 1, pk12, x, xbf, M, K, stream, err);
        if (!ok || err != hipSuccess) return true;
      }
      return true;
    }
  }
  return launch_decode_plan(segs, nseg, pk12, x, xbf, M, K, stream, err);
}

static bool launch_decode_plan(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                               hipStream_t stream, hipError_t& err) {
  DecodeArgs a;
  Plan p;
  if (!plan(segs, nseg, pk12, xbf, M, K, device_cu_count(), a, p)) return false;
  a.x = x;
  if (pk12) {
    if (p.ti == 3) err = launch_xdt<true, kCpl[3], 1, kDepth[3], kXpr[3]>(a, xbf, p.grid, p.lds, stream);
    else if (p.MT == 1) err = launch_xdt<true, kCpl[0], 1, kDepth[0], kXpr[0]>(a, xbf, p.grid, p.lds, stream);
    else if (p.MT == 2) err = launch_xdt<true, kCpl[1], 2, kDepth[1], kXpr[1]>(a, xbf, p.grid, p.lds, stream);
    else err = launch_xdt<true, kCpl[2], 4, kDepth[2], kXpr[2]>(a, xbf, p.grid, p.lds, stream);
  } else {
    if (p.ti == 3) err = launch_xdt<false, kCpl[3], 1, kDepth[3], kXpr[3]>(a, xbf, p.grid, p.lds, stream);
    else if (p.MT == 1) err = launch_xdt<false, kCpl[0], 1, kDepth[0], kXpr[0]>(a, xbf, p.grid, p.lds, stream);
    else if (p.MT == 2) err = launch_xdt<false, kCpl[1], 2, kDepth[1], kXpr[1]>(a, xbf, p.grid, p.lds, stream);
    else err = launch_xdt<false, kCpl[2], 4, kDepth[2], kXpr[2]>(a, xbf, p.grid, p.lds, stream);
  }
  return true;
}

bool decode_fits(const DecodeSeg* segs, int nseg, bool pk12, bool xbf, int M, int K) {
  DecodeArgs a;
  Plan p;
  return plan(segs, nseg, pk12, xbf, M, K, 256, a, p);
}

// More tokens than one pass takes: consecutive groups of G rows, G the
// largest of 4, 2, 1 whose group (and remainder) fits the kernel.  Rows
// m0 .. m0 + G - 1 of x and of every y are contiguous, so a group is the same
// call on x + m0 K and y + m0 N; each group streams the indices again.
bool launch_decode_chunked(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                           hipStream_t stream, hipError_t& err) {
  if (nseg < 1 || nseg > kMaxSegments || M < 1) return false;
  int G = 0;
  for (int c : {4, 2, 1}) {
    const int g = M < c ? M : c;
    if (decode_fits(segs, nseg, pk12, xbf, g, K) && (M % g == 0 || decode_fits(segs, nseg, pk12, xbf, M % g, K))) {
      G = g;
      break;
    }
  }
  if (G == 0) return false;
  const size_t xrow = (size_t)K * (xbf ? 2 : 4);
  for (int m0 = 0; m0 < M; m0 += G) {
    const int mc = M - m0 < G ? M - m0 : G;
    DecodeSeg cs[kMaxSegments];
    for (int i = 0; i < nseg; ++i) {
      cs[i] = segs[i];
      cs[i].y = segs[i].y + (size_t)m0 * segs[i].N;
    }
    hipError_t e = hipSuccess;
    if (!launch_decode(cs, nseg, pk12, static_cast<const char*>(x) + (size_t)m0 * xrow, xbf, mc, K, stream, e))
      return false;  // not reached: both group sizes were checked above
    if (e != hipSuccess) {
      err = e;
      return true;
    }
  }
  err = hipSuccess;
  return true;
}

}  // namespace hxq
