// Workgroup-cooperative fp32 GEMV for small token counts (u8 and pk12).
//
// y[m][n] = sum_k (C[idx[n][k]] + S[n][k]) x[m][k] + b[n]  (model cards, "What
// is HelixCode?"; HXQ whitepaper, "Method", sidecar outlier correction), with
// the weight never formed: every index becomes its codebook value in a
// register right before the multiply.
//
// One 512-thread workgroup per CU owns a contiguous range of output rows.
// LDS holds, for the whole kernel:
//   - the codebook: u8 as 64 copies with a 256-byte stride per entry (copy j of
//     entry e at byte e*256 + 4j, so lane j always reads bank j), pk12 as the
//     4096 pairs (8 bytes each);
//   - the MT token rows of x being processed, converted to fp32.
// Rows are processed in blocks.  A block is cut into units of R rows x one K
// slice (64 lanes x CPL chunks of 16 inputs); the 16 waves take the units
// round-robin and keep D units of index loads in flight.  Every global load
// is issued unconditionally (out-of-range reads are redirected to valid bytes
// and zeroed), so the compiler's wait counts stay exact and the index stream
// never stalls on a wait meant for something else.  Each unit's per-row
// sums are reduced across the wave (DPP) into an LDS table of partials; after
// a barrier one thread per row adds its partials in slice order, the row's
// sidecar triplets in their stored order (staged through LDS, looked up with
// one 1024-entry window read at the start of the block) and the bias, and
// writes y.  Results are bit-identical from run to run.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace wgv {
constexpr int THREADS = 512;
constexpr int WAVES = THREADS / kWave;
constexpr int SIDE_CAP = 256;  // sidecar triplets staged by the helper wave per block
constexpr int XMAX = 48 * 1024;  // bytes of x rows staged in LDS

struct Layout {
  int cb, xs, part, srow, scol, sd, rstart, rend, misc, total;
};

__host__ __device__ inline int align16(int v) { return (v + 15) & ~15; }

__host__ __device__ inline Layout layout(bool pk12, bool xbf, int MT, int kcp, int rb_rows, int slices) {
  Layout L;  // dynamic LDS, after the static codebook array
  L.cb = 0;
  L.xs = 0;
  L.part = L.xs + align16(MT * kcp * 16 * (xbf ? 2 : 4));
  L.srow = L.part + align16(rb_rows * slices * MT * 4);
  L.scol = L.srow + THREADS * 4;  // the overflow pass stages one triplet per thread
  L.sd = L.scol + THREADS * 4;
  L.rstart = L.sd + THREADS * 4;
  L.rend = L.rstart + align16(rb_rows * 4);
  L.misc = L.rend + align16(rb_rows * 4);
  L.total = L.misc + 64;
  return L;
}
}  // namespace wgv

template <bool PK12, int R, int CPL>
struct Unit {
  uint32_t w[R][CPL][PK12 ? 3 : 4];
};

// Index loads of one unit (one row, CPL chunks per lane).  `rowp` is the
// wave-uniform row start, so each load is a scalar base plus a 32-bit lane
// offset.  Always issued: a chunk past K re-reads the row's last chunk (its x
// is zero), so nothing is masked here -- a select on the loaded data would
// wait for it -- and the number of loads in flight is the same on every path.
template <bool PK12, int R, int CPL>
__device__ __forceinline__ void unit_load(Unit<PK12, R, CPL>& u, const uint8_t* rowp, int s, int lane,
                                          int kchunks) {
  static_assert(R == 1, "one row per unit");
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint32_t kc = (uint32_t)min((s * CPL + c) * kWave + lane, kchunks - 1);
    const uint8_t* p = rowp + kc * (PK12 ? 12u : 16u);
    if (PK12) {
      const uint3 v = *reinterpret_cast<const uint3*>(p);
      u.w[0][c][0] = v.x;
      u.w[0][c][1] = v.y;
      u.w[0][c][2] = v.z;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      u.w[0][c][0] = v.x;
      u.w[0][c][1] = v.y;
      u.w[0][c][2] = v.z;
      u.w[0][c][3] = v.w;
    }
  }
}

// x in LDS, "chunk-interleaved", so that the 64 lanes of a wave (consecutive
// chunks of 16 inputs) read consecutive addresses: no bank conflicts.
//   fp32: piece (m, q, kc) = inputs 16 kc + 4 q .. + 3 of token row m, 16 bytes,
//         at piece index (m * 4 + q) * kcp + kc;
//   bf16: piece (m, p, kc) = inputs 16 kc + 2 p, + 1, 4 bytes, at dword index
//         (m * 8 + p) * kcp + kc.
// kcp is the chunk count rounded up to whole K slices; the pieces past K are
// zero, so lanes past the end of a row multiply by zero without a test.
template <bool XBF>
__device__ __forceinline__ float4 xs_piece(const void* xs, int m, int q, int kc, int kcp) {
  if (XBF) {
    const uint32_t* d = static_cast<const uint32_t*>(xs);
    const uint32_t lo = d[(m * 8 + 2 * q) * kcp + kc];
    const uint32_t hi = d[(m * 8 + 2 * q + 1) * kcp + kc];
    return make_float4(bf16_to_f32(lo & 0xffffu), bf16_to_f32(lo >> 16), bf16_to_f32(hi & 0xffffu),
                       bf16_to_f32(hi >> 16));
  }
  return static_cast<const float4*>(xs)[(m * 4 + q) * kcp + kc];
}

template <bool XBF>
__device__ __forceinline__ float xs_elem(const void* xs, int m, int k, int kcp) {
  if (XBF) {
    const int dw = (m * 8 + ((k >> 1) & 7)) * kcp + (k >> 4);
    return bf16_to_f32(static_cast<const uint16_t*>(xs)[dw * 2 + (k & 1)]);
  }
  const int piece = (m * 4 + ((k >> 2) & 3)) * kcp + (k >> 4);
  return static_cast<const float*>(xs)[piece * 4 + (k & 3)];
}

template <bool PK12, int R, int CPL, int MT, bool XBF>
__device__ __forceinline__ void unit_compute(const Unit<PK12, R, CPL>& u, float (&acc)[R][MT],
                                             const unsigned char* cbs, const void* xs, int K, int s,
                                             int lane, uint32_t lane4, int kcp) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int kc = (s * CPL + c) * kWave + lane;  // < kcp
    float xv[MT][16];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = xs_piece<XBF>(xs, m, q, kc, kcp);
        xv[m][4 * q + 0] = v.x;
        xv[m][4 * q + 1] = v.y;
        xv[m][4 * q + 2] = v.z;
        xv[m][4 * q + 3] = v.w;
      }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float wv[16];
      if (PK12) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // the d-th 3-byte group of the 12 loaded bytes (upper bits unused)
          const uint32_t g = d == 0   ? u.w[r][c][0]
                             : d == 1 ? __builtin_amdgcn_alignbit(u.w[r][c][1], u.w[r][c][0], 24)
                             : d == 2 ? __builtin_amdgcn_alignbit(u.w[r][c][2], u.w[r][c][1], 16)
                                      : u.w[r][c][2] >> 8;
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
          const uint32_t wd = u.w[r][c][d];
          wv[4 * d + 0] = lds_load<float>(byte_addr256<0>(wd, lane4), cbs);
          wv[4 * d + 1] = lds_load<float>(byte_addr256<1>(wd, lane4), cbs);
          wv[4 * d + 2] = lds_load<float>(byte_addr256<2>(wd, lane4), cbs);
          wv[4 * d + 3] = lds_load<float>(byte_addr256<3>(wd, lane4), cbs);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float sacc = acc[r][m];
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc = fmaf(wv[j], xv[m][j], sacc);
        acc[r][m] = sacc;
      }
    }
  }
}

// Shared pointers into the dynamic LDS block.
struct WgLds {
  unsigned char* cbs;
  void* xs;
  float* part;
  int* srow;
  int* scol;
  float* sdl;
  int* rstart;
  int* rend;
  int* wcnt;  // per-wave window counts, [WAVES]
};

// One block of rows [rb0, rb1) for the token rows [m0, m0 + MT).  STAGE_CB /
// STAGE_X: this block also copies the codebook / the x rows into LDS.
//
// Wave 0 is a helper: it stages the codebook and x before the first barrier
// and the block's sidecar triplets after it, while waves 1.. stream the index
// units.  The unit waves issue nothing but index loads, in the same pattern
// before and inside their loop, so the compiler's wait counts stay exact and
// each wait covers only the unit about to be computed.
template <bool PK12, int R, int CPL, int MT, bool XBF, int D, bool STAGE_CB, bool STAGE_X>
__device__ __forceinline__ void wg_block(const LayerArgs& a, const WgLds& S, int slices, int64_t rb0, int64_t rb1,
                                         int m0) {
  using namespace wgv;
  constexpr int UW = WAVES - 1;  // unit waves
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: unit math stays scalar
  const bool helper = wave == 0;
  const int uw = wave - 1;
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int K = a.K;
  const int kchunks = K >> 4;
  const int kcp = slices * CPL * kWave;
  const int64_t row_bytes = PK12 ? (int64_t)3 * (K >> 2) : (int64_t)K;
  const int nrows = (int)(rb1 - rb0);
  const int units = ((nrows + R - 1) / R) * slices;
  const bool has_side = a.nnz > 0;

  // Unit u = (row u / slices, K slice u % slices).  Unit wave uw owns the
  // contiguous units [u_begin, u_end) and walks them in order: its position
  // and row pointer advance by one slice at a time, all wave-uniform.
  const int u_begin = (int)((int64_t)units * uw / UW);
  const int u_end = (int)((int64_t)units * (uw + 1) / UW);
  struct Pos {
    int u, g, s;
    const uint8_t* rowp;
  };
  auto advance = [&](Pos p) {
    p.u += 1;
    p.s += 1;
    if (p.s == slices) {
      p.s = 0;
      p.g += 1;
      p.rowp += row_bytes;
    }
    return p;
  };
  const int last = u_end > u_begin ? u_end - 1 : u_begin;
  const int last_s = last % slices;
  const uint8_t* last_rowp = a.indices + (rb0 + min(last / slices, nrows - 1)) * row_bytes;
  Unit<PK12, R, CPL> ring[D];
  auto load_unit = [&](Unit<PK12, R, CPL>& slot, const Pos& p) {
    const bool real = p.u < u_end;  // past the end: a repeat of the wave's last unit
    unit_load(slot, real ? p.rowp : last_rowp, real ? p.s : last_s, lane, kchunks);
  };
  const int g0 = u_begin / slices;
  Pos cur{u_begin, g0, u_begin % slices, a.indices + (rb0 + min(g0, nrows - 1)) * row_bytes};
  Pos nxt = cur;
  if (!helper) {
#pragma unroll
    for (int q = 0; q < D - 1; ++q) {
      load_unit(ring[q], nxt);
      nxt = advance(nxt);
    }
  } else {
    // ---- helper: codebook and x into LDS
    if (STAGE_CB) {
      if (PK12) {
        for (int c = 0; c < 32; ++c)  // 32 KB of pairs, 1 KB per instruction
          lds_dma16(static_cast<const unsigned char*>(a.codebook) + c * 1024 + lane * 16, S.cbs + c * 1024);
      } else {
        const float* cb = static_cast<const float*>(a.codebook);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = cb[lane + 64 * i];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int e = lane + 64 * i, slot = (j + lane) & 15;
            *reinterpret_cast<float4*>(S.cbs + e * 256 + slot * 16) = make_float4(v[i], v[i], v[i], v[i]);
          }
      }
    }
    if (STAGE_X) {
      // piece rows of kchunks pieces each, gathered from x 64 at a time
      constexpr int PR = XBF ? 8 : 4;   // piece rows per token row
      constexpr int PSZ = XBF ? 4 : 16;  // bytes per piece
      const int mrows = a.M - m0 < MT ? a.M - m0 : MT;
      const unsigned char* xb = static_cast<const unsigned char*>(a.x);
      unsigned char* dst = static_cast<unsigned char*>(S.xs);
      for (int mp = 0; mp < MT * PR; ++mp) {
        const int m = mp / PR, p = mp % PR;
        for (int kc0 = 0; kc0 < kcp; kc0 += kWave) {
          const int kc = kc0 + lane;
          unsigned char* d = dst + ((int64_t)mp * kcp + kc0) * PSZ;
          {
            if (m < mrows && kc < kchunks) {
              const int64_t e = (int64_t)(m0 + m) * K + (int64_t)kc * 16 + p * (16 / PR);
              if (XBF)
                lds_dma4(xb + e * 2, d);
              else
                lds_dma16(xb + e * 4, d);
            } else {
              if (XBF)
                reinterpret_cast<uint32_t*>(d)[lane] = 0u;
              else
                reinterpret_cast<uint4*>(d)[lane] = make_uint4(0, 0, 0, 0);
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // LDS copies landed
  }
  for (int i = tid; i < nrows; i += THREADS) {
    S.rstart[i] = 0;
    S.rend[i] = 0;
  }
  for (int i = tid; i < nrows * slices * MT; i += THREADS) S.part[i] = 0.f;
  __syncthreads();

  if (helper) {
    // ---- helper: the block's triplets [s_lo, s_hi) into LDS (first SIDE_CAP)
    int64_t s_lo = 0, s_hi = 0;
    if (has_side) {
      WindowProbe w0, w1;
      window_issue(w0, a.sc_rows, a.nnz, (int64_t)((double)a.nnz * (double)rb0 / (double)a.N));
      window_issue(w1, a.sc_rows, a.nnz, (int64_t)((double)a.nnz * (double)rb1 / (double)a.N));
      s_lo = window_resolve(w0, a.sc_rows, a.nnz, (int32_t)rb0);
      s_hi = window_resolve(w1, a.sc_rows, a.nnz, (int32_t)rb1);
      constexpr int NB = SIDE_CAP / kWave;
      int tr[NB], tc[NB], tp[NB], tn[NB];
      float td[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int64_t e = s_lo + b * kWave + lane;
        const bool ok = e < s_hi;
        const int64_t ec = ok ? e : s_lo;
        const int64_t ep = ok && e > s_lo ? e - 1 : ec;
        const int64_t en = ok && e + 1 < s_hi ? e + 1 : ec;
        tr[b] = ok ? a.sc_rows[ec] : INT_MAX;
        tc[b] = a.sc_cols[ec];
        td[b] = a.sc_deltas[ec];
        tp[b] = ok && e > s_lo ? a.sc_rows[ep] : INT_MIN;
        tn[b] = ok && e + 1 < s_hi ? a.sc_rows[en] : INT_MAX;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = b * kWave + lane;
        if (tr[b] != INT_MAX) {
          S.srow[i] = tr[b];
          S.scol[i] = tc[b];
          S.sdl[i] = td[b];
          if (tp[b] != tr[b]) S.rstart[tr[b] - rb0] = i;
          if (tn[b] != tr[b] || i + 1 == SIDE_CAP) S.rend[tr[b] - rb0] = i + 1;
        }
      }
    }
    if (lane == 0) {
      S.wcnt[0] = (int)(s_hi - s_lo);
      reinterpret_cast<int64_t*>(S.wcnt)[1] = s_lo;
    }
  } else {
    // ---- unit waves: D - 1 index units ahead.  A wave's units run row group
    // by row group; the sums of a group are reduced across the wave once,
    // when the wave leaves the group, into the partial slot of the first
    // slice it computed there (other slots of the table stay zero).
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
    int s_first = cur.s;
    for (int base = u_begin; base < u_end; base += D) {
#pragma unroll
      for (int q = 0; q < D; ++q) {
        load_unit(ring[(q + D - 1) % D], nxt);
        nxt = advance(nxt);
        if (cur.u < u_end) {
          unit_compute<PK12, R, CPL, MT, XBF>(ring[q], acc, S.cbs, S.xs, K, cur.s, lane, lane4, kcp);
          const Pos after = advance(cur);
          if (after.g != cur.g || after.u == u_end) {
            const int rl0 = cur.g * R;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                const float t = wave_sum_dpp(acc[r][m]);
                if (lane == r * MT + m && rl0 + r < nrows) S.part[((rl0 + r) * slices + s_first) * MT + m] = t;
                acc[r][m] = 0.f;
              }
            s_first = after.s;
          }
        }
        cur = advance(cur);
      }
    }
  }
  __syncthreads();

  // ---- one thread per row: partials in slice order, sidecar in triplet order, bias
  for (int rl = tid; rl < nrows; rl += THREADS) {
    const int64_t n = rb0 + rl;
    float out[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = 0.f;
      for (int s = 0; s < slices; ++s) v += S.part[(rl * slices + s) * MT + m];
      out[m] = v;
    }
    for (int i = S.rstart[rl]; i < S.rend[rl]; ++i) {
      const float d = S.sdl[i];
      const int c = S.scol[i];
#pragma unroll
      for (int m = 0; m < MT; ++m) out[m] = fmaf(d, xs_elem<XBF>(S.xs, m, c, kcp), out[m]);
    }
    const float b = a.bias ? a.bias[n] : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m0 + m < a.M) a.y[(int64_t)(m0 + m) * a.N + n] = out[m] + b;
  }
  // more triplets than the staging holds: applied afterwards in order, one
  // thread per row (same order as a single pass)
  const int s_cnt = S.wcnt[0];
  if (has_side && s_cnt > SIDE_CAP) {
    const int64_t s_lo = reinterpret_cast<const int64_t*>(S.wcnt)[1];
    const int64_t s_hi = s_lo + s_cnt;
    __syncthreads();
    for (int64_t e0 = s_lo + SIDE_CAP; e0 < s_hi; e0 += THREADS) {
      const int64_t e = e0 + tid;
      for (int i = tid; i < nrows; i += THREADS) {
        S.rstart[i] = 0;
        S.rend[i] = 0;
      }
      __syncthreads();
      if (e < s_hi) {
        const int r = a.sc_rows[e];
        S.srow[tid] = r;
        S.scol[tid] = a.sc_cols[e];
        S.sdl[tid] = a.sc_deltas[e];
        if (e == e0 || a.sc_rows[e - 1] != r) S.rstart[r - rb0] = tid;
        if (e + 1 == s_hi || tid + 1 == THREADS || a.sc_rows[e + 1] != r) S.rend[r - rb0] = tid + 1;
      }
      __syncthreads();
      for (int rl = tid; rl < nrows; rl += THREADS) {
        if (S.rend[rl] == S.rstart[rl]) continue;
        const int64_t n = rb0 + rl;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m0 + m >= a.M) break;
          float v = a.y[(int64_t)(m0 + m) * a.N + n];
          for (int i = S.rstart[rl]; i < S.rend[rl]; ++i)
            v = fmaf(S.sdl[i], xs_elem<XBF>(S.xs, m, S.scol[i], kcp), v);
          a.y[(int64_t)(m0 + m) * a.N + n] = v;
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();  // LDS tables are reused by the next block
}

template <bool PK12, int R, int CPL, int MT, bool XBF, int D>
__global__ __launch_bounds__(wgv::THREADS, 1) void gemv_wg(LayerArgs a, int slices, int rb_rows) {
  using namespace wgv;
  // The codebook is a static array: its LDS address is a constant, so each
  // gather's address is the byte-permute alone.
  __shared__ __align__(16) unsigned char cb_lds[PK12 ? 4096 * 8 : 256 * 256];
  extern __shared__ __align__(16) unsigned char smem[];
  const Layout Lo = layout(PK12, XBF, MT, slices * CPL * kWave, rb_rows, slices);
  WgLds S;
  S.cbs = cb_lds;
  S.xs = smem + Lo.xs;
  S.part = reinterpret_cast<float*>(smem + Lo.part);
  S.srow = reinterpret_cast<int*>(smem + Lo.srow);
  S.scol = reinterpret_cast<int*>(smem + Lo.scol);
  S.sdl = reinterpret_cast<float*>(smem + Lo.sd);
  S.rstart = reinterpret_cast<int*>(smem + Lo.rstart);
  S.rend = reinterpret_cast<int*>(smem + Lo.rend);
  S.wcnt = reinterpret_cast<int*>(smem + Lo.misc);

  const int64_t G = gridDim.x;
  const int64_t wr0 = (int64_t)blockIdx.x * a.N / G;
  const int64_t wr1 = (int64_t)(blockIdx.x + 1) * a.N / G;
  if (wr0 >= wr1) return;
  for (int64_t m0l = (int64_t)blockIdx.y * MT; m0l < a.M; m0l += (int64_t)gridDim.y * MT) {
    const int m0 = (int)m0l;
    const int64_t rb1 = wr0 + rb_rows < wr1 ? wr0 + rb_rows : wr1;
    if (m0l == (int64_t)blockIdx.y * MT)
      wg_block<PK12, R, CPL, MT, XBF, D, true, true>(a, S, slices, wr0, rb1, m0);
    else
      wg_block<PK12, R, CPL, MT, XBF, D, false, true>(a, S, slices, wr0, rb1, m0);
    for (int64_t rb0 = rb1; rb0 < wr1; rb0 += rb_rows) {
      const int64_t e1 = rb0 + rb_rows < wr1 ? rb0 + rb_rows : wr1;
      wg_block<PK12, R, CPL, MT, XBF, D, false, false>(a, S, slices, rb0, e1, m0);
    }
  }
}

// ------------------------------------------------------------------ launch

template <bool PK12, int R, int CPL, int MT, int D>
static hipError_t launch_wg_cfg(const LayerArgs& a, hipStream_t stream, int grid_x, int slices, int rb_rows,
                                int lds) {
  int64_t gy = ((int64_t)a.M + MT - 1) / MT;
  if (gy > 65535) gy = 65535;
  const dim3 grid((unsigned)grid_x, (unsigned)gy);
  if (a.x_bf16) {
    static const bool attr = ((void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_wg<PK12, R, CPL, MT, true, D>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024),
                              true);
    (void)attr;
    hipLaunchKernelGGL((gemv_wg<PK12, R, CPL, MT, true, D>), grid, dim3(wgv::THREADS), lds, stream, a, slices,
                       rb_rows);
  } else {
    static const bool attr = ((void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_wg<PK12, R, CPL, MT, false, D>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024),
                              true);
    (void)attr;
    hipLaunchKernelGGL((gemv_wg<PK12, R, CPL, MT, false, D>), grid, dim3(wgv::THREADS), lds, stream, a, slices,
                       rb_rows);
  }
  return hipGetLastError();
}

// Returns false when this kernel cannot take the call (x too large for LDS).
template <bool PK12, int R, int CPL, int MT, int D>
static bool try_wg(const LayerArgs& a, hipStream_t stream, hipError_t& err) {
  const int slices = (a.K / 16 + CPL * kWave - 1) / (CPL * kWave);
  const int cus = device_cu_count();
  int grid_x = cus;
  if ((int64_t)grid_x > a.N) grid_x = a.N;
  const int64_t rows_per_wg = ((int64_t)a.N + grid_x - 1) / grid_x;
  int rb_rows = (int)(rows_per_wg < 256 ? rows_per_wg : 256);
  constexpr int LDS_MAX = 160 * 1024;
  const int kcp = slices * CPL * kWave;
  while (rb_rows > 8 && wgv::layout(PK12, a.x_bf16, MT, kcp, rb_rows, slices).total + (PK12 ? 32768 : 65536) > LDS_MAX)
    rb_rows /= 2;
  const int lds = wgv::layout(PK12, a.x_bf16, MT, kcp, rb_rows, slices).total;
  const int64_t xbytes = (int64_t)MT * kcp * 16 * (a.x_bf16 ? 2 : 4);
  const int cb_bytes = PK12 ? 4096 * 8 : 256 * 256;
  if (lds + cb_bytes > LDS_MAX || xbytes > wgv::XMAX) return false;
  err = launch_wg_cfg<PK12, R, CPL, MT, D>(a, stream, grid_x, slices, rb_rows, lds);
  return true;
}

template <bool PK12>
static bool launch_wg_fmt(const LayerArgs& a, hipStream_t stream, hipError_t& err) {
  if (a.M == 1) return try_wg<PK12, 1, 2, 1, 5>(a, stream, err);
  if (a.M == 2) return try_wg<PK12, 1, 2, 2, 4>(a, stream, err);
  return try_wg<PK12, 1, 1, 4, 6>(a, stream, err);
}

bool launch_gemv_wg(const LayerArgs& a, bool pk12, hipStream_t stream, hipError_t& err) {
  return pk12 ? launch_wg_fmt<true>(a, stream, err) : launch_wg_fmt<false>(a, stream, err);
}

}  // namespace hxq
