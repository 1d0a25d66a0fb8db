// Input gradient of a frozen HelixLinear layer: the product with W itself.
//
//     dx[m][k] = sum_n dy[m][n] * (C[idx[n][k]] + S[n][k])
//
// The model cards ("Good to Know") keep the compressed weights frozen while
// LoRA adapters train through each HelixLinear; training through the layer
// needs the gradient of y = x W^T + b with respect to x, which is dY W.  W is
// the weight the forward uses ("What is HelixCode?"; HXQ whitepaper, "Method"
// and "2D vector quantization"), read here along its columns and never formed.
//
// bwdx_valu: the general kernel (fp32 or bf16 dy, any M, N, K).  A workgroup
// owns a column tile, a run of R rows and up to 8 tokens.  Tiles are 128
// columns (lane l holds columns 8 (l % 16) .. + 7 in one of four rows at a
// time, l / 16, so a load instruction reads a whole 128-byte line of four
// rows) or, for long rows, 512 columns (one row per instruction); the
// workgroup's row positions take
// interleaved rows of the run.  Per row a lane loads its 8 index bytes (u8)
// or 6 (pk12: four pairs), gathers the codebook values from LDS and adds
// dy[m][n] * w to its 8 x MT accumulators (dy staged in LDS).  The first
// index and dy loads are issued before the codebook is staged; later ones
// one group of rows ahead.  After the rows, the row positions of a wave are
// summed with lane shuffles and the waves' sums in LDS in wave order; the
// sidecar terms delta * dy[m][r] of the run's triplets in the tile's columns
// are added there with LDS atomics (the run's triplet range is looked up with
// loads issued at the start).  The tile is stored into dx, or, when the rows
// are split over several workgroups to fill the GPU, into its split of a
// caller-provided workspace, which a second kernel sums in split order.
// (Device-wide fp32 atomics are too slow to combine the splits: about a
// dozen per nanosecond over the whole chip.)

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>

namespace hxq {

namespace bx {
constexpr int THREADS = 256, WAVES = THREADS / 64;
}  // namespace bx

template <bool DYBF>
__device__ __forceinline__ float load_dy(const void* dy, int64_t off) {
  if (DYBF) return bf16_to_f32(static_cast<const uint16_t*>(dy)[off]);
  return static_cast<const float*>(dy)[off];
}

// The 8 index bytes (u8) or two 24-bit pair groups (pk12) of one lane and row.
// VEC: one 8-byte load (u8: K % 8 == 0; pk12: K % 16 == 0, so the row pitch
// is a multiple of 12 bytes and the lane's 6 bytes sit inside an aligned
// 8-byte window: bytes 0-5 for even lanes, 2-7 for odd ones).  Otherwise byte
// loads with the columns clamped to the row.  NT: the 8-byte loads are
// non-temporal (a launch that streams more than the L2s hold, once).
template <bool PK12, bool VEC, bool NT>
struct IdxLoad {
  const uint8_t* base;  // the lane's first byte in row 0 (VEC) or the row 0 start
  int64_t pitch;        // bytes per row
  int cl;               // first column of the lane
  int K;

  __device__ __forceinline__ uint2 load(int n) const {
    const uint8_t* p = base + (int64_t)n * pitch;
    if (VEC) {
      if (NT) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return make_uint2(v.x, v.y);
      }
      return *reinterpret_cast<const uint2*>(p);
    }
    if (PK12) {
      // groups t0 = cl / 4 and t0 + 1 (three bytes each), clamped to the row's last group
      const int tl = (K + 3) / 4 - 1;
      const int t0 = min(cl >> 2, tl), t1 = min((cl >> 2) + 1, tl);
      const uint32_t v0 = (uint32_t)p[3 * t0] | ((uint32_t)p[3 * t0 + 1] << 8) | ((uint32_t)p[3 * t0 + 2] << 16);
      const uint32_t v1 = (uint32_t)p[3 * t1] | ((uint32_t)p[3 * t1 + 1] << 8) | ((uint32_t)p[3 * t1 + 2] << 16);
      return make_uint2(v0, v1);
    }
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 |= (uint32_t)p[min(cl + j, K - 1)] << (8 * j);
      w1 |= (uint32_t)p[min(cl + 4 + j, K - 1)] << (8 * j);
    }
    return make_uint2(w0, w1);
  }
};

// The 8 weights of a lane for one row, from its loaded bytes.
template <bool PK12, bool VEC>
__device__ __forceinline__ void gather8(uint2 q, bool odd, const unsigned char* cbs, uint32_t lane4, float* w) {
  if (PK12) {
    uint32_t v0, v1;
    if (VEC && odd) {
      v0 = __builtin_amdgcn_alignbit(q.y, q.x, 16) & 0xffffffu;
      v1 = q.y >> 8;
    } else if (VEC) {
      v0 = q.x & 0xffffffu;
      v1 = __builtin_amdgcn_alignbit(q.y, q.x, 24) & 0xffffffu;
    } else {
      v0 = q.x;
      v1 = q.y;
    }
    const float2 p0 = lds_load<float2>((v0 & 0xfffu) << 3, cbs);
    const float2 p1 = lds_load<float2>((v0 >> 12) << 3, cbs);
    const float2 p2 = lds_load<float2>((v1 & 0xfffu) << 3, cbs);
    const float2 p3 = lds_load<float2>((v1 >> 12) << 3, cbs);
    w[0] = p0.x;
    w[1] = p0.y;
    w[2] = p1.x;
    w[3] = p1.y;
    w[4] = p2.x;
    w[5] = p2.y;
    w[6] = p3.x;
    w[7] = p3.y;
  } else {
    w[0] = lds_load<float>(byte_addr256<0>(q.x, lane4), cbs);
    w[1] = lds_load<float>(byte_addr256<1>(q.x, lane4), cbs);
    w[2] = lds_load<float>(byte_addr256<2>(q.x, lane4), cbs);
    w[3] = lds_load<float>(byte_addr256<3>(q.x, lane4), cbs);
    w[4] = lds_load<float>(byte_addr256<0>(q.y, lane4), cbs);
    w[5] = lds_load<float>(byte_addr256<1>(q.y, lane4), cbs);
    w[6] = lds_load<float>(byte_addr256<2>(q.y, lane4), cbs);
    w[7] = lds_load<float>(byte_addr256<3>(q.y, lane4), cbs);
  }
}

// LPR: lanes per row, 16 (a 128-column tile, four rows per wave instruction)
// or 64 (a 512-column tile, one row per instruction, for long rows)
template <bool PK12, bool DYBF, int MT, bool VEC, int LPR, bool NT>
__global__ __launch_bounds__(bx::THREADS) void bwdx_valu(BwdArgs ba) {
  using namespace bx;
  constexpr int UNR = MT >= 8 ? 4 : 8;        // rows per row position and group
  constexpr int CW = 8 * LPR;                 // columns per workgroup
  constexpr int RL = WAVES * (64 / LPR);      // row positions per workgroup
  constexpr int RC = 2048 / MT;               // rows of dy staged at a time
  constexpr int RPAD = RC + RL * UNR;         // zero rows past the end absorb clamped loads
  constexpr int DYV = (RPAD * MT + THREADS - 1) / THREADS;
  constexpr int CB = PK12 ? 4096 * 8 : 256 * 256;
  constexpr int SCQ = 4;                      // sidecar triplets per thread loaded early
  static_assert(MT * CW * 4 <= CB, "the partial sums reuse the codebook area");
  // u8: 64 fp32 copies per entry (entry e at byte 256 e, copy j at +4 j, one
  // bank per lane); pk12: the 4096 fp32 pairs
  __shared__ __align__(16) unsigned char cbs[CB];
  __shared__ __align__(16) float dys[RPAD * MT];  // [row][token]
  __shared__ int64_t lohi[2];
  float* red = reinterpret_cast<float*>(cbs);  // [MT][CW] after the rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const int ct = b % ba.CT, rest = b / ba.CT, s = rest % ba.S, mt = rest / ba.S;
  // the layer of split s (one layer unless the call is grouped)
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegments; ++i)
    if (i < ba.nseg && s >= ba.seg[i].split0) si = i;
  const BwdSeg& sg = ba.seg[si];
  const int M = ba.M, N = sg.N, K = ba.K;
  const int c0 = ct * CW, m0 = mt * MT;
  const int n_lo = (s - sg.split0) * sg.R, n_hi = min(N, n_lo + sg.R);
  const int rw = wave * (64 / LPR) + lane / LPR;  // the lane's row position
  const int cl = c0 + 8 * (lane % LPR);            // the lane's first column
  const uint32_t lane4 = (uint32_t)lane << 2;

  IdxLoad<PK12, VEC, NT> il;
  il.pitch = PK12 ? (int64_t)((K + 3) / 4) * 3 : (int64_t)K;
  il.cl = cl;
  il.K = K;
  if (VEC) {
    // lanes past the last column read column 0 (never stored)
    const int q = cl < K ? cl >> 3 : 0;
    il.base = sg.indices + (PK12 ? (int64_t)(6 * q - 2 * (q & 1)) : (int64_t)(cl < K ? cl : 0));
  } else {
    il.base = sg.indices;
  }
  const bool odd = (cl >> 3) & 1;

  // ---- first the index bytes of the first rows, dy of the first chunk and
  // the sidecar window around the run's ends (waves 0 and 1), then the
  // codebook, so the loads overlap the staging.  Row position p takes rows
  // r0 + p + RL u (+ RL UNR per group); rows past the chunk read its last row
  // and meet zero dy.
  int r0 = n_lo, rc = min(RC, n_hi - n_lo);
  uint2 cur[UNR], nxt[UNR];
  float dyv[DYV];
  auto load_chunk = [&]() {
#pragma unroll
    for (int u = 0; u < UNR; ++u) cur[u] = il.load(min(r0 + rw + RL * u, r0 + rc - 1));
#pragma unroll
    for (int v = 0; v < DYV; ++v) {
      const int e = tid + THREADS * v, i = e / MT, m = e % MT;
      dyv[v] = (i < rc && m0 + m < M) ? load_dy<DYBF>(sg.dy, (int64_t)(m0 + m) * N + r0 + i) : 0.f;
    }
  };
  load_chunk();
  WindowProbe probe;
  const int target = wave == 0 ? n_lo : n_hi;
  if (sg.nnz > 0 && wave < 2)
    window_issue(probe, sg.sc_rows, sg.nnz, (int64_t)((double)sg.nnz * (double)target / (double)N));
  if (PK12) {
    // (4-byte loads: the codebook is only required to be 4-byte aligned)
#pragma unroll
    for (int i = 0; i < 8192 / THREADS; ++i) {
      const int e = tid + THREADS * i;
      reinterpret_cast<float*>(cbs)[e] = sg.codebook[e];
    }
  } else {
    const float v = sg.codebook[tid];
    const float4 v4 = make_float4(v, v, v, v);
#pragma unroll
    for (int q = 0; q < 16; ++q) *reinterpret_cast<float4*>(cbs + tid * 256 + (((q + tid) & 15) << 4)) = v4;
  }

  float acc[MT][8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

  // the run's triplets: resolved before the first barrier, then loaded (up
  // to SCQ per thread) while the rows are processed
  if (sg.nnz > 0 && wave < 2) {
    const int64_t v = window_resolve(probe, sg.sc_rows, sg.nnz, target);
    if (lane == 0) lohi[wave] = v;
  }
  int64_t lo = 0, hi = 0;
  int tr[SCQ], tc[SCQ];
  float td[SCQ];
  bool first = true;
  while (true) {
#pragma unroll
    for (int v = 0; v < DYV; ++v) {
      const int e = tid + THREADS * v;
      if (e < RPAD * MT) dys[e] = dyv[v];
    }
    __syncthreads();
    if (first && sg.nnz > 0) {
      lo = lohi[0];
      hi = lohi[1];
#pragma unroll
      for (int q = 0; q < SCQ; ++q) {
        const int64_t e = min(lo + tid + THREADS * q, sg.nnz - 1);
        tr[q] = sg.sc_rows[e];
        tc[q] = sg.sc_cols[e];
        td[q] = sg.sc_deltas[e];
      }
    }
    first = false;
    const int groups = (rc + RL * UNR - 1) / (RL * UNR);
    for (int g = 0; g < groups; ++g) {
      const int i = g * RL * UNR;
      if (g + 1 < groups) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) nxt[u] = il.load(min(r0 + i + rw + RL * (UNR + u), r0 + rc - 1));
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float w[8];
        gather8<PK12, VEC>(cur[u], odd, cbs, lane4, w);
        const float* dr = dys + (i + rw + RL * u) * MT;
        float gv[MT];
        if (MT >= 4) {
#pragma unroll
          for (int m = 0; m < MT; m += 4) {
            const float4 t = *reinterpret_cast<const float4*>(dr + m);
            gv[m] = t.x;
            gv[m + 1] = t.y;
            gv[m + 2] = t.z;
            gv[m + 3] = t.w;
          }
        } else {
#pragma unroll
          for (int m = 0; m < MT; ++m) gv[m] = dr[m];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(gv[m], w[j], acc[m][j]);
      }
      if (g + 1 < groups) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) cur[u] = nxt[u];
      }
    }
    r0 += RC;
    if (r0 >= n_hi) break;
    rc = min(RC, n_hi - r0);
    load_chunk();
    __syncthreads();  // this chunk's readers of dy are done
  }

  // ---- the row positions of each wave (lane shuffles), then the waves in
  // wave order
  if (LPR < 64) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int o = LPR; o < 64; o *= 2) acc[m][j] += __shfl_xor(acc[m][j], o, 64);
  }
  __syncthreads();  // every wave is done with the codebook
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w && lane < LPR) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float4* p = reinterpret_cast<float4*>(red + m * CW + 8 * lane);
        float4 a = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
        float4 c = make_float4(acc[m][4], acc[m][5], acc[m][6], acc[m][7]);
        if (w > 0) {
          const float4 pa = p[0], pc = p[1];
          a = make_float4(pa.x + a.x, pa.y + a.y, pa.z + a.z, pa.w + a.w);
          c = make_float4(pc.x + c.x, pc.y + c.y, pc.z + c.z, pc.w + c.w);
        }
        p[0] = a;
        p[1] = c;
      }
    }
    __syncthreads();
  }

  // ---- sidecar terms of the run's triplets in these columns (LDS atomics):
  // the prefetched ones first, dy from LDS when the run was one chunk
  if (sg.nnz > 0) {
    const bool one_chunk = n_hi - n_lo <= RC;
#pragma unroll
    for (int q = 0; q < SCQ; ++q) {
      const int64_t e = lo + tid + THREADS * q;
      if (e < hi && tc[q] >= c0 && tc[q] < c0 + CW) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m0 + m < M) {
            const float g = one_chunk ? dys[(tr[q] - n_lo) * MT + m]
                                      : load_dy<DYBF>(sg.dy, (int64_t)(m0 + m) * N + tr[q]);
            atomicAdd(&red[m * CW + (tc[q] - c0)], td[q] * g);
          }
      }
    }
    for (int64_t e = lo + tid + THREADS * SCQ; e < hi; e += THREADS) {
      const int c = sg.sc_cols[e];
      if (c >= c0 && c < c0 + CW) {
        const int r = sg.sc_rows[e];
        const float d = sg.sc_deltas[e];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m0 + m < M) atomicAdd(&red[m * CW + (c - c0)], d * load_dy<DYBF>(sg.dy, (int64_t)(m0 + m) * N + r));
      }
    }
    __syncthreads();
  }

  // ---- store: into dx when the rows are not split, else into split s of
  // the workspace (in a grouped call the splits of all layers)
  float* out = ba.S > 1 ? ba.ws + (int64_t)s * M * K : ba.dx;
  for (int e = tid; e < MT * CW; e += THREADS) {
    const int m = e / CW, col = e % CW;
    if (m0 + m < M && c0 + col < K) out[(int64_t)(m0 + m) * K + c0 + col] = red[e];
  }
}

// dx[i] = sum over the splits of ws[s][i], added in split order.  VEC: four
// consecutive elements per thread (16-byte loads and stores), for large n;
// otherwise one element per thread, so a small reduction (one token: a few
// thousand elements) still spreads over several workgroups.
template <bool VEC>
__global__ __launch_bounds__(256) void bwdx_reduce(const float* __restrict__ ws, float* __restrict__ dx, int64_t n,
                                                   int S) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (VEC ? 4 : 1);
  if (i >= n) return;
  // loads go out 16 (four elements) or 32 (one element) splits at a time (a
  // plain loop would wait for each before issuing the next); the adds stay
  // in split order
  constexpr int B = VEC ? 16 : 32;
  if (VEC) {
    float4 v = *reinterpret_cast<const float4*>(ws + i);
    int s = 1;
    for (; s + B <= S; s += B) {
      float4 t[B];
#pragma unroll
      for (int u = 0; u < B; ++u) t[u] = *reinterpret_cast<const float4*>(ws + (int64_t)(s + u) * n + i);
#pragma unroll
      for (int u = 0; u < B; ++u) v = make_float4(v.x + t[u].x, v.y + t[u].y, v.z + t[u].z, v.w + t[u].w);
    }
    // the rest: loads clamped to the last split (unconditional, so they all
    // go out together), adds only for the splits that exist
    float4 t[B];
#pragma unroll
    for (int u = 0; u < B; ++u) t[u] = *reinterpret_cast<const float4*>(ws + (int64_t)min(s + u, S - 1) * n + i);
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (s + u < S) v = make_float4(v.x + t[u].x, v.y + t[u].y, v.z + t[u].z, v.w + t[u].w);
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(dx + i));
  } else {
    float v = ws[i];
    int s = 1;
    for (; s + B <= S; s += B) {
      float t[B];
#pragma unroll
      for (int u = 0; u < B; ++u) t[u] = ws[(int64_t)(s + u) * n + i];
#pragma unroll
      for (int u = 0; u < B; ++u) v += t[u];
    }
    float t[B];
#pragma unroll
    for (int u = 0; u < B; ++u) t[u] = ws[(int64_t)min(s + u, S - 1) * n + i];
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (s + u < S) v += t[u];
    dx[i] = v;
  }
}

__global__ __launch_bounds__(256) void fill_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

static bool vec_ok(const uint8_t* indices, int K, bool pk12) {
  const uintptr_t ip = reinterpret_cast<uintptr_t>(indices);
  return pk12 ? (K % 16 == 0 && ip % 4 == 0) : (K % 8 == 0 && ip % 8 == 0);
}

bool bwdx_vec_ok(const BwdArgs& a, bool pk12) { return vec_ok(a.indices, a.K, pk12); }

template <bool PK12, bool DYBF, bool VEC, int LPR, bool NT>
static hipError_t launch_bx(const BwdArgs& a, int mt, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1: hipLaunchKernelGGL((bwdx_valu<PK12, DYBF, 1, VEC, LPR, NT>), grid, dim3(bx::THREADS), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((bwdx_valu<PK12, DYBF, 2, VEC, LPR, NT>), grid, dim3(bx::THREADS), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((bwdx_valu<PK12, DYBF, 4, VEC, LPR, NT>), grid, dim3(bx::THREADS), 0, stream, a); break;
    default: hipLaunchKernelGGL((bwdx_valu<PK12, DYBF, 8, VEC, LPR, NT>), grid, dim3(bx::THREADS), 0, stream, a); break;
  }
  return hipGetLastError();
}

// nt: non-temporal index loads (8-byte loads only)
template <bool PK12, bool DYBF>
static hipError_t launch_bx_v(const BwdArgs& a, int mt, bool vec, bool nt, int lpr, dim3 grid, hipStream_t stream) {
  if (!vec)
    return lpr == 64 ? launch_bx<PK12, DYBF, false, 64, false>(a, mt, grid, stream)
                     : launch_bx<PK12, DYBF, false, 16, false>(a, mt, grid, stream);
  if (lpr == 64)
    return nt ? launch_bx<PK12, DYBF, true, 64, true>(a, mt, grid, stream)
              : launch_bx<PK12, DYBF, true, 64, false>(a, mt, grid, stream);
  return nt ? launch_bx<PK12, DYBF, true, 16, true>(a, mt, grid, stream)
            : launch_bx<PK12, DYBF, true, 16, false>(a, mt, grid, stream);
}

// The launch shape: tokens per workgroup, column tile width, and the number
// of row splits that gives about two workgroups per CU (one for layers of at
// most 4096 rows; at least 64 rows per split).  M, N, K > 0.
BwdPlan bwdx_plan(int M, int N, int K) {
  BwdPlan p;
  p.mt = M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : 8;
  p.lpr = K >= 8192 ? 64 : 16;
  p.mtiles = (M + p.mt - 1) / p.mt;
  p.ct = (K + 8 * p.lpr - 1) / (8 * p.lpr);
  const int64_t tiles = (int64_t)p.ct * p.mtiles;
  // about two workgroups per CU, one for layers of at most 4096 rows (fewer
  // splits to sum; measured at one token: 2048-row layers 8.7 -> 7.9 us,
  // 11008-row ones 10.9 -> 12.0 us with one)
  const int64_t target = (N <= 4096 ? 1 : 2) * (int64_t)device_cu_count();
  int64_t S = (target + tiles - 1) / tiles;
  int64_t smax = (N + 63) / 64;
  // rows a workgroup takes per group of loads; a layer of at most two such
  // groups is not split (one more round of loads costs less than the
  // reduction launch)
  const int group_rows = bx::WAVES * (64 / p.lpr) * (p.mt >= 8 ? 4 : 8);
  if (N <= 2 * group_rows) smax = 1;
  if (S > smax) S = smax;
  if (S > 64) S = 64;  // at most 64 splits (each M K floats of workspace)
  if (S < 1) S = 1;
  p.S = (int)S;
  return p;
}

int64_t bwdx_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const BwdPlan p = bwdx_plan(M, N, K);
  return p.S > 1 ? (int64_t)p.S * M * K * 4 : 0;
}

// One launch of the main kernel, then the reduction over the row splits when
// there are several (their partial sums go to the workspace; a workspace too
// small for the planned splits gets fewer).
static hipError_t launch_bx_any(const BwdArgs& a, const BwdPlan& p, bool pk12, bool vec, int64_t S,
                                hipStream_t stream) {
  const int64_t blocks = (int64_t)p.ct * p.mtiles * S;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  // index bytes read once (one token tile) and more of them than the L2s
  // hold: non-temporal loads (Qwen input-gradient step at one token 55.5 ->
  // 52.2 us with every launch so, gate|up the one that gains)
  int64_t ib = 0;
  for (int i = 0; i < a.nseg; ++i) ib += index_bytes(a.seg[i].N, a.K, pk12);
  const bool nt = p.mtiles == 1 && ib > kStreamPastCacheBytes;
  if (pk12)
    return a.dy_bf16 ? launch_bx_v<true, true>(a, p.mt, vec, nt, p.lpr, grid, stream)
                     : launch_bx_v<true, false>(a, p.mt, vec, nt, p.lpr, grid, stream);
  return a.dy_bf16 ? launch_bx_v<false, true>(a, p.mt, vec, nt, p.lpr, grid, stream)
                   : launch_bx_v<false, false>(a, p.mt, vec, nt, p.lpr, grid, stream);
}

hipError_t launch_bwdx_valu(const BwdArgs& a0, bool pk12, hipStream_t stream) {
  BwdArgs a = a0;
  const BwdPlan p = bwdx_plan(a.M, a.N, a.K);
  int64_t S = p.S;
  const int64_t per = (int64_t)a.M * a.K * 4;
  if (S > 1 && (a.ws == nullptr || a.ws_bytes < S * per)) S = a.ws ? a.ws_bytes / per : 1;
  if (S < 2) S = 1;
  if (S > 64) S = 64;
  const int64_t R = (a.N + S - 1) / S;
  S = (a.N + R - 1) / R;
  a.CT = p.ct;
  a.S = (int)S;
  a.R = (int)R;
  a.nseg = 1;
  a.seg[0] = {a.codebook, a.indices, a.sc_rows, a.sc_cols, a.sc_deltas, a.nnz, a.dy, a.N, 0, (int)R};
  const hipError_t e = launch_bx_any(a, p, pk12, bwdx_vec_ok(a, pk12), S, stream);
  if (e != hipSuccess || S == 1) return e;
  return launch_bwdx_reduce(a.ws, a.dx, (int64_t)a.M * a.K, (int)S, stream);
}

// Every layer is split into runs of one length R, chosen as for a single
// layer of all the group's rows (so a group of small layers still fills the
// GPU); a run never crosses into the next layer.  Ns[i] > 0.
BwdGroupPlan bwdx_group_plan(int M, const int* Ns, int nseg, int K) {
  BwdGroupPlan g;
  int64_t total = 0;
  for (int i = 0; i < nseg; ++i) total += Ns[i];
  g.p = bwdx_plan(M, (int)total, K);
  g.R = (int)((total + g.p.S - 1) / g.p.S);
  g.slots_total = 0;
  for (int i = 0; i < nseg; ++i) {
    g.S[i] = (Ns[i] + g.R - 1) / g.R;
    g.slots_total += g.S[i];
  }
  return g;
}

// One launch over the layers in a.seg (their fields set by the caller, split0
// and R set here), then the sum of all their splits into dx.  a.ws holds the
// plan's slots.
hipError_t launch_bwdx_valu_grouped(const BwdArgs& a0, bool pk12, hipStream_t stream) {
  BwdArgs a = a0;
  int Ns[kMaxSegments];
  for (int i = 0; i < a.nseg; ++i) Ns[i] = a.seg[i].N;
  const BwdGroupPlan g = bwdx_group_plan(a.M, Ns, a.nseg, a.K);
  if (a.ws == nullptr || a.ws_bytes < (int64_t)g.slots_total * a.M * a.K * 4) return hipErrorInvalidValue;
  bool vec = true;
  int split0 = 0;
  for (int i = 0; i < a.nseg; ++i) {
    vec = vec && vec_ok(a.seg[i].indices, a.K, pk12);
    a.seg[i].split0 = split0;
    a.seg[i].R = g.R;
    split0 += g.S[i];
  }
  a.CT = g.p.ct;
  a.S = g.slots_total;
  a.R = g.R;
  const hipError_t e = launch_bx_any(a, g.p, pk12, vec, g.slots_total, stream);
  if (e != hipSuccess) return e;
  return launch_bwdx_reduce(a.ws, a.dx, (int64_t)a.M * a.K, g.slots_total, stream);
}

hipError_t launch_bwdx_reduce(const float* ws, float* dx, int64_t n, int S, hipStream_t stream) {
  // four elements per thread only when that still gives a workgroup per CU
  const bool vec = n % 4 == 0 && reinterpret_cast<uintptr_t>(dx) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(ws) % 16 == 0 && n / 1024 >= device_cu_count();
  const int64_t rb = (n + (vec ? 1023 : 255)) / (vec ? 1024 : 256);
  if (rb > INT_MAX || S < 1 || S > 1024) return hipErrorInvalidConfiguration;
  if (vec)
    hipLaunchKernelGGL(bwdx_reduce<true>, dim3((unsigned)rb), dim3(256), 0, stream, ws, dx, n, S);
  else
    hipLaunchKernelGGL(bwdx_reduce<false>, dim3((unsigned)rb), dim3(256), 0, stream, ws, dx, n, S);
  return hipGetLastError();
}

}  // namespace hxq
