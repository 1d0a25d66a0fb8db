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

}  // namespace hxq
