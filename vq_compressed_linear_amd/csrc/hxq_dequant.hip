// Measurement helper: the dense bf16 weight of a HelixLinear layer, written to
// a caller-owned buffer.  Not part of the forward pass (which never forms the
// weight): it is the first half of the buffered design the HXQ whitepaper's
// inference paragraph describes (gather into a shared bf16 buffer, then a
// library matmul), so that design can be timed against the fused kernels.
//
// w[n][k] = bf16(C[idx[n][k]] + sum of the sidecar deltas at (n, k)), the
// deltas added in fp32 in stored order and the sum rounded once to nearest
// even: the same value the bf16 matrix-core GEMM feeds its matrix cores.
// Two launches on the stream: the codebook values for every weight, then the
// positions the sidecar names.

#include "hxq_device.h"
#include "hxq_launch.h"

namespace hxq {

namespace deq {
constexpr int THREADS = 256;
}

// One thread per 16 consecutive weights of a row (K % 16 == 0): 16 index bytes
// (u8) or 12 (pk12) in, 32 bytes of bf16 out.  The codebook sits in LDS as
// bf16 (u8: one value per entry in the low half; pk12: the pair as two halves).
template <bool PK12>
__global__ __launch_bounds__(deq::THREADS) void dequant_bf16_kernel(const float* __restrict__ codebook,
                                                                    const uint8_t* __restrict__ indices,
                                                                    uint16_t* __restrict__ w, int64_t groups,
                                                                    int64_t gpr) {
  __shared__ uint32_t cb[PK12 ? 4096 : 256];
  for (int e = threadIdx.x; e < (PK12 ? 4096 : 256); e += deq::THREADS) {
    if (PK12) {
      const float2 c = reinterpret_cast<const float2*>(codebook)[e];
      cb[e] = f32_to_bf16_rne(c.x) | (f32_to_bf16_rne(c.y) << 16);
    } else {
      cb[e] = f32_to_bf16_rne(codebook[e]);
    }
  }
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * deq::THREADS;
  for (int64_t gi = (int64_t)blockIdx.x * deq::THREADS + threadIdx.x; gi < groups; gi += stride) {
    const int64_t n = gi / gpr, j = gi - n * gpr;  // row, 16-weight group of the row
    uint32_t o[8];
    if (PK12) {
      // 8 pairs in 12 bytes: 24-bit group d holds pairs 2 d, 2 d + 1 as v & 0xfff, v >> 12
      const uint8_t* p = indices + n * (gpr * 12) + j * 12;
      const uint32_t w0 = *reinterpret_cast<const uint32_t*>(p), w1 = *reinterpret_cast<const uint32_t*>(p + 4),
                     w2 = *reinterpret_cast<const uint32_t*>(p + 8);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t v = d == 0 ? (w0 & 0xffffffu)
                         : d == 1 ? (__builtin_amdgcn_alignbit(w1, w0, 24) & 0xffffffu)
                         : d == 2 ? (__builtin_amdgcn_alignbit(w2, w1, 16) & 0xffffffu)
                                  : (w2 >> 8);
        o[2 * d] = cb[v & 0xfffu];
        o[2 * d + 1] = cb[v >> 12];
      }
    } else {
      const u32x4 q = *reinterpret_cast<const u32x4*>(indices + n * (gpr * 16) + j * 16);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t b = q[d];
        o[2 * d] = cb[b & 0xffu] | (cb[(b >> 8) & 0xffu] << 16);
        o[2 * d + 1] = cb[(b >> 16) & 0xffu] | (cb[b >> 24] << 16);
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(w + n * (gpr * 16) + j * 16);
    dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4{o[4], o[5], o[6], o[7]};
  }
}

// One thread per triplet; the first of each run of equal (row, col) writes
// bf16(C + its run's deltas in stored order).
template <bool PK12>
__global__ __launch_bounds__(deq::THREADS) void dequant_sidecar_kernel(const float* __restrict__ codebook,
                                                                       const uint8_t* __restrict__ indices,
                                                                       const int32_t* __restrict__ rows,
                                                                       const int32_t* __restrict__ cols,
                                                                       const float* __restrict__ deltas,
                                                                       int64_t nnz, uint16_t* __restrict__ w,
                                                                       int64_t K) {
  const int64_t e = (int64_t)blockIdx.x * deq::THREADS + threadIdx.x;
  if (e >= nnz) return;
  const int r = rows[e], c = cols[e];
  if (e > 0 && rows[e - 1] == r && cols[e - 1] == c) return;
  float v;
  if (PK12) {
    const uint8_t* p = indices + (int64_t)r * (K / 4 * 3) + (c >> 2) * 3;
    const uint32_t g = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
    const uint32_t pi = ((c >> 1) & 1) ? (g >> 12) : (g & 0xfffu);
    v = codebook[2 * pi + (c & 1)];
  } else {
    v = codebook[indices[(int64_t)r * K + c]];
  }
  v += deltas[e];
  for (int64_t e2 = e + 1; e2 < nnz && rows[e2] == r && cols[e2] == c; ++e2) v += deltas[e2];
  w[(int64_t)r * K + c] = (uint16_t)f32_to_bf16_rne(v);
}

hipError_t launch_dequant_bf16(bool pk12, const float* codebook, const uint8_t* indices, const int32_t* rows,
                               const int32_t* cols, const float* deltas, int64_t nnz, uint16_t* w, int64_t N,
                               int64_t K, hipStream_t stream) {
  const int64_t gpr = K / 16, groups = N * gpr;
  int64_t blocks = (groups + deq::THREADS - 1) / deq::THREADS;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  if (pk12)
    hipLaunchKernelGGL(dequant_bf16_kernel<true>, dim3((unsigned)blocks), dim3(deq::THREADS), 0, stream, codebook,
                       indices, w, groups, gpr);
  else
    hipLaunchKernelGGL(dequant_bf16_kernel<false>, dim3((unsigned)blocks), dim3(deq::THREADS), 0, stream, codebook,
                       indices, w, groups, gpr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nnz == 0) return err;
  const int64_t sb = (nnz + deq::THREADS - 1) / deq::THREADS;
  if (pk12)
    hipLaunchKernelGGL(dequant_sidecar_kernel<true>, dim3((unsigned)sb), dim3(deq::THREADS), 0, stream, codebook,
                       indices, rows, cols, deltas, nnz, w, K);
  else
    hipLaunchKernelGGL(dequant_sidecar_kernel<false>, dim3((unsigned)sb), dim3(deq::THREADS), 0, stream, codebook,
                       indices, rows, cols, deltas, nnz, w, K);
  return hipGetLastError();
}

}  // namespace hxq
