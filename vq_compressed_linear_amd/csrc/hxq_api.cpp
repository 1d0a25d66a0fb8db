// C entry points of libhxq: argument validation on the host, then dispatch to
// one kernel family.  Nothing here touches device memory or allocates.

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "../../include/hxq.h"
#include "hxq_launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)INT32_MAX - 65536;  // room for tile rounding in int32
constexpr int64_t kBwdMfmaMinM = 16;                       // input gradient: matrix cores from here

bool misaligned(const void* p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Checks shared by the forward entry points.  Returns HXQ_OK or an error.
int validate_forward(const void* codebook, const uint8_t* indices, const int32_t* sc_rows,
                     const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* x,
                     int x_dtype, const float* bias, const float* y, int64_t M, int64_t N,
                     int64_t K, bool pk12) {
  if (x_dtype != HXQ_F32 && x_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || nnz < 0) return HXQ_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || nnz > kMaxDim) return HXQ_ERR_SHAPE;
  if (pk12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return HXQ_OK;
  if (!y) return HXQ_ERR_NULL;
  if (K > 0 && (!x || !indices || !codebook)) return HXQ_ERR_NULL;
  if (nnz > 0 && (!sc_rows || !sc_cols || !sc_deltas)) return HXQ_ERR_NULL;
  const uintptr_t xs = x_dtype == HXQ_BF16 ? 2 : 4;
  if (misaligned(x, xs) || misaligned(y, 4) || misaligned(codebook, 4) || misaligned(bias, 4) ||
      misaligned(sc_rows, 4) || misaligned(sc_cols, 4) || misaligned(sc_deltas, 4))
    return HXQ_ERR_ALIGN;
  return HXQ_OK;
}

int select(bool pk12, bool x_bf16, int64_t M, int64_t K, bool gemv_ok, bool gemm_ok) {
  if (K == 0) return HXQ_VARIANT_GENERIC;
  if (x_bf16 && M > 16 && gemm_ok) return HXQ_VARIANT_GEMM_BF16;
  if (gemv_ok) return HXQ_VARIANT_GEMV_VALU;
  return HXQ_VARIANT_GENERIC;
}

int status_of(hipError_t e) { return e == hipSuccess ? HXQ_OK : HXQ_ERR_HIP; }

int forward(bool pk12, const void* codebook, const uint8_t* indices, const int32_t* sc_rows,
            const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* x, int x_dtype,
            const float* bias, float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream,
            int variant) {
  int st = validate_forward(codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias,
                            y, M, N, K, pk12);
  if (st != HXQ_OK) return st;
  if (variant < HXQ_VARIANT_AUTO || variant > HXQ_VARIANT_GENERIC) return HXQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return HXQ_OK;
  hxq::LayerArgs a;
  a.codebook = codebook;
  a.indices = indices;
  a.sc_rows = sc_rows;
  a.sc_cols = sc_cols;
  a.sc_deltas = sc_deltas;
  a.nnz = nnz;
  a.x = x;
  a.x_bf16 = x_dtype == HXQ_BF16;
  a.bias = bias;
  a.y = y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  const bool gemv_ok = K > 0 && hxq::gemv_fast_path_ok(a, pk12);
  const bool gemm_ok = K > 0 && (pk12 ? hxq::gemm2_path_ok(a, true) : hxq::gemm_path_ok(a));
  int v = variant;
  if (v == HXQ_VARIANT_AUTO) v = select(pk12, a.x_bf16, M, K, gemv_ok, gemm_ok);
  (void)hipGetLastError();  // start from a clean error state
  switch (v) {
    case HXQ_VARIANT_GEMV_VALU:
      if (!gemv_ok) return HXQ_ERR_UNSUPPORTED;
      return status_of(hxq::launch_gemv_valu(a, pk12, stream));
    case HXQ_VARIANT_GEMV_MFMA:
      if (!gemv_ok || !hxq::gemv_mfma_takes(a, pk12)) return HXQ_ERR_UNSUPPORTED;
      return status_of(hxq::launch_gemv_mfma_tokens(a, pk12, stream));
    case HXQ_VARIANT_GEMM_BF16:
      if (!gemm_ok) return HXQ_ERR_UNSUPPORTED;
      if (hxq::gemm2_path_ok(a, pk12)) return status_of(hxq::launch_gemm2_bf16(a, pk12, stream));
      return status_of(hxq::launch_gemm_bf16(a, stream));  // u8 only (pk12 passed the check above)
    case HXQ_VARIANT_GENERIC:
      return status_of(hxq::launch_generic(a, pk12, stream));
    default:
      return HXQ_ERR_UNSUPPORTED;
  }
}

int backward_x(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
               const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* dy, int dy_dtype,
               float* dx, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
               hipStream_t stream, int variant) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  const bool pk12 = fmt == HXQ_FMT_PK12;
  if (dy_dtype != HXQ_F32 && dy_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || nnz < 0 || workspace_bytes < 0) return HXQ_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || nnz > kMaxDim) return HXQ_ERR_SHAPE;
  if (pk12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  if (variant != HXQ_VARIANT_AUTO && variant != HXQ_VARIANT_GEMV_VALU && variant != HXQ_VARIANT_GEMM_BF16)
    return HXQ_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return HXQ_OK;
  if (!dx) return HXQ_ERR_NULL;
  if (N > 0 && (!dy || !indices || !codebook)) return HXQ_ERR_NULL;
  if (nnz > 0 && (!sc_rows || !sc_cols || !sc_deltas)) return HXQ_ERR_NULL;
  const uintptr_t ds = dy_dtype == HXQ_BF16 ? 2 : 4;
  if (misaligned(dy, ds) || misaligned(dx, 4) || misaligned(codebook, 4) || misaligned(sc_rows, 4) ||
      misaligned(sc_cols, 4) || misaligned(sc_deltas, 4) || misaligned(workspace, 4))
    return HXQ_ERR_ALIGN;
  (void)hipGetLastError();
  if (N == 0) return status_of(hxq::launch_fill_zero(dx, M * K, stream));
  hxq::BwdArgs a = {};
  a.codebook = codebook;
  a.indices = indices;
  a.sc_rows = sc_rows;
  a.sc_cols = sc_cols;
  a.sc_deltas = sc_deltas;
  a.nnz = nnz;
  a.dy = dy;
  a.dy_bf16 = dy_dtype == HXQ_BF16;
  a.dx = dx;
  a.ws = workspace ? static_cast<float*>(workspace) : nullptr;
  a.ws_bytes = workspace ? workspace_bytes : 0;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  // the bf16 matrix-core kernel past 16 tokens, when the shape, the pointers
  // and the workspace (row splits and sidecar bins) allow it
  bool mfma = hxq::bwdx_mfma_ok(a, pk12);
  if (mfma) {
    const hxq::BwdMPlan p = hxq::bwdx_mfma_plan(a.M, a.N, a.K, nnz);
    const int64_t need = p.split_bytes + p.bin_bytes;
    mfma = need == 0 || (workspace && workspace_bytes >= need);
  }
  if (variant == HXQ_VARIANT_GEMM_BF16 && !mfma) return HXQ_ERR_UNSUPPORTED;
  if (variant == HXQ_VARIANT_GEMM_BF16 || (variant == HXQ_VARIANT_AUTO && mfma && M >= kBwdMfmaMinM))
    return status_of(hxq::launch_bwdx_mfma(a, pk12, stream));
  return status_of(hxq::launch_bwdx_valu(a, pk12, stream));
}

}  // namespace

extern "C" {

int hxq_linear_bwd_x(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                     const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* dy, int dy_dtype,
                     float* dx, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                     hipStream_t stream) {
  return backward_x(fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, dy, dy_dtype, dx, M, N, K, workspace,
                    workspace_bytes, stream, HXQ_VARIANT_AUTO);
}

int64_t hxq_linear_bwd_x_workspace(int fmt, int dy_dtype, int64_t M, int64_t N, int64_t K, int64_t nnz) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  if (dy_dtype != HXQ_F32 && dy_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || nnz < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || nnz > kMaxDim)
    return HXQ_ERR_SHAPE;
  if (fmt == HXQ_FMT_PK12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0) return 0;
  // the kernel AUTO would pick with aligned pointers
  hxq::BwdArgs a = {};
  a.indices = reinterpret_cast<const uint8_t*>(uintptr_t(256));
  a.dy = reinterpret_cast<const void*>(uintptr_t(256));
  a.dx = reinterpret_cast<float*>(uintptr_t(256));
  a.dy_bf16 = dy_dtype == HXQ_BF16;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  if (M >= kBwdMfmaMinM && hxq::bwdx_mfma_ok(a, fmt == HXQ_FMT_PK12)) {
    const hxq::BwdMPlan p = hxq::bwdx_mfma_plan(a.M, a.N, a.K, nnz);
    return p.split_bytes + p.bin_bytes;
  }
  return hxq::bwdx_workspace_bytes((int)M, (int)N, (int)K);
}

int hxq_linear_bwd_x_ex(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                        const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* dy, int dy_dtype,
                        float* dx, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                        hipStream_t stream, int variant) {
  return backward_x(fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, dy, dy_dtype, dx, M, N, K, workspace,
                    workspace_bytes, stream, variant);
}

int hxq_linear_fwd_u8_ex(const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                         const int32_t* sc_cols, const float* sc_deltas, int64_t nnz,
                         const void* x, int x_dtype, const float* bias, float* y, int64_t M,
                         int64_t N, int64_t K, hipStream_t stream, int variant) {
  return forward(false, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y,
                 M, N, K, stream, variant);
}

int hxq_linear_fwd_pk12_ex(const float* codebook2, const uint8_t* packed, const int32_t* sc_rows,
                           const int32_t* sc_cols, const float* sc_deltas, int64_t nnz,
                           const void* x, int x_dtype, const float* bias, float* y, int64_t M,
                           int64_t N, int64_t K, hipStream_t stream, int variant) {
  return forward(true, codebook2, packed, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y, M,
                 N, K, stream, variant);
}

int hxq_linear_fwd_u8(const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                      const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* x,
                      int x_dtype, const float* bias, float* y, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
  return forward(false, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y,
                 M, N, K, stream, HXQ_VARIANT_AUTO);
}

int hxq_linear_fwd_pk12(const float* codebook2, const uint8_t* packed, const int32_t* sc_rows,
                        const int32_t* sc_cols, const float* sc_deltas, int64_t nnz,
                        const void* x, int x_dtype, const float* bias, float* y, int64_t M,
                        int64_t N, int64_t K, hipStream_t stream) {
  return forward(true, codebook2, packed, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y, M,
                 N, K, stream, HXQ_VARIANT_AUTO);
}

int hxq_linear_fwd_grouped(int fmt, const hxq_layer* layers, int count, const void* x, int x_dtype,
                           int64_t M, int64_t K, hipStream_t stream) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  if (count < 1 || count > HXQ_MAX_GROUP) return HXQ_ERR_SHAPE;
  if (!layers) return HXQ_ERR_NULL;
  const bool pk12 = fmt == HXQ_FMT_PK12;
  for (int i = 0; i < count; ++i) {
    const hxq_layer& l = layers[i];
    const int st = validate_forward(l.codebook, l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz, x,
                                    x_dtype, l.bias, l.y, M, l.N, K, pk12);
    if (st != HXQ_OK) return st;
  }
  if (M == 0) return HXQ_OK;
  // one launch when every non-empty layer fits the decode kernel
  hxq::DecodeSeg segs[hxq::kMaxSegments];
  int nseg = 0;
  bool fast = K > 0 && M <= hxq::kChunkMaxM;
  for (int i = 0; i < count && fast; ++i) {
    const hxq_layer& l = layers[i];
    if (l.N == 0) continue;
    hxq::LayerArgs a = {};
    a.codebook = l.codebook;
    a.indices = l.indices;
    a.x = x;
    a.x_bf16 = x_dtype == HXQ_BF16;
    a.M = (int)M;
    a.N = (int)l.N;
    a.K = (int)K;
    if (!hxq::gemv_fast_path_ok(a, pk12)) fast = false;
    segs[nseg++] = {l.codebook, l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz, l.bias, l.y, (int)l.N, 0, 0, 0.f};
  }
  if (fast && nseg == 0) return HXQ_OK;
  // From 5 to 64 tokens the matrix-core GEMVs, with the kernel a single-layer
  // call would pick for each layer (5 to 8 tokens: the 4x4-block GEMV where it
  // takes the layer, else the 16x16 one; u8 with bf16 x past 16 tokens goes to
  // the bf16 GEMM instead): one launch when every layer takes the same kernel
  // and the group fits one workgroup per CU, one launch per layer when they
  // take the same kernel but do not fit together, else the per-layer calls.
  const bool bf16_gemm = x_dtype == HXQ_BF16 && M > 16;
  if (K > 0 && M > 4 && M <= hxq::kGemvMfmaMaxM && !bf16_gemm) {
    hxq::GemvSeg gs[hxq::kMaxSegments];
    int ng = 0, n4 = 0, n16 = 0;
    for (int i = 0; i < count; ++i) {
      const hxq_layer& l = layers[i];
      if (l.N == 0) continue;
      hxq::LayerArgs a = {};
      a.codebook = l.codebook;
      a.indices = l.indices;
      a.x = x;
      a.x_bf16 = x_dtype == HXQ_BF16;
      a.M = (int)M;
      a.N = (int)l.N;
      a.K = (int)K;
      gs[ng] = {static_cast<const float*>(l.codebook), l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz,
                l.bias, l.y, (int)l.N, 0};
      if (hxq::gemv_fast_path_ok(a, pk12)) {
        if (M <= 8 && hxq::gemv_mfma4_ok(a, pk12) && hxq::gemv_mfma4_group_fits(&gs[ng], 1))
          ++n4;
        else if (hxq::gemv_mfma_ok(a, pk12))
          ++n16;
      }
      ++ng;
    }
    if (ng == 0) return HXQ_OK;
    const bool xbf = x_dtype == HXQ_BF16;
    if (n4 == ng) {
      (void)hipGetLastError();
      if (hxq::gemv_mfma4_group_fits(gs, ng))
        return status_of(hxq::launch_gemv_mfma4_grouped(gs, ng, pk12, x, xbf, (int)M, (int)K, stream));
      for (int i = 0; i < ng; ++i) {
        const hipError_t err = hxq::launch_gemv_mfma4_grouped(&gs[i], 1, pk12, x, xbf, (int)M, (int)K, stream);
        if (err != hipSuccess) return status_of(err);
      }
      return HXQ_OK;
    }
    if (n16 == ng) {
      (void)hipGetLastError();
      if (hxq::gemv_mfma_group_fits(gs, ng))
        return status_of(hxq::launch_gemv_mfma_grouped(gs, ng, pk12, x, xbf, (int)M, (int)K, stream));
      for (int i = 0; i < ng; ++i) {
        const hipError_t err = hxq::launch_gemv_mfma_grouped(&gs[i], 1, pk12, x, xbf, (int)M, (int)K, stream);
        if (err != hipSuccess) return status_of(err);
      }
      return HXQ_OK;
    }
    if (n4 + n16 > 0) fast = false;  // mixed kernels: the per-layer calls below
  }
  if (fast) {
    (void)hipGetLastError();
    hipError_t err = hipSuccess;
    const bool xbf = x_dtype == HXQ_BF16;
    const bool done = M <= 4 ? hxq::decode_fits(segs, nseg, pk12, xbf, (int)M, (int)K) &&
                                   hxq::launch_decode(segs, nseg, pk12, x, xbf, (int)M, (int)K, stream, err)
                             : hxq::launch_decode_chunked(segs, nseg, pk12, x, xbf, (int)M, (int)K, stream, err);
    if (done) return status_of(err);
  }
  // one matrix-core launch for bf16 x past the decode sizes when every layer takes it
  if (x_dtype == HXQ_BF16 && M > 16 && K > 0) {
    hxq::GemmSeg gs[hxq::kMaxSegments];
    int ng = 0;
    bool ok = true;
    for (int i = 0; i < count && ok; ++i) {
      const hxq_layer& l = layers[i];
      if (l.N == 0) continue;
      hxq::LayerArgs a = {};
      a.codebook = l.codebook;
      a.indices = l.indices;
      a.x = x;
      a.x_bf16 = true;
      a.y = l.y;
      a.M = (int)M;
      a.N = (int)l.N;
      a.K = (int)K;
      ok = hxq::gemm2_path_ok(a, pk12);
      gs[ng++] = {static_cast<const float*>(l.codebook), l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz,
                  l.bias, l.y, (int)l.N, 0};
    }
    if (ok && ng == 0) return HXQ_OK;
    if (ok) {
      (void)hipGetLastError();
      return status_of(hxq::launch_gemm_grouped(gs, ng, pk12, x, (int)M, (int)K, stream));
    }
  }
  for (int i = 0; i < count; ++i) {
    const hxq_layer& l = layers[i];
    const int st = forward(pk12, l.codebook, l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz, x, x_dtype,
                           l.bias, l.y, M, l.N, K, stream, HXQ_VARIANT_AUTO);
    if (st != HXQ_OK) return st;
  }
  return HXQ_OK;
}

int hxq_stream_read(const void* src, int64_t bytes, uint32_t* sink, int sink_words, hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0 || sink_words < 1) return HXQ_ERR_SHAPE;
  if (bytes == 0) return HXQ_OK;
  if (!src || !sink) return HXQ_ERR_NULL;
  if (misaligned(src, 16) || misaligned(sink, 4)) return HXQ_ERR_ALIGN;
  (void)hipGetLastError();
  return status_of(hxq::launch_stream_read(src, bytes, sink, sink_words, stream));
}

int hxq_dequant_bf16(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                     const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, uint16_t* w, int64_t N,
                     int64_t K, hipStream_t stream) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  const bool pk12 = fmt == HXQ_FMT_PK12;
  if (N < 0 || K < 0 || nnz < 0 || N > kMaxDim || K > kMaxDim || nnz > kMaxDim) return HXQ_ERR_SHAPE;
  if (pk12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  if (N == 0 || K == 0) return HXQ_OK;
  if (!codebook || !indices || !w) return HXQ_ERR_NULL;
  if (nnz > 0 && (!sc_rows || !sc_cols || !sc_deltas)) return HXQ_ERR_NULL;
  if (misaligned(indices, pk12 ? 4 : 16) || misaligned(codebook, pk12 ? 8 : 4) || misaligned(w, 16) ||
      misaligned(sc_rows, 4) || misaligned(sc_cols, 4) || misaligned(sc_deltas, 4))
    return HXQ_ERR_ALIGN;
  if (K % 16 != 0) return HXQ_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return status_of(hxq::launch_dequant_bf16(pk12, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, w, N, K,
                                            stream));
}

int hxq_sidecar_add(const int32_t* sc_rows, const int32_t* sc_cols, const float* sc_deltas,
                    int64_t nnz, const void* x, int x_dtype, float* y, int64_t M, int64_t N,
                    int64_t K, hipStream_t stream) {
  if (x_dtype != HXQ_F32 && x_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || nnz < 0) return HXQ_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || nnz > kMaxDim) return HXQ_ERR_SHAPE;
  if (M == 0 || N == 0 || nnz == 0) return HXQ_OK;
  if (!sc_rows || !sc_cols || !sc_deltas || !y) return HXQ_ERR_NULL;
  if (K > 0 && !x) return HXQ_ERR_NULL;
  const uintptr_t xs = x_dtype == HXQ_BF16 ? 2 : 4;
  if (misaligned(x, xs) || misaligned(y, 4) || misaligned(sc_rows, 4) || misaligned(sc_cols, 4) ||
      misaligned(sc_deltas, 4))
    return HXQ_ERR_ALIGN;
  hxq::LayerArgs a = {};
  a.sc_rows = sc_rows;
  a.sc_cols = sc_cols;
  a.sc_deltas = sc_deltas;
  a.nnz = nnz;
  a.x = x;
  a.x_bf16 = x_dtype == HXQ_BF16;
  a.y = y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  (void)hipGetLastError();
  return status_of(hxq::launch_sidecar_add(a, stream));
}

int hxq_select_variant(int fmt_pk12, int x_dtype, int64_t M, int64_t N, int64_t K) {
  if (x_dtype != HXQ_F32 && x_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return HXQ_ERR_SHAPE;
  if (fmt_pk12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  const bool gemv_ok = K > 0 && K % 16 == 0;
  const bool gemm_ok = x_dtype == HXQ_BF16 && K > 0 && K % (fmt_pk12 ? 64 : 32) == 0;
  return select(fmt_pk12 != 0, x_dtype == HXQ_BF16, M, K, gemv_ok, gemm_ok);
}

const char* hxq_status_str(int status) {
  switch (status) {
    case HXQ_OK: return "ok";
    case HXQ_ERR_NULL: return "required pointer is NULL";
    case HXQ_ERR_SHAPE: return "invalid shape";
    case HXQ_ERR_DTYPE: return "unknown activation dtype";
    case HXQ_ERR_ALIGN: return "misaligned pointer";
    case HXQ_ERR_UNSUPPORTED: return "unsupported combination";
    case HXQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int hxq_version(void) { return 100; }

}  // extern "C"
