// C entry points of libhxq: argument validation on the host, then dispatch to
// one kernel family.  Nothing here touches device memory or allocates.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "../../include/hxq.h"
#include "hxq_launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)INT32_MAX - 65536;  // room for tile rounding in int32
constexpr int64_t kBwdMfmaMinM = 16;                       // input gradient: matrix cores from here
constexpr int64_t kBwdG5MinM = 128;                        // and the 256 x 256 tile kernel (u8) from here

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

// bf16 x past 16 tokens: the bf16 GEMM, except up to 64 tokens on a layer
// with fewer than 32 output tiles of 128 x 128 (N <= 3968), which leaves most
// CUs idle in the GEMM; there the fp32 matrix-core GEMV (bf16 upcast exactly)
// is faster.  Decided per layer, so a grouped call picks what single calls do.
bool bf16_gemm_wanted(int64_t M, int64_t N) {
  if (M <= 16) return false;
  if (M > 64) return true;
  return ((M + 127) / 128) * ((N + 127) / 128) >= 32;
}

int select(bool pk12, bool x_bf16, int64_t M, int64_t N, int64_t K, bool gemv_ok, bool gemm_ok) {
  if (K == 0) return HXQ_VARIANT_GENERIC;
  if (x_bf16 && gemm_ok && M > 16 && (bf16_gemm_wanted(M, N) || !gemv_ok)) return HXQ_VARIANT_GEMM_BF16;
  if (gemv_ok) return HXQ_VARIANT_GEMV_VALU;
  return HXQ_VARIANT_GENERIC;
}

int status_of(hipError_t e) { return e == hipSuccess ? HXQ_OK : HXQ_ERR_HIP; }

// The 256 x 256 tile GEMM (gemm5) against the 128-token one (gemm3): per
// tile it does more work per LDS byte and per gather, but a launch with few
// tiles leaves CUs idle (the prefill layers at 2048 tokens: q|k|v, o and down
// have 64 to 80 such tiles, gate|up 688).  A round of gemm5 tiles over the
// CUs takes about as long as gemm3 needs for 0.59 CUs' worth of tiles
// (measured at K = 2048: one round 78-85 us; gemm3 54 us for 86 tiles, 102
// us for 172), so gemm5 takes a launch whose tiles fill its rounds to at
// least that (gate|up at 512 tokens: 172 tiles), and the shapes only it can
// take.
bool gemm5_preferred(const hxq::GemmSeg* segs, int nseg, int M) {
  const int64_t t = hxq::gemm5_tiles(segs, nseg, M), cus = hxq::device_cu_count();
  const int64_t rounds = (t + cus - 1) / cus;
  return 100 * t >= 59 * cus * rounds;
}

int forward(bool pk12, const void* codebook, const uint8_t* indices, const int32_t* sc_rows,
            const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* x, int x_dtype,
            const float* bias, float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream,
            int variant) {
  int st = validate_forward(codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias,
                            y, M, N, K, pk12);
  if (st != HXQ_OK) return st;
  if (variant < HXQ_VARIANT_AUTO || variant > HXQ_VARIANT_GEMM_BF16_T256) return HXQ_ERR_UNSUPPORTED;
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
  const bool gemm_ok = K > 0 && (hxq::gemm5_path_ok(a, pk12) || (pk12 ? hxq::gemm2_path_ok(a, true) : hxq::gemm_path_ok(a)));
  int v = variant;
  if (v == HXQ_VARIANT_AUTO) v = select(pk12, a.x_bf16, M, N, K, gemv_ok, gemm_ok);
  (void)hipGetLastError();  // start from a clean error state
  switch (v) {
    case HXQ_VARIANT_GEMV_VALU:
      if (!gemv_ok) return HXQ_ERR_UNSUPPORTED;
      return status_of(hxq::launch_gemv_valu(a, pk12, stream));
    case HXQ_VARIANT_GEMV_MFMA:
      if (!gemv_ok || !hxq::gemv_mfma_takes(a, pk12)) return HXQ_ERR_UNSUPPORTED;
      return status_of(hxq::launch_gemv_mfma_tokens(a, pk12, stream));
    case HXQ_VARIANT_GEMM_BF16:
    case HXQ_VARIANT_GEMM_BF16_T256: {
      if (!gemm_ok) return HXQ_ERR_UNSUPPORTED;
      const hxq::GemmSeg sg = {static_cast<const float*>(a.codebook), a.indices, a.sc_rows, a.sc_cols,
                               a.sc_deltas, a.nnz, a.bias, a.y, a.N, 0};
      const bool g5 = hxq::gemm5_path_ok(a, pk12);
      const bool g3 = hxq::gemm2_path_ok(a, pk12);
      if (v == HXQ_VARIANT_GEMM_BF16_T256) {
        if (!g5) return HXQ_ERR_UNSUPPORTED;
        return status_of(hxq::launch_gemm5_grouped(&sg, 1, pk12, a.x, a.M, a.K, stream));
      }
      if (g5 && (!g3 || gemm5_preferred(&sg, 1, a.M)))
        return status_of(hxq::launch_gemm5_grouped(&sg, 1, pk12, a.x, a.M, a.K, stream));
      if (g3) return status_of(hxq::launch_gemm2_bf16(a, pk12, stream));
      return status_of(hxq::launch_gemm_bf16(a, stream));  // u8 only (pk12 passed the check above)
    }
    case HXQ_VARIANT_GENERIC:
      return status_of(hxq::launch_generic(a, pk12, stream));
    default:
      return HXQ_ERR_UNSUPPORTED;
  }
}

// Argument checks of the input gradient (host only).  Returns HXQ_OK or an error.
int validate_bwd(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                 const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* dy, int dy_dtype,
                 const float* dx, int64_t M, int64_t N, int64_t K, const void* workspace, int64_t workspace_bytes,
                 int variant) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  const bool pk12 = fmt == HXQ_FMT_PK12;
  if (dy_dtype != HXQ_F32 && dy_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || nnz < 0 || workspace_bytes < 0) return HXQ_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || nnz > kMaxDim) return HXQ_ERR_SHAPE;
  if (pk12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  if (variant != HXQ_VARIANT_AUTO && variant != HXQ_VARIANT_GEMV_VALU && variant != HXQ_VARIANT_GEMM_BF16 &&
      variant != HXQ_VARIANT_GEMM_BF16_T256)
    return HXQ_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return HXQ_OK;
  if (!dx) return HXQ_ERR_NULL;
  if (N > 0 && (!dy || !indices || !codebook)) return HXQ_ERR_NULL;
  if (nnz > 0 && (!sc_rows || !sc_cols || !sc_deltas)) return HXQ_ERR_NULL;
  const uintptr_t ds = dy_dtype == HXQ_BF16 ? 2 : 4;
  if (misaligned(dy, ds) || misaligned(dx, 4) || misaligned(codebook, 4) || misaligned(sc_rows, 4) ||
      misaligned(sc_cols, 4) || misaligned(sc_deltas, 4) || misaligned(workspace, 4))
    return HXQ_ERR_ALIGN;
  return HXQ_OK;
}

int backward_x(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
               const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* dy, int dy_dtype,
               float* dx, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
               hipStream_t stream, int variant) {
  const int vst = validate_bwd(fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, dy, dy_dtype, dx, M, N, K,
                               workspace, workspace_bytes, variant);
  if (vst != HXQ_OK) return vst;
  const bool pk12 = fmt == HXQ_FMT_PK12;
  if (M == 0 || K == 0) return HXQ_OK;
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
  // the bf16 matrix-core kernels past 16 tokens (256 x 256 tiles from 128
  // tokens, u8), when the shape, the pointers and the workspace (row splits
  // and sidecar bins) allow them
  auto fits = [&](const hxq::BwdMPlan& p) {
    const int64_t need = p.split_bytes + p.bin_bytes;
    return need == 0 || (workspace && workspace_bytes >= need);
  };
  const bool g5 = hxq::bwdx_g5_ok(a, pk12) && fits(hxq::bwdx_g5_plan(a.M, a.N, a.K, nnz));
  const bool mfma = hxq::bwdx_mfma_ok(a, pk12) && fits(hxq::bwdx_mfma_plan(a.M, a.N, a.K, nnz));
  if (variant == HXQ_VARIANT_GEMM_BF16_T256)
    return g5 ? status_of(hxq::launch_bwdx_g5(a, stream)) : HXQ_ERR_UNSUPPORTED;
  if (variant == HXQ_VARIANT_GEMM_BF16)
    return mfma ? status_of(hxq::launch_bwdx_mfma(a, pk12, stream)) : HXQ_ERR_UNSUPPORTED;
  if (variant == HXQ_VARIANT_AUTO && M >= kBwdMfmaMinM) {
    if (g5 && M >= kBwdG5MinM) return status_of(hxq::launch_bwdx_g5(a, stream));
    if (mfma) return status_of(hxq::launch_bwdx_mfma(a, pk12, stream));
  }
  return status_of(hxq::launch_bwdx_valu(a, pk12, stream));
}

// The matrix-core kernel AUTO runs for one layer from kBwdMfmaMinM tokens
// (0: none takes it): 2 = 256 x 256 tiles, 1 = the 64-token kernel.
int bwd_mm_kernel(const hxq::BwdArgs& a, bool pk12) {
  if (a.M >= kBwdG5MinM && hxq::bwdx_g5_ok(a, pk12)) return 2;
  return hxq::bwdx_mfma_ok(a, pk12) ? 1 : 0;
}

hxq::BwdMPlan bwd_mm_plan(int kernel, const hxq::BwdArgs& a) {
  return kernel == 2 ? hxq::bwdx_g5_plan(a.M, a.N, a.K, a.nnz) : hxq::bwdx_mfma_plan(a.M, a.N, a.K, a.nnz);
}

// ---- forward with a workspace: the k split of the 256 x 256 tile GEMM

// The split plan AUTO would use for this layer with a workspace (S < 2: none).
hxq::Gemm5Split fwd_split_plan(bool pk12, const hxq::LayerArgs& a) {
  const hxq::Gemm5Split none = {1, 0, 0};
  if (!a.x_bf16 || a.K <= 0 || !hxq::gemm5_path_ok(a, pk12)) return none;
  const bool gemv_ok = hxq::gemv_fast_path_ok(a, pk12);
  if (select(pk12, true, a.M, a.N, a.K, gemv_ok, true) != HXQ_VARIANT_GEMM_BF16) return none;
  return hxq::gemm5_split_plan(a.M, a.N, a.K);
}

int forward_ws(int fmt, const void* codebook, const uint8_t* indices, const int32_t* sc_rows, const int32_t* sc_cols,
               const float* sc_deltas, int64_t nnz, const void* x, int x_dtype, const float* bias, float* y, int64_t M,
               int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  const bool pk12 = fmt == HXQ_FMT_PK12;
  const int st = validate_forward(codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y, M, N, K,
                                  pk12);
  if (st != HXQ_OK) return st;
  if (workspace_bytes < 0) return HXQ_ERR_SHAPE;
  if (misaligned(workspace, 16)) return HXQ_ERR_ALIGN;
  if (M > 0 && N > 0 && K > 0) {
    hxq::LayerArgs a = {};
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
    const hxq::Gemm5Split p = fwd_split_plan(pk12, a);
    if (p.S >= 2 && workspace && workspace_bytes >= p.bytes) {
      (void)hipGetLastError();
      const hxq::GemmSeg sg = {static_cast<const float*>(codebook), indices, sc_rows, sc_cols, sc_deltas, nnz, bias, y,
                               (int)N, 0};
      return status_of(hxq::launch_gemm5_split(sg, pk12, x, (int)M, (int)K, static_cast<float*>(workspace),
                                               workspace_bytes, stream));
    }
  }
  return forward(pk12, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y, M, N, K, stream,
                 HXQ_VARIANT_AUTO);
}

// ---- grouped input gradient: dx = sum over layers of dy_i W_i

hxq::BwdArgs bwd_args_of(const hxq_bwd_layer& l, bool dy_bf16, float* dx, int64_t M, int64_t K) {
  hxq::BwdArgs a = {};
  a.codebook = static_cast<const float*>(l.codebook);
  a.indices = l.indices;
  a.sc_rows = l.sc_rows;
  a.sc_cols = l.sc_cols;
  a.sc_deltas = l.sc_deltas;
  a.nnz = l.nnz;
  a.dy = l.dy;
  a.dy_bf16 = dy_bf16;
  a.dx = dx;
  a.M = (int)M;
  a.N = (int)l.N;
  a.K = (int)K;
  return a;
}

// The path of a call over n >= 2 layers with N > 0 and the workspace it
// needs: with matrix-core products the sidecar bins of one layer at a time
// (the layers run in turn) and then every layer's row splits; on the vector
// path the splits of its single launch.  aligned: plan for 16-byte aligned
// pointers (the workspace query) instead of the layers' own.
struct BwdGroupWs {
  bool mfma;
  bool g5group;               // every layer on the 256 x 256 tile kernel: one launch for all
  int kernel[HXQ_MAX_GROUP];  // per layer, with matrix cores: as bwd_mm_kernel
  int64_t bin_bytes;          // a multiple of 256: the split slots follow
  int slots;
  int64_t bytes;
};

BwdGroupWs plan_group(bool pk12, bool dy_bf16, const hxq_bwd_layer* act, int n, int64_t M, int64_t K, float* dx,
                      bool aligned) {
  const int64_t per = M * K * 4;
  bool mfma = dy_bf16 && M >= kBwdMfmaMinM;
  BwdGroupWs w = {};
  for (int i = 0; i < n && mfma; ++i) {
    hxq::BwdArgs a = bwd_args_of(act[i], dy_bf16, dx, M, K);
    if (aligned) {
      a.indices = reinterpret_cast<const uint8_t*>(uintptr_t(256));
      a.dy = reinterpret_cast<const void*>(uintptr_t(256));
      a.dx = reinterpret_cast<float*>(uintptr_t(256));
    }
    w.kernel[i] = bwd_mm_kernel(a, pk12);
    mfma = w.kernel[i] != 0;
  }
  w.mfma = mfma;
  w.g5group = mfma;
  for (int i = 0; i < n && mfma; ++i) w.g5group = w.g5group && w.kernel[i] == 2;
  if (w.g5group) {
    int Ns[hxq::kMaxSegments];
    int64_t nnzs[hxq::kMaxSegments];
    for (int i = 0; i < n; ++i) {
      Ns[i] = (int)act[i].N;
      nnzs[i] = act[i].nnz;
    }
    const hxq::BwdG5Group g = hxq::bwdx_g5_group_plan((int)M, (int)K, Ns, nnzs, n);
    w.bin_bytes = g.bin_total;
    w.slots = g.slots;
  } else if (mfma) {
    for (int i = 0; i < n; ++i) {
      const hxq::BwdMPlan p = bwd_mm_plan(w.kernel[i], bwd_args_of(act[i], dy_bf16, dx, M, K));
      w.bin_bytes = std::max(w.bin_bytes, p.bin_bytes);
      w.slots += p.S;
    }
  } else {
    int Ns[hxq::kMaxSegments];
    for (int i = 0; i < n; ++i) Ns[i] = (int)act[i].N;
    w.slots = hxq::bwdx_group_plan((int)M, Ns, n, (int)K).slots_total;
  }
  w.bytes = w.bin_bytes + (int64_t)w.slots * per;
  return w;
}

int check_group(int fmt, const hxq_bwd_layer* layers, int count, int dy_dtype) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  if (count < 1 || count > HXQ_MAX_GROUP) return HXQ_ERR_SHAPE;
  if (dy_dtype != HXQ_F32 && dy_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (!layers) return HXQ_ERR_NULL;
  return HXQ_OK;
}

int backward_x_grouped(int fmt, const hxq_bwd_layer* layers, int count, int dy_dtype, float* dx, int64_t M,
                       int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  int st = check_group(fmt, layers, count, dy_dtype);
  if (st != HXQ_OK) return st;
  for (int i = 0; i < count; ++i) {
    const hxq_bwd_layer& l = layers[i];
    st = validate_bwd(fmt, static_cast<const float*>(l.codebook), l.indices, l.sc_rows, l.sc_cols, l.sc_deltas,
                      l.nnz, l.dy, dy_dtype, dx, M, l.N, K, workspace, workspace_bytes, HXQ_VARIANT_AUTO);
    if (st != HXQ_OK) return st;
  }
  if (misaligned(workspace, 16)) return HXQ_ERR_ALIGN;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += layers[i].N;
  if (rows > kMaxDim) return HXQ_ERR_SHAPE;  // the layers' rows are split as one range
  if (M == 0 || K == 0) return HXQ_OK;
  hxq_bwd_layer act[HXQ_MAX_GROUP];
  int n = 0;
  for (int i = 0; i < count; ++i)
    if (layers[i].N > 0) act[n++] = layers[i];
  if (n <= 1) {
    if (n == 0) {
      (void)hipGetLastError();
      return status_of(hxq::launch_fill_zero(dx, M * K, stream));
    }
    const hxq_bwd_layer& l = act[0];
    return backward_x(fmt, static_cast<const float*>(l.codebook), l.indices, l.sc_rows, l.sc_cols, l.sc_deltas,
                      l.nnz, l.dy, dy_dtype, dx, M, l.N, K, workspace, workspace_bytes, stream, HXQ_VARIANT_AUTO);
  }
  const bool pk12 = fmt == HXQ_FMT_PK12, dy_bf16 = dy_dtype == HXQ_BF16;
  const BwdGroupWs w = plan_group(pk12, dy_bf16, act, n, M, K, dx, false);
  if (workspace == nullptr || workspace_bytes < w.bytes) return HXQ_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  unsigned char* wb = static_cast<unsigned char*>(workspace);
  if (w.g5group) {
    hxq::BwdArgs ls[HXQ_MAX_GROUP];
    for (int i = 0; i < n; ++i) ls[i] = bwd_args_of(act[i], dy_bf16, dx, M, K);
    float* slots = reinterpret_cast<float*>(wb + w.bin_bytes);
    const hipError_t e = hxq::launch_bwdx_g5_grouped(ls, n, slots, wb, stream);
    if (e != hipSuccess) return status_of(e);
    return status_of(hxq::launch_bwdx_reduce(slots, dx, M * K, w.slots, stream));
  }
  if (w.mfma) {
    float* slots = reinterpret_cast<float*>(wb + w.bin_bytes);
    int slot0 = 0;
    for (int i = 0; i < n; ++i) {
      hxq::BwdArgs a = bwd_args_of(act[i], dy_bf16, dx, M, K);
      a.ws = reinterpret_cast<float*>(wb);
      a.ws_bytes = w.bin_bytes;
      a.slots = slots;
      a.slot0 = slot0;
      const hipError_t e = w.kernel[i] == 2 ? hxq::launch_bwdx_g5(a, stream) : hxq::launch_bwdx_mfma(a, pk12, stream);
      if (e != hipSuccess) return status_of(e);
      slot0 += bwd_mm_plan(w.kernel[i], a).S;
    }
    return status_of(hxq::launch_bwdx_reduce(slots, dx, M * K, slot0, stream));
  }
  hxq::BwdArgs a = bwd_args_of(act[0], dy_bf16, dx, M, K);
  a.ws = reinterpret_cast<float*>(wb);
  a.ws_bytes = workspace_bytes;
  a.nseg = n;
  for (int i = 0; i < n; ++i) {
    const hxq_bwd_layer& l = act[i];
    a.seg[i] = {static_cast<const float*>(l.codebook), l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz, l.dy,
                (int)l.N, 0, 0};
  }
  return status_of(hxq::launch_bwdx_valu_grouped(a, pk12, stream));
}

// ---- device scratch of the allocation-free input gradient.  One array per
// GPU (each device holds its own copy of this module's globals), kept until
// the process ends.  In host code `scratch` only names the symbol: its
// device address comes from hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) unsigned char scratch[HXQ_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address (set up on the first call on that
// device, with it current).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HXQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HXQ_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HXQ_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return HXQ_OK;
}

}  // namespace

extern "C" {

int hxq_linear_bwd_x_noalloc(int fmt, const float* codebook, const uint8_t* indices, const int32_t* sc_rows,
                             const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* dy,
                             int dy_dtype, float* dx, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int vst = validate_bwd(fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, dy, dy_dtype, dx, M, N, K,
                               nullptr, 0, HXQ_VARIANT_AUTO);
  if (vst != HXQ_OK) return vst;
  if (M == 0 || K == 0) return HXQ_OK;
  // the workspace the allocating entry point would be given
  const int64_t need = hxq_linear_bwd_x_workspace(fmt, dy_dtype, M, N, K, nnz);
  if (need < 0) return (int)need;
  if (need > (int64_t)HXQ_SCRATCH_BYTES) return HXQ_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != HXQ_OK) return st;
  }
  return backward_x(fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, dy, dy_dtype, dx, M, N, K, ws, need,
                    stream, HXQ_VARIANT_AUTO);
}

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
  a.nnz = nnz;
  const int kernel = M >= kBwdMfmaMinM ? bwd_mm_kernel(a, fmt == HXQ_FMT_PK12) : 0;
  if (kernel != 0) {
    const hxq::BwdMPlan p = bwd_mm_plan(kernel, a);
    return p.split_bytes + p.bin_bytes;
  }
  return hxq::bwdx_workspace_bytes((int)M, (int)N, (int)K);
}

int hxq_linear_bwd_x_grouped(int fmt, const hxq_bwd_layer* layers, int count, int dy_dtype, float* dx, int64_t M,
                             int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return backward_x_grouped(fmt, layers, count, dy_dtype, dx, M, K, workspace, workspace_bytes, stream);
}

int64_t hxq_linear_bwd_x_grouped_workspace(int fmt, int dy_dtype, const hxq_bwd_layer* layers, int count, int64_t M,
                                           int64_t K) {
  const int st = check_group(fmt, layers, count, dy_dtype);
  if (st != HXQ_OK) return st;
  if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return HXQ_ERR_SHAPE;
  if (fmt == HXQ_FMT_PK12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  hxq_bwd_layer act[HXQ_MAX_GROUP];
  int n = 0;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) {
    const hxq_bwd_layer& l = layers[i];
    if (l.N < 0 || l.N > kMaxDim || l.nnz < 0 || l.nnz > kMaxDim) return HXQ_ERR_SHAPE;
    rows += l.N;
    if (l.N > 0) act[n++] = l;
  }
  if (rows > kMaxDim) return HXQ_ERR_SHAPE;
  if (M == 0 || K == 0 || n == 0) return 0;
  if (n == 1) return hxq_linear_bwd_x_workspace(fmt, dy_dtype, M, act[0].N, K, act[0].nnz);
  return plan_group(fmt == HXQ_FMT_PK12, dy_dtype == HXQ_BF16, act, n, M, K, nullptr, true).bytes;
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

int hxq_linear_fwd_ws(int fmt, const void* codebook, const uint8_t* indices, const int32_t* sc_rows,
                      const int32_t* sc_cols, const float* sc_deltas, int64_t nnz, const void* x, int x_dtype,
                      const float* bias, float* y, int64_t M, int64_t N, int64_t K, void* workspace,
                      int64_t workspace_bytes, hipStream_t stream) {
  return forward_ws(fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, nnz, x, x_dtype, bias, y, M, N, K, workspace,
                    workspace_bytes, stream);
}

int64_t hxq_linear_fwd_workspace(int fmt, int x_dtype, int64_t M, int64_t N, int64_t K) {
  if (fmt != HXQ_FMT_U8 && fmt != HXQ_FMT_PK12) return HXQ_ERR_SHAPE;
  if (x_dtype != HXQ_F32 && x_dtype != HXQ_BF16) return HXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return HXQ_ERR_SHAPE;
  if (fmt == HXQ_FMT_PK12 && (K % 2) != 0) return HXQ_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0) return 0;
  // the plan for 16-byte aligned pointers
  hxq::LayerArgs a = {};
  a.indices = reinterpret_cast<const uint8_t*>(uintptr_t(256));
  a.codebook = reinterpret_cast<const void*>(uintptr_t(256));
  a.x = reinterpret_cast<const void*>(uintptr_t(256));
  a.y = reinterpret_cast<float*>(uintptr_t(256));
  a.x_bf16 = x_dtype == HXQ_BF16;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  const hxq::Gemm5Split p = fwd_split_plan(fmt == HXQ_FMT_PK12, a);
  return p.S >= 2 ? p.bytes : 0;
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
  // From 2 to 64 tokens the matrix-core GEMVs, with the kernel a single-layer
  // call would pick for each layer (2 to 8 tokens: the 4x4-block GEMV where it
  // takes the layer, else the 16x16 one from 5 tokens and the decode kernel up
  // to 4; u8 with bf16 x past 16 tokens goes to
  // the bf16 GEMM instead where it wants the layer): one launch when every
  // layer takes the same kernel and the group fits one workgroup per CU, one
  // launch per layer when they take the same kernel but do not fit together,
  // else the per-layer calls.
  int want_gemm = 0, want_gemv = 0;
  if (x_dtype == HXQ_BF16 && M > 16)
    for (int i = 0; i < count; ++i)
      if (layers[i].N > 0) ++(bf16_gemm_wanted(M, layers[i].N) ? want_gemm : want_gemv);
  if (K > 0 && M >= 2 && M <= hxq::kGemvMfmaMaxM && want_gemm == 0) {
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
        else if (M > 4 && hxq::gemv_mfma_ok(a, pk12))
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
  // one matrix-core launch for bf16 x past the decode sizes when every layer
  // takes it and wants it
  if (x_dtype == HXQ_BF16 && M > 16 && K > 0 && want_gemv == 0) {
    hxq::GemmSeg gs[hxq::kMaxSegments];
    int ng = 0;
    bool ok5 = true, ok3 = true, ok = true;
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
      ok5 = ok5 && hxq::gemm5_path_ok(a, pk12);
      ok3 = ok3 && hxq::gemm2_path_ok(a, pk12);
      ok = ok5 || ok3;
      gs[ng++] = {static_cast<const float*>(l.codebook), l.indices, l.sc_rows, l.sc_cols, l.sc_deltas, l.nnz,
                  l.bias, l.y, (int)l.N, 0};
    }
    if (ok && ng == 0) return HXQ_OK;
    if (ok) {
      (void)hipGetLastError();
      if (ok5 && (!ok3 || gemm5_preferred(gs, ng, (int)M)))
        return status_of(hxq::launch_gemm5_grouped(gs, ng, pk12, x, (int)M, (int)K, stream));
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

static int stream_read(const void* src, int64_t bytes, uint32_t* sink, int sink_words, bool nt,
                       hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0 || sink_words < 8) return HXQ_ERR_SHAPE;
  if (bytes == 0) return HXQ_OK;
  if (!src || !sink) return HXQ_ERR_NULL;
  if (misaligned(src, 16) || misaligned(sink, 4)) return HXQ_ERR_ALIGN;
  (void)hipGetLastError();
  return status_of(hxq::launch_stream_read(src, bytes, sink, sink_words, nt, stream));
}

int hxq_stream_read(const void* src, int64_t bytes, uint32_t* sink, int sink_words, hipStream_t stream) {
  return stream_read(src, bytes, sink, sink_words, false, stream);
}

int hxq_stream_read_nt(const void* src, int64_t bytes, uint32_t* sink, int sink_words, hipStream_t stream) {
  return stream_read(src, bytes, sink, sink_words, true, stream);
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
  const bool gemm_ok = x_dtype == HXQ_BF16 && K > 0 && K % 32 == 0;
  return select(fmt_pk12 != 0, x_dtype == HXQ_BF16, M, N, K, gemv_ok, gemm_ok);
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
    case HXQ_ERR_SCRATCH: return "the call needs more device scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int hxq_version(void) { return 100; }

#ifndef HXQ_SOURCE_DIGEST
#define HXQ_SOURCE_DIGEST "unknown"
#endif

const char* hxq_source_digest(void) { return HXQ_SOURCE_DIGEST; }

}  // extern "C"
