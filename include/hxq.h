/*
 * libhxq: the HelixLinear forward pass computed from the compressed weights.
 *
 * A HelixLinear layer (model cards "Zamba2-1.2B-HXQ", "Mamba2-1.3B-HXQ",
 * "Qwen2.5-3B-Instruct-HXQ", section "What is HelixCode?") replaces an
 * nn.Linear weight W [N out, K in] by a float32 codebook, an index per weight
 * and sparse sidecar corrections, and computes codebook[indices] @ x without
 * forming W.  The HXQ whitepaper (J. P. Fellows, Echo Labs, 2026) gives the
 * two index formats ("Method"; "2D vector quantization"):
 *   u8   - 256-entry float32 codebook, one uint8 index per weight;
 *   pk12 - 4096-entry codebook of float32 pairs over adjacent weights, two
 *          12-bit indices packed into 3 bytes;
 * and the sidecar: sparse (row, col, delta) triplets that correct the weights
 * with the largest reconstruction error ("Method", sidecar outlier
 * correction).  Every entry point computes, for m < M and n < N,
 *
 *     y[m][n] = sum_k (C[idx[n][k]] + S[n][k]) * x[m][k] + bias[n]
 *
 * where S[n][k] is the sum of the deltas of the triplets at (n, k).
 *
 * Conventions shared by all entry points
 *   - Every pointer is device memory owned by the caller.  The library
 *     allocates nothing, keeps no per-call state and never reads device memory
 *     on the host.  Work is queued on `stream` (0 = the null stream) and the
 *     call returns without waiting for it.
 *   - Row-major layouts: indices [N][K] (u8) or [N][3*ceil(K/4)] (pk12),
 *     x [M][K], y [M][N].  y must not overlap any input.
 *   - x_dtype: HXQ_F32 (float) or HXQ_BF16 (bf16 bit patterns, uint16).
 *     y is always float32.
 *   - Sidecar: sc_rows / sc_cols int32, sc_deltas float32, nnz entries,
 *     sorted by (row, col) in non-decreasing order; repeated coordinates add.
 *     Entries out of range or out of order are undefined behaviour (they are
 *     never checked on the device).  With nnz == 0 the three pointers may be
 *     NULL.
 *   - bias may be NULL (no bias).
 *   - M == 0 or N == 0: nothing is launched, HXQ_OK.  K == 0: y = bias (or 0).
 *   - Arithmetic: fp32 activations are multiplied in fp32 with fp32
 *     accumulation (vector FMAs for one token, fp32 matrix-core products
 *     from two, which are exact fp32 products summed in fp32; up to 4 tokens
 *     vector FMAs again where the matrix-core GEMV does not take the layer:
 *     K % 256 != 0 or misaligned pointers); bf16 activations
 *     are upcast exactly and take the same fp32 path, except with M > 64, or
 *     17 <= M <= 64 on a layer with N > 3968 (at least 32 output tiles of
 *     128 x 128), which runs on bf16 matrix cores with fp32 accumulation
 *     (K % 32 == 0 for both formats).  There the weight operand at (n, k) is the codebook value
 *     plus every sidecar delta at (n, k), summed in fp32 in stored order and
 *     rounded once to bf16 (nearest, ties to even): the sidecar correction is
 *     folded into the operand, so an outlier's corrected weight carries one
 *     bf16 rounding like every other weight (relative 2^-9), instead of
 *     entering as an exact fp32 delta * x term.  (A 256 x 256 output tile
 *     of the 256-token kernel with more than 4096 sidecar entries, or with
 *     K > 12288, instead uses the plain codebook operand and adds
 *     x * (bf16(C + deltas) - bf16(C)) per distinct (n, k) in fp32 after the
 *     matrix ops: the same products, summed in another order.)  The
 *     tolerance of that path, 8e-3 of |X| |W|^T, covers it.
 *   - Errors are returned as a negative hxq_status before anything is
 *     launched; HXQ_ERR_HIP reports a failed launch.
 */
#ifndef HXQ_H
#define HXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* the same tag HIP uses */

enum hxq_status {
  HXQ_OK = 0,
  HXQ_ERR_NULL = -1,        /* a required pointer is NULL while its extent is > 0 */
  HXQ_ERR_SHAPE = -2,       /* negative M, N, K or nnz; odd K for pk12; M, N, K >= 2^31 */
  HXQ_ERR_DTYPE = -3,       /* x_dtype is not HXQ_F32 or HXQ_BF16 */
  HXQ_ERR_ALIGN = -4,       /* x not aligned to its element size, or y / codebook / bias /
                               sidecar arrays not 4-byte aligned */
  HXQ_ERR_UNSUPPORTED = -5, /* a combination this version does not implement */
  HXQ_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  HXQ_ERR_SCRATCH = -7      /* hxq_linear_bwd_x_noalloc: the call needs more than HXQ_SCRATCH_BYTES */
};

enum hxq_dtype { HXQ_F32 = 0, HXQ_BF16 = 1 };

/* Forward pass, 1D VQ (u8).
 *   codebook  [256] float32 (model cards, "What is HelixCode?").
 *   indices   [N][K] uint8, row-major, one index per weight.
 *   sc_*      sidecar triplets as described above.
 *   x         [M][K] float32 or bf16; bias [N] float32 or NULL; y [M][N] float32,
 *             overwritten. */
int hxq_linear_fwd_u8(const float* codebook, const uint8_t* indices,
                      const int32_t* sc_rows, const int32_t* sc_cols,
                      const float* sc_deltas, int64_t nnz,
                      const void* x, int x_dtype, const float* bias, float* y,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Forward pass, 2D VQ with 12-bit indices (pk12).
 *   codebook2 [4096][2] float32 pairs (HXQ whitepaper, "2D vector quantization").
 *             Weights (2j, 2j+1) of a row take components 0 and 1 of the entry
 *             selected by that row's index j.
 *   packed    [N][3*ceil(K/4)] uint8.  Group t of a row (its bytes 3t..3t+2)
 *             holds the row's indices 2t (a) and 2t+1 (b) as the little-endian
 *             24-bit word v = a | b << 12: byte0 = a[7:0], byte1 = a[11:8] | b[3:0] << 4,
 *             byte2 = b[11:4].  When K = 2 (mod 4) the last group's b is 0 and unused
 *             (HXQ whitepaper, "Method", 12-bit index packing; the byte order is this
 *             library's choice).
 *   K must be even.  All other arguments as for hxq_linear_fwd_u8.  bf16 x is
 *   accepted at every M and takes the fp32 path or the bf16 matrix cores by
 *   the same rule as the u8 format (weights rounded to bf16 as described
 *   above); K % 32 != 0 always takes the fp32 path. */
int hxq_linear_fwd_pk12(const float* codebook2, const uint8_t* packed,
                        const int32_t* sc_rows, const int32_t* sc_cols,
                        const float* sc_deltas, int64_t nnz,
                        const void* x, int x_dtype, const float* bias, float* y,
                        int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* The forward of either format (fmt: HXQ_FMT_U8 or HXQ_FMT_PK12; codebook
 * and indices as for hxq_linear_fwd_u8 / hxq_linear_fwd_pk12) with a caller
 * workspace.  A layer with bf16 x that the matrix-core GEMM takes but whose
 * 256 x 256 output tiles are too few to fill the GPU while K is long
 * (K >= 4096: the 11008 -> 2048 down projection at 512 or 2048 tokens) then
 * splits its sum over k into runs of at least 24 32-deep stages: each run's
 * partial sums go to the workspace, and a second launch adds them into y in
 * run order (the bias and, on the sidecar's walk path, its terms in the
 * first run).  The result is within the bf16 tolerance of the single-launch
 * product, not bitwise the same (another summation order).  Any other call,
 * or a workspace smaller than hxq_linear_fwd_workspace gives, computes
 * exactly what hxq_linear_fwd_u8 / hxq_linear_fwd_pk12 compute.
 *   workspace  caller-owned device memory, 16-byte aligned, workspace_bytes
 *              long (NULL with 0: none); contents on entry ignored and on
 *              return unspecified; two calls in flight at once need separate
 *              workspaces.
 * Errors: those of hxq_linear_fwd_u8 / _pk12, HXQ_ERR_SHAPE for an unknown fmt
 * or negative workspace_bytes, HXQ_ERR_ALIGN for a misaligned workspace. */
int hxq_linear_fwd_ws(int fmt, const void* codebook, const uint8_t* indices,
                      const int32_t* sc_rows, const int32_t* sc_cols,
                      const float* sc_deltas, int64_t nnz,
                      const void* x, int x_dtype, const float* bias, float* y,
                      int64_t M, int64_t N, int64_t K,
                      void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace hxq_linear_fwd_ws uses on the current device for these
 * sizes with 16-byte aligned pointers (0 when it would not split), or a
 * negative hxq_status for arguments it would reject (HXQ_ERR_SHAPE,
 * HXQ_ERR_DTYPE).  Host only. */
int64_t hxq_linear_fwd_workspace(int fmt, int x_dtype, int64_t M, int64_t N, int64_t K);

/* The sidecar term alone, accumulated into y:
 *     y[m][r] += sum over triplets (r, c, d) of d * x[m][c]      (fp32)
 * (HXQ whitepaper, "Method", sidecar outlier correction, applied to the
 * activations instead of the weights).  y [M][N] is read and written; the
 * sidecar must be sorted as above.  Deterministic: each output element is
 * summed in triplet order by one thread. */
int hxq_sidecar_add(const int32_t* sc_rows, const int32_t* sc_cols,
                    const float* sc_deltas, int64_t nnz,
                    const void* x, int x_dtype, float* y,
                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Several layers applied to the same activations in one call, for instance
 * the query, key and value projections of an attention block or the gate and
 * up projections of an MLP block.  Each layer keeps its own codebook, indices,
 * sidecar, bias and output (the HXQ whitepaper fits one codebook per weight
 * tensor, "Method"); all share the format, x, M and K.  Each layer's y is what
 * hxq_linear_fwd_u8 / hxq_linear_fwd_pk12 would compute for it, within the
 * same tolerance (bitwise the same where the single-layer call would run the
 * same kernel); the layers normally run in a single launch (up to 64 tokens,
 * and with bf16 x at any M where K % 32 == 0), otherwise one after another on
 * `stream`.
 *   fmt     HXQ_FMT_U8 or HXQ_FMT_PK12.
 *   layers  host array of `count` descriptors, 1 <= count <= HXQ_MAX_GROUP,
 *           read during the call only.  Each field means what the argument of
 *           the same name means for the single-layer entry points; a layer
 *           with N == 0 is skipped.
 *   x, x_dtype, M, K, stream as for the single-layer entry points.
 * Errors: HXQ_ERR_SHAPE for count out of range or an unknown fmt, otherwise the
 * first error the single-layer entry point would return for any layer;
 * nothing is launched when an error is returned. */
enum hxq_format { HXQ_FMT_U8 = 0, HXQ_FMT_PK12 = 1 };

#define HXQ_MAX_GROUP 8

typedef struct hxq_layer {
  const void* codebook;     /* u8: float[256]; pk12: float[4096][2] */
  const uint8_t* indices;   /* u8: [N][K]; pk12: [N][3*ceil(K/4)] */
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const float* bias;        /* [N] or NULL */
  float* y;                 /* [M][N] float32, overwritten */
  int64_t N;
} hxq_layer;

int hxq_linear_fwd_grouped(int fmt, const hxq_layer* layers, int count,
                           const void* x, int x_dtype, int64_t M, int64_t K,
                           hipStream_t stream);

/* Measurement helper, not part of the forward pass: reads `bytes` bytes of
 * device memory at `src` once with sink_words / 8 workgroups of 512 threads
 * (fewer when the buffer needs fewer, at most 65535; 16-byte loads, the whole
 * grid sweeping the buffer in order, four loads in flight per thread and the
 * next four requested before they are used), and each wave stores a 32-bit
 * digest of what it read into `sink` (device memory, `sink_words` entries;
 * word 8 g + w for wave w of workgroup g; the words of workgroups not
 * launched are left as they were, so with a zeroed sink the XOR of all words
 * is the XOR of all 32-bit words read).  Timed over a sweep of grid sizes it
 * gives the attainable read bandwidth that the decode kernels' HBM fraction
 * is compared against.
 * Errors: HXQ_ERR_SHAPE if bytes < 0 or not a multiple of 16 or sink_words < 8,
 * HXQ_ERR_NULL for a NULL pointer with bytes > 0, HXQ_ERR_ALIGN if src is not
 * 16-byte aligned or sink not 4-byte aligned. */
int hxq_stream_read(const void* src, int64_t bytes, uint32_t* sink, int sink_words,
                    hipStream_t stream);

/* The same read with non-temporal loads (the form the decode and
 * input-gradient kernels use for launches that stream more index bytes than
 * the L2 caches hold); same arguments, digest and errors.  The attainable
 * read bandwidth is the better of the two over the grid sweep. */
int hxq_stream_read_nt(const void* src, int64_t bytes, uint32_t* sink, int sink_words,
                       hipStream_t stream);

/* Measurement helper, not part of the forward pass: the dense bf16 weight of
 * one layer, for timing the buffered design the HXQ whitepaper's inference
 * paragraph describes (gather the weight into a shared bf16 buffer, then a
 * library matmul) against the fused kernels, which never form it.
 *   w[n][k] = bf16(C[idx[n][k]] + the sidecar deltas at (n, k)), the deltas
 *   added in fp32 in stored order and the sum rounded once to nearest even
 *   (the value the bf16 matrix-core GEMM uses).
 *   fmt      HXQ_FMT_U8 or HXQ_FMT_PK12; codebook, indices and sidecar as for
 *            the forward entry points (sidecar sorted by (row, col)).
 *   w        [N][K] bf16 bit patterns, caller-owned device memory, 16-byte
 *            aligned, overwritten.
 * Work is two launches on `stream`.  Errors: HXQ_ERR_SHAPE for an unknown fmt,
 * negative or oversized N, K, nnz, or odd K with pk12; HXQ_ERR_NULL;
 * HXQ_ERR_ALIGN (indices 16-byte (u8) or 4-byte (pk12), codebook 4 / 8-byte,
 * w 16-byte, sidecar 4-byte); HXQ_ERR_UNSUPPORTED if K % 16 != 0; N == 0 or
 * K == 0 is a no-op. */
int hxq_dequant_bf16(int fmt, const float* codebook, const uint8_t* indices,
                     const int32_t* sc_rows, const int32_t* sc_cols,
                     const float* sc_deltas, int64_t nnz, uint16_t* w,
                     int64_t N, int64_t K, hipStream_t stream);

/* Input gradient of a frozen layer: the product with W itself (not W^T),
 *
 *     dx[m][k] = sum_n dy[m][n] * (C[idx[n][k]] + S[n][k])     (m < M, k < K)
 *
 * which is the gradient of the forward's y with respect to x.  The model cards
 * ("Good to Know") keep the compressed weights frozen while LoRA adapters
 * train through each HelixLinear (via HelixLinearSTE), so training needs this
 * product and no gradient for the codebook, indices or sidecar.  There is no
 * bias term.
 *   fmt        HXQ_FMT_U8 or HXQ_FMT_PK12.
 *   codebook, indices, sc_*  as for the forward entry points of that format
 *              (the layer's N x K weight; pk12 needs even K).
 *   dy         [M][N] float32 or bf16 bit patterns (dy_dtype), row-major.
 *   dx         [M][K] float32, overwritten; must not overlap any input.
 *   workspace  device memory for the partial sums when the sum over n is split
 *              over several workgroups to fill the GPU, workspace_bytes long
 *              (hxq_linear_bwd_x_workspace gives the size the call would use;
 *              with less, or NULL, it splits less, down to not at all, which
 *              is slower for small M).  Caller-owned, 4-byte aligned, contents
 *              on entry ignored and on return unspecified; two calls in flight
 *              at once need separate workspaces.
 * Arithmetic: fp32 products with fp32 accumulation (bf16 dy upcast exactly);
 * with bf16 dy from 16 tokens, on shapes and pointers the bf16 matrix-core
 * kernel takes (see hxq_linear_bwd_x_ex) and with its workspace, bf16
 * products with fp32 accumulation, the weight value being the codebook value
 * plus the sidecar deltas at that position (added in fp32 in stored order)
 * rounded once to bf16, as in the forward bf16 GEMM.  Row splits are added in
 * a fixed order; on the vector path, sidecar terms that land in the same
 * column of one workgroup's tile are added in no fixed order.
 * N == 0 sets dx to zero; M == 0 or K == 0 does nothing.  Work is one to
 * three launches on `stream` (sidecar binning, the product, the sum of the
 * row splits).
 * Errors: HXQ_ERR_SHAPE for an unknown fmt, negative or oversized M, N, K, nnz,
 * negative workspace_bytes, or odd K with pk12; HXQ_ERR_DTYPE for an unknown
 * dy_dtype; HXQ_ERR_NULL; HXQ_ERR_ALIGN (dy to its element size, dx, codebook,
 * workspace and sidecar 4-byte); nothing is launched when an error is
 * returned. */
int hxq_linear_bwd_x(int fmt, const float* codebook, const uint8_t* indices,
                     const int32_t* sc_rows, const int32_t* sc_cols,
                     const float* sc_deltas, int64_t nnz,
                     const void* dy, int dy_dtype, float* dx,
                     int64_t M, int64_t N, int64_t K,
                     void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the input
 * gradient of hxq_linear_bwd_x without a workspace argument.  Its row-split
 * partial sums and sidecar bins live in a device array the library owns,
 * HXQ_SCRATCH_BYTES per GPU (each GPU the library runs on holds its own copy
 * until the process ends; nothing is allocated at call time).
 *   Arguments, arithmetic and result as for hxq_linear_bwd_x with a workspace
 *   of hxq_linear_bwd_x_workspace(...) bytes: the same kernels run.
 *   Calls on one GPU share its array and its contents are left behind: two
 *   calls that overlap on one GPU (two streams, or two host threads without
 *   ordering between their streams) race and give undefined results.
 *   The first call on a device looks up the array's device address with that
 *   device current (HXQ_ERR_HIP if that fails).
 * Errors: those of hxq_linear_bwd_x, and HXQ_ERR_SCRATCH (nothing launched)
 * when the workspace query exceeds HXQ_SCRATCH_BYTES. */
#define HXQ_SCRATCH_BYTES (96 * 1024 * 1024)

int hxq_linear_bwd_x_noalloc(int fmt, const float* codebook, const uint8_t* indices,
                             const int32_t* sc_rows, const int32_t* sc_cols,
                             const float* sc_deltas, int64_t nnz,
                             const void* dy, int dy_dtype, float* dx,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Bytes of workspace hxq_linear_bwd_x uses on the current device for these
 * sizes with pointers aligned to 16 bytes (0 when it needs none), or a
 * negative hxq_status for arguments it would reject (HXQ_ERR_SHAPE,
 * HXQ_ERR_DTYPE).  Host only. */
int64_t hxq_linear_bwd_x_workspace(int fmt, int dy_dtype, int64_t M, int64_t N,
                                   int64_t K, int64_t nnz);

/* The input gradient of several layers that read the same activations (the
 * query, key and value projections; the gate and up projections), their
 * contributions summed:
 *
 *     dx[m][k] = sum over layers i of sum_n dy_i[m][n] * W_i[n][k]
 *
 * which is the gradient with respect to the shared x of what
 * hxq_linear_fwd_grouped computes (each layer's W as for hxq_linear_bwd_x).
 *   fmt        HXQ_FMT_U8 or HXQ_FMT_PK12.
 *   layers     host array of `count` descriptors, 1 <= count <= HXQ_MAX_GROUP,
 *              read during the call only: codebook, indices, sidecar and N as
 *              for hxq_linear_bwd_x, dy the layer's [M][N] gradient
 *              (dy_dtype).  A layer with N == 0 adds nothing.
 *   dy_dtype, dx, M, K, stream  as for hxq_linear_bwd_x; dx receives the sum.
 *   workspace  caller-owned device memory, 16-byte aligned, of at least the
 *              size hxq_linear_bwd_x_grouped_workspace gives (which assumes
 *              16-byte aligned dy, dx and indices); contents on entry ignored
 *              and on return unspecified.  It holds a partial sum of dx for
 *              every run of rows the layers are split into.
 * Arithmetic: as hxq_linear_bwd_x for every layer (the bf16 matrix-core
 * products when every layer's shape and pointers allow them, else fp32
 * products for all); the partial sums are added in a fixed order (layer
 * order, then row order).  With a single layer of N > 0 the result is that of
 * hxq_linear_bwd_x with the same workspace.  Work is one or two launches on
 * `stream` (the product over all layers, the sum), or with bf16 matrix-core
 * products one or two per layer (sidecar binning, product) and the sum.
 * Errors: HXQ_ERR_SHAPE for count out of range, an unknown fmt or layers
 * with more than INT32_MAX - 65536 rows together, HXQ_ERR_NULL for NULL
 * layers, otherwise the first error hxq_linear_bwd_x would return for any
 * layer; HXQ_ERR_UNSUPPORTED when the workspace is smaller than the call
 * needs; nothing is launched when an error is returned. */
typedef struct hxq_bwd_layer {
  const void* codebook;     /* u8: float[256]; pk12: float[4096][2] */
  const uint8_t* indices;   /* u8: [N][K]; pk12: [N][3*ceil(K/4)] */
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const void* dy;           /* [M][N] float32 or bf16 bits */
  int64_t N;
} hxq_bwd_layer;

int hxq_linear_bwd_x_grouped(int fmt, const hxq_bwd_layer* layers, int count,
                             int dy_dtype, float* dx, int64_t M, int64_t K,
                             void* workspace, int64_t workspace_bytes,
                             hipStream_t stream);

/* Bytes of workspace hxq_linear_bwd_x_grouped needs on the current device for
 * these layers (only their N and nnz are read) with 16-byte aligned pointers,
 * or a negative hxq_status for arguments it would reject (HXQ_ERR_SHAPE,
 * HXQ_ERR_DTYPE, HXQ_ERR_NULL).  Host only. */
int64_t hxq_linear_bwd_x_grouped_workspace(int fmt, int dy_dtype, const hxq_bwd_layer* layers,
                                           int count, int64_t M, int64_t K);

/* The same with the kernel family forced: HXQ_VARIANT_AUTO;
 * HXQ_VARIANT_GEMV_VALU, the vector-FMA kernel (any shape);
 * HXQ_VARIANT_GEMM_BF16, the 64-token bf16 matrix-core kernel (bf16 dy,
 * N % 32 == 0, K % 128 == 0, K <= 16384, dy and dx 16-byte and indices
 * 8-byte (u8) or 4-byte (pk12) aligned, and the workspace the query gives);
 * or HXQ_VARIANT_GEMM_BF16_T256, the 256 x 256 tile bf16 matrix-core kernel
 * (u8 only; the same shapes, indices 4-byte aligned), which AUTO takes from
 * 128 tokens.  A forced kernel that cannot take the call returns
 * HXQ_ERR_UNSUPPORTED; any other value returns HXQ_ERR_UNSUPPORTED. */
int hxq_linear_bwd_x_ex(int fmt, const float* codebook, const uint8_t* indices,
                        const int32_t* sc_rows, const int32_t* sc_cols,
                        const float* sc_deltas, int64_t nnz,
                        const void* dy, int dy_dtype, float* dx,
                        int64_t M, int64_t N, int64_t K,
                        void* workspace, int64_t workspace_bytes, hipStream_t stream,
                        int variant);

/* Kernel selection, for tests and measurement.  HXQ_VARIANT_AUTO is what the
 * entry points above use; the others force one kernel family and return
 * HXQ_ERR_UNSUPPORTED when it cannot take the call. */
enum hxq_variant {
  HXQ_VARIANT_AUTO = 0,
  HXQ_VARIANT_GEMV_VALU = 1,  /* fp32 GEMV family: vector FMAs for one token (and up to 4 where the
                                 matrix-core GEMV does not fit), fp32 matrix cores beyond */
  HXQ_VARIANT_GEMV_MFMA = 2,  /* fp32 matrix-core GEMV (16x16x4 fp32 MFMA) at any M; needs K % 64 == 0 */
  HXQ_VARIANT_GEMM_BF16 = 3,  /* bf16 matrix-core GEMM (bf16 x only; K % 32 == 0) */
  HXQ_VARIANT_GENERIC = 4,    /* any shape or alignment, one wave per output row */
  HXQ_VARIANT_GEMM_BF16_T256 = 5  /* the bf16 matrix-core GEMM with 256 x 256 tiles (bf16 x only,
                                     K % 32 == 0); AUTO and HXQ_VARIANT_GEMM_BF16 take it for
                                     launches whose tiles fill their rounds over the CUs to at
                                     least 59% */
};

int hxq_linear_fwd_u8_ex(const float* codebook, const uint8_t* indices,
                         const int32_t* sc_rows, const int32_t* sc_cols,
                         const float* sc_deltas, int64_t nnz,
                         const void* x, int x_dtype, const float* bias, float* y,
                         int64_t M, int64_t N, int64_t K, hipStream_t stream,
                         int variant);

int hxq_linear_fwd_pk12_ex(const float* codebook2, const uint8_t* packed,
                           const int32_t* sc_rows, const int32_t* sc_cols,
                           const float* sc_deltas, int64_t nnz,
                           const void* x, int x_dtype, const float* bias, float* y,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream,
                           int variant);

/* The kernel family AUTO picks for these arguments (an hxq_variant), or a
 * negative hxq_status if the call would be rejected.  Host only. */
int hxq_select_variant(int fmt_pk12, int x_dtype, int64_t M, int64_t N, int64_t K);

/* Static text for a status code. */
const char* hxq_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int hxq_version(void);

/* Digest of the sources this library was built from (static text, 32 hex
 * digits, or "unknown" for a build that did not record it), so a caller can
 * tell a stale build from a current one. */
const char* hxq_source_digest(void);

#ifdef __cplusplus
}
#endif

#endif /* HXQ_H */
