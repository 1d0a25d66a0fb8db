// Host-side launchers of the libhxq kernels.  Arguments are validated by the
// C entry points before any of these is called; each launcher only computes a
// grid and queues the kernel on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hxq {

struct LayerArgs {
  const void* codebook;      // u8: float[256]; pk12: float[4096][2]
  const uint8_t* indices;    // u8: [N][K]; pk12: [N][3*ceil(K/4)]
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const void* x;             // [M][K] fp32 or bf16 bits
  bool x_bf16;
  const float* bias;         // [N] or nullptr
  float* y;                  // [M][N]
  int M, N, K;
};

int device_cu_count();

// fp32-arithmetic GEMV on the vector ALUs, u8 or pk12; needs K % 16 == 0 and
// 16-byte (u8) / 4-byte (pk12) aligned index rows, 16-byte aligned x rows.
hipError_t launch_gemv_valu(const LayerArgs& a, bool pk12, hipStream_t stream);

bool gemv_fast_path_ok(const LayerArgs& a, bool pk12);

// One layer of a decode launch.  The launcher fills in the row split and the
// sidecar density.
constexpr int kMaxSegments = 8;

// Index bytes of one launch past which the streaming kernels (one-token and
// few-token decode, the vector input gradient) load them non-temporally: a
// launch that reads more than the eight XCDs' L2 caches hold (8 x 4 MB) and
// never reads a byte twice gains from not allocating it (Qwen gate|up, 45.8
// MB, and the decode step around it), while smaller launches (down, 22.9 MB;
// q|k|v, o) were slower that way on their own.
constexpr int64_t kStreamPastCacheBytes = (int64_t)32 << 20;
// Bytes of one layer's index matrix.
inline int64_t index_bytes(int64_t N, int64_t K, bool pk12) { return N * (pk12 ? K / 4 * 3 : K); }
struct DecodeSeg {
  const void* codebook;
  const uint8_t* indices;
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const float* bias;
  float* y;  // [M][N]
  int N;
  int rows_q, rows_r;  // workgroup j owns rows_q rows, plus one when j < rows_r
  float side_per_row;  // nnz / N, to guess where a row's triplets start
};

struct DecodeArgs {
  int wg0[kMaxSegments];  // first workgroup of each layer; INT_MAX past the last
  int grid;               // workgroups in the launch
  int M, K;
  int S;                  // K slices
  int rows_cap;           // most rows owned by one workgroup
  const void* x;          // [M][K], shared by all layers
  DecodeSeg seg[kMaxSegments];
};

// Decode GEMV for M <= 4 over up to kMaxSegments layers that share x and K
// (one 1024-thread workgroup per CU, x and the codebook staged in LDS).
// Returns false without launching when the call does not fit (M > 4, x too
// large for LDS); needs the fast-path shape and alignment rules.
bool launch_decode(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                   hipStream_t stream, hipError_t& err);
bool decode_fits(const DecodeSeg* segs, int nseg, bool pk12, bool xbf, int M, int K);
// The lean decode kernel for one token row and K <= 4096 (K % 1024 == 0):
// takes = it runs this layer in a single-layer call; launch returns false
// without launching when the layers do not fit one launch.
bool decode1_takes(const DecodeSeg& s, bool pk12, bool xbf, int M, int K, const void* x);
bool launch_decode1(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                    hipStream_t stream, hipError_t& err);
// Matrix-core GEMV for M <= kGemvMfmaMaxM (u8 or pk12, K % 64 == 0): fp32
// products on v_mfma_f32_16x16x4_f32, one launch per layer.
constexpr int kGemvMfmaMaxM = 64;
struct GemvSeg {
  const float* codebook;
  const uint8_t* indices;
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const float* bias;
  float* y;
  int N;
  int nfrag;  // 16-row fragments (set by the launcher)
};
struct GemvMArgs {
  const void* x;
  int M, K;
  int nseg;
  int wg0[kMaxSegments];  // first workgroup of each layer; INT_MAX past the last
  GemvSeg seg[kMaxSegments];
};
bool gemv_mfma_ok(const LayerArgs& a, bool pk12);
hipError_t launch_gemv_mfma(const LayerArgs& a, bool pk12, hipStream_t stream);
// Matrix-core GEMV on 4x4 fp32 blocks for up to 8 tokens (u8 or pk12,
// K % 256 == 0, x 16-byte aligned): 4-row fragments, one workgroup per CU.
// The group check is false when the layers need more than one workgroup per
// CU at the kernel's fragment limit.
bool gemv_mfma4_ok(const LayerArgs& a, bool pk12);
bool gemv_mfma4_group_fits(const GemvSeg* segs, int nseg);
hipError_t launch_gemv_mfma4_grouped(const GemvSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M,
                                     int K, hipStream_t stream);
// Any M >= 1: one launch up to kGemvMfmaMaxM tokens, launches of that many
// tokens beyond (takes: the shape and alignment rules hold for such launches).
bool gemv_mfma_takes(const LayerArgs& a, bool pk12);
hipError_t launch_gemv_mfma_tokens(const LayerArgs& a, bool pk12, hipStream_t stream);
// Several layers sharing x in one launch (each must pass gemv_mfma_ok); the
// fits check is false when the layers need more fragments per workgroup than
// the kernel takes (then launch them one by one).
bool gemv_mfma_group_fits(const GemvSeg* segs, int nseg);
hipError_t launch_gemv_mfma_grouped(const GemvSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M,
                                    int K, hipStream_t stream);

// M up to kChunkMaxM through the decode kernel in groups of up to four tokens
// (indices streamed once per group); false when it does not fit.
constexpr int kChunkMaxM = 16;
bool launch_decode_chunked(const DecodeSeg* segs, int nseg, bool pk12, const void* x, bool xbf, int M, int K,
                           hipStream_t stream, hipError_t& err);

// Measurement helper: the dense bf16 weight (K % 16 == 0), two launches.
hipError_t launch_dequant_bf16(bool pk12, const float* codebook, const uint8_t* indices, const int32_t* rows,
                               const int32_t* cols, const float* deltas, int64_t nnz, uint16_t* w, int64_t N,
                               int64_t K, hipStream_t stream);

// Any shape and alignment: one wave per output row.
hipError_t launch_generic(const LayerArgs& a, bool pk12, hipStream_t stream);

// bf16 matrix-core GEMM for u8 with bf16 x; needs K % 32 == 0 and 16-byte
// aligned index and x rows.
hipError_t launch_gemm_bf16(const LayerArgs& a, hipStream_t stream);
bool gemm_path_ok(const LayerArgs& a);
// The same product with per-wave weight operands built in registers, u8 or
// pk12; needs K % 64 == 0, index rows 16-byte (u8) or 4-byte (pk12) aligned.
hipError_t launch_gemm2_bf16(const LayerArgs& a, bool pk12, hipStream_t stream);
bool gemm2_path_ok(const LayerArgs& a, bool pk12);

// Several layers of one format sharing bf16 x in one launch of that kernel
// (each must pass gemm2_path_ok); tile0 is filled in by the launcher.
struct GemmSeg {
  const float* codebook;
  const uint8_t* indices;
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const float* bias;
  float* y;
  int N;
  int tile0;
};
struct GemmArgs {
  const void* x;
  int M, K;
  int tiles_m;
  int nseg;
  GemmSeg seg[kMaxSegments];
  // the 256 x 256 tile kernel's split of k (one layer only): S runs of sst
  // stages, run s storing into ws + s * slot_stride (S == 1: into y)
  int S, sst;
  float* ws;
  int64_t slot_stride;
};
hipError_t launch_gemm_grouped(const GemmSeg* segs, int nseg, bool pk12, const void* x, int M, int K,
                               hipStream_t stream);
// The 256-token x 256-output tile GEMM, four waves of 128 x 128 with the
// weight tile built in LDS two stages ahead (u8 or pk12, bf16 x, K % 32 == 0,
// x 16-byte and index rows 16-byte (u8) / 4-byte (pk12) aligned); several
// layers sharing x in one launch.
bool gemm5_path_ok(const LayerArgs& a, bool pk12);
int64_t gemm5_tiles(const GemmSeg* segs, int nseg, int M);
hipError_t launch_gemm5_grouped(const GemmSeg* segs, int nseg, bool pk12, const void* x, int M, int K,
                                hipStream_t stream);
// One layer with its sum over k split into S runs (S >= 2 when the layer has
// too few tiles to fill the CUs and K is long enough), the runs' partial
// sums in a workspace of S M N floats, added into y in run order.
struct Gemm5Split {
  int S, sst;
  int64_t bytes;
};
Gemm5Split gemm5_split_plan(int M, int N, int K);
hipError_t launch_gemm5_split(const GemmSeg& sg, bool pk12, const void* x, int M, int K, float* ws, int64_t ws_bytes,
                              hipStream_t stream);

// y += S x.
hipError_t launch_sidecar_add(const LayerArgs& a, hipStream_t stream);

// Reads `bytes` (a multiple of 16) of src once; one word per wave into sink
// (sink_words / 8 workgroups at most); nt: non-temporal loads.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int sink_words, bool nt,
                              hipStream_t stream);

// ---- input gradient dx = dy W (hxq_bwd.hip, hxq_bwd_mfma.hip)
// One layer of a vector-kernel launch: its rows split into runs of R rows,
// the first of them split `split0` of the launch.
struct BwdSeg {
  const float* codebook;
  const uint8_t* indices;
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const void* dy;            // [M][N] fp32 or bf16 bits
  int N, split0, R;
};

struct BwdArgs {
  const float* codebook;     // u8: float[256]; pk12: float[4096][2]
  const uint8_t* indices;    // u8: [N][K]; pk12: [N][3*ceil(K/4)]
  const int32_t* sc_rows;
  const int32_t* sc_cols;
  const float* sc_deltas;
  int64_t nnz;
  const void* dy;            // [M][N] fp32 or bf16 bits
  bool dy_bf16;
  float* dx;                 // [M][K]
  int M, N, K;
  float* ws;                 // workspace for the partial sums of row splits, or nullptr
  int64_t ws_bytes;
  int CT, S, R;              // set by the launcher: column tiles, row splits, rows per split
  // grouped calls (dx = the sum over layers of dy_i W_i): the matrix-core
  // launcher writes this layer's splits into slots + slot0 (M K floats each)
  // and leaves the sum to the caller; the vector kernel reads its layers
  // from seg (nseg of them; the launcher fills seg[0] for one layer)
  float* slots;
  int slot0;
  int nseg;
  BwdSeg seg[kMaxSegments];
};

struct BwdPlan {
  int mt, lpr, mtiles, ct, S;
};

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
bool bwdx_vec_ok(const BwdArgs& a, bool pk12);
BwdPlan bwdx_plan(int M, int N, int K);
int64_t bwdx_workspace_bytes(int M, int N, int K);
hipError_t launch_bwdx_valu(const BwdArgs& a, bool pk12, hipStream_t stream);
// Several layers sharing dy's tokens and K: dx = sum_i dy_i W_i.  The group
// plan splits every layer into runs of one common length; slots_total is the
// number of partial sums (M K floats each) the workspace must hold.
struct BwdGroupPlan {
  BwdPlan p;
  int R, slots_total;
  int S[kMaxSegments];
};
BwdGroupPlan bwdx_group_plan(int M, const int* Ns, int nseg, int K);
hipError_t launch_bwdx_valu_grouped(const BwdArgs& a, bool pk12, hipStream_t stream);
hipError_t launch_bwdx_reduce(const float* ws, float* dx, int64_t n, int S, hipStream_t stream);

struct BwdMPlan {
  int ctw, mtiles, S, R, CT;
  int64_t split_bytes, bin_bytes;
};
bool bwdx_mfma_ok(const BwdArgs& a, bool pk12);
BwdMPlan bwdx_mfma_plan(int M, int N, int K, int64_t nnz);
hipError_t launch_bwdx_mfma(const BwdArgs& a, bool pk12, hipStream_t stream);
// The sidecar patch words of every 32-row step, binned by 128-column bin
// (CT = K / 128 bins per step; binstart [N / 32][CT + 1], bpat [nnz]).
hipError_t launch_bwdx_bin(const BwdArgs& a, bool pk12, int CT, int* binstart, uint32_t* bpat, hipStream_t stream);

// 256-token x 256-column tiles (hxq_bwd_g5.hip), u8 only.  One launch can
// take several layers of a grouped call (all with the same M and K): layer
// i owns workgroups wg0 .. and stores its split s into slot slot0 + s.
struct BwdG5Seg {
  const float* codebook;
  const uint8_t* indices;
  const uint16_t* dy;        // [M][N] bf16
  const int* binstart;       // sidecar bins (CT > 0)
  const uint32_t* bpat;      // patch words, or a stand-in word when nnz == 0
  int N, nnz, CT, R;         // rows, words (>= 1), bins per step (K / 128; 0 = no sidecar), rows per split
  int wg0, slot0;
};
struct BwdG5Args {
  float* out;                // dx, or slot 0
  int64_t slot_stride;       // floats between slots (0: one split into dx)
  int M, K, tiles_m, tiles_k, nseg;
  BwdG5Seg seg[kMaxSegments];
};
bool bwdx_g5_ok(const BwdArgs& a, bool pk12);
BwdMPlan bwdx_g5_plan(int M, int N, int K, int64_t nnz);
// Several layers in one launch: one run length for all (about one workgroup
// per CU over the group's rows), each layer's splits and sidecar bins.
struct BwdG5Group {
  int S[kMaxSegments], R[kMaxSegments];
  int64_t bins[kMaxSegments];  // workspace bytes of each layer's bins (multiples of 256)
  int slots;
  int64_t bin_total;
};
BwdG5Group bwdx_g5_group_plan(int M, int K, const int* Ns, const int64_t* nnzs, int n);
// Bins into `bins` (bin_total bytes), then one launch whose splits go to
// slots 0 .. slots - 1 (M K floats each) of `slots`; not summed here.
hipError_t launch_bwdx_g5_grouped(const BwdArgs* ls, int n, float* slots, unsigned char* bins, hipStream_t stream);
hipError_t launch_bwdx_g5(const BwdArgs& a, hipStream_t stream);

}  // namespace hxq
