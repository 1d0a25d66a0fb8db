// Input gradient dx = dy W on bf16 matrix cores (bf16 dy, training-size M).
//
//     dx[m][k] = sum_n dy[m][n] * Wq[n][k],   Wq = bf16(C[idx] + S)
//
// (model cards, "Good to Know": LoRA trains through frozen HelixLinear layers,
// which needs this product; W as in "What is HelixCode?" and the HXQ
// whitepaper's "Method" and "2D vector quantization").  The weight value fed
// to the matrix cores is the codebook value plus any sidecar deltas at that
// position, added in fp32 in stored order and rounded once to bf16 (nearest,
// ties to even): the same value the forward bf16 GEMM uses.  fp32 accumulation.
//
// v_mfma_f32_16x16x32_bf16 with the weight as the A operand: its 16 rows are
// output columns, its 32-long contraction runs over n.  A workgroup owns 64
// tokens (four 16-token blocks) and 512 columns (128 per wave) and sweeps its
// run of rows 32 at a time.  Per step lane l (group g = l / 16, l16 = l % 16)
// loads 8 index bytes (u8) or 6 (pk12, four pairs) from each of the rows
// n0 + 8 g .. + 7 at columns kc + 8 l16 .. + 7, gathers their bf16 codebook
// values from LDS and packs them row pairs to a word: fragment f (0..7) then
// holds column kc + 8 i + f in its row i.  The lane's 8 dy values of those
// rows per token block (16 bytes) are the B operand.  In the result, lane l
// holds for token 16 b + l16 the 32 consecutive columns kc + 32 g .. + 31, so
// the epilogue is whole float4 stores.  Index bytes, dy and the sidecar
// patches of a step are loaded two steps ahead.
//
// Sidecar: a prologue kernel turns every distinct (row, col) of the triplets
// into a patch word, bf16(C + deltas) with the lane, fragment and operand
// half that hold that weight, sorted into (32-row step, 128-column) bins in
// the workspace.  A wave reads its bin for the step (its start from LDS);
// each lane with a word passes it to the owner lane through an LDS slot, and
// the owner overwrites the operand half it names.
//
// Row splits (to fill the GPU) store into the workspace and are summed by
// the reduction kernel of the vector path.

#include "hxq_device.h"
#include "hxq_launch.h"

#include <climits>
#include <type_traits>

namespace hxq {

namespace bm {
constexpr int THREADS = 256, WAVES = 4;
constexpr int TM = 64;              // tokens per workgroup
constexpr int CWW = 128;            // columns per wave = sidecar bin width
constexpr int CW = WAVES * CWW;     // columns per workgroup
constexpr int STEP = 32;            // rows per step
constexpr int MAXCT = 128;          // bins per step: K <= 16384
constexpr int MAXST = 1024;         // steps per row split (bin starts kept in LDS)
}  // namespace bm

// ---- sidecar patches: one 256-thread workgroup per 32-row step.  Every
// distinct (row, col) of the step becomes one patch word, placed in its
// 128-column bin: the owner lane (bits 0-5: 16 (row / 8 in
// the step) + column / 8 in the bin), the fragment (6-8: column % 8), the
// operand word (9-10) and half (11) of its row, and the bf16 value (16-31)
// of the codebook value plus the run's deltas, added in fp32 in stored order
// and rounded once to nearest even.
template <bool PK12>
__global__ __launch_bounds__(256) void bwdx_bin(const float* __restrict__ codebook, const uint8_t* __restrict__ indices,
                                               const int32_t* __restrict__ rows, const int32_t* __restrict__ cols,
                                               const float* __restrict__ deltas, int64_t nnz, int N, int K, int CT,
                                               int* __restrict__ binstart, uint32_t* __restrict__ bpat) {
  __shared__ int off[bm::MAXCT];
  __shared__ int run[bm::MAXCT];
  const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int r_lo = s * bm::STEP, r_hi = min(N, r_lo + bm::STEP);
  const int64_t lo = wave_lower_bound_rows_near(rows, nnz, r_lo, (int64_t)((double)nnz * r_lo / N));
  const int64_t hi = wave_lower_bound_rows_near(rows, nnz, r_hi, (int64_t)((double)nnz * r_hi / N));
  for (int i = tid; i < bm::MAXCT; i += 256) {
    off[i] = 0;
    run[i] = 0;
  }
  __syncthreads();
  // a triplet heads its run when the one before it has another coordinate
  auto head = [&](int64_t e, int r, int c) { return e == 0 || rows[e - 1] != r || cols[e - 1] != c; };
  for (int64_t e = lo + tid; e < hi; e += 256) {
    const int r = rows[e], c = cols[e];
    if (head(e, r, c)) atomicAdd(&off[c / bm::CWW], 1);
  }
  __syncthreads();
  // exclusive prefix over the bin counts, two bins per lane of wave 0
  const int b0 = 2 * lane, b1 = 2 * lane + 1;
  int c0 = 0, c1 = 0, inc = 0;
  if (tid < 64) {
    c0 = b0 < CT ? off[b0] : 0;
    c1 = b1 < CT ? off[b1] : 0;
    inc = c0 + c1;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int t = __shfl_up(inc, d, 64);
      if (lane >= d) inc += t;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int exc = inc - c0 - c1;
    if (b0 < CT) off[b0] = exc;
    if (b1 < CT) off[b1] = exc + c0;
    int* bs = binstart + (int64_t)s * (CT + 1);
    if (b0 < CT) bs[b0] = (int)lo + exc;
    if (b1 < CT) bs[b1] = (int)lo + exc + c0;
    const int total = __shfl(inc, 63, 64);  // distinct coordinates in the step
    if (lane == 0) bs[CT] = (int)lo + total;
  }
  __syncthreads();
  const int64_t pitch = PK12 ? (int64_t)((K + 3) / 4) * 3 : (int64_t)K;
  // the words, 256 triplets at a time
  for (int64_t base = lo; base < hi; base += 256) {
    const int64_t e = base + tid;
    const bool v = e < hi;
    const int64_t ec = v ? e : hi - 1;
    const int r = rows[ec], c = cols[ec];
    const bool h = v && head(ec, r, c);
    uint32_t word = 0;
    if (h) {
      float cv;
      if (PK12) {
        const uint8_t* pb = indices + (int64_t)r * pitch + (c >> 2) * 3;
        const uint32_t g = (uint32_t)pb[0] | ((uint32_t)pb[1] << 8) | ((uint32_t)pb[2] << 16);
        const uint32_t pi = ((c >> 1) & 1) ? (g >> 12) : (g & 0xfffu);
        cv = codebook[2 * pi + (c & 1)];
      } else {
        cv = codebook[indices[(int64_t)r * K + c]];
      }
      float val = cv + deltas[ec];
      for (int64_t e2 = ec + 1; e2 < hi && rows[e2] == r && cols[e2] == c; ++e2) val += deltas[e2];
      const int jj = r - r_lo, cw = c % bm::CWW;
      word = (uint32_t)(16 * (jj >> 3) + (cw >> 3)) | ((uint32_t)(cw & 7) << 6) | ((uint32_t)((jj & 7) >> 1) << 9) |
             ((uint32_t)(jj & 1) << 11) | (f32_to_bf16_rne(val) << 16);
    }
    // a word's place within its bin does not matter (each names its own
    // operand half), so positions come from an LDS counter per bin
    int pos = 0;
    if (h) pos = off[c / bm::CWW] + atomicAdd(&run[c / bm::CWW], 1);
    if (h) bpat[lo + pos] = word;
  }
}

struct Rows8 {
  uint2 v[8];
};

struct Hits {  // a wave's patch bin for one step: start, count, word `lane`
  int b, n;
  uint32_t w;
};

struct BwdMArgs {
  const float* codebook;
  const uint8_t* indices;
  const uint16_t* dy;   // [M][N] bf16
  float* out;           // dx, or the workspace splits when S > 1
  int out_final;        // out is dx itself (stored past the cache), not slots summed afterwards
  int M, N, K;
  int ctw, mtiles, S, R;
  int CT;               // sidecar bins per step (K / 128); 0 = no sidecar
  int nnz;
  const int* binstart;
  const uint32_t* bpat;
};

template <bool PK12>
__global__ __launch_bounds__(bm::THREADS, 1) void bwdx_mfma(BwdMArgs a) {
  using namespace bm;
  // u8: 64 bf16 copies per entry (copy j at byte 256 e + 4 j, value in the
  // upper half); pk12: entry e at byte 4 e, component 0 low, 1 high
  __shared__ __align__(16) unsigned char cbs[PK12 ? 4096 * 4 : 256 * 256];
  __shared__ float cbf[PK12 ? 8192 : 256];  // fp32 codebook for the patches
  __shared__ int bsl[MAXST * 5];             // per step: bin starts of the 4 waves and the end
  __shared__ int ovf;
  __shared__ uint32_t pslot[WAVES * 64];     // patch words on their way to their owner lanes

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int M = a.M, N = a.N, K = a.K;
  const int b = blockIdx.x;
  const int ctw = b % a.ctw, rest = b / a.ctw, mt = rest % a.mtiles, s = rest / a.mtiles;
  const int kc = ctw * CW + wave * CWW;
  const bool wave_ok = kc < K;
  const int kcc = wave_ok ? kc : 0;
  const int m0 = mt * TM;
  const int n_lo = s * a.R, n_hi = min(N, n_lo + a.R);
  const int steps = (n_hi - n_lo) / STEP;
  const uint32_t lane4 = (uint32_t)lane << 2;

  // ---- operand addresses
  const int64_t pitch = PK12 ? (int64_t)(K / 4) * 3 : (int64_t)K;
  const uint8_t* ib;
  if (PK12) {
    const int q = kcc / 8 + l16;
    ib = a.indices + (6 * q - 2 * (q & 1)) + (int64_t)(8 * g) * pitch;
  } else {
    ib = a.indices + kcc + 8 * l16 + (int64_t)(8 * g) * pitch;
  }
  const bool odd = l16 & 1;
  const uint16_t* db[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) db[t] = a.dy + (int64_t)min(m0 + 16 * t + l16, M - 1) * N + 8 * g;

  // (the rows travel by value: through pointers the compiler keeps them in scratch memory)
  auto load_I = [&](int st) {
    Rows8 I;
    const uint8_t* p = ib + (int64_t)(n_lo + st * STEP) * pitch;
#pragma unroll
    for (int j = 0; j < 8; ++j) I.v[j] = *reinterpret_cast<const uint2*>(p + j * pitch);
    return I;
  };
  auto load_B = [&](int st, u32x4* B) {
#pragma unroll
    for (int t = 0; t < 4; ++t) B[t] = *reinterpret_cast<const u32x4*>(db[t] + n_lo + st * STEP);
  };
  // the step's sidecar bin for this wave (its start and count from LDS, so
  // that making them uniform waits for no global load) and entry `lane` of it
  auto load_H = [&](int st, Hits& h) {
    h.n = 0;
    if (a.CT > 0) {
      h.b = __builtin_amdgcn_readfirstlane(bsl[st * 5 + wave]);
      h.n = __builtin_amdgcn_readfirstlane(bsl[st * 5 + wave + 1]) - h.b;
      const int e = min(h.b + min(lane, max(h.n - 1, 0)), a.nnz - 1);  // an empty last bin starts at nnz
      h.w = a.bpat[e];
    }
  };

  // loads run two steps ahead: index rows for step st + 1 and st + 2, dy for
  // st .. st + 2, sidecar bins for st + 1 and st + 2
  Rows8 I1 = {}, I2 = {};
  u32x4 B0[4], B1[4], B2[4];
  Hits H1 = {}, H2 = {};
  const Rows8 I0 = load_I(0);
  if (steps > 1) I1 = load_I(1);
  load_B(0, B0);
  if (steps > 1) load_B(1, B1);

  // ---- bin starts of this workgroup's steps: the bins of its four waves and the end
  if (a.CT > 0) {
    const int ct0 = ctw * WAVES;
    for (int i = tid; i < steps * 5; i += THREADS) {
      const int st = i / 5, w = i - st * 5;
      bsl[i] = a.binstart[(int64_t)((n_lo / STEP) + st) * (a.CT + 1) + min(ct0 + w, a.CT)];
    }
  }
  // ---- codebooks
  if (PK12) {
#pragma unroll
    for (int i = 0; i < 4096 / THREADS; ++i) {
      const int e = tid + THREADS * i;
      const float c0 = a.codebook[2 * e], c1 = a.codebook[2 * e + 1];
      reinterpret_cast<uint32_t*>(cbs)[e] = f32_to_bf16_rne(c0) | (f32_to_bf16_rne(c1) << 16);
      cbf[2 * e] = c0;
      cbf[2 * e + 1] = c1;
    }
  } else {
    const float cv = a.codebook[tid];
    const float vb = __uint_as_float(f32_to_bf16_rne(cv) << 16);
    const float4 v4 = make_float4(vb, vb, vb, vb);
#pragma unroll
    for (int q = 0; q < 16; ++q) *reinterpret_cast<float4*>(cbs + tid * 256 + (((q + tid) & 15) << 4)) = v4;
    cbf[tid] = cv;
  }
  __syncthreads();

  // ---- A operand of one step from its index bytes
  u32x4 A[8];
  auto build_A = [&](Rows8 I) {
    if (PK12) {
      uint32_t P[8][4];  // row j, pair p: bf16 pair word
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint2 q = I.v[j];
        uint32_t v0, v1;
        if (odd) {
          v0 = __builtin_amdgcn_alignbit(q.y, q.x, 16) & 0xffffffu;
          v1 = q.y >> 8;
        } else {
          v0 = q.x & 0xffffffu;
          v1 = __builtin_amdgcn_alignbit(q.y, q.x, 24) & 0xffffffu;
        }
        P[j][0] = lds_load<uint32_t>((v0 & 0xfffu) << 2, cbs);
        P[j][1] = lds_load<uint32_t>((v0 >> 12) << 2, cbs);
        P[j][2] = lds_load<uint32_t>((v1 & 0xfffu) << 2, cbs);
        P[j][3] = lds_load<uint32_t>((v1 >> 12) << 2, cbs);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          A[2 * p][q] = __builtin_amdgcn_perm(P[2 * q + 1][p], P[2 * q][p], 0x05040100u);
          A[2 * p + 1][q] = __builtin_amdgcn_perm(P[2 * q + 1][p], P[2 * q][p], 0x07060302u);
        }
    } else {
      uint32_t V[8][8];  // row j, column f: the gathered word (bf16 in the upper half)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        V[j][0] = lds_load<uint32_t>(byte_addr256<0>(I.v[j].x, lane4), cbs);
        V[j][1] = lds_load<uint32_t>(byte_addr256<1>(I.v[j].x, lane4), cbs);
        V[j][2] = lds_load<uint32_t>(byte_addr256<2>(I.v[j].x, lane4), cbs);
        V[j][3] = lds_load<uint32_t>(byte_addr256<3>(I.v[j].x, lane4), cbs);
        V[j][4] = lds_load<uint32_t>(byte_addr256<0>(I.v[j].y, lane4), cbs);
        V[j][5] = lds_load<uint32_t>(byte_addr256<1>(I.v[j].y, lane4), cbs);
        V[j][6] = lds_load<uint32_t>(byte_addr256<2>(I.v[j].y, lane4), cbs);
        V[j][7] = lds_load<uint32_t>(byte_addr256<3>(I.v[j].y, lane4), cbs);
      }
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) A[f][q] = __builtin_amdgcn_perm(V[2 * q + 1][f], V[2 * q][f], 0x07060302u);
    }
  };

  // ---- sidecar patches of one step: word t names the owner lane, the
  // fragment, the operand word (uniform, so it picks the register) and half,
  // and the bf16 value
  auto patch_one = [&](uint32_t ent) {
    const uint32_t keep = (ent & 2048u) ? 0x0000ffffu : 0xffff0000u;
    const uint32_t put = ((ent >> 16) * 0x10001u) & ~keep;
    const bool mine = lane == (int)(ent & 63u);
    // the operand word by a switch on the uniform (fragment, word): a few
    // scalar branches and one select, where an indexed register access
    // would cost a mode switch per fragment
    switch (((ent >> 6) & 7u) * 4u + ((ent >> 9) & 3u)) {
#define HXQ_PATCH_CASE(F, Q)                                        \
  case (F) * 4 + (Q):                                               \
    A[F][Q] = mine ? ((A[F][Q] & keep) | put) : A[F][Q];            \
    break;
#define HXQ_PATCH_ROW(F) HXQ_PATCH_CASE(F, 0) HXQ_PATCH_CASE(F, 1) HXQ_PATCH_CASE(F, 2) HXQ_PATCH_CASE(F, 3)
      HXQ_PATCH_ROW(0) HXQ_PATCH_ROW(1) HXQ_PATCH_ROW(2) HXQ_PATCH_ROW(3)
      HXQ_PATCH_ROW(4) HXQ_PATCH_ROW(5) HXQ_PATCH_ROW(6) HXQ_PATCH_ROW(7)
#undef HXQ_PATCH_ROW
#undef HXQ_PATCH_CASE
      default:
        break;
    }
  };
  // the bin's first 64 words are in lanes 0..63 (one each): every lane with
  // a word writes it to its owner lane's LDS slot, every lane applies the word
  // it finds in its own slot (per-lane selects, no branches), and a round
  // repeats only for the rare words that lost a slot to another word of the
  // same owner
  uint32_t* slot = pslot + wave * 64;
  auto patch = [&](const Hits& h, auto rare_c) {
    // (the empty asm uses the word here, in straight-line code, so the wait
    // for its load counts only what was issued after it)
    uint32_t hw = h.w;
    asm volatile("" : "+v"(hw));
    if (h.n == 0) return;
    const uint32_t tagged = hw | 0x1000u;  // bit 12: slot holds a word
    bool pending = lane < min(h.n, 64);
    while (__ballot(pending)) {
      if (pending) slot[hw & 63u] = tagged;
      const uint32_t w = slot[lane];
      if (w & 0x1000u) {
        const uint32_t fq = ((w >> 6) & 7u) * 4u + ((w >> 9) & 3u);
        const uint32_t keep = (w & 2048u) ? 0x0000ffffu : 0xffff0000u;
        const uint32_t put = ((w >> 16) * 0x10001u) & ~keep;
#pragma unroll
        for (int ff = 0; ff < 8; ++ff)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            if (fq == (uint32_t)(ff * 4 + qq)) A[ff][qq] = (A[ff][qq] & keep) | put;
      }
      if (pending && slot[hw & 63u] == tagged) pending = false;
      slot[lane] = 0u;
    }
    // words past the first 64 of a bin: only in the copy of the loop for
    // workgroups that have such bins (scalar loads, waited for in the same
    // asm block)
    if (!decltype(rare_c)::value) return;
    for (int i = 64; i < h.n; ++i) {
      const uint32_t* wp = a.bpat + h.b + i;
      uint32_t word;
      asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(word) : "s"(wp) : "memory");
      patch_one(word);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[t][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto main_loop = [&](auto rare_c) {
  if (steps > 0) {
    Hits H0 = {};
    load_H(0, H0);
    if (steps > 1) load_H(1, H1);
    build_A(I0);
    patch(H0, rare_c);
  }
  for (int st = 0; st < steps; ++st) {
    if (st + 2 < steps) {
      I2 = load_I(st + 2);
      load_B(st + 2, B2);
      load_H(st + 2, H2);
    }
    // this step's matrix ops and the next step's operand gathers in one
    // block, interleaved (one matrix op, then two LDS reads (u8; one for
    // pk12, which gathers half as often) and two vector ops), so the gathers
    // run while the matrix unit is busy; past the last step the gathers read
    // a stand-in row and go unused
    const u32x4 Acur[8] = {A[0], A[1], A[2], A[3], A[4], A[5], A[6], A[7]};
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, Acur[f]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, B0[t]), acc[t][f], 0, 0, 0);
    }
    build_A(I1);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // matrix op
      __builtin_amdgcn_sched_group_barrier(0x0100, PK12 ? 1 : 2, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x0002, 2, 0);  // vector op
    }
    if (st + 1 < steps) {
      patch(H1, rare_c);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        B0[t] = B1[t];
        B1[t] = B2[t];
      }
      I1 = I2;
      H1 = H2;
    }
  }
  };
  // does any bin of this workgroup hold more than 64 patch words?
  if (tid == 0) ovf = 0;
  pslot[tid] = 0u;
  __syncthreads();
  if (a.CT > 0)
    for (int i = tid; i < steps * 4; i += THREADS) {
      const int st = i >> 2, w = i & 3;
      if (bsl[st * 5 + w + 1] - bsl[st * 5 + w] > 64) ovf = 1;
    }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(ovf))
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  // ---- epilogue: lane l holds token m0 + 16 t + l16, columns kc + 32 g + 8 r + f
  if (!wave_ok) return;
  float* out = a.out + (a.S > 1 ? (int64_t)s * M * K : 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + 16 * t + l16;
    if (m >= M) continue;
    float* p = out + (int64_t)m * K + kc + 32 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 lo4 = {acc[t][0][r], acc[t][1][r], acc[t][2][r], acc[t][3][r]};
      const f32x4 hi4 = {acc[t][4][r], acc[t][5][r], acc[t][6][r], acc[t][7][r]};
      if (!a.out_final) {  // a partial sum the reduction reads back soon: keep it in the cache
        *reinterpret_cast<f32x4*>(p + 8 * r) = lo4;
        *reinterpret_cast<f32x4*>(p + 8 * r + 4) = hi4;
      } else {
        __builtin_nontemporal_store(lo4, reinterpret_cast<f32x4*>(p + 8 * r));
        __builtin_nontemporal_store(hi4, reinterpret_cast<f32x4*>(p + 8 * r + 4));
      }
    }
  }
}

// The shapes and pointers this kernel takes.
bool bwdx_mfma_ok(const BwdArgs& a, bool pk12) {
  if (!a.dy_bf16 || a.M < 1 || a.N < bm::STEP || a.K < bm::CWW) return false;
  if (a.N % bm::STEP != 0 || a.K % bm::CWW != 0 || a.K > bm::MAXCT * bm::CWW) return false;
  if ((int64_t)a.N > (int64_t)64 * bm::MAXST * bm::STEP) return false;  // at most 64 splits of 1024 steps
  const uintptr_t ip = reinterpret_cast<uintptr_t>(a.indices), dp = reinterpret_cast<uintptr_t>(a.dy);
  const uintptr_t xp = reinterpret_cast<uintptr_t>(a.dx);
  if (dp % 16 != 0 || xp % 16 != 0 || ip % (pk12 ? 4 : 8) != 0) return false;
  return true;
}

// Launch shape: column tiles x token tiles x row splits, splits added until
// the launch has one workgroup per CU (at most 64, at least 256 rows each,
// and at most 1024 steps each).
BwdMPlan bwdx_mfma_plan(int M, int N, int K, int64_t nnz) {
  BwdMPlan p;
  p.ctw = (K + bm::CW - 1) / bm::CW;
  p.mtiles = (M + bm::TM - 1) / bm::TM;
  const int64_t tiles = (int64_t)p.ctw * p.mtiles;
  const int64_t cus = device_cu_count();
  int64_t S = (cus + tiles - 1) / tiles;
  const int64_t smax = N / 256 > 0 ? N / 256 : 1;  // at least 8 steps per split
  if (S > smax) S = smax;
  if (S > 64) S = 64;  // at most 64 splits (each M K floats of workspace)
  const int64_t smin = (N / bm::STEP + bm::MAXST - 1) / bm::MAXST;  // bin starts of a split fit LDS
  if (S < smin) S = smin;
  if (S < 1) S = 1;
  const int nsteps = N / bm::STEP;
  const int spp = (nsteps + (int)S - 1) / (int)S;  // steps per split
  p.R = spp * bm::STEP;
  p.S = (nsteps + spp - 1) / spp;
  p.CT = nnz > 0 ? K / bm::CWW : 0;
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  p.split_bytes = p.S > 1 ? al((int64_t)p.S * M * K * 4) : 0;
  p.bin_bytes = nnz > 0 ? al((int64_t)nsteps * (p.CT + 1) * 4) + al(nnz * 4) : 0;
  return p;
}

hipError_t launch_bwdx_bin(const BwdArgs& a, bool pk12, int CT, int* binstart, uint32_t* bpat, hipStream_t stream) {
  const int nsteps = a.N / bm::STEP;
  if (pk12)
    hipLaunchKernelGGL(bwdx_bin<true>, dim3((unsigned)nsteps), dim3(256), 0, stream, a.codebook, a.indices, a.sc_rows,
                       a.sc_cols, a.sc_deltas, a.nnz, a.N, a.K, CT, binstart, bpat);
  else
    hipLaunchKernelGGL(bwdx_bin<false>, dim3((unsigned)nsteps), dim3(256), 0, stream, a.codebook, a.indices, a.sc_rows,
                       a.sc_cols, a.sc_deltas, a.nnz, a.N, a.K, CT, binstart, bpat);
  return hipGetLastError();
}

// a.slots set (grouped calls): the splits go to slots a.slot0 .. + S - 1 and
// are not summed here; the workspace then holds only the sidecar bins.
hipError_t launch_bwdx_mfma(const BwdArgs& a, bool pk12, hipStream_t stream) {
  const BwdMPlan p = bwdx_mfma_plan(a.M, a.N, a.K, a.nnz);
  const bool grouped = a.slots != nullptr;
  const int64_t split_bytes = grouped ? 0 : p.split_bytes;
  if (a.ws_bytes < split_bytes + p.bin_bytes || (split_bytes + p.bin_bytes > 0 && a.ws == nullptr))
    return hipErrorInvalidValue;
  unsigned char* w = reinterpret_cast<unsigned char*>(a.ws);
  BwdMArgs m = {};
  m.codebook = a.codebook;
  m.indices = a.indices;
  m.dy = static_cast<const uint16_t*>(a.dy);
  m.out = grouped ? a.slots + (int64_t)a.slot0 * a.M * a.K : p.S > 1 ? reinterpret_cast<float*>(w) : a.dx;
  m.out_final = !grouped && p.S <= 1;
  m.M = a.M;
  m.N = a.N;
  m.K = a.K;
  m.ctw = p.ctw;
  m.mtiles = p.mtiles;
  m.S = p.S;
  m.R = p.R;
  m.CT = p.CT;
  m.nnz = (int)a.nnz;
  if (a.nnz > 0) {
    const int nsteps = a.N / bm::STEP;
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    unsigned char* q = w + split_bytes;
    int* binstart = reinterpret_cast<int*>(q);
    q += al((int64_t)nsteps * (p.CT + 1) * 4);
    uint32_t* bpat = reinterpret_cast<uint32_t*>(q);
    const hipError_t e = launch_bwdx_bin(a, pk12, p.CT, binstart, bpat, stream);
    if (e != hipSuccess) return e;
    m.binstart = binstart;
    m.bpat = bpat;
  }
  const int64_t blocks = (int64_t)p.ctw * p.mtiles * p.S;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  if (pk12)
    hipLaunchKernelGGL(bwdx_mfma<true>, dim3((unsigned)blocks), dim3(bm::THREADS), 0, stream, m);
  else
    hipLaunchKernelGGL(bwdx_mfma<false>, dim3((unsigned)blocks), dim3(bm::THREADS), 0, stream, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1 || grouped) return e;
  return launch_bwdx_reduce(m.out, a.dx, (int64_t)a.M * a.K, p.S, stream);
}

}  // namespace hxq
