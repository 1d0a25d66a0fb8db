// Host-only driver for the sanitizer build of the C ABI's validation and
// planning layer: every call here is rejected, or answered, on the host
// before anything would be queued on a GPU (workspace queries, kernel choice,
// status strings), over shapes up to the 2^31 limit.  Built with host
// AddressSanitizer and UndefinedBehaviorSanitizer (no recovery), so an
// out-of-bounds access, an overflow or a division by zero in that layer ends
// the run.  Prints "host sanitize: N checks ok" and exits 0 on success.

#include <stdint.h>
#include <stdio.h>

#include "hxq.h"

static int fails = 0, checks = 0;

static void expect(int got, int want, const char* what) {
  ++checks;
  if (got != want) {
    ++fails;
    printf("FAIL %s: got %d want %d\n", what, got, want);
  }
}

int main() {
  // a non-null, 16-byte aligned address that is never dereferenced
  const uintptr_t F = 0x100000;
  const float* cb = reinterpret_cast<const float*>(F);
  const uint8_t* ix = reinterpret_cast<const uint8_t*>(F);
  const int32_t* ri = reinterpret_cast<const int32_t*>(F);
  const float* dl = reinterpret_cast<const float*>(F);
  const void* x = reinterpret_cast<const void*>(F);
  float* y = reinterpret_cast<float*>(F);
  const int64_t BIG = (int64_t)1 << 31;

  // forward: dtype, shapes, pointers, alignment, forced variants
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, 0, x, 2, dl, y, 1, 1, 16, nullptr), HXQ_ERR_DTYPE, "fwd dtype");
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, -1, 1, 16, nullptr), HXQ_ERR_SHAPE, "fwd M<0");
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, BIG, 1, 16, nullptr), HXQ_ERR_SHAPE, "fwd M 2^31");
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, -1, x, HXQ_F32, dl, y, 1, 1, 16, nullptr), HXQ_ERR_SHAPE, "fwd nnz<0");
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, nullptr, 1, 1, 16, nullptr), HXQ_ERR_NULL, "fwd y");
  expect(hxq_linear_fwd_u8(cb, ix, nullptr, ri, dl, 3, x, HXQ_F32, dl, y, 1, 1, 16, nullptr), HXQ_ERR_NULL,
         "fwd rows");
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, 0, (const char*)x + 2, HXQ_F32, dl, y, 1, 1, 16, nullptr),
         HXQ_ERR_ALIGN, "fwd x align");
  expect(hxq_linear_fwd_pk12(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 1, 1, 15, nullptr), HXQ_ERR_SHAPE,
         "pk12 odd K");
  expect(hxq_linear_fwd_u8(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 0, 7, 16, nullptr), HXQ_OK, "fwd M=0");
  expect(hxq_linear_fwd_u8_ex(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 1, 1, 16, nullptr, 9), HXQ_ERR_UNSUPPORTED,
         "fwd variant 9");
  expect(hxq_linear_fwd_u8_ex(cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 1, 1, 16, nullptr, -1),
         HXQ_ERR_UNSUPPORTED, "fwd variant -1");
  expect(hxq_linear_fwd_ws(5, cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 1, 1, 16, nullptr, 0, nullptr), HXQ_ERR_SHAPE,
         "ws fmt");
  expect(hxq_linear_fwd_ws(HXQ_FMT_U8, cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 1, 1, 16, (void*)(F + 4), 64, nullptr),
         HXQ_ERR_ALIGN, "ws align");
  expect(hxq_linear_fwd_ws(HXQ_FMT_U8, cb, ix, ri, ri, dl, 0, x, HXQ_F32, dl, y, 1, 1, 16, (void*)F, -1, nullptr),
         HXQ_ERR_SHAPE, "ws bytes<0");
  expect(hxq_sidecar_add(ri, ri, dl, 4, x, 3, y, 1, 1, 16, nullptr), HXQ_ERR_DTYPE, "sidecar dtype");
  expect(hxq_sidecar_add(nullptr, ri, dl, 4, x, HXQ_F32, y, 1, 1, 16, nullptr), HXQ_ERR_NULL, "sidecar rows");
  expect(hxq_stream_read(x, 15, (uint32_t*)F, 8, nullptr), HXQ_ERR_SHAPE, "stream bytes");
  expect(hxq_stream_read_nt(x, 16, (uint32_t*)F, 7, nullptr), HXQ_ERR_SHAPE, "stream nt words");
  expect(hxq_stream_read_nt(nullptr, 16, (uint32_t*)F, 8, nullptr), HXQ_ERR_NULL, "stream nt src");

  // grouped forward: counts, layers
  hxq_layer L[9];
  for (int i = 0; i < 9; ++i) L[i] = hxq_layer{cb, ix, ri, ri, dl, 0, dl, y, 16};
  expect(hxq_linear_fwd_grouped(HXQ_FMT_U8, L, 9, x, HXQ_F32, 1, 16, nullptr), HXQ_ERR_SHAPE, "grouped count 9");
  expect(hxq_linear_fwd_grouped(HXQ_FMT_U8, nullptr, 2, x, HXQ_F32, 1, 16, nullptr), HXQ_ERR_NULL, "grouped null");
  L[1].N = -3;
  expect(hxq_linear_fwd_grouped(HXQ_FMT_U8, L, 2, x, HXQ_F32, 1, 16, nullptr), HXQ_ERR_SHAPE, "grouped N<0");
  L[1].N = 16;

  // input gradient: dtype, shapes, variants
  expect(hxq_linear_bwd_x(HXQ_FMT_U8, cb, ix, ri, ri, dl, 0, x, 4, y, 1, 1, 16, nullptr, 0, nullptr), HXQ_ERR_DTYPE,
         "bwd dtype");
  expect(hxq_linear_bwd_x(HXQ_FMT_U8, cb, ix, ri, ri, dl, 0, x, HXQ_F32, y, 1, -2, 16, nullptr, 0, nullptr),
         HXQ_ERR_SHAPE, "bwd N<0");
  expect(hxq_linear_bwd_x(HXQ_FMT_PK12, cb, ix, ri, ri, dl, 0, x, HXQ_F32, y, 1, 1, 15, nullptr, 0, nullptr),
         HXQ_ERR_SHAPE, "bwd pk12 odd K");
  expect(hxq_linear_bwd_x_ex(HXQ_FMT_U8, cb, ix, ri, ri, dl, 0, x, HXQ_F32, y, 1, 1, 16, nullptr, 0, nullptr, 2),
         HXQ_ERR_UNSUPPORTED, "bwd variant 2");
  hxq_bwd_layer B[9];
  for (int i = 0; i < 9; ++i) B[i] = hxq_bwd_layer{cb, ix, ri, ri, dl, 0, x, 16};
  expect(hxq_linear_bwd_x_grouped(HXQ_FMT_U8, B, 9, HXQ_F32, y, 1, 16, nullptr, 0, nullptr), HXQ_ERR_SHAPE,
         "bwd grouped count 9");
  // rows of a group that together pass int32
  for (int i = 0; i < 2; ++i) B[i].N = (int64_t)1 << 30;
  expect((int)hxq_linear_bwd_x_grouped_workspace(HXQ_FMT_U8, HXQ_BF16, B, 2, 2048, 2048), HXQ_ERR_SHAPE,
         "bwd grouped rows overflow");

  // host planning over shapes up to the limits: workspace sizes and the
  // kernel choice must be answered (or the shape refused with HXQ_ERR_SHAPE,
  // as products past the kernels' index range are) without overflow or a fault
  const int64_t dims[] = {0, 1, 2, 5, 16, 17, 64, 127, 128, 300, 512, 2048, 4096, 11008, 25600, 65535, 1 << 20,
                          BIG - 1};
  const int64_t Ks[] = {16, 64, 2048, 11008, 12288, 33024, (BIG - 1) / 64 * 64};
  for (int64_t M : dims)
    for (int64_t N : dims)
      for (int64_t K : Ks) {
        for (int fmt = 0; fmt < 2; ++fmt)
          for (int xd = 0; xd < 2; ++xd) {
            const int64_t w = hxq_linear_fwd_workspace(fmt, xd, M, N, K);
            ++checks;
            if (w < 0 && w != HXQ_ERR_SHAPE) {
              ++fails;
              printf("FAIL fwd workspace fmt=%d x=%d M=%lld N=%lld K=%lld: %lld\n", fmt, xd, (long long)M,
                     (long long)N, (long long)K, (long long)w);
            }
            const int64_t wb = hxq_linear_bwd_x_workspace(fmt, xd, M, N, K, N / 1000);
            ++checks;
            if (wb < 0 && wb != HXQ_ERR_SHAPE) {
              ++fails;
              printf("FAIL bwd workspace fmt=%d dy=%d M=%lld N=%lld K=%lld: %lld\n", fmt, xd, (long long)M,
                     (long long)N, (long long)K, (long long)wb);
            }
            const int v = hxq_select_variant(fmt, xd, M, N, K);
            ++checks;
            if (v < HXQ_VARIANT_AUTO && v != HXQ_ERR_SHAPE) {
              ++fails;
              printf("FAIL select fmt=%d x=%d M=%lld N=%lld K=%lld: %d\n", fmt, xd, (long long)M, (long long)N,
                     (long long)K, v);
            }
          }
      }
  expect((int)hxq_linear_fwd_workspace(3, HXQ_F32, 1, 1, 16), HXQ_ERR_SHAPE, "fwd workspace fmt");
  expect((int)hxq_linear_bwd_x_workspace(HXQ_FMT_U8, 7, 1, 1, 16, 0), HXQ_ERR_DTYPE, "bwd workspace dtype");
  for (int s = -8; s <= 0; ++s) {
    ++checks;
    if (!hxq_status_str(s)) ++fails;
  }
  ++checks;
  if (hxq_version() < 100 || !hxq_source_digest()) ++fails;

  if (fails) {
    printf("host sanitize: %d of %d checks failed\n", fails, checks);
    return 1;
  }
  printf("host sanitize: %d checks ok\n", checks);
  return 0;
}
