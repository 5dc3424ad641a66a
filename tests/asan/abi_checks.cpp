// Host-only harness for the argument checks of the forward C ABI
// (fa_api.hip), built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (tests/test_asan_abi.py builds and runs it). The kernel
// launchers are stubs that count their calls, so every case runs without a
// GPU: a call with valid arguments ends at the device check (FA_ERR_DEVICE
// without a gfx950) or, on a gfx950, in the launcher stub (FA_OK, one call).
// The tensor pointers point into host buffers that the checks never
// dereference; cu_seqlens is never read on the host either.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "fa.h"
#include "fa_check.h"
#include "fa_launch.h"

namespace fa {
static int g_launches = 0;
static FwdArgs g_last{};
int launch_fwd(FwdArgs a, int, int, bool, hipStream_t) {
  ++g_launches;
  g_last = a;
  return FA_OK;
}
int launch_fwd_split(FwdArgs, int, int, bool, int, hipStream_t) { return FA_ERR_LAUNCH; }
int launch_fwd_mfma_sums(FwdArgs, hipStream_t) { return FA_ERR_LAUNCH; }
}  // namespace fa

static int g_fail = 0, g_cases = 0;

static void expect(const char* what, int got, int want) {
  ++g_cases;
  if (got != want) {
    std::printf("FAIL %s: got %d, want %d\n", what, got, want);
    ++g_fail;
  }
}

// a call with valid arguments: the device check, or the launcher
static void expect_valid(const char* what, int got) {
  ++g_cases;
  if (got != FA_ERR_DEVICE && got != FA_OK) {
    std::printf("FAIL %s: got %d, want FA_OK or FA_ERR_DEVICE\n", what, got);
    ++g_fail;
  }
}

int main() {
  const int B = 2, H = 3, N = 40, d = 64;
  const size_t elems = (size_t)B * H * N * d;
  // 16-byte aligned host buffers, separate for each tensor
  std::vector<uint64_t> bq(elems / 4 + 2), bk(elems / 4 + 2), bv(elems / 4 + 2), bo(elems / 4 + 2);
  std::vector<float> blse((size_t)B * H * N + 4);
  std::vector<int32_t> bcu(8, 0);
  auto al16 = [](void* p) {
    return reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(p) + 15) & ~uintptr_t(15));
  };
  char* q = static_cast<char*>(al16(bq.data()));
  char* k = static_cast<char*>(al16(bk.data()));
  char* v = static_cast<char*>(al16(bv.data()));
  char* o = static_cast<char*>(al16(bo.data()));
  float* lse = static_cast<float*>(al16(blse.data()));
  const float sc = 0.125f, nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();

  // ---- fa_fwd ----
  expect("fwd B<0", fa_fwd(q, k, v, o, lse, -1, H, N, d, sc, 0, FA_F16, nullptr), FA_ERR_DIM);
  expect("fwd N<0", fa_fwd(q, k, v, o, lse, B, H, -5, d, sc, 0, FA_F16, nullptr), FA_ERR_DIM);
  expect("fwd B*H*N*d overflow", fa_fwd(q, k, v, o, lse, 1 << 20, 1 << 20, 1 << 20, d, sc, 0, FA_F16, nullptr),
         FA_ERR_DIM);
  expect("fwd d=32", fa_fwd(q, k, v, o, lse, B, H, N, 32, sc, 0, FA_F16, nullptr), FA_ERR_UNSUPPORTED);
  expect("fwd dtype 7", fa_fwd(q, k, v, o, lse, B, H, N, d, sc, 0, 7, nullptr), FA_ERR_UNSUPPORTED);
  expect("fwd scale NaN", fa_fwd(q, k, v, o, lse, B, H, N, d, nan, 0, FA_F16, nullptr), FA_ERR_SCALE);
  expect("fwd scale inf", fa_fwd(q, k, v, o, lse, B, H, N, d, -inf, 0, FA_BF16, nullptr), FA_ERR_SCALE);
  expect("fwd empty, null pointers", fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, B, H, 0, d, sc, 0,
                                            FA_F16, nullptr),
         FA_OK);
  expect("fwd q null", fa_fwd(nullptr, k, v, o, lse, B, H, N, d, sc, 0, FA_F16, nullptr), FA_ERR_NULL);
  expect("fwd lse null", fa_fwd(q, k, v, o, nullptr, B, H, N, d, sc, 0, FA_F16, nullptr), FA_ERR_NULL);
  expect("fwd q misaligned", fa_fwd(q + 2, k, v, o, lse, B, H, N, d, sc, 0, FA_F16, nullptr), FA_ERR_ALIGN);
  expect("fwd lse misaligned",
         fa_fwd(q, k, v, o, reinterpret_cast<float*>(reinterpret_cast<char*>(lse) + 2), B, H, N, d, sc, 0,
                FA_F16, nullptr),
         FA_ERR_ALIGN);
  expect("fwd o == q", fa_fwd(q, k, v, q, lse, B, H, N, d, sc, 0, FA_F16, nullptr), FA_ERR_ALIAS);
  expect("fwd o over the tail of v", fa_fwd(q, k, v, v + 64, lse, B, H, N, d, sc, 0, FA_F16, nullptr),
         FA_ERR_ALIAS);
  expect("fwd lse inside o",
         fa_fwd(q, k, v, o, reinterpret_cast<float*>(o + 4096), B, H, N, d, sc, 0, FA_F16, nullptr), FA_ERR_ALIAS);
  expect_valid("fwd valid", fa_fwd(q, k, v, o, lse, B, H, N, d, sc, 1, FA_BF16, nullptr));
  expect_valid("fwd q == k == v", fa_fwd(q, q, q, o, lse, B, H, N, d, -sc, 0, FA_F16, nullptr));

  // ---- fa_fwd_strided: [B, N, H, d] views ----
  const int64_t rs = (int64_t)H * d, hs = d, bs = (int64_t)N * H * d;
  auto strided = [&](const void* qq, void* oo, float* ll, int64_t q_sr, int64_t o_sb, int64_t o_sh, int64_t o_sr,
                     int n = N) {
    return fa_fwd_strided(qq, k, v, oo, ll, B, H, n, d, sc, 0, FA_F16, bs, hs, q_sr, bs, hs, rs, bs, hs, rs, o_sb,
                          o_sh, o_sr, nullptr);
  };
  expect_valid("strided bnhd", strided(q, o, lse, rs, bs, hs, rs));
  expect("strided negative stride", strided(q, o, lse, -rs, bs, hs, rs), FA_ERR_DIM);
  expect("strided row stride > 2^24", strided(q, o, lse, (INT64_C(1) << 24) + 8, bs, hs, rs), FA_ERR_DIM);
  expect("strided stride not a multiple of 8", strided(q, o, lse, rs + 4, bs, hs, rs), FA_ERR_ALIGN);
  expect("strided span past 2^62",
         fa_fwd_strided(q, k, v, o, lse, 1 << 20, H, N, d, sc, 0, FA_F16, INT64_C(1) << 44, hs, rs, bs, hs, rs, bs,
                        hs, rs, bs, hs, rs, nullptr),
         FA_ERR_DIM);
  expect("strided output rows overlap (o_sr < d)", strided(q, o, lse, rs, bs, hs, d - 8), FA_ERR_ALIAS);
  expect("strided output heads collide (o_sh = 0)", strided(q, o, lse, rs, bs, 0, rs), FA_ERR_ALIAS);
  expect("strided o inside k's span", strided(q, k + 128, lse, rs, bs, hs, rs), FA_ERR_ALIAS);
  expect("strided lse inside o's span", strided(q, o, reinterpret_cast<float*>(o + 256), rs, bs, hs, rs),
         FA_ERR_ALIAS);
  expect("strided empty", strided(nullptr, nullptr, nullptr, rs, bs, hs, rs, 0), FA_OK);

  // ---- fa_fwd_varlen ----
  int32_t* cu = static_cast<int32_t*>(al16(bcu.data()));
  const int T = B * N;  // rows of the packed tensors fit the buffers: T*H*d = elems
  auto varlen = [&](const int32_t* c, int b, int t, int maxs, int h) {
    return fa_fwd_varlen(q, k, v, o, lse, c, b, t, maxs, h, d, sc, 1, FA_BF16, nullptr);
  };
  expect("varlen T<0", varlen(cu, 2, -1, 4, H), FA_ERR_DIM);
  expect("varlen max_seqlen<0", varlen(cu, 2, T, -1, H), FA_ERR_DIM);
  expect("varlen B<0", varlen(cu, -1, T, N, H), FA_ERR_DIM);
  expect("varlen B=0", varlen(cu, 0, T, N, H), FA_OK);
  expect("varlen max_seqlen > T", varlen(cu, 2, T, T + 1, H), FA_ERR_DIM);
  expect("varlen H*d > 2^24", varlen(cu, 2, 1, 1, 1 << 19), FA_ERR_DIM);
  expect("varlen cu_seqlens null", varlen(nullptr, 2, T, N, H), FA_ERR_NULL);
  expect("varlen cu_seqlens misaligned",
         varlen(reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(cu) + 2), 2, T, N, H), FA_ERR_ALIGN);
  expect_valid("varlen valid", varlen(cu, 2, T, N, H));

  // ---- the helpers ----
  int64_t x = 0;
  expect("mul_ok 2^31 * (2^31 - 1)", fa::mul_ok(INT64_C(1) << 31, (INT64_C(1) << 31) - 1, &x), 1);
  expect("mul_ok 2^31 * (2^31 - 1) value", x == (INT64_C(1) << 62) - (INT64_C(1) << 31), 1);
  expect("mul_ok 2^31 * 2^31 (2^62 is out of range)", fa::mul_ok(INT64_C(1) << 31, INT64_C(1) << 31, &x), 0);
  expect("mul_ok 2^40 * 2^30", fa::mul_ok(INT64_C(1) << 40, INT64_C(1) << 30, &x), 0);
  expect("mul_ok negative", fa::mul_ok(-1, 5, &x), 0);
  expect("rows_disjoint bhnd", fa::rows_disjoint((int64_t)H * N * d, (int64_t)N * d, d, B, H, N, d), 1);
  expect("rows_disjoint bnhd", fa::rows_disjoint(bs, hs, rs, B, H, N, d), 1);
  expect("rows_disjoint heads overlap", fa::rows_disjoint(bs, 8, rs, B, H, N, d), 0);
  expect("rows_disjoint one head, zero head stride", fa::rows_disjoint(bs, 0, rs, B, 1, N, d), 1);
  const fa::FwdArgs a = fa::contiguous_args(q, k, v, o, lse, B, H, N, d, -sc);
  expect("contiguous strides",
         a.q_sb == (int64_t)H * N * d && a.q_sh == (int64_t)N * d && a.q_sr == d && a.lse_sb == (int64_t)H * N &&
             a.lse_sh == N,
         1);
  expect("negative scale flips Q signs", a.qsign == 0x80008000u && a.c > 0.f, 1);

  std::printf("%d cases, %d failed, %d launches\n", g_cases, g_fail, fa::g_launches);
  return g_fail == 0 ? 0 : 1;
}
