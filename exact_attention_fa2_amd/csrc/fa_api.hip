// C ABI of libfa.so: argument validation (host only, before any HIP call),
// kernel-variant selection and launch on the caller's stream. See fa.h for
// the contract of each entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa.h"
#include "fa_check.h"
#include "fa_fwd_kernel.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// validation helpers (pure host logic)
// ---------------------------------------------------------------------------
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > (INT64_C(1) << 62) / a) return false;
  *out = a * b;
  return *out < (INT64_C(1) << 62);
}

bool head_dim_ok(int d) { return d == 64 || d == 96 || d == 128 || d == 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

// True when the rows (b, h, i) of a strided [B, H, N, d] tensor share no
// element: with the axes of extent above 1 sorted by stride, each stride must
// reach past everything the smaller axes span (a row spans d elements). This
// is sufficient; layouts it rejects would have several workgroups write the
// same bytes of an output.
bool rows_disjoint(int64_t sb, int64_t sh, int64_t sr, int B, int H, int N, int d) {
  int64_t ax[3][2] = {{sr, N}, {sh, H}, {sb, B}};
  for (int i = 0; i < 3; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && ax[j][0] < ax[j - 1][0]; --j)
      for (int c = 0; c < 2; ++c) {
        const int64_t t = ax[j][c];
        ax[j][c] = ax[j - 1][c];
        ax[j - 1][c] = t;
      }
  int64_t reach = d;
  for (int i = 0; i < 3; ++i) {
    if (ax[i][1] <= 1) continue;
    if (ax[i][0] < reach) return false;
    reach += ax[i][0] * (ax[i][1] - 1);  // no overflow: bounded by the span check
  }
  return true;
}

// Common checks of (B, H, N, d, scale, dtype); returns FA_OK or an error and
// the element count B*H*N*d in *elems.
int check_problem(int B, int H, int N, int d, float scale, int dtype, int64_t* elems) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_DIM;
  int64_t bh, bhn, all;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &bhn) || !mul_ok(bhn, d, &all)) return FA_ERR_DIM;
  if (!head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  *elems = all;
  return FA_OK;
}

// Per-device check that the current device is a gfx950 (cached).
int device_ok() {
  static std::atomic<int> state[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (dev < 64) {
    const int s = state[dev].load(std::memory_order_relaxed);
    if (s != 0) return s > 0 ? FA_OK : FA_ERR_DEVICE;
  }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FA_ERR_DEVICE;
  const bool ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) state[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? FA_OK : FA_ERR_DEVICE;
}

// The kernels run the softmax in the log2 domain with c = |scale| * log2(e) and
// fold a negative scale into Q's sign. c is kept >= 1e-30 so that a masked
// score (-inf) times c stays -inf; for scale 0 every |s * c| is then below
// 2^-60 and exp2 of it rounds to exactly 1, i.e. uniform weights as required.
void fill_scale(FwdArgs& a, float scale) {
  a.c = std::fmax(std::fabs(scale) * kLog2e, 1e-30f);
  a.qsign = scale < 0.f ? 0x80008000u : 0u;
}

FwdArgs contiguous_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                        int N, int d, float scale) {
  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  const int64_t sr = d, sh = (int64_t)N * d, sb = (int64_t)H * N * d;
  a.q_sb = a.k_sb = a.v_sb = a.o_sb = sb;
  a.q_sh = a.k_sh = a.v_sh = a.o_sh = sh;
  a.q_sr = a.k_sr = a.v_sr = a.o_sr = sr;
  a.lse_sb = (int64_t)H * N;
  a.lse_sh = N;
  a.cu_seqlens = nullptr;
  a.B = B;
  a.H = H;
  a.N = N;
  fill_scale(a, scale);
  return a;
}

}  // namespace fa

using namespace fa;

extern "C" {

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_DIM: return "invalid or overflowing size or stride";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim or dtype (d in {64,96,128,256}; fp16/bf16)";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ALIAS: return "an output overlaps an input, the other output or itself";
    case FA_ERR_DEVICE: return "current device is not a usable gfx950";
    case FA_ERR_TOO_LARGE: return "B*H*N exceeds the static scratch of fa_bwd_noalloc (FA_BWD_NOALLOC_MAX_ROWS)";
    default: return "unknown fa_status";
  }
}

int fa_version(void) { return (1 << 16) | 0; }

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, int dtype, void* stream) {
  int64_t elems = 0;
  int rc = check_problem(B, H, N, d, scale, dtype, &elems);
  if (rc != FA_OK) return rc;
  if (elems == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return FA_ERR_ALIGN;
  const int64_t nbytes = elems * 2, lbytes = (elems / d) * 4;
  if (overlap(o, nbytes, q, nbytes) || overlap(o, nbytes, k, nbytes) ||
      overlap(o, nbytes, v, nbytes) || overlap(lse, lbytes, q, nbytes) ||
      overlap(lse, lbytes, k, nbytes) || overlap(lse, lbytes, v, nbytes) ||
      overlap(lse, lbytes, o, nbytes))
    return FA_ERR_ALIAS;
  if ((rc = device_ok()) != FA_OK) return rc;

  const FwdArgs a = contiguous_args(q, k, v, o, lse, B, H, N, d, scale);
  return launch_fwd(a, d, dtype, causal != 0, static_cast<hipStream_t>(stream));
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float scale, int causal, int dtype, int64_t q_sb, int64_t q_sh,
                   int64_t q_sr, int64_t k_sb, int64_t k_sh, int64_t k_sr, int64_t v_sb,
                   int64_t v_sh, int64_t v_sr, int64_t o_sb, int64_t o_sh, int64_t o_sr,
                   void* stream) {
  int64_t elems = 0;
  int rc = check_problem(B, H, N, d, scale, dtype, &elems);
  if (rc != FA_OK) return rc;
  if (elems == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const int64_t st[12] = {q_sb, q_sh, q_sr, k_sb, k_sh, k_sr, v_sb, v_sh, v_sr, o_sb, o_sh, o_sr};
  for (int i = 0; i < 12; ++i) {
    if (st[i] < 0) return FA_ERR_DIM;
    if (i % 3 == 2 && st[i] > kMaxRowStride) return FA_ERR_DIM;
    if (st[i] % 8) return FA_ERR_ALIGN;
  }
  // the largest element offset reached must stay addressable; span[t] is the
  // element count from a tensor's base to just past its last element
  const int64_t ext[3] = {B, H, N};
  int64_t span[4];
  for (int t = 0; t < 4; ++t) {
    int64_t far = d, x = 0;
    for (int i = 0; i < 3; ++i) {
      if (!mul_ok(ext[i] - 1, st[3 * t + i], &x)) return FA_ERR_DIM;
      far += x;
      if (far >= (INT64_C(1) << 62)) return FA_ERR_DIM;
    }
    span[t] = far;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return FA_ERR_ALIGN;
  // o's and lse's address ranges must not meet q's, k's or v's, nor each other
  const void* in[3] = {q, k, v};
  const int64_t lbytes = elems / d * 4;
  for (int t = 0; t < 3; ++t)
    if (overlap(o, span[3] * 2, in[t], span[t] * 2) || overlap(lse, lbytes, in[t], span[t] * 2))
      return FA_ERR_ALIAS;
  if (overlap(lse, lbytes, o, span[3] * 2)) return FA_ERR_ALIAS;
  if (!rows_disjoint(o_sb, o_sh, o_sr, B, H, N, d)) return FA_ERR_ALIAS;
  if ((rc = device_ok()) != FA_OK) return rc;

  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.q_sb = q_sb; a.q_sh = q_sh; a.q_sr = q_sr;
  a.k_sb = k_sb; a.k_sh = k_sh; a.k_sr = k_sr;
  a.v_sb = v_sb; a.v_sh = v_sh; a.v_sr = v_sr;
  a.o_sb = o_sb; a.o_sh = o_sh; a.o_sr = o_sr;
  a.lse_sb = (int64_t)H * N;
  a.lse_sh = N;
  a.cu_seqlens = nullptr;
  a.B = B;
  a.H = H;
  a.N = N;
  fill_scale(a, scale);
  return launch_fwd(a, d, dtype, causal != 0, static_cast<hipStream_t>(stream));
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens, int B, int T, int max_seqlen, int H, int d,
                  float scale, int causal, int dtype, void* stream) {
  if (max_seqlen < 0 || T < 0) return FA_ERR_DIM;
  int64_t elems = 0;
  int rc = check_problem(1, H, T, d, scale, dtype, &elems);
  if (rc != FA_OK) return rc;
  if (B < 0) return FA_ERR_DIM;
  if (B == 0 || elems == 0 || max_seqlen == 0) return FA_OK;
  if (max_seqlen > T) return FA_ERR_DIM;
  if ((int64_t)H * d > kMaxRowStride) return FA_ERR_DIM;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3))
    return FA_ERR_ALIGN;
  const int64_t nbytes = elems * 2, lbytes = (elems / d) * 4;
  if (overlap(o, nbytes, q, nbytes) || overlap(o, nbytes, k, nbytes) ||
      overlap(o, nbytes, v, nbytes) || overlap(lse, lbytes, o, nbytes) ||
      overlap(lse, lbytes, q, nbytes) || overlap(lse, lbytes, k, nbytes) ||
      overlap(lse, lbytes, v, nbytes))
    return FA_ERR_ALIAS;
  if ((rc = device_ok()) != FA_OK) return rc;

  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  const int64_t sr = (int64_t)H * d;
  a.q_sb = a.k_sb = a.v_sb = a.o_sb = 0;  // batch offset comes from cu_seqlens
  a.q_sh = a.k_sh = a.v_sh = a.o_sh = d;
  a.q_sr = a.k_sr = a.v_sr = a.o_sr = sr;
  a.lse_sb = 0;
  a.lse_sh = T;
  a.cu_seqlens = cu_seqlens;
  a.B = B;
  a.H = H;
  a.N = max_seqlen;
  fill_scale(a, scale);
  return launch_fwd(a, d, dtype, causal != 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"
