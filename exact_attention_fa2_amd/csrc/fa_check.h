// Host-side argument checks and argument packing shared by the C-ABI entry
// points (defined in fa_api.hip). None of these makes a HIP call except
// device_ok().
#pragma once
#include <stdint.h>

#include "fa_fwd_kernel.h"

namespace fa {
// Largest row stride (elements) of any tensor: the kernels address a tile of
// up to 64 rows with 32-bit byte offsets.
constexpr int64_t kMaxRowStride = INT64_C(1) << 24;
bool mul_ok(int64_t a, int64_t b, int64_t* out);
bool head_dim_ok(int d);
bool aligned16(const void* p);
bool overlap(const void* a, int64_t na, const void* b, int64_t nb);
// the rows of a strided [B, H, N, d] tensor share no element
bool rows_disjoint(int64_t sb, int64_t sh, int64_t sr, int B, int H, int N, int d);
// checks of (B, H, N, d, scale, dtype); *elems = B*H*N*d on success
int check_problem(int B, int H, int N, int d, float scale, int dtype, int64_t* elems);
// FA_OK when the current device is a gfx950 (cached per device)
int device_ok();
void fill_scale(FwdArgs& a, float scale);
// kernel arguments for contiguous [B, H, N, d] tensors and [B, H, N] LSE
FwdArgs contiguous_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                        int N, int d, float scale);
}  // namespace fa
