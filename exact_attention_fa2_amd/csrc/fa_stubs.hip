#include <hip/hip_runtime.h>
#include "fa.h"
extern "C" {
int fa_bwd(const void*, const void*, const void*, const void*, const void*, const float*, void*,
           void*, void*, void*, int, int, int, int, float, int, int, void*) {
  return FA_ERR_UNSUPPORTED;
}
int64_t fa_bwd_workspace_bytes(int, int, int, int) { return -1; }
}
