// Host-side helpers shared by the C-ABI translation units (argument checks,
// error text).  Nothing here calls the HIP runtime.
#pragma once

#include <hip/hip_runtime.h>

#define DA_HIP_STREAM_DEFINED
#include "da.h"
#include "internal.h"

namespace da {

da_status fail(da_status st, const char *fmt, ...);
da_status ok();
da_status hip_fail(hipError_t e, const char *what);
da_status check_shape(const da_attn_shape *s, bool kv4);
da_status check_ptr(const void *p, const char *name);
int esize(int dtype);
enum SplitMode { SPLIT_DENSE = 0, SPLIT_U4 = 1, SPLIT_PAGED = 2 };
int32_t split_tokens_of(const da_attn_shape *s, int mode);
AttnLaunch dense_launch(const da_attn_shape *s, int kv_fmt, int mode);

}  // namespace da

#define DA_TRY(x)                              \
    do {                                       \
        da_status _st = (x);                   \
        if (_st != DA_OK) return _st;          \
    } while (0)
