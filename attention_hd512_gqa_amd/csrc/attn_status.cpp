// Status strings of the C ABI.
#include "../../include/attn_hd512.h"

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "a count or size is out of range or inconsistent";
        case ATTN_ERR_UNSUPPORTED: return "outside the supported set (head_dim 512, page 64, dtypes)";
        case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
        case ATTN_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}
