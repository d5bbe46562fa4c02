// Host-side pieces shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/attn_hd512.h"
