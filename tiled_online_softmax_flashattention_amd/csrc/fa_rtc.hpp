// Caller-defined score_mods (internal to the library): creation, release and
// launches of the run-time compiled kernels (fa_custom.hpp).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/fa_mi355x.h"
#include "fa_common.hpp"

namespace fa {

fa_status custom_create(const char* source, fa_score_mod* out, char* log, size_t log_bytes);
fa_status custom_destroy(fa_score_mod mod);

// Launches pass 0 (forward), 1 (query pass), 2 (key/value pass) or 3 (the
// forward over one key chunk per workgroup, writing partials) of the
// configuration (dtype, D, causal, key mask, block mask) over `grid`
// workgroups of 256 threads with `shared_bytes` of dynamic LDS (the fp32
// kernels'; 0 for the 16-bit ones), compiling and loading it for the current
// device on first use.
fa_status custom_launch(fa_score_mod mod, int pass, int dtype, int D, bool causal, bool mask, bool blk,
                        const AttnArgs& a, unsigned grid, size_t shared_bytes, hipStream_t st);

}  // namespace fa
