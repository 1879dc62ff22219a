// Kernels of the external-prefix (tree-tail) mode of the verify step.
#pragma once

#include "ddtv_internal.hpp"

namespace ddtv {

// tail_rows[b] = the tree rows of batch row b as a row without prefix:
// {kv_off + prefix, 0, Q}.
hipError_t launch_tail_rows(const ddtv_row* rows, ddtv_row* tail_rows, int B, int Q, hipStream_t stream);

// Over n query rows: out (the tree rows' result, merged in place) and lse_tail
// merged with the caller's prefix result (prefix_out normalised, prefix_lse
// natural log); the merged lse goes to lse (may be null).
hipError_t launch_tail_merge(float* out, const float* lse_tail, float* lse, const float* prefix_out,
                             const float* prefix_lse, int64_t n, hipStream_t stream);

}  // namespace ddtv
