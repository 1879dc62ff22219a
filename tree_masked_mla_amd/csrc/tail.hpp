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

// Everything the tree-sparse tail kernel needs (passed by value).
struct TailSparseArgs {
    const float* q_abs;         // [B][Q][H][512]
    const float* q_rope;        // [B][Q][H][64]
    const void* ckv;            // [total_kv][512] of the cache dtype
    const void* k_rope;         // [total_kv][64]
    const uint32_t* bits;       // [B][Q][W]
    const ddtv_row* rows;       // [B]
    const float* prefix_out;    // [B][Q][H][512], normalised
    const float* prefix_lse;    // [B][Q][H], natural log
    float* out;                 // [B][Q][H][512]
    float* lse;                 // [B][Q][H] or null
    int B, Q, H, W;
    float scale_log2;           // scale * log2(e)
};

// Attention of every tree node over its own ancestors-or-self only, merged with
// the caller's prefix result, in one launch (one workgroup per node).
hipError_t launch_tail_sparse(const TailSparseArgs& a, int kv_dtype, hipStream_t stream);

}  // namespace ddtv
