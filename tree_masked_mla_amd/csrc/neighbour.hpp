// Internal declarations of the steps around the attention (query preparation,
// value projection, appended cache rows), shared by api.hip and neighbour.hip.
#pragma once

#include "ddtv_internal.hpp"

namespace ddtv {

// A per-head projection GEMM (absorb or value), optionally with the query's
// rotary step (passed by value).  A[m][h][k] = A[m * lda + h * a_head + k];
// the head-h block of B is [K][N] (absorb) or [N][K] (value);
// C[m][h][n] = C[m * ldc + h * c_head + n].
struct ProjArgs {
    const float* A;
    int64_t lda, a_head;
    const float* B;
    int64_t b_head;
    float* C;
    int64_t ldc, c_head;
    int64_t M;
    int K, N, H;
    float* rope_out;            // [M][H][64], or null: no rotary step
    const int32_t* positions;   // [M], or null: prefix + depth from the masks
    const uint32_t* bits;       // [B][Q][W] ancestor-or-self masks
    const ddtv_row* rows;       // [B]
    int Q, W;
    double inv_freq[32];        // rotary frequency of each pair
};

// The tree nodes' new cache rows (passed by value).
struct AppendArgs {
    const float* latent;        // [B][Q][512]
    const float* k_pe;          // [B][Q][64], not yet rotated
    const int32_t* positions;   // [B][Q], or null: prefix + depth from the masks
    const uint32_t* bits;       // [B][Q][W]
    const ddtv_row* rows;       // [B]
    void* ckv;                  // [total_kv][512] f32 or bf16
    void* k_rope;               // [total_kv][64]
    int B, Q, W;
    int dtype;                  // ddtv_dtype of the caches
    double inv_freq[32];
};

// cus: compute units of the device (small grids take narrower tiles)
hipError_t launch_proj(const ProjArgs& p, bool b_trans, int cus, hipStream_t stream);
hipError_t launch_append_kv(const AppendArgs& p, hipStream_t stream);

}  // namespace ddtv
