// Internal declarations shared by the HIP translation units of libddtv.
// gfx950 (CDNA4) only: wave64, 160 KiB LDS per workgroup, MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddtv.h"

namespace ddtv {

constexpr int kDLat = DDTV_D_LATENT;      // 512
constexpr int kDRope = DDTV_D_ROPE;       // 64
constexpr int kDQK = kDLat + kDRope;      // 576
constexpr int kMaxQ = DDTV_MAX_Q;         // 256
constexpr int kMaxW = kMaxQ / 32;         // 8 mask words
constexpr int kTile = 32;                 // KV positions per LDS tile (both kernels)
constexpr int kSplitQuantum = kTile / 2;  // split lengths are multiples of half a tile
constexpr int kVisChunk = 64;             // batch rows described per visibility launch
constexpr int kXcds = 8;                  // MI355X: 8 XCDs, workgroups dealt round-robin

// Everything the attention kernels need (passed by value).
struct AttnArgs {
    const float* q_abs;      // [B][Q][H][512]
    const float* q_rope;     // [B][Q][H][64]
    const void* ckv;         // [total_kv][512] f32 or bf16
    const void* k_rope;      // [total_kv][64]
    const uint32_t* bits;    // [B][Q][W]
    const ddtv_row* rows;    // [B]
    const int32_t* order;    // [B] batch row of each grid slot, or null for the identity
    float* out;              // [B][Q][H][512]
    float* lse;              // [B][Q][H] or null
    float* part_o;           // [B][n_split][R][512]   (n_split > 1)
    float2* part_ml;         // [B][n_split][R]  {m (log2 units), l}
    int B, Q, H, W, R;       // R = Q*H query rows per batch row
    int n_rt;                // row tiles per batch row
    int split_len;           // KV positions per split (multiple of kSplitQuantum)
    int n_split;             // splits per batch row in the grid (max over rows)
    int spread;              // 1: work item = workgroup id; 0: XCD-local order (xcd_remap)
    int halves;              // 1: row-half mode (32 rows per workgroup, halves combined in it; matrix kernel)
    float scale_log2;        // scale * log2(e)
    int absorb;              // a row's last split also takes a remainder of up to this many positions
                             // (row-half mode; 0 for the other kernels, whose splits stop at split_len)
};

// Everything the draft-tree builder needs (passed by value).
struct TreeArgs {
    const float* logp;       // [B][D][K], any order within each [b][d]
    const int32_t* tokens;   // [B][D][K] or null
    int32_t* parent;         // [B][Q]
    int32_t* depth;          // [B][Q] or null
    int32_t* rank;           // [B][Q] or null
    int32_t* token;          // [B][Q] or null
    float* score;            // [B][Q] or null
    int B, D, K, Q;
};
constexpr int kMaxTreeK = 64;   // choices per depth the builder accepts

// Everything the tree-accept step needs (passed by value).
struct AcceptArgs {
    const float* logits;     // [B][Q][V]
    const int32_t* parent;   // [B][Q]
    const int32_t* token;    // [B][Q] draft tokens
    const ddtv_row* rows;    // [B] cache geometry (compaction)
    int32_t* pred;           // [B][Q] out
    int32_t* path;           // [B][Q] out
    int32_t* out_tokens;     // [B][Q] out
    int32_t* accept_len;     // [B] out
    void* ckv;               // [total_kv][512] or null: no compaction
    void* k_rope;            // [total_kv][64]
    int kv_elem;             // bytes per cache element (4 or 2)
    int B, Q, V;
};

struct VisChunk {
    int64_t kv_off[kVisChunk];
    int32_t prefix[kVisChunk];
    int32_t order[kVisChunk];   // entries b0 .. b0+nb-1 of the longest-first row order
};

// Launchers (return the launch error, never synchronise).
hipError_t launch_visibility(const int32_t* parent, int b0, int nb, int Q, int W, uint32_t* bits,
                             ddtv_row* rows, int32_t* status, int32_t* order, const VisChunk& chunk,
                             hipStream_t stream);
hipError_t launch_attn_valu(const AttnArgs& a, int kv_dtype, int64_t grid, hipStream_t stream);
hipError_t launch_attn_mfma(const AttnArgs& a, int kv_dtype, int64_t grid, hipStream_t stream);
int mfma_rows_per_workgroup(int kv_dtype);   // query rows per workgroup of the fp32 MFMA kernel
hipError_t launch_attn_mfma_bf16(const AttnArgs& a, int64_t grid, hipStream_t stream);
int bf16_rows_per_workgroup();   // query rows per workgroup of the bf16 MFMA kernel
hipError_t launch_merge(const AttnArgs& a, hipStream_t stream);
hipError_t launch_tree_build(const TreeArgs& a, hipStream_t stream);
hipError_t launch_tree_accept(const AcceptArgs& a, hipStream_t stream);

constexpr int kValuRows = 16;   // query rows per VALU workgroup

// Splits of a batch row of kv_len positions at split length L: split s starts at
// s * L and ends L later, except the last, which ends at kv_len; it also takes a
// remainder of up to `absorb` positions rather than leaving them to a split of
// their own (a row one position past a multiple of L would otherwise hold up a
// whole extra workgroup of the grid for that position).
__host__ __device__ __forceinline__ int splits_of(int kv_len, int L, int absorb) {
    const int n = (kv_len + L - 1 - absorb) / L;
    return kv_len <= 0 ? 0 : (n < 1 ? 1 : n);
}

// Work item of workgroup i in the XCD-local order: consecutive work items land
// on the same XCD (the dispatcher deals workgroup i to XCD i % 8).  Bijective for
// any grid.  Also used by the host planner to simulate the dispatch.
__host__ __device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t G) {
    const int64_t q = G / kXcds, r = G % kXcds;
    const int64_t x = i % kXcds, k = i / kXcds;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)

// Work item of this workgroup under the planned order.
__device__ __forceinline__ int64_t work_item(const AttnArgs& a) {
    return a.spread ? (int64_t)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
}

// Batch row of grid slot `slot` (the slowest-varying part of the work item).
__device__ __forceinline__ int batch_row(const AttnArgs& a, int slot) { return a.order ? a.order[slot] : slot; }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Four FP8 E4M3 ("fn") bytes of v (lowest byte first) -> float32, exactly, with
// gfx950's packed conversion (v_cvt_pk_f32_fp8, two values per instruction).  Its
// decoding was checked against the OCP E4M3 definition on all 256 codes (NaN for
// 0x7F and 0xFF) by an in-bounds probe on the device; the parity tests cover it
// through every FP8 path.
__device__ __forceinline__ float4 fp8x4(uint32_t v) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
    return make_float4(lo[0], lo[1], hi[0], hi[1]);
}

// Wave-level butterflies (wave64).
__device__ __forceinline__ float wave_xor(float v, int m) { return __shfl_xor(v, m, 64); }

#endif

}  // namespace ddtv
