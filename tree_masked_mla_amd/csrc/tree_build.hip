// Best-first draft-tree builder: per-depth top-K drafter log-probabilities in,
// the tree of the Q best choice paths out, as parent arrays that the visibility
// builder reads directly (the tree builder of "The Moment of Truth: Validating a
// Custom CUDA Attention Kernel for Speculative Decoding", section "Context:
// Building a Native DDTree Inference Engine", which builds the draft tree on the
// device in place of a per-request CPU heap).
//
// Definition (the pages name the builder but not its rule; this is the reading
// the library documents):
//  * depth d = 1..D offers K choices with log-probabilities logp[d-1][0..K-1],
//    sorted in descending order; a node's score is its parent's score plus its
//    choice's log-probability, summed in float32; the root scores 0;
//  * best first: the next node is the candidate with the highest score; equal
//    scores go to the candidate whose parent was taken first, then to the better
//    rank (the order in which candidates appear when a taken node offers all K
//    children at once);
//  * taking node (d, r) offers its first child (d+1, rank 0) when d < D and its
//    next sibling (same parent, rank r+1) when r+1 < K.  With sorted inputs that
//    takes the same nodes, in the same order, as offering all K children at once.
//
// Organisation: one wave per batch row, no barriers and no LDS traffic in the
// loop beyond two reads of the staged log-probabilities per node.
//  * The candidate set never holds more than Q+1 entries (each step removes one
//    and adds at most two, one of them in the removed slot), so it lives in
//    registers: 5 slots per lane.  A candidate is a unique 64-bit key whose
//    order is the best-first order: the score mapped to an order-preserving
//    unsigned integer (high half), then the inverted (parent, rank) code with
//    the candidate's depth below it (low half).
//  * A step is a wave maximum of the high halves (4 DPP steps inside 16-lane rows
//    plus 4 readlanes); the low halves are compared only when several lanes hold
//    the top score.  Then the winner's slot takes the new first child and an
//    appended slot the new sibling.
//  * Taken nodes' scores also live in registers (node i: lane i & 63, slot
//    i >> 6), so the parent's score for a sibling's key is one readlane.
//  * The log-probabilities the tree can reach (min(D, Q) depths x min(K, Q)
//    ranks) are staged in LDS once.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

// Register slots per lane: kSlots candidate slots (64 * kSlots >= Q + 1 candidates)
// and kNodeSlots taken-node slots (64 * kNodeSlots >= Q), instantiated per tree
// size so small trees scan fewer slots per step: (2, 1) for Q <= 64, (3, 2) for
// Q <= 128, (5, 4) up to kMaxQ.
constexpr int kMaxSlots = 5;              // 64 lanes x 5 >= kMaxQ + 1 candidates
static_assert(64 * kMaxSlots >= kMaxQ + 1, "candidate slots");

// float -> unsigned with the same order (-0 and +0 map to the same value)
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// (parent, rank, depth) -> low half: larger for an earlier parent, then a better
// rank (the depth follows from the parent and only rides along); never 0, which
// marks an empty slot
__device__ __forceinline__ uint32_t tie_key(int parent, int rank, int depth) {
    return 0x7fffffffu - (uint32_t)(((parent + 1) << 16) | ((rank < 0 ? 0 : rank) << 8) | depth);
}

// Maximum over the wave, returned to every lane: within each 16-lane row by DPP
// (quad swaps, then rotations by 4 and 8), across the 4 rows by readlane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false));    // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false));    // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xf, 0xf, false));   // row_ror 4
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, false));   // row_ror 8
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

template <int kSlots, int kNodeSlots>
__global__ __launch_bounds__(64) void tree_build_kernel(TreeArgs a) {
    extern __shared__ float slp[];       // [Ds][Ks] staged log-probabilities
    __shared__ uint32_t ncode[kMaxQ];    // taken node i: (parent + 1) << 16 | (rank + 1) << 8 | depth
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int Ds = min(a.D, a.Q), Ks = min(a.K, a.Q);
    const float* lp = a.logp + (int64_t)b * a.D * a.K;
    for (int i = lane; i < Ds * Ks; i += 64) slp[i] = lp[(i / Ks) * a.K + (i % Ks)];
    for (int i = lane; i < a.Q; i += 64) ncode[i] = 0u;
    __syncthreads();

    uint64_t key[kSlots];   // 0 = empty
#pragma unroll
    for (int j = 0; j < kSlots; ++j) key[j] = 0u;
    if (lane == 0) key[0] = ((uint64_t)score_key(0.f) << 32) | tie_key(-1, -1, 0);   // the root
    float nsc[kNodeSlots];  // score of taken node i: lane i & 63, slot i >> 6
#pragma unroll
    for (int j = 0; j < kNodeSlots; ++j) nsc[j] = 0.f;
    int napp = 1;   // slots handed out in append order: lane napp & 63, slot napp >> 6

    for (int i = 0; i < a.Q; ++i) {
        // this lane's best candidate and its slot (branch-free)
        uint64_t best = key[0];
        int bslot = 0;
#pragma unroll
        for (int j = 1; j < kSlots; ++j) {
            const bool gt = key[j] > best;
            best = gt ? key[j] : best;
            bslot = gt ? j : bslot;
        }
        const uint32_t bh = (uint32_t)(best >> 32);
        const uint32_t wh = wave_max(bh);
        if (wh == 0u) break;   // no candidate left (the host's size check rules this out)
        // the low half decides only between lanes that hold the top score (rare)
        const uint64_t top = __ballot(bh == wh);
        uint32_t wl;
        if (__popcll(top) == 1) {
            wl = __builtin_amdgcn_readlane((uint32_t)best, __ffsll((unsigned long long)top) - 1);
        } else {
            wl = wave_max(bh == wh ? (uint32_t)best : 0u);
        }
        const uint64_t win = ((uint64_t)wh << 32) | wl;
        const int own_lane = __ffsll((unsigned long long)__ballot(best == win)) - 1;
        const int own_slot = __builtin_amdgcn_readlane(bslot, own_lane);

        const float s = key_score(wh);
        const uint32_t code = 0x7fffffffu - wl;
        const int p = (int)(code >> 16) - 1;
        const int r = p < 0 ? -1 : (int)((code >> 8) & 255u);
        const int d = (int)(code & 255u);
        const bool last = i + 1 == a.Q;
        const bool child = !last && d < a.D;
        // a rank >= Q is never reached: the tree fills first
        const bool sib = !last && d >= 1 && r + 1 < a.K && r + 1 < Ks;
        const float lc = child ? slp[d * Ks] : 0.f;                  // both reads issued at once
        const float lsb = sib ? slp[(d - 1) * Ks + r + 1] : 0.f;

        // the parent's score (for the sibling), then record node i
        float ps = 0.f;
        if (p >= 0) {
            const int ps_slot = p >> 6;
            float mine = nsc[0];
#pragma unroll
            for (int j = 1; j < kNodeSlots; ++j) mine = ps_slot == j ? nsc[j] : mine;
            ps = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), p & 63));   // bits, not value
        }
        if (lane == (i & 63)) {
#pragma unroll
            for (int j = 0; j < kNodeSlots; ++j) nsc[j] = j == (i >> 6) ? s : nsc[j];
        }
        if (lane == 0) ncode[i] = ((uint32_t)(p + 1) << 16) | ((uint32_t)(r + 1) << 8) | (uint32_t)d;
        if (last) break;

        // offer the first child into the freed slot, the next sibling into an
        // appended one (or the freed slot when there is no child)
        const uint64_t kc = child ? ((uint64_t)score_key(s + lc) << 32) | tie_key(i, 0, d + 1) : 0u;
        const uint64_t ks = sib ? ((uint64_t)score_key(ps + lsb) << 32) | tie_key(p, r + 1, d) : 0u;
        const bool two = child && sib;
        const uint64_t kf = child ? kc : ks;
        const int app_lane = napp & 63, app_slot = napp >> 6;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            key[j] = (lane == own_lane && j == own_slot) ? kf : key[j];
            key[j] = (two && lane == app_lane && j == app_slot) ? ks : key[j];
        }
        napp += two ? 1 : 0;
    }
    __syncthreads();

    // outputs: lane l writes nodes l, l + 64, ...
    const int64_t base = (int64_t)b * a.Q;
#pragma unroll
    for (int j = 0; j < kNodeSlots; ++j) {
        const int i = j * 64 + lane;
        if (i < a.Q) {
            const uint32_t c = ncode[i];
            const int p = (int)(c >> 16) - 1;
            const int r = (int)((c >> 8) & 255u) - 1;
            const int d = (int)(c & 255u);
            a.parent[base + i] = p;
            if (a.depth) a.depth[base + i] = d;
            if (a.rank) a.rank[base + i] = r;
            if (a.score) a.score[base + i] = nsc[j];
            if (a.token) {
                const bool chosen = d >= 1 && d <= a.D && r >= 0 && r < a.K;
                a.token[base + i] =
                    !chosen ? -1 : (a.tokens ? a.tokens[((int64_t)b * a.D + d - 1) * a.K + r] : r);
            }
        }
    }
}

}  // namespace

size_t tree_build_lds_bytes(int D, int K, int Q) { return sizeof(float) * (size_t)min(D, Q) * (size_t)min(K, Q); }

hipError_t launch_tree_build(const TreeArgs& a, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    const size_t lds = tree_build_lds_bytes(a.D, a.K, a.Q);
    if (a.Q <= 64)
        hipLaunchKernelGGL((tree_build_kernel<2, 1>), dim3((unsigned)a.B), dim3(64), lds, stream, a);
    else if (a.Q <= 128)
        hipLaunchKernelGGL((tree_build_kernel<3, 2>), dim3((unsigned)a.B), dim3(64), lds, stream, a);
    else
        hipLaunchKernelGGL((tree_build_kernel<kMaxSlots, kMaxQ / 64>), dim3((unsigned)a.B), dim3(64), lds, stream,
                           a);
    return hipGetLastError();
}

}  // namespace ddtv
