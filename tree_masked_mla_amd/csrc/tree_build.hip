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
// Organisation: one wave per batch row.  The candidate set never holds more than
// Q+1 entries (each step removes one and adds at most two, one of which reuses
// the removed slot), so it lives in registers: 5 slots per lane.  A candidate is
// a unique 64-bit key whose order is the best-first order -- the score mapped to
// an order-preserving unsigned integer (high half), then the inverted
// (parent, rank) code (low half) -- so a step is a two-phase wave maximum (high
// halves, then low halves among the lanes that hold the high maximum), one slot
// clear and up to two slot writes.  The log-probabilities the tree can reach
// (min(D, Q) depths x min(K, Q) ranks) are staged in LDS once.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

constexpr int kSlots = 5;   // 64 lanes x 5 >= kMaxQ + 1 candidates
static_assert(64 * kSlots >= kMaxQ + 1, "candidate slots");

// float -> unsigned with the same order (-0 and +0 map to the same value)
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// (parent, rank) -> low half, larger for an earlier parent, then a better rank;
// never 0 (0 marks an empty slot)
__device__ __forceinline__ uint32_t tie_key(int parent, int rank) {
    return 0x7fffffffu - (uint32_t)(((parent + 1) << 8) | (rank < 0 ? 0 : rank));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
    return v;
}

__global__ __launch_bounds__(64) void tree_build_kernel(TreeArgs a) {
    extern __shared__ float slp[];   // [Ds][Ks] staged log-probabilities
    __shared__ float nscore[kMaxQ];
    __shared__ int32_t ndepth[kMaxQ], nparent[kMaxQ], nrank[kMaxQ];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int Ds = min(a.D, a.Q), Ks = min(a.K, a.Q);
    const float* lp = a.logp + (int64_t)b * a.D * a.K;
    for (int i = lane; i < Ds * Ks; i += 64) slp[i] = lp[(i / Ks) * a.K + (i % Ks)];
    for (int i = lane; i < a.Q; i += 64) {
        nscore[i] = 0.f;
        ndepth[i] = 0;
        nparent[i] = -1;
        nrank[i] = -1;
    }
    __syncthreads();

    uint32_t kh[kSlots], kl[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) kh[j] = kl[j] = 0u;
    if (lane == 0) {   // the root
        kh[0] = score_key(0.f);
        kl[0] = tie_key(-1, -1);
    }
    int napp = 1;   // slots handed out in append order: lane napp & 63, slot napp >> 6

    for (int i = 0; i < a.Q; ++i) {
        uint32_t bh = 0u, bl = 0u;
#pragma unroll
        for (int j = 0; j < kSlots; ++j)
            if (kh[j] > bh || (kh[j] == bh && kl[j] > bl)) {
                bh = kh[j];
                bl = kl[j];
            }
        const uint32_t wh = wave_max(bh);
        if (wh == 0u) break;   // no candidate left (the host's size check rules this out)
        const uint32_t wl = wave_max(bh == wh ? bl : 0u);
        const float s = key_score(wh);
        const uint32_t code = 0x7fffffffu - wl;
        const int p = (int)(code >> 8) - 1;
        const int r = p < 0 ? -1 : (int)(code & 255u);

        int own = -1;   // the slot that held the winner (keys are unique)
#pragma unroll
        for (int j = 0; j < kSlots; ++j)
            if (kh[j] == wh && kl[j] == wl) {
                kh[j] = kl[j] = 0u;
                own = j;
            }
        const uint64_t holders = __ballot(own >= 0);
        const int own_lane = __ffsll((unsigned long long)holders) - 1;
        const int own_slot = __shfl(own, own_lane, 64);

        const int d = p < 0 ? 0 : ndepth[p] + 1;
        const float ps = p < 0 ? 0.f : nscore[p];
        __syncthreads();   // every lane has read the node arrays before lane 0 extends them
        if (lane == 0) {
            nscore[i] = s;
            ndepth[i] = d;
            nparent[i] = p;
            nrank[i] = r;
        }

        // offer the first child, then the next sibling
        const bool child = d < a.D;
        const bool sib = d >= 1 && r + 1 < a.K;
        uint32_t ch = 0u, cl = 0u, sh = 0u, sl = 0u;
        if (child) {
            ch = score_key(s + slp[d * Ks]);
            cl = tie_key(i, 0);
        }
        if (sib && r + 1 < Ks) {   // a rank >= Q is never reached: the tree fills first
            sh = score_key(ps + slp[(d - 1) * Ks + r + 1]);
            sl = tie_key(p, r + 1);
        }
        const bool two = ch != 0u && sh != 0u;
        const uint32_t fh = ch != 0u ? ch : sh, fl = ch != 0u ? cl : sl;   // goes into the freed slot
        const int app_lane = napp & 63, app_slot = napp >> 6;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            if (fh != 0u && lane == own_lane && j == own_slot) {
                kh[j] = fh;
                kl[j] = fl;
            }
            if (two && lane == app_lane && j == app_slot) {
                kh[j] = sh;
                kl[j] = sl;
            }
        }
        napp += two ? 1 : 0;
        __syncthreads();
    }

    // outputs
    const int64_t base = (int64_t)b * a.Q;
    for (int i = lane; i < a.Q; i += 64) {
        const int d = ndepth[i], r = nrank[i];
        a.parent[base + i] = nparent[i];
        if (a.depth) a.depth[base + i] = d;
        if (a.rank) a.rank[base + i] = r;
        if (a.score) a.score[base + i] = nscore[i];
        if (a.token) {
            const bool chosen = d >= 1 && d <= a.D && r >= 0 && r < a.K;
            a.token[base + i] = !chosen ? -1 : (a.tokens ? a.tokens[((int64_t)b * a.D + d - 1) * a.K + r] : r);
        }
    }
}

}  // namespace

size_t tree_build_lds_bytes(int D, int K, int Q) { return sizeof(float) * (size_t)min(D, Q) * (size_t)min(K, Q); }

hipError_t launch_tree_build(const TreeArgs& a, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(tree_build_kernel, dim3((unsigned)a.B), dim3(64), tree_build_lds_bytes(a.D, a.K, a.Q), stream,
                       a);
    return hipGetLastError();
}

}  // namespace ddtv
