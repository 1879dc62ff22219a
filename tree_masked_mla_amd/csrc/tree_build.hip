// Best-first draft-tree builder: per-depth drafter log-probabilities in, the tree
// of the Q best choice paths out, as parent arrays that the visibility builder
// reads directly (the tree builder of "The Moment of Truth: Validating a Custom
// CUDA Attention Kernel for Speculative Decoding", section "Context: Building a
// Native DDTree Inference Engine", which builds the draft tree on the device in
// place of a per-request CPU heap).
//
// Definition (the pages name the builder but not its rule; this is the reading
// the library documents):
//  * depth d = 1..D offers K choices with log-probabilities logp[d-1][0..K-1] in
//    any order; they are ranked by descending value, equal values by index;
//  * a node's score is its parent's score plus its choice's log-probability,
//    summed in float32; the root scores 0;
//  * best first over every child of every taken node: the next node is the
//    candidate with the highest score; equal scores go to the candidate whose
//    parent was taken first, then to the better rank.
//
// One workgroup (16 waves) per tree, in three phases.
//  1. Ranking.  Each depth's choices are ranked in LDS; the first min(K, Q) ranks
//     are kept as value and choice-index tables in rank order.
//  2. Level pass (all waves).  When every value is <= 0, a child never scores
//     above its parent, so the tree is the root plus the Q-1 best nodes of the
//     whole choice lattice, in score order, when no two of the nodes involved
//     tie.  The pass keeps the best Q-1 nodes found so far (T, sorted), and for
//     depth d = 1, 2, ... scores the children of T's nodes of depth d-1 and keeps
//     those that beat T's last score once T is full; they join T by a merge in
//     which every element's new position is counted.  A parent that T drops
//     takes its lower-scoring children with it, so T's nodes of each depth are
//     exactly the parents the next depth needs.  Any equal scores among the nodes
//     compared, a positive value, or more candidates than the buffers hold end
//     the pass without a result.
//  3. Sequential pass (wave 0), when the level pass gave no result: best first
//     one node per step.  Taking node (d, r) offers its first child (d+1, rank 0)
//     and its next sibling (same parent, rank r+1): with choices in rank order
//     that takes the same nodes, in the same order, as offering all K children
//     at once, since a parent's children are offered in the order in which best
//     first would take them.
//     * The candidate set never holds more than Q+1 entries (each step removes
//       one and adds at most two, one of them in the removed slot), so it lives in
//       registers: a candidate is a unique 64-bit key whose order is the
//       best-first order -- the score mapped to an order-preserving unsigned
//       integer (high half), then the inverted (parent, rank) code with the
//       candidate's depth below it (low half).
//     * A step is a wave maximum of the high halves (4 DPP steps inside 16-lane
//       rows plus 4 readlanes); the low halves are compared only when several
//       lanes hold the top score.  The winner's slot takes the new first child and
//       an appended slot the new sibling.
//     * Taken nodes' scores also live in registers (node i: lane i & 63, slot
//       i >> 6), so the parent's score for a sibling's key is one readlane.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

constexpr int kThreads = 1024;         // 16 waves per tree
constexpr int kNewCap = 1024;          // children one depth of the level pass may keep
constexpr int kStoreCap = 2048;        // nodes the level pass may create in all
constexpr int kMaxSlots = 5;           // 64 lanes x 5 >= kMaxQ + 1 candidates
static_assert(64 * kMaxSlots >= kMaxQ + 1, "candidate slots");

enum : int { kPositive = 1, kTie = 2, kOverflow = 4, kBroken = 8 };

struct TreeLds {
    alignas(16) float t_score[2][kMaxQ];   // T (sorted by descending score once merged; double-buffered)
    uint16_t t_gid[2][kMaxQ];          // node id (index into s_*) of each T entry
    alignas(16) float n_score[kNewCap];   // this depth's kept children (node id = base + slot)
    int16_t e_pos[kNewCap + kMaxQ];    // merge: each element's position in the merged T (Qm: dropped)
    uint16_t e_gid[kNewCap + kMaxQ];   //        and its node id
    float p_score[kMaxQ];              // T's nodes of the previous depth: the parents
    uint16_t p_gid[kMaxQ];
    uint16_t s_parent[kStoreCap];      // node id -> parent's node id (0xffff for the root)
    uint8_t s_depth[kStoreCap];
    uint8_t s_rank[kStoreCap];
    uint16_t index_of[kStoreCap];      // node id -> tree index
    int16_t node_parent[kMaxQ];        // the result, tree index order
    uint8_t node_depth[kMaxQ];
    int8_t node_rank[kMaxQ];
    float node_score[kMaxQ];
    float staging[kThreads];           // raw log-probabilities of the depths being ranked
    int n_new[2], n_next[2];           // per-depth counters, alternating between depths
    // flags, one word per phase: each is read (after a barrier) only when no thread
    // can be writing it
    int flags;                         // ranking: kPositive
    int gflags;                        // generating children: kTie, kOverflow
    int mflags;                        // merging: kTie
    int bflags;                        // tree indices: kBroken
};

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

// Slot of each lane that wants one in an array filled through `counter`: one LDS
// atomic per wave.  Every lane of the wave must call it.
__device__ __forceinline__ int wave_append(int* counter, bool want) {
    const uint64_t mask = __ballot(want);
    if (mask == 0) return -1;
    const int leader = __ffsll((unsigned long long)mask) - 1;
    int base = 0;
    if ((int)__lane_id() == leader) base = atomicAdd(counter, (int)__popcll(mask));
    base = __builtin_amdgcn_readlane(base, leader);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    return want ? base + below : -1;
}

// Number of entries of ns[0..n) above x among the groups of 16 numbered k,
// k + S, k + 2S, ..., read with the next group in flight.  ns is 16-byte aligned
// and its entries from n to the next multiple of 16 hold NaN, which is never
// above anything.
__device__ __forceinline__ int count16(const float4& a, const float4& b, const float4& c, const float4& d, float x) {
    return ((a.x > x) + (a.y > x) + (a.z > x) + (a.w > x)) + ((b.x > x) + (b.y > x) + (b.z > x) + (b.w > x)) +
           ((c.x > x) + (c.y > x) + (c.z > x) + (c.w > x)) + ((d.x > x) + (d.y > x) + (d.z > x) + (d.w > x));
}
__device__ __forceinline__ int count_above(const float* ns, int n, float x, int k, int S) {
    const float4* v = reinterpret_cast<const float4*>(__builtin_assume_aligned(ns, 16));
    const int groups = (n + 15) >> 4;
    int c0 = 0, c1 = 0;   // two sums: shorter dependency chains
    if (k < groups) {
        float4 a = v[4 * k], b = v[4 * k + 1], c = v[4 * k + 2], d = v[4 * k + 3];
        bool odd = false;
        for (int g = k + S; g < groups; g += S) {
            const float4 na = v[4 * g], nb = v[4 * g + 1], nc = v[4 * g + 2], nd = v[4 * g + 3];
            if (odd) c1 += count16(a, b, c, d, x);
            else c0 += count16(a, b, c, d, x);
            odd = !odd;
            a = na;
            b = nb;
            c = nc;
            d = nd;
        }
        c0 += count16(a, b, c, d, x);
    }
    return c0 + c1;
}

// Sum over each aligned group of S lanes (S = 1, 2, 4 or 8), returned to every
// lane of the group: DPP quad swaps, then the mirror within 8 lanes.
__device__ __forceinline__ int group_sum(int v, int S) {
    if (S >= 2) v += __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, false);    // quad_perm 1,0,3,2
    if (S >= 4) v += __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, false);    // quad_perm 2,3,0,1
    if (S >= 8) v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false);   // row_half_mirror
    return v;
}

// Phase 2: the level pass.  Returns true (the same on every thread) when it has
// written the tree to L.node_*.
__device__ __forceinline__ bool level_pass(TreeLds& L, const float* sv, int D, int Ds, int Ks, int Q, int tid) {
    const int Qm = Q - 1;   // nodes besides the root
    // unused New slots and T entries hold NaN, so counts can read whole groups of 16
    for (int i = tid; i < kNewCap; i += kThreads) L.n_score[i] = __builtin_nanf("");
    for (int i = tid; i < kMaxQ; i += kThreads) L.t_score[0][i] = __builtin_nanf("");
    if (tid == 0) {
        L.p_score[0] = 0.f;
        L.p_gid[0] = 0;
        L.s_parent[0] = 0xffff;
        L.s_depth[0] = 0;
        L.s_rank[0] = 0xff;
        L.n_new[0] = L.n_new[1] = 0;
        L.n_next[0] = L.n_next[1] = 0;
        L.gflags = L.mflags = L.bflags = 0;
    }
    __syncthreads();
    int m = 0, np = 1, cur = 0, n_store = 1;
    bool sorted = true;      // T in descending order (false while nodes are only appended)
    float cut = -INFINITY;   // T's last score once T is full
    for (int d = 1; d <= Ds && np > 0; ++d) {
        const int par = d & 1;
        // the children of the parents that can still enter T
        const bool full = m == Qm;
        const float* row = sv + (d - 1) * Ks;
        const int pairs = np * Ks;
        for (int e0 = 0; e0 < pairs; e0 += kThreads) {   // same trip count on every thread
            const int e = e0 + tid;
            const int pi = e / Ks, r = e - pi * Ks;
            const float s = e < pairs ? L.p_score[pi] + row[r] : -INFINITY;
            if (e < pairs && full && s == cut) atomicOr(&L.gflags, kTie);
            const int slot = wave_append(&L.n_new[par], e < pairs && (!full || s > cut));
            if (slot < 0) continue;
            if (slot >= kNewCap || n_store + slot >= kStoreCap) {
                atomicOr(&L.gflags, kOverflow);
                continue;
            }
            L.n_score[slot] = s;
            const int g = n_store + slot;
            L.s_parent[g] = L.p_gid[pi];
            L.s_depth[g] = (uint8_t)d;
            L.s_rank[g] = (uint8_t)r;
        }
        __syncthreads();
        if (L.gflags) return false;
        const int n = L.n_new[par];
        if (n == 0) break;
        if (tid == 0) {   // the next depth's counters: their last reads preceded the barrier above
            L.n_new[par ^ 1] = 0;
            L.n_next[par ^ 1] = 0;
        }
        if (m + n < Qm) {
            // T cannot overflow yet: append the children unsorted; all are parents next
            for (int j = tid; j < n; j += kThreads) {
                const float x = L.n_score[j];
                L.n_score[j] = __builtin_nanf("");   // back to unused
                L.t_score[cur][m + j] = x;
                L.t_gid[cur][m + j] = (uint16_t)(n_store + j);
                L.p_score[j] = x;
                L.p_gid[j] = (uint16_t)(n_store + j);
            }
            __syncthreads();
            sorted = false;
            n_store += n;
            m += n;
            np = d < D ? n : 0;
            continue;
        }
        // merge: every element's position in T u New is the number of elements
        // above it.  Each element's count is split over S adjacent lanes (each
        // takes every S-th group of 16 values) and summed with DPP.  Two equal
        // scores would take the same position, so every writer checks its entry
        // after the barrier (a lost write means a tie).
        const int nxt = cur ^ 1;
        const int u = n + m;   // elements: New j at e = j, T entry i at e = n + i
        int S = 1;
        while (S < 8 && u * (2 * S) <= kThreads) S *= 2;
        const int per_pass = kThreads / S;
        const int k = tid & (S - 1);
        for (int e0 = 0; e0 < u; e0 += per_pass) {   // same trip count on every thread
            const int e = e0 + tid / S;
            const bool valid = e < u, is_new = e < n;
            float x = 0.f;
            int cnt = 0;
            if (valid) {
                x = is_new ? L.n_score[e] : L.t_score[cur][e - n];
                cnt = count_above(L.n_score, n, x, k, S);
                if (!sorted) cnt += count_above(L.t_score[cur], m, x, k, S);
            }
            cnt = group_sum(cnt, S);
            int pos = Qm;
            if (valid && k == 0) {
                if (!sorted) {
                    pos = cnt;
                } else if (!is_new) {
                    pos = (e - n) + cnt;   // T entries above a T entry: the ones before it
                } else {
                    int lo = 0, hi = m;    // T entries above x (T is sorted)
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (L.t_score[cur][mid] > x) lo = mid + 1;
                        else hi = mid;
                    }
                    if (lo < m && L.t_score[cur][lo] == x) atomicOr(&L.mflags, kTie);
                    pos = lo + cnt;
                }
                pos = min(pos, Qm);
                const int g = is_new ? n_store + e : L.t_gid[cur][e - n];
                L.e_pos[e] = (int16_t)pos;
                L.e_gid[e] = (uint16_t)g;
                if (pos < Qm) {
                    L.t_score[nxt][pos] = x;
                    L.t_gid[nxt][pos] = (uint16_t)g;
                }
            }
            const int q = wave_append(&L.n_next[par], valid && k == 0 && is_new && pos < Qm && d < D);
            if (q >= 0) {   // a parent for the next depth
                L.p_score[q] = x;
                L.p_gid[q] = (uint16_t)(n_store + e);
            }
        }
        __syncthreads();
        for (int e = tid; e < u; e += kThreads) {
            const int pos = L.e_pos[e];
            if (pos < Qm && L.t_gid[nxt][pos] != L.e_gid[e]) atomicOr(&L.mflags, kTie);
            if (e < n) L.n_score[e] = __builtin_nanf("");   // back to unused (its readers passed the barrier above)
        }
        __syncthreads();
        if (L.mflags) return false;
        sorted = true;
        n_store += n;
        m = min(m + n, Qm);
        cur = nxt;
        cut = m == Qm ? L.t_score[cur][Qm - 1] : -INFINITY;
        np = L.n_next[par];
    }
    if (m != Qm || !sorted) return false;   // cannot happen once Q fits the tree (the host checks)
    // node ids -> tree indices, then each node's parent index (parents precede
    // their children: a parent scores above each of its children)
    for (int g = tid; g < n_store; g += kThreads) L.index_of[g] = 0xffff;
    __syncthreads();
    for (int i = tid; i < Qm; i += kThreads) L.index_of[L.t_gid[cur][i]] = (uint16_t)(i + 1);
    if (tid == 0) L.index_of[0] = 0;
    __syncthreads();
    for (int i = tid; i < Qm; i += kThreads) {
        const int g = L.t_gid[cur][i];
        const int p = L.index_of[L.s_parent[g]];
        if (p > i) atomicOr(&L.bflags, kBroken);
        L.node_parent[i + 1] = (int16_t)p;
        L.node_depth[i + 1] = L.s_depth[g];
        L.node_rank[i + 1] = (int8_t)L.s_rank[g];
        L.node_score[i + 1] = L.t_score[cur][i];
    }
    __syncthreads();
    return L.bflags == 0;
}

// Phase 3: one node per step on wave 0 (see the file comment).
template <int kSlots, int kNodeSlots>
__device__ __forceinline__ void sequential_pass(TreeLds& L, const float* sv, int D, int Ks, int K, int Q, int lane) {
    uint64_t key[kSlots];   // 0 = empty
#pragma unroll
    for (int j = 0; j < kSlots; ++j) key[j] = 0u;
    if (lane == 0) key[0] = ((uint64_t)score_key(0.f) << 32) | tie_key(-1, -1, 0);   // the root
    float nsc[kNodeSlots];  // score of taken node i: lane i & 63, slot i >> 6
#pragma unroll
    for (int j = 0; j < kNodeSlots; ++j) nsc[j] = 0.f;
    int napp = 1;   // slots handed out in append order: lane napp & 63, slot napp >> 6

    for (int i = 0; i < Q; ++i) {
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
        const bool last = i + 1 == Q;
        const bool child = !last && d < D;
        // a rank >= Q is never reached: the tree fills first
        const bool sib = !last && d >= 1 && r + 1 < K && r + 1 < Ks;
        const float lc = child ? sv[d * Ks] : 0.f;                  // both reads issued at once
        const float lsb = sib ? sv[(d - 1) * Ks + r + 1] : 0.f;

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
        if (lane == 0) {
            L.node_parent[i] = (int16_t)p;
            L.node_depth[i] = (uint8_t)d;
            L.node_rank[i] = (int8_t)r;
        }
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
#pragma unroll
    for (int j = 0; j < kNodeSlots; ++j) {
        const int i = j * 64 + lane;
        if (i < Q) L.node_score[i] = nsc[j];
    }
}

template <int kSlots, int kNodeSlots>
__global__ __launch_bounds__(kThreads) void tree_build_kernel(TreeArgs a) {
    extern __shared__ float dyn[];       // [Ds][Ks] values in rank order, then [Ds][Ks] choice indices
    __shared__ TreeLds L;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int Ds = min(a.D, a.Q), Ks = min(a.K, a.Q);
    float* sv = dyn;
    uint8_t* so = reinterpret_cast<uint8_t*>(dyn + Ds * Ks);
    const float* lp = a.logp + (int64_t)b * a.D * a.K;

    // Phase 1: rank each depth's choices (descending value, equal values by index)
    if (tid == 0) L.flags = 0;
    const int per = kThreads / a.K;   // depths ranked together (K <= 64, so at least 4)
    bool positive = false;
    for (int d0 = 0; d0 < Ds; d0 += per) {
        const int ne = min(per, Ds - d0) * a.K;
        __syncthreads();   // the previous group's readers are done with the staging area
        float v = 0.f;
        if (tid < ne) {
            v = lp[(int64_t)d0 * a.K + tid];
            L.staging[tid] = v;
        }
        __syncthreads();
        if (tid < ne) {
            const int k = tid % a.K;
            const float* row = L.staging + (tid - k);
            int r = 0;
            for (int j = 0; j < a.K; ++j) {
                const float u = row[j];
                r += (u > v || (u == v && j < k)) ? 1 : 0;
            }
            const int d = d0 + tid / a.K;
            if (r < Ks) {
                sv[d * Ks + r] = v;
                so[d * Ks + r] = (uint8_t)k;
            }
            positive |= v > 0.f;
        }
    }
    if (positive) atomicOr(&L.flags, kPositive);
    __syncthreads();

    // Phase 2, else phase 3
    bool done = false;
    if (a.Q > 1 && !(L.flags & kPositive)) done = level_pass(L, sv, a.D, Ds, Ks, a.Q, tid);
    if (!done) {
        if (tid < 64) sequential_pass<kSlots, kNodeSlots>(L, sv, a.D, Ks, a.K, a.Q, tid);
        __syncthreads();
    }
    if (done && tid == 0) {   // the root (the level pass writes nodes 1..Q-1)
        L.node_parent[0] = -1;
        L.node_depth[0] = 0;
        L.node_rank[0] = -1;
        L.node_score[0] = 0.f;
    }
    __syncthreads();

    // outputs
    const int64_t base = (int64_t)b * a.Q;
    for (int i = tid; i < a.Q; i += kThreads) {
        const int p = L.node_parent[i];
        const int d = L.node_depth[i];
        const int r = L.node_rank[i];
        a.parent[base + i] = p;
        if (a.depth) a.depth[base + i] = d;
        if (a.rank) a.rank[base + i] = r;
        if (a.score) a.score[base + i] = L.node_score[i];
        if (a.token) {
            const bool chosen = d >= 1 && d <= Ds && r >= 0 && r < Ks;
            const int k = chosen ? so[(d - 1) * Ks + r] : -1;
            a.token[base + i] = !chosen ? -1 : (a.tokens ? a.tokens[((int64_t)b * a.D + d - 1) * a.K + k] : k);
        }
    }
}

template <int kSlots, int kNodeSlots>
hipError_t launch_instance(const TreeArgs& a, size_t lds, hipStream_t stream) {
    const void* fn = reinterpret_cast<const void*>(&tree_build_kernel<kSlots, kNodeSlots>);
    if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((tree_build_kernel<kSlots, kNodeSlots>), dim3((unsigned)a.B), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

// Dynamic LDS: the rank-ordered values (float) and choice indices (byte) of the
// first min(D, Q) depths and min(K, Q) ranks.
size_t tree_build_lds_bytes(int D, int K, int Q) {
    const size_t n = (size_t)min(D, Q) * (size_t)min(K, Q);
    return n * sizeof(float) + (n + 3) / 4 * 4;
}

hipError_t launch_tree_build(const TreeArgs& a, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    const size_t lds = tree_build_lds_bytes(a.D, a.K, a.Q);
    if (a.Q <= 64) return launch_instance<2, 1>(a, lds, stream);
    if (a.Q <= 128) return launch_instance<3, 2>(a, lds, stream);
    return launch_instance<kMaxSlots, kMaxQ / 64>(a, lds, stream);
}

}  // namespace ddtv
