// Greedy tree acceptance after the verify step, and the KV compaction that
// follows it (the tree-accept step of "The Moment of Truth: Validating a Custom
// CUDA Attention Kernel for Speculative Decoding", section "Context: Building a
// Native DDTree Inference Engine"; the compaction that drops unaccepted branches,
// "The Architecture of an Inference Engine: Designing the Model Structure for
// DDTree Speculative Decoding", section "Input Knowledge Required").
//
// Definition (the reading the library documents):
//  * the target's prediction after node i is the argmax of its float32 logits
//    (the lowest index among equal maxima);
//  * from the root, repeatedly move to the lowest-index child whose draft token
//    equals the current node's prediction; stop where there is none;
//  * k = accepted draft tokens; output tokens = their draft tokens, then the last
//    accepted node's prediction;
//  * compaction: cache row prefix + path[j] moves to prefix + j, j = 1..k.
//
// Launches on the caller's stream (two when the caches are given: the walk and the
// compaction then run as one, accept_walk_compact_kernel below):
//  * accept_argmax_kernel: one 256-thread workgroup per (batch row, node); each
//    thread keeps the first maximum of its strided share of the V logits
//    (coalesced, 16-byte loads four at a time when V is a multiple of 4), then a
//    workgroup reduction keeps the larger value, and on equal values the lower
//    index.  This part reads B*Q*V floats and is HBM-bound for a real vocabulary.
//  * accept_walk_kernel: one wave per batch row; at each step all lanes test the
//    candidate children in parallel (64 node indices per ballot) and the lowest
//    matching index is taken.
//  * accept_compact_kernel: one workgroup per (batch row, 256-byte column window of
//    the latent or rope rows); it reads the k accepted rows' window into LDS, then
//    writes them to their new rows.  Windows are disjoint, and every read of a
//    window precedes every write to it, so the in-place move is safe even though
//    a destination row can be another accepted node's source row.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

constexpr int kArgmaxThreads = 256;
constexpr int kWindowChunks = 16;   // 16-byte chunks per compaction window (256 B)

__global__ __launch_bounds__(kArgmaxThreads) void accept_argmax_kernel(const float* __restrict__ logits, int V,
                                                                       int32_t* __restrict__ pred) {
    __shared__ float sv[kArgmaxThreads];
    __shared__ int si[kArgmaxThreads];
    const int64_t row = blockIdx.x;   // b * Q + node
    const float* x = logits + row * V;
    const int t = threadIdx.x;
    float best = -INFINITY;
    int bi = -1;
    auto take = [&](float y, int v) {   // first maximum in the order visited
        if (bi < 0 || y > best) {
            best = y;
            bi = v;
        }
    };
    if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) {
        // 16-byte loads (rows start 16-byte aligned), four in flight per thread; a thread visits its chunks in
        // increasing order and each chunk's elements in order
        const float4* x4 = reinterpret_cast<const float4*>(x);
        const int n4 = V >> 2;
        int c = t;
        for (; c + 3 * kArgmaxThreads < n4; c += 4 * kArgmaxThreads) {
            float4 q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = x4[c + u * kArgmaxThreads];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = 4 * (c + u * kArgmaxThreads);
                take(q[u].x, v);
                take(q[u].y, v + 1);
                take(q[u].z, v + 2);
                take(q[u].w, v + 3);
            }
        }
        for (; c < n4; c += kArgmaxThreads) {
            const float4 q = x4[c];
            take(q.x, 4 * c);
            take(q.y, 4 * c + 1);
            take(q.z, 4 * c + 2);
            take(q.w, 4 * c + 3);
        }
    } else {
        for (int v = t; v < V; v += kArgmaxThreads) take(x[v], v);
    }
    sv[t] = best;
    si[t] = bi;
    __syncthreads();
    for (int s = kArgmaxThreads / 2; s > 0; s >>= 1) {
        if (t < s) {
            const float ov = sv[t + s];
            const int oi = si[t + s];
            if (oi >= 0 && (si[t] < 0 || ov > sv[t] || (ov == sv[t] && oi < si[t]))) {
                sv[t] = ov;
                si[t] = oi;
            }
        }
        __syncthreads();
    }
    if (t == 0) pred[row] = si[0];
}

__global__ __launch_bounds__(64) void accept_walk_kernel(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ token,
                                                         const int32_t* __restrict__ pred, int Q,
                                                         int32_t* __restrict__ path, int32_t* __restrict__ out_tokens,
                                                         int32_t* __restrict__ accept_len) {
    __shared__ int32_t sp[kMaxQ], st[kMaxQ], sq[kMaxQ];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)b * Q;
    for (int i = lane; i < Q; i += 64) {
        sp[i] = parent[base + i];
        st[i] = token[base + i];
        sq[i] = pred[base + i];
        path[base + i] = -1;
        out_tokens[base + i] = -1;
    }
    __syncthreads();
    int cur = 0, k = 0;
    for (;;) {
        const int want = sq[cur];
        int next = -1;
        for (int c0 = cur + 1; c0 < Q && next < 0; c0 += 64) {   // children have larger indices
            const int c = c0 + lane;
            const uint64_t hit = __ballot(c < Q && sp[c] == cur && st[c] == want);
            if (hit) next = c0 + __ffsll((unsigned long long)hit) - 1;
        }
        if (next < 0) break;
        ++k;
        if (lane == 0) {
            path[base + k] = next;
            out_tokens[base + k - 1] = st[next];
        }
        cur = next;
    }
    if (lane == 0) {
        path[base] = 0;
        out_tokens[base + k] = sq[cur];
        accept_len[b] = k;
    }
}

// One window of 16-byte chunks [w * 16, w * 16 + 16) of the concatenated chunk
// space: latent chunks first (lat_chunks per row), then rope chunks.
__global__ __launch_bounds__(256) void accept_compact_kernel(char* ckv, char* k_rope, int lat_chunks,
                                                             int rope_chunks, const ddtv_row* __restrict__ rows,
                                                             const int32_t* __restrict__ path,
                                                             const int32_t* __restrict__ accept_len, int Q) {
    __shared__ uint4 buf[kMaxQ - 1][kWindowChunks];   // 255 rows x 256 B
    const int b = blockIdx.y;
    const int w = blockIdx.x;
    const int k = accept_len[b];
    if (k <= 0) return;
    const int c_lo = w * kWindowChunks;
    const bool lat = c_lo < lat_chunks;
    char* base = lat ? ckv : k_rope;
    const int row_chunks = lat ? lat_chunks : rope_chunks;
    const int c0 = lat ? c_lo : c_lo - lat_chunks;
    const int nc = min(kWindowChunks, row_chunks - c0);
    const ddtv_row rd = rows[b];
    const int64_t first = rd.kv_off + rd.prefix;   // cache row of tree node 0
    const int32_t* pb = path + (int64_t)b * Q;
    uint4* arr = reinterpret_cast<uint4*>(base);
    for (int e = threadIdx.x; e < k * kWindowChunks; e += 256) {
        const int j = e / kWindowChunks, c = e % kWindowChunks;
        if (c < nc) buf[j][c] = arr[(first + pb[j + 1]) * row_chunks + c0 + c];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < k * kWindowChunks; e += 256) {
        const int j = e / kWindowChunks, c = e % kWindowChunks;
        if (c < nc) arr[(first + j + 1) * row_chunks + c0 + c] = buf[j][c];
    }
}

// The walk and the compaction in one launch (when the caches are given): every
// workgroup of batch row b repeats the walk on its first wave -- a few ballots
// over at most 256 nodes -- into LDS, the one with window 0 writes the walk's
// outputs, and each then moves its window of the accepted rows as
// accept_compact_kernel does.  One launch fewer per step than walk + compact.
__global__ __launch_bounds__(256) void accept_walk_compact_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ token, const int32_t* __restrict__ pred, int Q,
    int32_t* __restrict__ path, int32_t* __restrict__ out_tokens, int32_t* __restrict__ accept_len, char* ckv,
    char* k_rope, int lat_chunks, int rope_chunks, const ddtv_row* __restrict__ rows) {
    __shared__ int32_t sp[kMaxQ], st[kMaxQ], sq[kMaxQ], spath[kMaxQ];
    __shared__ int32_t sk;
    __shared__ uint4 buf[kMaxQ - 1][kWindowChunks];   // 255 rows x 256 B
    const int b = blockIdx.y;
    const int w = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t base = (int64_t)b * Q;
    for (int i = t; i < Q; i += 256) {
        sp[i] = parent[base + i];
        st[i] = token[base + i];
        sq[i] = pred[base + i];
    }
    __syncthreads();
    if (t < 64) {   // the walk, on the first wave (as accept_walk_kernel)
        const int lane = t;
        int cur = 0, k = 0;
        for (;;) {
            const int want = sq[cur];
            int next = -1;
            for (int c0 = cur + 1; c0 < Q && next < 0; c0 += 64) {   // children have larger indices
                const int c = c0 + lane;
                const uint64_t hit = __ballot(c < Q && sp[c] == cur && st[c] == want);
                if (hit) next = c0 + __ffsll((unsigned long long)hit) - 1;
            }
            if (next < 0) break;
            ++k;
            if (lane == 0) spath[k] = next;
            cur = next;
        }
        if (lane == 0) {
            spath[0] = 0;
            sk = k;
            if (w == 0) {
                out_tokens[base + k] = sq[cur];
                accept_len[b] = k;
            }
        }
    }
    __syncthreads();
    const int k = sk;
    if (w == 0) {
        for (int i = t; i < Q; i += 256) {
            path[base + i] = i <= k ? spath[i] : -1;
            if (i < k) out_tokens[base + i] = st[spath[i + 1]];
            else if (i > k) out_tokens[base + i] = -1;
        }
    }
    if (k <= 0) return;
    const int c_lo = w * kWindowChunks;
    const bool lat = c_lo < lat_chunks;
    char* cbase = lat ? ckv : k_rope;
    const int row_chunks = lat ? lat_chunks : rope_chunks;
    const int c0 = lat ? c_lo : c_lo - lat_chunks;
    const int nc = min(kWindowChunks, row_chunks - c0);
    const ddtv_row rd = rows[b];
    const int64_t first = rd.kv_off + rd.prefix;   // cache row of tree node 0
    uint4* arr = reinterpret_cast<uint4*>(cbase);
    for (int e = t; e < k * kWindowChunks; e += 256) {
        const int j = e / kWindowChunks, c = e % kWindowChunks;
        if (c < nc) buf[j][c] = arr[(first + spath[j + 1]) * row_chunks + c0 + c];
    }
    __syncthreads();
    for (int e = t; e < k * kWindowChunks; e += 256) {
        const int j = e / kWindowChunks, c = e % kWindowChunks;
        if (c < nc) arr[(first + j + 1) * row_chunks + c0 + c] = buf[j][c];
    }
}

}  // namespace

hipError_t launch_tree_accept(const AcceptArgs& a, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(accept_argmax_kernel, dim3((unsigned)((int64_t)a.B * a.Q)), dim3(kArgmaxThreads), 0, stream,
                       a.logits, a.V, a.pred);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int lat_chunks = kDLat * a.kv_elem / 16, rope_chunks = kDRope * a.kv_elem / 16;
    const int windows = (lat_chunks + kWindowChunks - 1) / kWindowChunks +
                        (rope_chunks + kWindowChunks - 1) / kWindowChunks;
    if (a.ckv) {
        hipLaunchKernelGGL(accept_walk_compact_kernel, dim3((unsigned)windows, (unsigned)a.B), dim3(256), 0, stream,
                           a.parent, a.token, a.pred, a.Q, a.path, a.out_tokens, a.accept_len,
                           static_cast<char*>(a.ckv), static_cast<char*>(a.k_rope), lat_chunks, rope_chunks, a.rows);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(accept_walk_kernel, dim3((unsigned)a.B), dim3(64), 0, stream, a.parent, a.token, a.pred, a.Q,
                       a.path, a.out_tokens, a.accept_len);
    e = hipGetLastError();
    if (e != hipSuccess || !a.ckv) return e;
    hipLaunchKernelGGL(accept_compact_kernel, dim3((unsigned)windows, (unsigned)a.B), dim3(256), 0, stream,
                       static_cast<char*>(a.ckv), static_cast<char*>(a.k_rope), lat_chunks, rope_chunks, a.rows,
                       a.path, a.accept_len, a.Q);
    return hipGetLastError();
}

}  // namespace ddtv
