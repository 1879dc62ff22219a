// S1 -- visibility builder: parent arrays -> packed ancestor-or-self bits.
//
// A node sees the shared prefix, its tree ancestors and itself ("The Verify-Attn
// Kernel: A Single File Write ...", section "The Design Journey: From Concept to
// CUDA").  The prefix is implicit; only tree columns get bits.
//
// One workgroup per batch row.  The tree (Q <= 256 nodes) is staged in LDS and the
// ancestor sets are built by pointer jumping: after round r every node holds the
// nodes within distance < 2^r up its chain, and ceil(log2 Q) rounds cover any depth.
// Malformed nodes get no jump pointer, so a chain stops at them (their own bit
// included) and they see only themselves.  The lowest malformed node of the row is
// written to status[b] (-1 if none) without atomics across workgroups.
#include "ddtv_internal.hpp"

namespace ddtv {

__global__ __launch_bounds__(256) void visibility_kernel(const int32_t* __restrict__ parent, int b0,
                                                         int Q, int W, uint32_t* __restrict__ bits,
                                                         ddtv_row* __restrict__ rows,
                                                         int32_t* __restrict__ status,
                                                         int32_t* __restrict__ order, VisChunk chunk) {
    __shared__ uint32_t sbits[2][kMaxQ][kMaxW];
    __shared__ int32_t sjump[2][kMaxQ];
    __shared__ int32_t sbad;

    const int lb = blockIdx.x;          // index inside this launch's chunk
    const int b = b0 + lb;
    const int i = threadIdx.x;          // node
    if (i == 0) sbad = Q;
    __syncthreads();

    if (i < Q) {
        const int32_t p = parent[(int64_t)b * Q + i];
        const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
        if (!ok) atomicMin(&sbad, i);
        sjump[0][i] = (ok && i != 0) ? p : -1;
#pragma unroll
        for (int w = 0; w < kMaxW; ++w) sbits[0][i][w] = (w == (i >> 5)) ? (1u << (i & 31)) : 0u;
    }
    __syncthreads();

    int cur = 0;
    for (int span = 1; span < Q; span <<= 1) {
        if (i < Q) {
            const int j = sjump[cur][i];
            uint32_t nb[kMaxW];
#pragma unroll
            for (int w = 0; w < kMaxW; ++w) nb[w] = sbits[cur][i][w];
            int nj = -1;
            if (j >= 0) {
#pragma unroll
                for (int w = 0; w < kMaxW; ++w) nb[w] |= sbits[cur][j][w];
                nj = sjump[cur][j];
            }
#pragma unroll
            for (int w = 0; w < kMaxW; ++w) sbits[cur ^ 1][i][w] = nb[w];
            sjump[cur ^ 1][i] = nj;
        }
        __syncthreads();
        cur ^= 1;
    }

    if (i < Q) {
        uint32_t* dst = bits + ((int64_t)b * Q + i) * W;
        for (int w = 0; w < W; ++w) dst[w] = sbits[cur][i][w];
    }
    if (i == 0) {
        ddtv_row r;
        r.kv_off = chunk.kv_off[lb];
        r.prefix = chunk.prefix[lb];
        r.kv_len = chunk.prefix[lb] + Q;
        rows[b] = r;
        status[b] = (sbad < Q) ? sbad : -1;
        order[b] = chunk.order[lb];
    }
}

hipError_t launch_visibility(const int32_t* parent, int b0, int nb, int Q, int W, uint32_t* bits,
                             ddtv_row* rows, int32_t* status, int32_t* order, const VisChunk& chunk,
                             hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(visibility_kernel, dim3(nb), dim3(256), 0, stream, parent, b0, Q, W, bits,
                       rows, status, order, chunk);
    return hipGetLastError();
}

}  // namespace ddtv
