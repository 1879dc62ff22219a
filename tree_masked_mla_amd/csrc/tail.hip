// External-prefix mode of the verify step: the caller brings the attention of
// every query row over the shared prefix (from any prefix kernel), this library
// attends only the tree rows and merges the two by log-sum-exp -- the production
// split the pages plan, a prefix kernel for the long prefix and the masked kernel
// for the tree tail ("The Verify-Attn Kernel: A Single File Write ...", section
// "Design Decisions and Trade-Offs").
//
// Two small kernels around the ordinary attention launch:
//  * tail_rows_kernel rewrites the row table so each batch row's tree rows look
//    like a row without prefix (the attention kernels then touch Q cache rows
//    per batch row);
//  * tail_merge_kernel folds the prefix result into out, in place (each thread
//    reads and writes only its own float4), and writes the merged lse: with
//    M = max(lse_t, lse_p), out = (e^(lse_t - M) o_t + e^(lse_p - M) o_p) /
//    (e^(lse_t - M) + e^(lse_p - M)) and lse = M + ln(the denominator); an empty
//    side (lse = -inf) has weight 0.  128 threads per query row, one float4 each.
#include "tail.hpp"

namespace ddtv {

namespace {

__global__ __launch_bounds__(64) void tail_rows_kernel(const ddtv_row* __restrict__ rows,
                                                       ddtv_row* __restrict__ tail_rows, int B, int Q) {
    const int b = blockIdx.x * 64 + threadIdx.x;
    if (b >= B) return;
    const ddtv_row r = rows[b];
    ddtv_row t;
    t.kv_off = r.kv_off + r.prefix;
    t.prefix = 0;
    t.kv_len = Q;
    tail_rows[b] = t;
}

__global__ __launch_bounds__(256) void tail_merge_kernel(float* __restrict__ out, const float* __restrict__ lse_tail,
                                                         float* __restrict__ lse, const float* __restrict__ prefix_out,
                                                         const float* __restrict__ prefix_lse, int64_t n) {
    const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
    if (row >= n) return;
    const int c = threadIdx.x & 127;
    const float lt = lse_tail[row], lp = prefix_lse[row];
    const float M = fmaxf(lt, lp);
    float4* o = reinterpret_cast<float4*>(out) + row * 128 + c;   // each thread owns its float4
    if (M == -INFINITY) {   // neither side sees anything
        *o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lse && c == 0) lse[row] = -INFINITY;
        return;
    }
    const float wt = lt == -INFINITY ? 0.f : expf(lt - M);
    const float wp = lp == -INFINITY ? 0.f : expf(lp - M);
    const float inv = 1.f / (wt + wp);
    const float4 a = *o;
    const float4 p = reinterpret_cast<const float4*>(prefix_out)[row * 128 + c];
    *o = make_float4((wt * a.x + wp * p.x) * inv, (wt * a.y + wp * p.y) * inv, (wt * a.z + wp * p.z) * inv,
                     (wt * a.w + wp * p.w) * inv);
    if (lse && c == 0) lse[row] = M + logf(wt + wp);
}

}  // namespace

hipError_t launch_tail_rows(const ddtv_row* rows, ddtv_row* tail_rows, int B, int Q, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(tail_rows_kernel, dim3((unsigned)((B + 63) / 64)), dim3(64), 0, stream, rows, tail_rows, B, Q);
    return hipGetLastError();
}

hipError_t launch_tail_merge(float* out, const float* lse_tail, float* lse, const float* prefix_out,
                             const float* prefix_lse, int64_t n, hipStream_t stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(tail_merge_kernel, dim3((unsigned)((n + 1) / 2)), dim3(256), 0, stream, out, lse_tail, lse,
                       prefix_out, prefix_lse, n);
    return hipGetLastError();
}

}  // namespace ddtv
