// External-prefix mode of the verify step: the caller brings the attention of
// every query row over the shared prefix (from any prefix kernel), this library
// attends only the tree rows and merges the two by log-sum-exp -- the production
// split the pages plan, a prefix kernel for the long prefix and the masked kernel
// for the tree tail ("The Verify-Attn Kernel: A Single File Write ...", section
// "Design Decisions and Trade-Offs").
//
// Two routes.  The default one, tail_sparse_kernel, visits only what each node
// sees: one workgroup per tree node reads the node's mask, walks its ancestors-
// or-self (depth + 1 cache rows), runs the online softmax over them for every
// head and merges the prefix result in the same pass.  The dense route, taken
// when the caller forces a path or a split length, runs the ordinary attention
// kernels over a tree-rows-only view with two small kernels around them:
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

// ---- tree-sparse route ------------------------------------------------------
// A workgroup of 8 waves takes one tree node and 16 of its heads, a wave 2 of
// them; lane l holds latent dims 8l .. 8l+7 and rope dim l of the query and of
// each visited cache row, so a cache row is read once per wave for 2 heads and a
// score is a 9-term lane product plus a wave sum.  The next row's loads are in
// flight while the current one is scored.
constexpr int kSparseHeads = 2;
constexpr int kSparseWaves = 8;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <int KV>
__device__ __forceinline__ void load_cache_row(const TailSparseArgs& a, int64_t row, int lane, float v[8], float& r) {
    if (KV == DDTV_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.ckv) + row * kDLat) + 2 * lane;
        const float4 x = p[0], y = p[1];
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
        r = static_cast<const float*>(a.k_rope)[row * kDRope + lane];
    } else if (KV == DDTV_BF16) {
        const uint4 u = reinterpret_cast<const uint4*>(a.ckv)[row * (kDLat / 8) + lane];
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
        r = bf16_lo(static_cast<const uint16_t*>(a.k_rope)[row * kDRope + lane]);
    } else {
        const uint2 u = reinterpret_cast<const uint2*>(a.ckv)[row * (kDLat / 8) + lane];
        const float4 x = fp8x4(u.x), y = fp8x4(u.y);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
        r = fp8x4(static_cast<const uint8_t*>(a.k_rope)[row * kDRope + lane]).x;
    }
}

template <int KV>
__global__ __launch_bounds__(kSparseWaves * 64) void tail_sparse_kernel(TailSparseArgs a) {
    // workgroup = (tree node, group of kSparseWaves * kSparseHeads heads)
    const int n_hg = (a.H + kSparseWaves * kSparseHeads - 1) / (kSparseWaves * kSparseHeads);
    const int64_t node = blockIdx.x / n_hg;
    const int hg = (int)(blockIdx.x % n_hg);
    const int b = (int)(node / a.Q);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const ddtv_row rd = a.rows[b];
    const int64_t base = rd.kv_off + rd.prefix;          // cache row of tree node 0
    const uint32_t* mw = a.bits + node * a.W;

    {
        const int h0 = (hg * kSparseWaves + wave) * kSparseHeads;
        if (h0 >= a.H) return;
        float qa[kSparseHeads][8], qr[kSparseHeads], m[kSparseHeads], l[kSparseHeads], acc[kSparseHeads][8];
#pragma unroll
        for (int k = 0; k < kSparseHeads; ++k) {
            const int h = min(h0 + k, a.H - 1);           // surplus heads repeat the last one, unwritten
            const int64_t qrow = node * a.H + h;
            const float4* p = reinterpret_cast<const float4*>(a.q_abs + qrow * kDLat) + 2 * lane;
            const float4 x = p[0], y = p[1];
            qa[k][0] = x.x * a.scale_log2; qa[k][1] = x.y * a.scale_log2;
            qa[k][2] = x.z * a.scale_log2; qa[k][3] = x.w * a.scale_log2;
            qa[k][4] = y.x * a.scale_log2; qa[k][5] = y.y * a.scale_log2;
            qa[k][6] = y.z * a.scale_log2; qa[k][7] = y.w * a.scale_log2;
            qr[k] = a.q_rope[qrow * kDRope + lane] * a.scale_log2;
            m[k] = -INFINITY;
            l[k] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
        }
        // the ancestors-or-self in index order (set bits of the mask), the next
        // row's loads in flight while the current one is scored
        int w = 0;
        uint32_t word = mw[0];
        auto next_anc = [&]() -> int {   // -1 once the mask is exhausted
            while (word == 0u) {
                if (++w >= a.W) return -1;
                word = mw[w];
            }
            const int anc = 32 * w + __builtin_ctz(word);
            word &= word - 1;
            return anc;
        };
        int cur = next_anc();
        float v[8], r = 0.f;
        if (cur >= 0) load_cache_row<KV>(a, base + cur, lane, v, r);
        while (cur >= 0) {
            const int nxt = next_anc();
            float vn[8], rn = 0.f;
            if (nxt >= 0) load_cache_row<KV>(a, base + nxt, lane, vn, rn);
#pragma unroll
            for (int k = 0; k < kSparseHeads; ++k) {
                float s = qr[k] * r;
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(qa[k][e], v[e], s);
                s = wave_sum(s);                       // score in log2 units
                const float mn = fmaxf(m[k], s);
                const float alpha = exp2f(m[k] - mn);  // 0 on the first row (m = -inf)
                const float pr = exp2f(s - mn);
                l[k] = l[k] * alpha + pr;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[k][e] = fmaf(pr, v[e], acc[k][e] * alpha);
                m[k] = mn;
            }
            cur = nxt;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = vn[e];
            r = rn;
        }
        // merge with the prefix result: weights e^(lse - M) of both sides
#pragma unroll
        for (int k = 0; k < kSparseHeads; ++k) {
            const int h = h0 + k;
            if (h >= a.H) break;
            const int64_t qrow = node * a.H + h;
            const float lt = l[k] > 0.f ? (m[k] + log2f(l[k])) * 0.69314718055994531f : -INFINITY;
            const float lp = a.prefix_lse[qrow];
            const float M = fmaxf(lt, lp);
            float4* o = reinterpret_cast<float4*>(a.out + qrow * kDLat) + 2 * lane;
            if (M == -INFINITY) {   // neither side sees anything
                o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
                o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a.lse && lane == 0) a.lse[qrow] = -INFINITY;
                continue;
            }
            const float wt = lt == -INFINITY ? 0.f : expf(lt - M);
            const float wp = lp == -INFINITY ? 0.f : expf(lp - M);
            const float inv = 1.f / (wt + wp);
            const float ft = lt == -INFINITY ? 0.f : wt * inv / l[k];   // tail weight per unnormalised sum
            const float fp = wp * inv;
            const float4* po = reinterpret_cast<const float4*>(a.prefix_out + qrow * kDLat) + 2 * lane;
            float4 p0 = make_float4(0.f, 0.f, 0.f, 0.f), p1 = p0;
            if (wp > 0.f) { p0 = po[0]; p1 = po[1]; }
            o[0] = make_float4(ft * acc[k][0] + fp * p0.x, ft * acc[k][1] + fp * p0.y,
                               ft * acc[k][2] + fp * p0.z, ft * acc[k][3] + fp * p0.w);
            o[1] = make_float4(ft * acc[k][4] + fp * p1.x, ft * acc[k][5] + fp * p1.y,
                               ft * acc[k][6] + fp * p1.z, ft * acc[k][7] + fp * p1.w);
            if (a.lse && lane == 0) a.lse[qrow] = M + logf(wt + wp);
        }
    }
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

namespace ddtv {

hipError_t launch_tail_sparse(const TailSparseArgs& a, int kv_dtype, hipStream_t stream) {
    (void)hipGetLastError();
    const int n_hg = (a.H + kSparseWaves * kSparseHeads - 1) / (kSparseWaves * kSparseHeads);
    const dim3 grid((unsigned)((int64_t)a.B * a.Q * n_hg));
    if (kv_dtype == DDTV_BF16)
        hipLaunchKernelGGL(tail_sparse_kernel<DDTV_BF16>, grid, dim3(kSparseWaves * 64), 0, stream, a);
    else if (kv_dtype == DDTV_FP8_E4M3)
        hipLaunchKernelGGL(tail_sparse_kernel<DDTV_FP8_E4M3>, grid, dim3(kSparseWaves * 64), 0, stream, a);
    else
        hipLaunchKernelGGL(tail_sparse_kernel<DDTV_F32>, grid, dim3(kSparseWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ddtv
