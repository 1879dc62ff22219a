// S7 -- log-sum-exp merge of split-KV partials.
//
// A long cache is cut into splits that are attended independently; each split
// leaves an unnormalised partial (running max m, running sum l, weighted latent
// sum o).  They combine exactly: with M = max m_s, L = sum exp2(m_s - M) l_s,
// out = sum exp2(m_s - M) o_s / L and lse = (M + log2 L) ln 2.  This is the
// prefix/tail log-sum-exp combination the pages plan for long contexts ("The
// Verify-Attn Kernel: A Single File Write ...", section "Design Decisions and
// Trade-Offs"), applied to any number of splits.
//
// 128 threads per query row (one float4 of the 512-d output each), 2 rows per
// workgroup.  Rows whose batch row needed a single split were finished by the
// attention kernel and are skipped (except in row-half mode, where every split
// leaves two partials).  The splits are read in batches of kBatch
// independent loads and folded in with an online rescale (the running maximum
// moves batch by batch), so up to kBatch splits cost one memory round trip.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

constexpr int kBatch = 16;

__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
    const int64_t gr = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);   // b * R + row
    const int64_t total = (int64_t)a.B * a.R;
    if (gr >= total) return;
    const int b = (int)(gr / a.R);
    const int row = (int)(gr - (int64_t)b * a.R);
    const int kv_len = a.rows[b].kv_len;
    const int hm = a.halves ? 2 : 1;                   // partials per split
    const int n_b = hm * ((kv_len + a.split_len - 1) / a.split_len);
    if (n_b <= 1) return;
    const int c = threadIdx.x & 127;
    const int64_t pbase = (int64_t)b * hm * a.n_split * a.R + row;   // partial s at pbase + s * R
    const float4* po = reinterpret_cast<const float4*>(a.part_o);

    float M = -INFINITY, L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < n_b; s0 += kBatch) {
        float2 ml[kBatch];
        float4 v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const bool in = s0 + k < n_b;
            const int64_t p = pbase + (int64_t)(in ? s0 + k : 0) * a.R;
            ml[k] = in ? a.part_ml[p] : make_float2(-INFINITY, 0.f);
            v[k] = in ? po[p * 128 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) Mb = fmaxf(Mb, ml[k].x);
        if (Mb == -INFINITY) continue;          // nothing visible so far
        // an empty split (m = -inf) has l = 0 and o = 0: weight 0
        const float r = (M == -INFINITY) ? 0.f : exp2f(M - Mb);
        L *= r;
        o.x *= r;
        o.y *= r;
        o.z *= r;
        o.w *= r;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const float wgt = (ml[k].x == -INFINITY) ? 0.f : exp2f(ml[k].x - Mb);
            L = fmaf(wgt, ml[k].y, L);
            o.x = fmaf(wgt, v[k].x, o.x);
            o.y = fmaf(wgt, v[k].y, o.y);
            o.z = fmaf(wgt, v[k].z, o.z);
            o.w = fmaf(wgt, v[k].w, o.w);
        }
        M = Mb;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    reinterpret_cast<float4*>(a.out)[gr * 128 + c] = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (a.lse && c == 0) a.lse[gr] = L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    const int64_t rows = (int64_t)a.B * a.R;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ddtv
