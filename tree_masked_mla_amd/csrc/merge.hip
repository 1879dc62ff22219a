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
// attention kernel and are skipped.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
    const int64_t gr = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);   // b * R + row
    const int64_t total = (int64_t)a.B * a.R;
    if (gr >= total) return;
    const int b = (int)(gr / a.R);
    const int row = (int)(gr - (int64_t)b * a.R);
    const int kv_len = a.rows[b].kv_len;
    const int n_b = (kv_len + a.split_len - 1) / a.split_len;
    if (n_b <= 1) return;
    const int c = threadIdx.x & 127;
    const int64_t pbase = (int64_t)b * a.n_split * a.R + row;   // split s at pbase + s * R

    float M = -INFINITY;
    for (int s = 0; s < n_b; ++s) M = fmaxf(M, a.part_ml[pbase + (int64_t)s * a.R].x);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
        for (int s = 0; s < n_b; ++s) {
            const float2 ml = a.part_ml[pbase + (int64_t)s * a.R];
            if (ml.x == -INFINITY) continue;
            const float wgt = exp2f(ml.x - M);
            L += wgt * ml.y;
            const float4 v = reinterpret_cast<const float4*>(a.part_o)[(pbase + (int64_t)s * a.R) * 128 + c];
            o.x = fmaf(wgt, v.x, o.x);
            o.y = fmaf(wgt, v.y, o.y);
            o.z = fmaf(wgt, v.z, o.z);
            o.w = fmaf(wgt, v.w, o.w);
        }
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
