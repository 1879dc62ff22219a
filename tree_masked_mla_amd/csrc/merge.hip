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
// 128 threads per query row and partial group (one float4 of the 512-d output
// each).  Rows whose batch row needed a single split were finished by the
// attention kernel and are skipped.  The splits are read in batches of kBatch independent
// loads and folded in with an online rescale (the running maximum moves batch by
// batch), so up to kBatch splits cost one memory round trip.  With many partials
// and few rows (decode shapes) G groups of 128 threads share a row, each taking
// a contiguous share of its partials; the G (m, l, o) results are then combined
// in LDS in group order, the same exact combination one level up.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

constexpr int kBatch = 16;

// G partial groups per row: 2 rows per 256-thread workgroup for G = 1, else one
// row per workgroup of 128 G threads.
template <int G>
__global__ __launch_bounds__(G == 1 ? 256 : 128 * G) void merge_kernel(AttnArgs a) {
    constexpr int kRowsPerWG = G == 1 ? 2 : 1;
    const int grp = G == 1 ? 0 : (int)(threadIdx.x >> 7);
    const int64_t gr = (int64_t)blockIdx.x * kRowsPerWG + (G == 1 ? (threadIdx.x >> 7) : 0);   // b * R + row
    const int64_t total = (int64_t)a.B * a.R;
    if (gr >= total) return;   // (G > 1: uniform over the workgroup)
    const int b = (int)(gr / a.R);
    const int row = (int)(gr - (int64_t)b * a.R);
    const int kv_len = a.rows[b].kv_len;
    const int n_b = splits_of(kv_len, a.split_len, a.absorb);   // this batch row's partials
    if (n_b <= 1) return;
    const int c = threadIdx.x & 127;
    const int64_t pbase = (int64_t)b * a.n_split * a.R + row;   // partial s at pbase + s * R
    const float4* po = reinterpret_cast<const float4*>(a.part_o);
    // this group's partials: [s_lo, s_hi)
    const int per = (n_b + G - 1) / G;
    const int s_lo = min(n_b, grp * per), s_hi = min(n_b, s_lo + per);

    float M = -INFINITY, L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = s_lo; s0 < s_hi; s0 += kBatch) {
        float2 ml[kBatch];
        float4 v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const bool in = s0 + k < s_hi;
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
    if constexpr (G > 1) {
        __shared__ float4 so[G][128];
        __shared__ float2 sml[G];
        so[grp][c] = o;
        if (c == 0) sml[grp] = make_float2(M, L);
        __syncthreads();
        if (grp != 0) return;
        float Mt = -INFINITY;
#pragma unroll
        for (int k = 0; k < G; ++k) Mt = fmaxf(Mt, sml[k].x);
        M = Mt;
        L = 0.f;
        o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (Mt != -INFINITY) {
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const float2 mk = sml[k];
                const float wgt = (mk.x == -INFINITY) ? 0.f : exp2f(mk.x - Mt);
                const float4 ok = so[k][c];
                L = fmaf(wgt, mk.y, L);
                o.x = fmaf(wgt, ok.x, o.x);
                o.y = fmaf(wgt, ok.y, o.y);
                o.z = fmaf(wgt, ok.z, o.z);
                o.w = fmaf(wgt, ok.w, o.w);
            }
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
    // Partial groups per row: enough that each group's share is one batch of
    // loads, used only while the rows alone leave most CUs without a workgroup.
    const int n_part = a.n_split;
    int G = 1;
    while (G < 8 && n_part > G * kBatch && rows * G < 2048) G *= 2;
    switch (G) {
    case 1: hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(merge_kernel<2>, dim3((unsigned)rows), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)rows), dim3(512), 0, stream, a); break;
    default: hipLaunchKernelGGL(merge_kernel<8>, dim3((unsigned)rows), dim3(1024), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace ddtv
