// S2..S6 on the vector ALUs -- the path for batch rows with fewer than 16 query rows (H * q_len < 16).
//
// Score = scale * (absorbed query . latent + rope query . rope key); softmax over
// the node's visible positions; output = weighted sum of latents ("The Verify-Attn
// Kernel: A Single File Write ...", section "The Design Journey: From Concept to
// CUDA").  Unlike the pages' one-block-per-(b,h,q) design with every score kept in
// shared memory, this kernel streams the cache in 32-row tiles with an online
// (running max / running sum) softmax, so any prefix length works, and every tile
// is shared by the 16 query rows of the workgroup (all heads share one latent
// cache).
//
// Workgroup: 256 threads = 4 waves; 16 query rows (4 per wave) of one batch row,
// one KV split.  Within a wave, lane l scores cache row (l & 31) of the tile over
// half (l >> 5) of the 576 dims; the halves are summed with one cross-half swap.
// For the weighted sum every lane owns 8 of the 512 latent dims and reads the
// probabilities of the 32 tile rows with readlane (SGPR operands).
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

constexpr int kRows = kValuRows;            // 16
constexpr int kChunks = kDQK / 4;           // 144 float4 per cache row
constexpr int kStride = kChunks + 1;        // padded LDS row (580 floats)

template <int KV>
__device__ __forceinline__ void load_kv_tile(float4 (*skv)[kStride], const AttnArgs& a, int64_t kv_base,
                                             int t0, int kv_last, int tid) {
    if (KV == DDTV_F32) {
        const float4* ck = reinterpret_cast<const float4*>(a.ckv);
        const float4* kr = reinterpret_cast<const float4*>(a.k_rope);
        for (int idx = tid; idx < kTile * kChunks; idx += 256) {
            const int r = idx / kChunks, c = idx - r * kChunks;
            const int64_t row = kv_base + min(t0 + r, kv_last);
            skv[r][c] = (c < 128) ? ck[row * 128 + c] : kr[row * 16 + (c - 128)];
        }
    } else if (KV == DDTV_FP8_E4M3) {
        // 16 FP8 values (16 bytes) per load -> four float4 chunks
        const uint4* ck = reinterpret_cast<const uint4*>(a.ckv);
        const uint4* kr = reinterpret_cast<const uint4*>(a.k_rope);
        constexpr int kB8 = kChunks / 4;    // 36 x 16 B per row
        for (int idx = tid; idx < kTile * kB8; idx += 256) {
            const int r = idx / kB8, c = idx - r * kB8;
            const int64_t row = kv_base + min(t0 + r, kv_last);
            const uint4 v = (c < 32) ? ck[row * 32 + c] : kr[row * 4 + (c - 32)];
            skv[r][4 * c] = fp8x4(v.x);
            skv[r][4 * c + 1] = fp8x4(v.y);
            skv[r][4 * c + 2] = fp8x4(v.z);
            skv[r][4 * c + 3] = fp8x4(v.w);
        }
    } else {
        // 8 bf16 (16 bytes) per load -> two float4 chunks
        const uint4* ck = reinterpret_cast<const uint4*>(a.ckv);
        const uint4* kr = reinterpret_cast<const uint4*>(a.k_rope);
        constexpr int kB16 = kChunks / 2;   // 72 x 16 B per row
        for (int idx = tid; idx < kTile * kB16; idx += 256) {
            const int r = idx / kB16, c = idx - r * kB16;
            const int64_t row = kv_base + min(t0 + r, kv_last);
            const uint4 v = (c < 64) ? ck[row * 64 + c] : kr[row * 8 + (c - 64)];
            skv[r][2 * c] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
            skv[r][2 * c + 1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
        }
    }
}

template <int KV>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
    __shared__ float4 sq[kRows][kChunks];     // 36 KiB: the workgroup's query rows
    __shared__ float4 skv[kTile][kStride];    // 72.5 KiB: one cache tile
    __shared__ uint32_t smask[kRows][kMaxW];

    const int64_t w = work_item(a);
    const int rt = (int)(w % a.n_rt);
    const int s = (int)((w / a.n_rt) % a.n_split);
    const int b = batch_row(a, (int)(w / ((int64_t)a.n_rt * a.n_split)));
    const ddtv_row rowd = a.rows[b];
    const int kv_len = rowd.kv_len, P = rowd.prefix;
    const int n_b = (kv_len + a.split_len - 1) / a.split_len;
    if (s >= n_b) return;
    const int kv_lo = s * a.split_len;
    const int kv_hi = min(kv_len, kv_lo + a.split_len);
    const int row0 = rt * kRows;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // Stage the query rows (zero beyond R) and their mask words.
    for (int idx = tid; idx < kRows * kChunks; idx += 256) {
        const int r = idx / kChunks, c = idx - r * kChunks;
        const int gr = row0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gr < a.R) {
            const int64_t qrow = (int64_t)b * a.R + gr;
            v = (c < 128) ? reinterpret_cast<const float4*>(a.q_abs)[qrow * 128 + c]
                          : reinterpret_cast<const float4*>(a.q_rope)[qrow * 16 + (c - 128)];
        }
        sq[r][c] = v;
    }
    if (tid < kRows * kMaxW) {
        const int r = tid / kMaxW, k = tid % kMaxW;
        const int gr = row0 + r;
        uint32_t m = 0;
        if (gr < a.R && k < a.W) m = a.bits[((int64_t)b * a.Q + gr / a.H) * a.W + k];
        smask[r][k] = m;
    }

    const int kvl = lane & 31, half = lane >> 5;
    float m_run[4], l_run[4];
    float4 o[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.f;
        o[r][0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[r][1] = o[r][0];
    }

    for (int t0 = kv_lo; t0 < kv_hi; t0 += kTile) {
        __syncthreads();   // previous tile fully consumed (and staging above visible)
        load_kv_tile<KV>(skv, a, rowd.kv_off, t0, kv_len - 1, tid);
        __syncthreads();

        // scores of cache row t0 + kvl against the wave's 4 query rows
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        const float4* krow = &skv[kvl][half * 72];
#pragma unroll 4
        for (int c = 0; c < 72; ++c) {
            const float4 k = krow[c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float4 q = sq[wave * 4 + r][half * 72 + c];
                acc[r] = fmaf(q.x, k.x, acc[r]);
                acc[r] = fmaf(q.y, k.y, acc[r]);
                acc[r] = fmaf(q.z, k.z, acc[r]);
                acc[r] = fmaf(q.w, k.w, acc[r]);
            }
        }
        const int j = t0 + kvl;
        float p[4], alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sc = (acc[r] + wave_xor(acc[r], 32)) * a.scale_log2;
            const int rr = wave * 4 + r;
            bool vis = (row0 + rr < a.R) && (j < kv_hi);
            if (vis && j >= P) vis = ((smask[rr][(j - P) >> 5] >> ((j - P) & 31)) & 1u) != 0u;
            sc = vis ? sc : -INFINITY;
            float tm = sc;
#pragma unroll
            for (int m = 1; m < 32; m <<= 1) tm = fmaxf(tm, wave_xor(tm, m));
            const float m_new = fmaxf(m_run[r], tm);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[r] = exp2f(m_run[r] - m_use);
            p[r] = vis ? exp2f(sc - m_use) : 0.f;
            float ps = p[r];
#pragma unroll
            for (int m = 1; m < 32; m <<= 1) ps += wave_xor(ps, m);
            l_run[r] = l_run[r] * alpha[r] + ps;
            m_run[r] = m_new;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o[r][0].x *= alpha[r]; o[r][0].y *= alpha[r]; o[r][0].z *= alpha[r]; o[r][0].w *= alpha[r];
            o[r][1].x *= alpha[r]; o[r][1].y *= alpha[r]; o[r][1].z *= alpha[r]; o[r][1].w *= alpha[r];
        }
        // weighted latent sum: lane owns latent dims 8*lane .. 8*lane+7
#pragma unroll 8
        for (int k = 0; k < kTile; ++k) {
            const float4 v0 = skv[k][2 * lane];
            const float4 v1 = skv[k][2 * lane + 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[r]), k));
                o[r][0].x = fmaf(pk, v0.x, o[r][0].x); o[r][0].y = fmaf(pk, v0.y, o[r][0].y);
                o[r][0].z = fmaf(pk, v0.z, o[r][0].z); o[r][0].w = fmaf(pk, v0.w, o[r][0].w);
                o[r][1].x = fmaf(pk, v1.x, o[r][1].x); o[r][1].y = fmaf(pk, v1.y, o[r][1].y);
                o[r][1].z = fmaf(pk, v1.z, o[r][1].z); o[r][1].w = fmaf(pk, v1.w, o[r][1].w);
            }
        }
    }

    const float kLn2 = 0.69314718055994530942f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gr = row0 + wave * 4 + r;
        if (gr >= a.R) continue;
        const int64_t orow = (int64_t)b * a.R + gr;
        if (n_b == 1) {
            const float inv = l_run[r] > 0.f ? 1.f / l_run[r] : 0.f;
            float4* dst = reinterpret_cast<float4*>(a.out) + orow * 128 + 2 * lane;
            dst[0] = make_float4(o[r][0].x * inv, o[r][0].y * inv, o[r][0].z * inv, o[r][0].w * inv);
            dst[1] = make_float4(o[r][1].x * inv, o[r][1].y * inv, o[r][1].z * inv, o[r][1].w * inv);
            if (a.lse && lane == 0)
                a.lse[orow] = l_run[r] > 0.f ? (m_run[r] + log2f(l_run[r])) * kLn2 : -INFINITY;
        } else {
            const int64_t prow = ((int64_t)b * a.n_split + s) * a.R + gr;
            float4* dst = reinterpret_cast<float4*>(a.part_o) + prow * 128 + 2 * lane;
            dst[0] = o[r][0];
            dst[1] = o[r][1];
            if (lane == 0) a.part_ml[prow] = make_float2(m_run[r], l_run[r]);
        }
    }
}

}  // namespace

hipError_t launch_attn_valu(const AttnArgs& a, int kv_dtype, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    if (kv_dtype == DDTV_BF16)
        hipLaunchKernelGGL(attn_valu_kernel<DDTV_BF16>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    else if (kv_dtype == DDTV_FP8_E4M3)
        hipLaunchKernelGGL(attn_valu_kernel<DDTV_FP8_E4M3>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(attn_valu_kernel<DDTV_F32>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ddtv
