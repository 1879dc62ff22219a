// The steps around the verify attention: the query split with NeoX rotary
// embedding and the w_kc absorb before it, the w_vc value projection after it,
// and the tree nodes' new cache rows (latent plus rotated rope key).
//   Pages: "The Query-Split Kernel: A Pivotal Edit in Building a Native DDTree
//   Inference Engine", sections "The Reasoning Chain" and "Input Knowledge"
//   (the query projection of each token and head holds a nope part and a rope
//   part; the rope part is rotated NeoX style with float64 angles; the nope part
//   meets the latent through the absorbed w_kc); "The Verify-Attn Kernel ...",
//   section "Design Decisions and Trade-Offs" (the attention emits the latent, a
//   separate per-head GEMM with w_vc follows).  The pages split the query into
//   contiguous nope/rope buffers with one kernel, rotate with another and absorb
//   with a GEMM; here one launch reads the projection once and writes both
//   attention operands.
//
// Both projections are per-head fp32 GEMMs on the matrix cores
// (v_mfma_f32_16x16x4_f32), C[m][n] = sum_k A[m][k] B[k][n] for every head:
//   absorb:  A = q[m][h][0..d_nope), B = w_kc[h] ([d_nope][512]), C = q_abs[m][h]
//   value:   A = latent[m][h][0..512), B = w_vc[h]^T (w_vc[h] is [d_v][512]),
//            C = v[m][h]
// A workgroup (8 waves) owns a 64 x 128 output tile of one head and walks K in
// stages of 32, double-buffered through LDS: 16-byte global loads, the next
// stage loaded into registers while the current one feeds the MFMAs.  Each wave
// owns 32 x 32 of the tile (2 x 2 blocks of 16 x 16); two workgroups fit a CU,
// so every SIMD holds up to four waves to cover LDS reads and barriers.  Small
// grids (fewer wide workgroups than CUs) take 2-wave workgroups over 64 x 32
// tiles instead, so the work spreads over four times as many CUs.
// LDS layouts (4-byte words; 64 banks on gfx950):
//   A stage   [64 m][36]   : lane (i, kk) of an A operand reads m = i, k = kk;
//                            row stride 36 words puts the 16 x 4 lanes on 64
//                            distinct banks;
//   B stage   absorb: [32 k][BN + 16] (n contiguous; a stride of 16 mod 64 puts
//                            the four k rows of an operand on disjoint bank groups)
//             value:  [128 n][36] (k contiguous, as A).
#include <math.h>

#include "ddtv_internal.hpp"
#include "neighbour.hpp"

namespace ddtv {
namespace {

constexpr int kBM = 64, kBK = 32;
constexpr int kAStride = 36;             // words per m row of an A stage
constexpr int kBStrideNK = 36;           // words per n row of an [n][k] B stage
constexpr int kAStage = kBM * kAStride;  // 2304 words

// Workgroup shape.  Wide: 8 waves over a 64 x 128 output tile (2 x 4 waves of
// 32 x 32).  Narrow: 2 waves over 64 x 32, four times the workgroups, for grids
// that would leave most CUs idle with wide tiles (few tree nodes and heads).
template <bool kWide>
struct Geo {
    static constexpr int Threads = kWide ? 512 : 128;
    static constexpr int BN = kWide ? 128 : 32;
    static constexpr int WavesN = BN / 32;              // waves across the columns
    static constexpr int BStrideKN = BN + 16;           // words per k row of a [k][n] B stage (16 mod 64)
    static constexpr int BStage = (kBK * BStrideKN > BN * kBStrideNK) ? kBK * BStrideKN : BN * kBStrideNK;
    static constexpr int ALoads = kBM * kBK / 4 / Threads;   // float4 per thread
    static constexpr int BLoads = BN * kBK / 4 / Threads;
    static constexpr int RopeRows = Threads / 16;
    static_assert(kDLat / BN * RopeRows >= kBM, "the rotary slice covers a row tile with its column-tile workgroups");
};

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Global -> registers for one K stage.  A: 64 rows x 32 k = 512 float4 (8 threads
// per row, 128 contiguous bytes).  B: 32 k x BN n, as [k][n] rows of 4 BN bytes
// (absorb) or [n][k] rows of 128 bytes (value).  Rows past M and columns past N
// read the last valid row or column instead of a zero fill: they feed only
// outputs that are never stored, and unconditional loads let the compiler keep
// them in flight across the stage instead of waiting at each predicated load.
template <bool kWide>
struct Stage {
    float4 a[Geo<kWide>::ALoads];
    float4 b[Geo<kWide>::BLoads];
};

template <bool kBTrans, bool kWide>
__device__ __forceinline__ void load_stage(const ProjArgs& p, int h, int m0, int n0, int k0, Stage<kWide>& s,
                                           int t) {
    using G = Geo<kWide>;
#pragma unroll
    for (int r = 0; r < G::ALoads; ++r) {
        const int idx = t + r * G::Threads;
        const int row = idx >> 3, kq = (idx & 7) * 4;
        const int64_t m = min((int64_t)m0 + row, p.M - 1);
        s.a[r] = ld4(p.A + m * p.lda + (int64_t)h * p.a_head + k0 + kq);
    }
#pragma unroll
    for (int r = 0; r < G::BLoads; ++r) {
        const int idx = t + r * G::Threads;
        if (!kBTrans) {
            const int k = idx / (G::BN / 4), nq = (idx % (G::BN / 4)) * 4;
            const int n = min(n0 + nq, p.N - 4);           // N is a multiple of 4 here (512)
            s.b[r] = ld4(p.B + (int64_t)h * p.b_head + (int64_t)(k0 + k) * p.N + n);
        } else {
            const int nl = idx >> 3, kq = (idx & 7) * 4;       // 8 float4 per n row
            const int n = min(n0 + nl, p.N - 1);
            s.b[r] = ld4(p.B + (int64_t)h * p.b_head + (int64_t)n * p.K + k0 + kq);
        }
    }
}

template <bool kBTrans, bool kWide>
__device__ __forceinline__ void store_stage(float* As, float* Bs, const Stage<kWide>& s, int t) {
    using G = Geo<kWide>;
#pragma unroll
    for (int r = 0; r < G::ALoads; ++r) {
        const int idx = t + r * G::Threads;
        const int row = idx >> 3, kq = (idx & 7) * 4;
        *reinterpret_cast<float4*>(As + row * kAStride + kq) = s.a[r];
    }
#pragma unroll
    for (int r = 0; r < G::BLoads; ++r) {
        const int idx = t + r * G::Threads;
        if (!kBTrans) {
            const int k = idx / (G::BN / 4), nq = (idx % (G::BN / 4)) * 4;
            *reinterpret_cast<float4*>(Bs + k * G::BStrideKN + nq) = s.b[r];
        } else {
            const int nl = idx >> 3, kq = (idx & 7) * 4;
            *reinterpret_cast<float4*>(Bs + nl * kBStrideNK + kq) = s.b[r];
        }
    }
}

// NeoX rotation of the rope part of kThreads / 16 query rows from m0, every head.
// 16 lanes per row, two pairs per lane: each (row, pair) angle is computed once
// and used for all heads.  Angles, their sine and cosine, and the rotation run
// in float64; the result is rounded once to float32.
__device__ void rope_rows(const ProjArgs& p, int64_t m0) {
    const int64_t m = m0 + (threadIdx.x >> 4);
    const int i = (threadIdx.x & 15) * 2;
    if (m >= p.M) return;
    int32_t pos;
    if (p.positions) {
        pos = p.positions[m];
    } else {   // prefix length plus depth: the ancestor-or-self mask holds depth + 1 bits
        const int b = (int)(m / p.Q), q = (int)(m % p.Q);
        const uint32_t* w = p.bits + ((int64_t)b * p.Q + q) * p.W;
        int pc = 0;
        for (int k = 0; k < p.W; ++k) pc += __popc(w[k]);
        pos = p.rows[b].prefix + pc - 1;
    }
    double s0, c0, s1, c1;
    sincos((double)pos * p.inv_freq[i], &s0, &c0);
    sincos((double)pos * p.inv_freq[i + 1], &s1, &c1);
    const float* x = p.A + m * p.lda + p.K + i;
    float* y = p.rope_out + m * p.H * kDRope + i;
#pragma unroll 4
    for (int h = 0; h < p.H; ++h) {
        const float2 lo = *reinterpret_cast<const float2*>(x + (int64_t)h * p.a_head);
        const float2 hi = *reinterpret_cast<const float2*>(x + (int64_t)h * p.a_head + 32);
        float2 ylo, yhi;
        ylo.x = (float)((double)lo.x * c0 - (double)hi.x * s0);
        yhi.x = (float)((double)hi.x * c0 + (double)lo.x * s0);
        ylo.y = (float)((double)lo.y * c1 - (double)hi.y * s1);
        yhi.y = (float)((double)hi.y * c1 + (double)lo.y * s1);
        *reinterpret_cast<float2*>(y + (int64_t)h * kDRope) = ylo;
        *reinterpret_cast<float2*>(y + (int64_t)h * kDRope + 32) = yhi;
    }
}

template <bool kBTrans, bool kWide>
__global__ __launch_bounds__(Geo<kWide>::Threads) void proj_gemm_kernel(ProjArgs p) {
    using G = Geo<kWide>;
    __shared__ float As[2][kAStage];
    __shared__ float Bs[2][G::BStage];
    // With the rotary step, slice z = 0 rotates (dispatched first, short) and
    // slice z = 1 + h multiplies head h.
    int h = blockIdx.z;
    if (!kBTrans && p.rope_out) {
        if (h == 0) {
            if (blockIdx.y * G::RopeRows < kBM)
                rope_rows(p, (int64_t)blockIdx.x * kBM + blockIdx.y * G::RopeRows);
            return;
        }
        --h;
    }
    const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * G::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave / G::WavesN) * 32, wn = (wave % G::WavesN) * 32;
    const int li = lane & 15, lk = lane >> 4;

    floatx4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    Stage<kWide> st;
    load_stage<kBTrans, kWide>(p, h, m0, n0, 0, st, threadIdx.x);
    store_stage<kBTrans, kWide>(As[0], Bs[0], st, threadIdx.x);
    __syncthreads();
    const int n_stage = p.K / kBK;
    for (int s = 0; s < n_stage; ++s) {
        const int cur = s & 1;
        if (s + 1 < n_stage) load_stage<kBTrans, kWide>(p, h, m0, n0, (s + 1) * kBK, st, threadIdx.x);
        const float* A = As[cur];
        const float* Bm = Bs[cur];
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 4) {
            float a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = A[(wm + i * 16 + li) * kAStride + kk + lk];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = kBTrans ? Bm[(wn + j * 16 + li) * kBStrideNK + kk + lk]
                               : Bm[(kk + lk) * G::BStrideKN + wn + j * 16 + li];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < n_stage) {
            store_stage<kBTrans, kWide>(As[cur ^ 1], Bs[cur ^ 1], st, threadIdx.x);
            __syncthreads();
        }
    }
    // D block (i, j): lane holds rows 4*lk + r, column li.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = (int64_t)m0 + wm + i * 16 + 4 * lk + r;
            if (m >= p.M) continue;
            float* c = p.C + m * p.ldc + (int64_t)h * p.c_head;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + wn + j * 16 + li;
                if (n < p.N) c[n] = acc[i][j][r];
            }
        }
    }
}

// Small grids with a long contraction (the value projection of a few tree nodes:
// one 64-row tile and 4 column tiles per head, K = 512): four groups of 128
// threads share one 64 x 32 output tile, group g taking the K stages g, g + 4,
// ...; then groups 1..3 park their sums in LDS and group 0 adds them in group
// order (deterministic) and writes C.  Four times the waves per workgroup and a
// quarter of the stages each, where the narrow kernel ran 16 dependent stages on
// 2 waves.
constexpr int kSplitGroups = 4;

template <bool kBTrans>
__global__ __launch_bounds__(kSplitGroups * 128) void proj_gemm_splitk_kernel(ProjArgs p) {
    using G = Geo<false>;
    static_assert(G::Threads == 128 && G::WavesN == 1, "one narrow tile per group");
    __shared__ float As[kSplitGroups][2][kAStage];
    __shared__ float Bs[kSplitGroups][2][G::BStage];
    const int h = blockIdx.z;
    const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * G::BN;
    const int grp = threadIdx.x >> 7, t = threadIdx.x & 127;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave * 32;
    const int li = lane & 15, lk = lane >> 4;

    floatx4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int n_stage = p.K / kBK;
    const int rounds = (n_stage + kSplitGroups - 1) / kSplitGroups;   // the same for every group
    Stage<false> st;
    if (grp < n_stage) {
        load_stage<kBTrans, false>(p, h, m0, n0, grp * kBK, st, t);
        store_stage<kBTrans, false>(As[grp][0], Bs[grp][0], st, t);
    }
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
        const int s = grp + r * kSplitGroups, sn = s + kSplitGroups;
        const int cur = r & 1;
        if (sn < n_stage) load_stage<kBTrans, false>(p, h, m0, n0, sn * kBK, st, t);
        if (s < n_stage) {
            const float* A = As[grp][cur];
            const float* Bm = Bs[grp][cur];
#pragma unroll
            for (int kk = 0; kk < kBK; kk += 4) {
                float a[2], b[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) a[i] = A[(wm + i * 16 + li) * kAStride + kk + lk];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    b[j] = kBTrans ? Bm[(j * 16 + li) * kBStrideNK + kk + lk] : Bm[(kk + lk) * G::BStrideKN + j * 16 + li];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
        if (r + 1 < rounds) {
            if (sn < n_stage) store_stage<kBTrans, false>(As[grp][cur ^ 1], Bs[grp][cur ^ 1], st, t);
            __syncthreads();
        }
    }
    __syncthreads();   // every group is done with the stage buffers
    float* park = &As[0][0][0];   // 3 groups x 16 values x 128 threads (24 KiB of the 36 KiB of A buffers)
    static_assert((kSplitGroups - 1) * 16 * 128 <= kSplitGroups * 2 * kAStage, "parking fits the A buffers");
    if (grp > 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) park[((grp - 1) * 16 + (i * 2 + j) * 4 + r) * 128 + t] = acc[i][j][r];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < kSplitGroups; ++g)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] += park[((g - 1) * 16 + (i * 2 + j) * 4 + r) * 128 + t];
    // D block (i, j): lane holds rows 4*lk + r, column li.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = (int64_t)m0 + wm + i * 16 + 4 * lk + r;
            if (m >= p.M) continue;
            float* c = p.C + m * p.ldc + (int64_t)h * p.c_head;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + j * 16 + li;
                if (n < p.N) c[n] = acc[i][j][r];
            }
        }
    }
}

// Float32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Float32 -> FP8 E4M3 ("fn") byte, round to nearest, ties to even; magnitudes
// above 464 (which round past the largest finite value, 448) saturate to 448.
//  - normal results (|x| >= 2^-6): the float32 exponent/mantissa fields are
//    rounded to 3 mantissa bits by adding half an fp8 ulp minus one plus the
//    kept lsb, then rebased (bias 127 -> 7); a carry out of the mantissa moves
//    into the exponent, as it should;
//  - subnormal results: round |x| * 2^9 to an integer (0..8; 8 is the smallest
//    normal, 0x08, so the code is that integer either way).
__device__ __forceinline__ uint32_t to_fp8(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a > 0x43e80000u) {                       // > 464
        code = 0x7eu;
    } else if (a >= 0x3c800000u) {               // >= 2^-6
        const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    } else {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

__device__ __forceinline__ void store_cache(void* base, int dtype, int64_t idx, float v) {
    if (dtype == DDTV_BF16)
        reinterpret_cast<uint16_t*>(base)[idx] = to_bf16(v);
    else if (dtype == DDTV_FP8_E4M3)
        reinterpret_cast<uint8_t*>(base)[idx] = (uint8_t)to_fp8(v);
    else
        reinterpret_cast<float*>(base)[idx] = v;
}

// One wave per tree node: its latent row and its rotated rope key go to cache
// row kv_off + prefix + node.
__global__ __launch_bounds__(64) void append_kv_kernel(AppendArgs p) {
    const int64_t node = blockIdx.x;
    const int b = (int)(node / p.Q), q = (int)(node % p.Q);
    const int lane = threadIdx.x;
    const ddtv_row row = p.rows[b];
    const int64_t r = row.kv_off + row.prefix + q;
    int32_t pos;
    if (p.positions) {
        pos = p.positions[node];
    } else {
        const uint32_t* w = p.bits + node * p.W;
        int pc = 0;
        for (int k = 0; k < p.W; ++k) pc += __popc(w[k]);
        pos = row.prefix + pc - 1;
    }
    const float* lat = p.latent + node * kDLat;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = (lane + u * 64) * 4;
        const float4 v = ld4(lat + c);
        if (p.dtype == DDTV_BF16) {
            uint16_t* d = reinterpret_cast<uint16_t*>(p.ckv) + r * kDLat + c;
            ushort4 o;
            o.x = to_bf16(v.x); o.y = to_bf16(v.y); o.z = to_bf16(v.z); o.w = to_bf16(v.w);
            *reinterpret_cast<ushort4*>(d) = o;
        } else if (p.dtype == DDTV_FP8_E4M3) {
            uint32_t* d = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.ckv) + r * kDLat + c);
            *d = to_fp8(v.x) | (to_fp8(v.y) << 8) | (to_fp8(v.z) << 16) | (to_fp8(v.w) << 24);
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.ckv) + r * kDLat + c) = v;
        }
    }
    if (lane < 32) {
        const float* x = p.k_pe + node * kDRope;
        const double x0 = (double)x[lane], x1 = (double)x[lane + 32];
        double sn, cs;
        sincos((double)pos * p.inv_freq[lane], &sn, &cs);
        const float y0 = (float)(x0 * cs - x1 * sn), y1 = (float)(x1 * cs + x0 * sn);
        store_cache(p.k_rope, p.dtype, r * kDRope + lane, y0);
        store_cache(p.k_rope, p.dtype, r * kDRope + lane + 32, y1);
    }
}

}  // namespace


template <bool kBTrans, bool kWide>
static void launch_proj_as(const ProjArgs& p, hipStream_t stream) {
    using G = Geo<kWide>;
    const dim3 grid((unsigned)((p.M + kBM - 1) / kBM), (unsigned)((p.N + G::BN - 1) / G::BN),
                    (unsigned)(p.H + (!kBTrans && p.rope_out ? 1 : 0)));
    hipLaunchKernelGGL((proj_gemm_kernel<kBTrans, kWide>), grid, dim3(G::Threads), 0, stream, p);
}

hipError_t launch_proj(const ProjArgs& p, bool b_trans, int cus, hipStream_t stream) {
    // narrow tiles when wide ones would give fewer workgroups than CUs
    const int64_t wide_wgs = (p.M + kBM - 1) / kBM * ((p.N + Geo<true>::BN - 1) / Geo<true>::BN) * p.H;
    const bool wide = wide_wgs >= cus;
    (void)hipGetLastError();   // report only this launch's error
    // value projection of few rows: narrow tiles would still leave most CUs idle
    // and run 16 dependent K stages each -- split K inside the workgroup instead
    const int64_t narrow_wgs = (p.M + kBM - 1) / kBM * ((p.N + Geo<false>::BN - 1) / Geo<false>::BN) * p.H;
    if (b_trans && !wide && 2 * narrow_wgs <= cus && p.K / kBK >= 2 * kSplitGroups) {
        const dim3 grid((unsigned)((p.M + kBM - 1) / kBM), (unsigned)((p.N + Geo<false>::BN - 1) / Geo<false>::BN),
                        (unsigned)p.H);
        hipLaunchKernelGGL((proj_gemm_splitk_kernel<true>), grid, dim3(kSplitGroups * 128), 0, stream, p);
        return hipGetLastError();
    }
    if (b_trans)
        wide ? launch_proj_as<true, true>(p, stream) : launch_proj_as<true, false>(p, stream);
    else
        wide ? launch_proj_as<false, true>(p, stream) : launch_proj_as<false, false>(p, stream);
    return hipGetLastError();
}

hipError_t launch_append_kv(const AppendArgs& p, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)((int64_t)p.B * p.Q)), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ddtv
