// S2..S6 on the matrix cores -- the path once a batch row has 16 or more query rows (H * q_len).
//
// Same arithmetic as the VALU path (score = scale * (absorbed query . latent + rope
// query . rope key), softmax over visible positions, weighted latent sum -- "The
// Verify-Attn Kernel: A Single File Write ...", section "The Design Journey: From
// Concept to CUDA"), organised for CDNA4 MFMA (v_mfma_f32_16x16x4_f32):
//
//  * A workgroup (8 waves) owns 64 query rows of one batch row and one KV split.
//    All heads share one latent cache, so one LDS tile of 32 cache rows (576 floats
//    each) feeds all 64 rows, and its first 512 columns serve as the value too:
//    each cache row crosses HBM->LDS once per workgroup.
//  * Waves come in pairs; a pair owns 16 query rows.  For the scores the pair
//    splits the 576-long contraction (wave h holds query dims 288h .. 288h+287 in
//    VGPRs for the whole split) and swaps partial sums through LDS; for the
//    weighted sum it splits the 512 output dims (wave h accumulates dims
//    256h .. 256h+255).  No MFMA is duplicated, and each wave needs ~half the
//    registers a single owner of 16 rows would, which leaves room for two waves
//    per SIMD.
//  * Scores are produced transposed, S^T = K Q^T: the cache tile is the A operand,
//    the query the B operand.  In that layout each lane holds probabilities of ONE
//    query row, exactly the A-operand layout of P.V, so no shuffle is needed
//    between the two contractions.  The contraction order is permuted the same way
//    on both operands so every LDS operand fetch is a conflict-free 16-byte read.
//    The swizzle reduces to 4 per-lane base offsets per operand kind plus
//    compile-time immediates (TileOffsets); addressing it that way instead of
//    through the swizzle function leaves the register allocator ~20 VGPRs and made
//    the kernel ~2 % faster.
//  * Row maxima cross lanes with permlane swaps; exponentials are the raw v_exp_f32;
//    the query is pre-scaled by scale*log2(e) when it is loaded.
//  * Online softmax in exp2 units with lazy rescaling (the running max moves only
//    when a tile beats it by more than 2^8).
//  * Row-half mode, for batch rows of at most 32 query rows (decode-like shapes,
//    where the cache stream is the bound): a workgroup owns 32 rows, and wave
//    pairs 2k and 2k + 1 both own rows 16k .. 16k + 15 but take cache rows 0..15
//    and 16..31 of every tile respectively, each with its own online softmax.
//    The two halves are combined inside the workgroup at the end (through LDS),
//    so a split leaves one partial like the usual mode.  With 16 rows this puts pairs 0 and 1 (waves 0..3, one per
//    SIMD) to work where otherwise one pair (two SIMDs) would do all the matrix
//    work of the tile; the idle waves 4..7 then issue every tile load, and the
//    score-swap barrier waits for LDS work only, so the next tile streams in
//    during P.V.
//  * fp32 caches go HBM->LDS with global_load_lds_dwordx4 (no VGPR staging),
//    double buffered; bf16 and FP8 caches are widened exactly to fp32 through
//    VGPRs on the way in.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRows = 64;                     // query rows per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTileChunks = kTile * kDQK / 4; // 4608 x 16 B per tile (72 KiB)

// LDS tile layout (fp32, 16-byte chunks): a latent region of 32 rows x 128 chunks
// followed by a rope region of 32 rows x 16 chunks.  Chunk c of row r is stored at
// position c ^ (r & 15) of its row, so the 16 rows read together by an MFMA operand
// fetch hit 16 different bank groups.
constexpr int kRopeBase = kTile * 128;

__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int lat_at(int r, int c) { return r * 128 + swz(r, c); }
__device__ __forceinline__ int rope_at(int r, int c) { return kRopeBase + r * 16 + swz(r, c); }

// max over the 4 lanes holding one query row (lanes l, l^16, l^32, l^48), with
// lane swaps on the vector ALU instead of LDS permutes
__device__ __forceinline__ float row_max4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(x, fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(x, fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])));
}

// fp32 cache straight into LDS.  Per wave: 8 instructions for the latent region
// (half a row each, 1 KiB contiguous in HBM) and 1 for the rope region (4 rows x
// 256 B).  Row indices and swizzle constants are wave-uniform; only the lane's
// 16-byte column varies.
__device__ __forceinline__ void issue_tile_f32(f32x4* buf, const AttnArgs& a, int64_t kv_base, int t0,
                                               int kv_last, int wave, int lane) {
    const float* ck = reinterpret_cast<const float*>(a.ckv);
    const float* kr = reinterpret_cast<const float*>(a.k_rope);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = wave * 4 + (k >> 1);
        const int p = (k & 1) * 64 + lane;
        const int64_t row = kv_base + min(t0 + r, kv_last);
        __builtin_amdgcn_global_load_lds(ck + row * kDLat + 4 * swz(r, p),
                                         (lds_void*)(buf + r * 128 + (k & 1) * 64), 16, 0, 0);
    }
    {
        const int r0 = wave * 4;
        const int r = r0 + (lane >> 4);
        const int64_t row = kv_base + min(t0 + r, kv_last);
        __builtin_amdgcn_global_load_lds(kr + row * kDRope + 4 * swz(r, lane & 15),
                                         (lds_void*)(buf + kRopeBase + r0 * 16), 16, 0, 0);
    }
}

// bf16 and FP8 caches: 16-byte loads (8 or 16 values) into VGPRs ...
struct NarrowStage {
    uint4 v[5];
};

__device__ __forceinline__ void load_tile_bf16(NarrowStage& st, const AttnArgs& a, int64_t kv_base, int t0,
                                               int kv_last, int tid) {
    const uint4* ck = reinterpret_cast<const uint4*>(a.ckv);
    const uint4* kr = reinterpret_cast<const uint4*>(a.k_rope);
#pragma unroll
    for (int k = 0; k < 4; ++k) {   // latent: 32 rows x 64 pieces
        const int r = k * 8 + (tid >> 6), c = tid & 63;
        st.v[k] = ck[(kv_base + min(t0 + r, kv_last)) * 64 + c];
    }
    if (tid < 256) {                // rope: 32 rows x 8 pieces
        const int r = tid >> 3, c = tid & 7;
        st.v[4] = kr[(kv_base + min(t0 + r, kv_last)) * 8 + c];
    }
}

// ... then widened and written to the swizzled fp32 layout.
__device__ __forceinline__ void store_tile_bf16(f32x4* buf, const NarrowStage& st, int tid) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        if (k == 4 && tid >= 256) break;
        const uint4 v = st.v[k];
        const f32x4 lo = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        const f32x4 hi = {bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        if (k < 4) {
            const int r = k * 8 + (tid >> 6), c = tid & 63;
            buf[lat_at(r, 2 * c)] = lo;
            buf[lat_at(r, 2 * c + 1)] = hi;
        } else {
            const int r = tid >> 3, c = tid & 7;
            buf[rope_at(r, 2 * c)] = lo;
            buf[rope_at(r, 2 * c + 1)] = hi;
        }
    }
}

// FP8: a tile is 32 rows x 32 latent pieces + 32 rows x 4 rope pieces of 16 bytes.
__device__ __forceinline__ void load_tile_fp8(NarrowStage& st, const AttnArgs& a, int64_t kv_base, int t0,
                                              int kv_last, int tid) {
    const uint4* ck = reinterpret_cast<const uint4*>(a.ckv);
    const uint4* kr = reinterpret_cast<const uint4*>(a.k_rope);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = k * 16 + (tid >> 5), c = tid & 31;
        st.v[k] = ck[(kv_base + min(t0 + r, kv_last)) * 32 + c];
    }
    if (tid < 128) {
        const int r = tid >> 2, c = tid & 3;
        st.v[2] = kr[(kv_base + min(t0 + r, kv_last)) * 4 + c];
    }
}

__device__ __forceinline__ f32x4 fp8_chunk(uint32_t w) {
    const float4 f = fp8x4(w);
    return f32x4{f.x, f.y, f.z, f.w};
}

__device__ __forceinline__ void store_tile_fp8(f32x4* buf, const NarrowStage& st, int tid) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = k * 16 + (tid >> 5), c = tid & 31;
        const uint4 v = st.v[k];
        buf[lat_at(r, 4 * c)] = fp8_chunk(v.x);
        buf[lat_at(r, 4 * c + 1)] = fp8_chunk(v.y);
        buf[lat_at(r, 4 * c + 2)] = fp8_chunk(v.z);
        buf[lat_at(r, 4 * c + 3)] = fp8_chunk(v.w);
    }
    if (tid < 128) {
        const int r = tid >> 2, c = tid & 3;
        const uint4 v = st.v[2];
        buf[rope_at(r, 4 * c)] = fp8_chunk(v.x);
        buf[rope_at(r, 4 * c + 1)] = fp8_chunk(v.y);
        buf[rope_at(r, 4 * c + 2)] = fp8_chunk(v.z);
        buf[rope_at(r, 4 * c + 3)] = fp8_chunk(v.w);
    }
}

// One tile of a narrow (bf16 or FP8) cache: load into VGPRs, then widen into LDS.
template <int KV>
__device__ __forceinline__ void load_tile_narrow(NarrowStage& st, const AttnArgs& a, int64_t kv_base, int t0,
                                                 int kv_last, int tid) {
    if (KV == DDTV_FP8_E4M3)
        load_tile_fp8(st, a, kv_base, t0, kv_last, tid);
    else
        load_tile_bf16(st, a, kv_base, t0, kv_last, tid);
}
template <int KV>
__device__ __forceinline__ void store_tile_narrow(f32x4* buf, const NarrowStage& st, int tid) {
    if (KV == DDTV_FP8_E4M3)
        store_tile_fp8(buf, st, tid);
    else
        store_tile_bf16(buf, st, tid);
}

struct Smem {
    f32x4 kv[2][kTileChunks];        // 2 x 72 KiB, double-buffered cache tile
    f32x4 sx[kWaves][2][64];         // 16 KiB, partial scores swapped inside a wave pair
};

// Per-lane byte offsets inside a tile buffer, derived from the swizzle (chunk c
// of row r at c ^ (r & 15)); with them every operand read is one register plus
// a compile-time immediate.  Lane (g, n), x = g ^ (n & 3), y = (n >> 2) & 3:
//  score operand, latent step tg = 4a + b, cache row n:  qoff[b] + 256 a   (row 16+n: +32 KiB)
//  score operand, rope step 32 + t, cache row n:          roff[t]           (row 16+n: +4 KiB)
//  value operand, cache row 16h + 4g + j, dims 16 blk + n: voff[j] + 256 blk (h = 1: +32 KiB)
struct TileOffsets {
    uint32_t qoff[4], roff[4], voff[4];
};

__device__ __forceinline__ TileOffsets tile_offsets(int g, int n) {
    TileOffsets o;
    const int x = g ^ (n & 3), y = (n >> 2) & 3;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        o.qoff[b] = n * 2048 + ((b ^ y) << 6) + (x << 4);
        o.roff[b] = kRopeBase * 16 + n * 256 + ((b ^ y) << 6) + (x << 4);
        o.voff[b] = (4 * g + b) * 2048 + ((n ^ (4 * g + b)) << 4);
    }
    return o;
}

__device__ __forceinline__ f32x4 lds16(const char* base, uint32_t off) {
    return *reinterpret_cast<const f32x4*>(base + off);
}

// Partial S^T of the tile at Kb over this wave's half of the contraction (two
// independent accumulators: cache rows n and 16 + n; in row-half mode one, cache
// row 16 rh + n), stored to the wave's swap area; issue() starts the next tile's
// loads part-way through.
template <int HALF, bool kHv, class Issue>
__device__ __forceinline__ void qk_slot(const char* Kb, const TileOffsets& to, const f32x4 (&qreg)[18],
                                        f32x4* sx_mine, int lane, Issue&& issue, int rh) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    auto kchunk = [&](int row_hi, int t) -> f32x4 {
        const int tg = 18 * HALF + t;
        return (tg < 32) ? lds16(Kb, to.qoff[tg & 3] + 256 * (tg >> 2) + row_hi * 32768)
                         : lds16(Kb, to.roff[tg - 32] + row_hi * 4096);
    };
    if constexpr (kHv) {
        f32x4 a0 = kchunk(rh, 0);
#pragma unroll
        for (int t = 0; t < 18; ++t) {
            const f32x4 c0 = a0;
            if (t + 1 < 18) a0 = kchunk(rh, t + 1);
#pragma unroll
            for (int u = 0; u < 4; ++u) s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(c0[u], qreg[t][u], s0, 0, 0, 0);
            if (t == 2) issue();
        }
        sx_mine[lane] = s0;
        return;
    }
    f32x4 a0 = kchunk(0, 0), a1 = kchunk(1, 0);
#pragma unroll
    for (int t = 0; t < 18; ++t) {
        const f32x4 c0 = a0, c1 = a1;
        if (t + 1 < 18) {
            a0 = kchunk(0, t + 1);
            a1 = kchunk(1, t + 1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(c0[u], qreg[t][u], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(c1[u], qreg[t][u], s1, 0, 0, 0);
        }
        // The next tile's loads go out here, behind a queue of MFMAs: issuing them
        // (9 address computations and global_load_lds per wave) right after the
        // barrier would delay the first MFMA by a few hundred cycles.  Measured
        // on the 8-batch-row, 32768-prefix workload: after step 2 of 18 beats steps
        // 1, 3 and 5 and a three-way split.
        if (t == 2) issue();
    }
    sx_mine[lane] = s0;
    sx_mine[64 + lane] = s1;
}

// Full scores of the tile starting at cache position t0 (own partial and the
// partner's, both from LDS), online softmax, then O += P V over this wave's 256 dims.
// Row-half mode: only the 16 cache rows of half rh.  kPF pins the value reads
// one step ahead (off for the widened bf16 cache, whose registers it would spill).
template <int HALF, bool kHv, bool kPF>
__device__ __forceinline__ void sm_pv_slot(f32x4 (&oacc)[16], const f32x4* sx_mine, const f32x4* sx_partner,
                                           const char* Kb, const TileOffsets& to, float& m_run, float& l_lane,
                                           const uint32_t* mrow, int g, int n, int lane, int t0, int P,
                                           int kv_hi, int rh) {
    constexpr int NE = kHv ? 4 : 8;   // scores per lane: cache rows 16 (e >> 2) + 4g + (e & 3), or 16 rh + 4g + e
    // value operands of step e (cache row vr(e), this wave's 256 dims); read one
    // step ahead of their MFMAs, the first step's before the softmax arithmetic
    auto vread = [&](int e, f32x4 (&v)[4]) {
#pragma unroll
        for (int T = 0; T < 4; ++T)
            v[T] = lds16(Kb, to.voff[e & 3] + (kHv ? rh : (e >> 2)) * 32768 + 256 * (4 * HALF + T));
    };
    f32x4 vf[4];
    float sv[8];
    {
        const f32x4 a0 = sx_mine[lane] + sx_partner[lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = a0[e];
        if constexpr (!kHv) {
            const f32x4 a1 = sx_mine[64 + lane] + sx_partner[64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[4 + e] = a1[e];
        }
    }
    vread(0, vf);
    if constexpr (kPF) __builtin_amdgcn_sched_barrier(0);   // (the scheduler would sink the reads to their MFMAs)
    const bool full = (t0 + kTile <= P) && (t0 + kTile <= kv_hi);
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        float x = sv[e];
        if (!full) {
            const int j = t0 + (kHv ? rh : (e >> 2)) * 16 + 4 * g + (e & 3);
            bool vis = j < kv_hi;
            if (vis && j >= P) vis = (mrow[(j - P) >> 5] >> ((j - P) & 31)) & 1u;
            x = vis ? x : -INFINITY;
        }
        sv[e] = x;
        tmax = fmaxf(tmax, x);
    }
    tmax = row_max4(tmax);
    const bool raise = tmax > m_run + 8.f;
    if (__any(raise)) {
        const float m_new = raise ? tmax : m_run;
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_lane *= alpha;
        float aj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, 4 * g + j, 64);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            oacc[c][0] *= aj[0];
            oacc[c][1] *= aj[1];
            oacc[c][2] *= aj[2];
            oacc[c][3] *= aj[3];
        }
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        sv[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
        l_lane += sv[e];
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const float pv = sv[e];
        f32x4 vn[4];
        if (e + 1 < NE) vread(e + 1, vn);
        if constexpr (kPF) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            oacc[4 * T + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, vf[T][0], oacc[4 * T + 0], 0, 0, 0);
            oacc[4 * T + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, vf[T][1], oacc[4 * T + 1], 0, 0, 0);
            oacc[4 * T + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, vf[T][2], oacc[4 * T + 2], 0, 0, 0);
            oacc[4 * T + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, vf[T][3], oacc[4 * T + 3], 0, 0, 0);
        }
        if (e + 1 < NE) {
#pragma unroll
            for (int T = 0; T < 4; ++T) vf[T] = vn[T];
        }
    }
}

// Barrier at the score swap.  With tile loads in flight it waits for LDS work
// only, so the loads stay in flight across it (__syncthreads would first wait for
// them, and P.V would start only after the next tile had landed).  Narrow caches
// in the usual mode keep __syncthreads.
template <bool kLdsOnly>
__device__ __forceinline__ void swap_barrier() {
    if constexpr (kLdsOnly)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        __syncthreads();
}

// Row-half mode: pairs 2k and 2k + 1 hold the same 16 query rows, each with its
// own online softmax over one half of every tile.  Pair 2k + 1 hands its running
// max, sums and weighted sums to pair 2k through LDS (the tile buffers are free
// once every wave has left the loop), and pair 2k folds them into its own with
// the log-sum-exp combination the split merge uses.  So a split leaves one
// partial, and a batch row with a single split gets its output here.
template <int HALF>
__device__ __forceinline__ void combine_halves(Smem& sm, f32x4 (&oacc)[16], float& m_run, float& l_lane, int wave,
                                               int lane) {
    const int pair = wave >> 1, slot = (pair >> 1) * 2 + HALF, rh = pair & 1;
    f32x4* xo = &sm.kv[0][0] + slot * 16 * 64;                           // 16 KiB per slot
    float2* xml = reinterpret_cast<float2*>(&sm.kv[1][0]) + slot * 64;
    __syncthreads();   // every wave is done with the tile buffers
    if (rh) {
#pragma unroll
        for (int c = 0; c < 16; ++c) xo[c * 64 + lane] = oacc[c];
        xml[lane] = make_float2(m_run, l_lane);
    }
    __syncthreads();
    if (!rh) {
        // lane (g, n): statistics of row n; accumulators of rows 4g + j
        const float2 pm = xml[lane];
        const float M = fmaxf(m_run, pm.x);
        const float a0 = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);   // an empty half weighs 0
        const float a1 = (pm.x == -INFINITY) ? 0.f : exp2f(pm.x - M);
        l_lane = a0 * l_lane + a1 * pm.y;
        m_run = M;
        const int g = lane >> 4;
        float w0[4], w1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w0[j] = __shfl(a0, 4 * g + j, 64);
            w1[j] = __shfl(a1, 4 * g + j, 64);
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const f32x4 x = xo[c * 64 + lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) oacc[c][j] = w0[j] * oacc[c][j] + w1[j] * x[j];
        }
    }
}

// One workgroup's work; HALF is the wave's half of the pair (wave-uniform);
// kHv selects row-half mode.
template <int KV, int HALF, bool kHv, bool kHalfLast>
__device__ __forceinline__ void attn_body(const AttnArgs& a, Smem& sm, int b, int s, int rt, int wave,
                                          int lane) {
    const int tid = wave * 64 + lane;
    const int g = lane >> 4;     // lane group
    const int n = lane & 15;     // query row (score layout) within the pair's 16
    const int pair = wave >> 1;
    constexpr int kRowsWG = kHv ? 32 : kRows;      // query rows per workgroup
    const int rgrp = kHv ? (pair >> 1) : pair;     // the pair's 16-row group
    const int rh = kHv ? (pair & 1) : 0;           // row-half mode: the pair's half of each tile

    const ddtv_row rowd = a.rows[b];
    const int kv_len = rowd.kv_len, P = rowd.prefix;
    // (row-half mode: the last split takes the remainder a.absorb allows; the usual
    // mode's plans set no remainder)
    const int n_b = kHv ? splits_of(kv_len, a.split_len, a.absorb) : (kv_len + a.split_len - 1) / a.split_len;
    const int kv_lo = s * a.split_len;
    const int kv_hi = kHv ? (s == n_b - 1 ? kv_len : kv_lo + a.split_len) : min(kv_len, kv_lo + a.split_len);
    const int ntiles = (kv_hi - kv_lo + kTile - 1) / kTile;
    const int64_t kv_base = rowd.kv_off;

    NarrowStage stage;
    if (KV == DDTV_F32)
        issue_tile_f32(sm.kv[0], a, kv_base, kv_lo, kv_len - 1, wave, lane);
    else
        load_tile_narrow<KV>(stage, a, kv_base, kv_lo, kv_len - 1, tid);

    // Query half: register t holds dims 16(18*HALF + t) + 4g .. +3 of row n (this
    // permutation of the contraction index matches the cache-operand reads),
    // pre-multiplied by scale*log2(e) so the scores come out in exp2 units.
    const int myrow = rt * kRowsWG + rgrp * 16 + n;
    const bool row_ok = myrow < a.R;
    // The 18 loads are unconditional (a row past the end reads row 0 and scales it
    // by 0), so they issue back to back under one wait; a per-load row test made
    // the compiler branch around each load and wait for it in turn.
    f32x4 qreg[18];
    {
        const int64_t qrow = (int64_t)b * a.R + (row_ok ? myrow : 0);
        const f32x4* qa = reinterpret_cast<const f32x4*>(a.q_abs) + qrow * 128;
        const f32x4* qr = reinterpret_cast<const f32x4*>(a.q_rope) + qrow * 16;
        const float sc = row_ok ? a.scale_log2 : 0.f;
#pragma unroll
        for (int t = 0; t < 18; ++t) {
            const int tg = 18 * HALF + t;
            const f32x4 v = (tg < 32) ? qa[4 * tg + g] : qr[4 * (tg - 32) + g];
            qreg[t] = v * sc;
        }
    }
    // mask words of this row's node (read only in the tiles that reach the tree)
    const uint32_t* mrow = a.bits + ((int64_t)b * a.Q + (row_ok ? myrow / a.H : 0)) * a.W;
    f32x4 oacc[16];   // output dims 256*HALF + 64T' + 4n + (c & 3) for block c = 4T' + (c & 3)
#pragma unroll
    for (int c = 0; c < 16; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max of row n (exp2 units)
    float l_lane = 0.f;        // this lane's share of the running sum of row n

    if (KV != DDTV_F32) store_tile_narrow<KV>(sm.kv[0], stage, tid);

    const TileOffsets to = tile_offsets(g, n);
    f32x4* sx_mine = &sm.sx[wave][0][0];
    const f32x4* sx_partner = &sm.sx[wave ^ 1][0][0];
    // Row-half mode with at most 16 query rows: waves 4..7 are idle, and on fp32
    // caches they issue every tile load (their own rows and those of waves 0..3)
    // right after the loop-top barrier, so the computing waves issue none.
    const bool helpers = KV == DDTV_F32 && kHv && a.R <= 16;
    // Usual mode, fp32 cache: each SIMD holds waves w and w + 4, and the older
    // waves 0..3 finish their scores thousands of cycles before 4..7, then wait at
    // the score swap.  They issue the whole next tile there (their rows and those
    // of waves 4..7), so the waves on the critical path issue no loads.
    constexpr bool early_issue = KV == DDTV_F32 && !kHv;
    // A pair whose 16 rows all lie beyond the batch row's H*Q query rows (small
    // trees, few heads) only loads its share of the tiles and meets the barriers:
    // its matrix work would be discarded, and skipping it frees the SIMDs for the
    // pairs with rows.  (A separate loop, so the main loop's code is unchanged.)
    if (rt * kRowsWG + rgrp * 16 >= a.R) {
        for (int it = 0; it < ntiles; ++it) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const bool more = it + 1 < ntiles;
            if (more) {
                if (KV == DDTV_F32) {
                    f32x4* nb = sm.kv[(it + 1) & 1];
                    const int t1 = kv_lo + (it + 1) * kTile;
                    if (helpers) issue_tile_f32(nb, a, kv_base, t1, kv_len - 1, wave - 4, lane);
                    issue_tile_f32(nb, a, kv_base, t1, kv_len - 1, wave, lane);
                } else
                    load_tile_narrow<KV>(stage, a, kv_base, kv_lo + (it + 1) * kTile, kv_len - 1, tid);
            }
            swap_barrier<kHv>();
            if (KV != DDTV_F32 && more) store_tile_narrow<KV>(sm.kv[(it + 1) & 1], stage, tid);
        }
        if constexpr (kHv) combine_halves<HALF>(sm, oacc, m_run, l_lane, wave, lane);   // (its barriers)
        return;   // no rows to write
    }
    // kHalfLast: a last tile with at most 16 rows (a split that ends mid-tile, or
    // a short end of the cache) runs as half a tile -- one score block and half of
    // P.V; the other half would only add zeros.  (Its own instantiation, so the
    // loop of the other kernels is compiled exactly as before.)
    const int t_last = kv_lo + (ntiles - 1) * kTile;
    const int nloop = (kHalfLast && kv_hi - t_last <= kTile / 2) ? ntiles - 1 : ntiles;
    for (int it = 0; it < nloop; ++it) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                                  // tile `it` is in LDS
        const bool more = it + 1 < ntiles;
        auto issue = [&]() {
            if (more && !helpers && !early_issue) {
                if (KV == DDTV_F32)
                    issue_tile_f32(sm.kv[(it + 1) & 1], a, kv_base, kv_lo + (it + 1) * kTile, kv_len - 1, wave, lane);
                else
                    load_tile_narrow<KV>(stage, a, kv_base, kv_lo + (it + 1) * kTile, kv_len - 1, tid);
            }
        };
        const char* Kb = reinterpret_cast<const char*>(sm.kv[it & 1]);
        qk_slot<HALF, kHv>(Kb, to, qreg, sx_mine, lane, issue, rh);
        if (early_issue && more && wave < 4) {
            f32x4* nb = sm.kv[(it + 1) & 1];
            const int t1 = kv_lo + (it + 1) * kTile;
            issue_tile_f32(nb, a, kv_base, t1, kv_len - 1, wave, lane);
            issue_tile_f32(nb, a, kv_base, t1, kv_len - 1, wave + 4, lane);
        }
        // Narrow caches: the next tile goes into its buffer (free since the loop-top
        // barrier) before the score swap, where the waves that finish their scores
        // first would otherwise wait for the others.
        if (KV != DDTV_F32 && more) store_tile_narrow<KV>(sm.kv[(it + 1) & 1], stage, tid);
        swap_barrier<kHv || early_issue>();               // partner's partial scores are in LDS
        sm_pv_slot<HALF, kHv, KV != DDTV_BF16>(oacc, sx_mine, sx_partner, Kb, to, m_run, l_lane, mrow, g, n, lane, kv_lo + it * kTile,
                              P, kv_hi, rh);
    }
    if constexpr (kHalfLast) {
        if (nloop < ntiles) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();                              // the last tile is in LDS
            const char* Kb = reinterpret_cast<const char*>(sm.kv[nloop & 1]);
            qk_slot<HALF, true>(Kb, to, qreg, sx_mine, lane, [] {}, 0);
            swap_barrier<early_issue>();
            sm_pv_slot<HALF, true, KV != DDTV_BF16>(oacc, sx_mine, sx_partner, Kb, to, m_run, l_lane, mrow, g, n,
                                                    lane, t_last, P, kv_hi, 0);
        }
    }

    if constexpr (kHv) {
        combine_halves<HALF>(sm, oacc, m_run, l_lane, wave, lane);
        if (rh) return;   // pair 2k writes the combined rows
    }

    // ---- epilogue: output rows pair*16 + 4g + j of the tile, dims 256*HALF + 64T + 4n + (0..3)
    float l_row = l_lane + wave_xor(l_lane, 16);
    l_row += wave_xor(l_row, 32);
    const float kLn2 = 0.69314718055994530942f;
    const int orow_base = rt * kRowsWG + rgrp * 16 + 4 * g;
    if (n_b == 1) {
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float ij = __shfl(inv, 4 * g + j, 64);
            const int orow = orow_base + j;
            if (orow < a.R) {
                f32x4* dst = reinterpret_cast<f32x4*>(a.out) + ((int64_t)b * a.R + orow) * 128 + 64 * HALF;
#pragma unroll
                for (int T = 0; T < 4; ++T)
                    dst[16 * T + n] = f32x4{oacc[4 * T + 0][j] * ij, oacc[4 * T + 1][j] * ij,
                                            oacc[4 * T + 2][j] * ij, oacc[4 * T + 3][j] * ij};
            }
        }
        if (HALF == 0 && a.lse && g == 0 && row_ok)
            a.lse[(int64_t)b * a.R + myrow] = l_row > 0.f ? (m_run + log2f(l_row)) * kLn2 : -INFINITY;
    } else {
        // partial entry of this split
        const int64_t pbase = ((int64_t)b * a.n_split + s) * a.R;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int orow = orow_base + j;
            if (orow < a.R) {
                f32x4* dst = reinterpret_cast<f32x4*>(a.part_o) + (pbase + orow) * 128 + 64 * HALF;
#pragma unroll
                for (int T = 0; T < 4; ++T)
                    dst[16 * T + n] = f32x4{oacc[4 * T + 0][j], oacc[4 * T + 1][j], oacc[4 * T + 2][j],
                                            oacc[4 * T + 3][j]};
            }
        }
        if (HALF == 0 && g == 0 && row_ok) a.part_ml[pbase + myrow] = make_float2(m_run, l_row);
    }
}

// kHv: row-half mode (its own kernel, so the code of the usual mode is unchanged).
template <int KV, bool kHv, bool kHalfLast>
__global__ __launch_bounds__(kThreads, 1) void attn_mfma_kernel(AttnArgs a) {
    __shared__ Smem sm;
    const int64_t w = work_item(a);
    const int rt = (int)(w % a.n_rt);
    const int s = (int)((w / a.n_rt) % a.n_split);
    const int b = batch_row(a, (int)(w / ((int64_t)a.n_rt * a.n_split)));
    const int kv_len = a.rows[b].kv_len;
    if (kHv ? s >= splits_of(kv_len, a.split_len, a.absorb) : s * a.split_len >= kv_len)
        return;   // this batch row needs fewer splits
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wave & 1)
        attn_body<KV, 1, kHv, kHalfLast>(a, sm, b, s, rt, wave, lane);
    else
        attn_body<KV, 0, kHv, kHalfLast>(a, sm, b, s, rt, wave, lane);
}

template <int KV>
void launch_kv(const AttnArgs& a, int64_t grid, hipStream_t stream) {
    if (a.halves)
        hipLaunchKernelGGL((attn_mfma_kernel<KV, true, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else if (KV == DDTV_F32 && a.split_len % kTile != 0)   // splits end mid-tile: half last tiles
        hipLaunchKernelGGL((attn_mfma_kernel<KV, false, KV == DDTV_F32>), dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((attn_mfma_kernel<KV, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
}

}  // namespace

int mfma_rows_per_workgroup(int /*kv_dtype*/) { return kRows; }

hipError_t launch_attn_mfma(const AttnArgs& a, int kv_dtype, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    if (kv_dtype == DDTV_BF16)
        launch_kv<DDTV_BF16>(a, grid, stream);
    else if (kv_dtype == DDTV_FP8_E4M3)
        launch_kv<DDTV_FP8_E4M3>(a, grid, stream);
    else
        launch_kv<DDTV_F32>(a, grid, stream);
    return hipGetLastError();
}

}  // namespace ddtv
