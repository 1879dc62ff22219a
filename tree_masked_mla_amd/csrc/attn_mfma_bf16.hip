// S2..S6 for bf16 caches on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulate) -- the dense-tree path when the latent cache is bf16.
//
// Same definition as the other attention kernels (score = scale * (absorbed query
// . latent + rope query . rope key), softmax over visible positions, weighted
// latent sum -- "The Verify-Attn Kernel: A Single File Write ...", section "The
// Design Journey: From Concept to CUDA").  Arithmetic: the cache is used as
// stored (bf16); the query, pre-multiplied by scale*log2(e), is rounded to bf16
// once when it is loaded; the probabilities are rounded to bf16 before the
// weighted sum; every product is accumulated in fp32 and the softmax statistics
// are fp32.
//
// Organisation (the launched geometry: 8 waves = 4 wave pairs, 64 query rows per
// workgroup, one workgroup per CU):
//  * A wave pair owns 16 query rows of one batch row and KV split.  For the scores
//    the pair splits the 576-long contraction (wave h keeps query dims 288h ..
//    288h+287 of its rows in 36 VGPRs as bf16) and swaps partial sums through LDS;
//    for P.V it splits the 512 output dims (wave h accumulates dims 256h ..
//    256h+255).  No MFMA is duplicated; 196 VGPRs, two waves per SIMD.  The
//    template also builds 32 rows per pair (RB = 2: every cache fragment read from
//    LDS feeds two MFMAs), which needs one wave per SIMD and ran slower.
//  * Scores are produced transposed, S^T = K Q^T: A = 16 cache rows x 32 dims read
//    from LDS (16 bytes per lane), B = the query fragment in VGPRs.  Each lane then
//    holds the scores of ONE query row for 8 cache positions -- the A-operand
//    layout of P.V -- so the probabilities never move between lanes.
//  * P.V needs, per lane, 8 consecutive cache positions of one latent dim: the
//    transpose read ds_read_b64_tr_b16 delivers exactly that from the row-major
//    tile (lane l reads row l>>2, dims 4(l&3)..+3 of a 16-dim block; inside each
//    16-lane group lane i receives element i&3 of the words read by lanes
//    4e + (i>>2)), so the tile is stored once.
//  * LDS: latent rows of 1024 B and rope rows of 128 B, XOR-swizzled in 32-byte
//    units so both the score reads and the transpose reads spread over the banks.
//    Every per-lane LDS offset is computed once; inside the loop only the tile
//    base changes, and block / dim selection folds into instruction offsets.
//  * Tiles arrive with global_load_lds_dwordx4 into a ring of 4 buffers (144 KiB),
//    3 tiles ahead.  Barriers are raw s_barrier with only the waits they need (the
//    loop-top one waits for the oldest tile alone, the score-swap one for LDS
//    only), so prefetches stay in flight across them.
//  * Row maxima cross lanes with v_permlane32_swap / v_permlane16_swap (no LDS).
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kLatChunks = kTile * 64;               // 16-byte chunks of the latent region (32 KiB)
constexpr int kTileChunks = kLatChunks + kTile * 8;  // + rope region (4 KiB)

// Kernel geometry.  RB: 16-row blocks per wave pair; WAVES: waves per workgroup
// (pairs); RING: tile buffers.  The configuration the library launches is below.
template <int RB, int WAVES, int RING>
struct Geo {
    static constexpr int kThreads = WAVES * 64;
    static constexpr int kRows = (WAVES / 2) * 16 * RB;     // query rows per workgroup
    static constexpr int kLatRows = kTile / WAVES;          // latent rows loaded per wave per tile
    static constexpr int kRopeLanes = kTile * 8 / WAVES;    // rope chunks loaded per wave per tile
    static constexpr int kLoadsPerTile = kLatRows + 1;      // global_load_lds per wave per tile
    static_assert(kRopeLanes <= 64 && kRopeLanes % 8 == 0, "one rope instruction per wave");
};

#ifndef DDTV_BF16_RB
#define DDTV_BF16_RB 1
#endif
#ifndef DDTV_BF16_WAVES
#define DDTV_BF16_WAVES 8
#endif
#ifndef DDTV_BF16_RING
#define DDTV_BF16_RING 4
#endif
using GeoL = Geo<DDTV_BF16_RB, DDTV_BF16_WAVES, DDTV_BF16_RING>;

template <int RB, int WAVES, int RING>
struct Smem {
    f32x4 kv[RING][kTileChunks];    // ring of cache tiles (36 KiB each)
    f32x4 sx[WAVES][2 * RB][64];    // partial scores swapped inside a wave pair
};

// Barrier after this wave's LDS writes have landed; vector-memory loads (tile
// prefetches) stay in flight.  The asm's memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier once this wave has at most N vector-memory loads outstanding (loads
// retire in order, so every older tile has landed).
template <int N>
__device__ __forceinline__ void vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Transpose read of 8 bytes per lane (ds_read_b64_tr_b16) at LDS byte address
// addr + OFF.  Issued as inline asm: the builtin form makes the compiler wait for
// every in-flight LDS DMA (the tile prefetches) before each transpose read.  The
// result is NOT ready when this returns -- see lgkm_wait_tied.
template <int OFF>
__device__ __forceinline__ void tr_read(s16x4& r, uint32_t addr) {
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
}

// Wait until at most N LDS operations of this wave are outstanding; the eight
// values are tied through the asm so nothing reads them before the wait.  (The
// loop issues no scalar-memory loads, so the LDS counter is in program order.)
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(s16x4 (&v)[8]) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "n"(N));
}

// Transpose reads for four 16-dim blocks (first block C of this half): rows
// 4g..4g+3 (v[2i]) and 16+4g..16+4g+3 (v[2i+1]) of latent dims 16(16*HALF+C+i) + n.
template <int HALF, int C>
__device__ __forceinline__ void tr_batch(s16x4 (&v)[8], const uint32_t (&va)[8]) {
    constexpr int c0 = 16 * HALF + C, c1 = c0 + 1, c2 = c0 + 2, c3 = c0 + 3;
    tr_read<256 * (c0 >> 3)>(v[0], va[c0 & 7]);
    tr_read<256 * (c0 >> 3) + 16384>(v[1], va[c0 & 7]);
    tr_read<256 * (c1 >> 3)>(v[2], va[c1 & 7]);
    tr_read<256 * (c1 >> 3) + 16384>(v[3], va[c1 & 7]);
    tr_read<256 * (c2 >> 3)>(v[4], va[c2 & 7]);
    tr_read<256 * (c2 >> 3) + 16384>(v[5], va[c2 & 7]);
    tr_read<256 * (c3 >> 3)>(v[6], va[c3 & 7]);
    tr_read<256 * (c3 >> 3) + 16384>(v[7], va[c3 & 7]);
}

__device__ __forceinline__ bf16x8 cat8(s16x4 lo, s16x4 hi) {
    const bf16x4 b0 = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 b1 = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
}

// four 16-dim blocks (first C) for every row block: each value fragment feeds RB MFMAs
template <int C, int RB>
__device__ __forceinline__ void pv_batch(f32x4 (&oacc)[RB][16], const bf16x8 (&pa)[RB], const s16x4 (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x8 vb = cat8(v[2 * i], v[2 * i + 1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            oacc[rb][C + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[rb], vb, oacc[rb][C + i], 0, 0, 0);
    }
}

// max over the 4 lanes holding one query row (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float row_max4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(x, fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(x, fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])));
}

template <class G>
__device__ __forceinline__ void issue_tile(f32x4* buf, const AttnArgs& a, int64_t kv_base, int t0, int kv_last,
                                           int wave, int lane) {
    const char* ck = reinterpret_cast<const char*>(a.ckv);
    const char* kr = reinterpret_cast<const char*>(a.k_rope);
#pragma unroll
    for (int k = 0; k < G::kLatRows; ++k) {       // latent: one 1 KiB row per instruction
        const int r = wave * G::kLatRows + k;
        const int64_t row = kv_base + min(t0 + r, kv_last);
        const int c = (((lane >> 1) ^ (r & 7)) << 1) + (lane & 1);   // logical chunk stored at `lane`
        __builtin_amdgcn_global_load_lds(ck + row * 1024 + c * 16, (lds_void*)(buf + r * 64), 16, 0, 0);
    }
    {                                             // rope: kRopeLanes / 8 rows of 128 B
        const int slot = wave * G::kRopeLanes + min(lane, G::kRopeLanes - 1);
        const int r = slot >> 3, p = slot & 7;
        const int64_t row = kv_base + min(t0 + r, kv_last);
        const int c = (((p >> 1) ^ ((r >> 1) & 3)) << 1) + (p & 1);
        if (lane < G::kRopeLanes)
            __builtin_amdgcn_global_load_lds(kr + row * 128 + c * 16,
                                             (lds_void*)(buf + kLatChunks + wave * G::kRopeLanes), 16, 0, 0);
    }
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 a, f32x4 b, float s) {
    bf16x8 r;
    r[0] = (__bf16)(a[0] * s); r[1] = (__bf16)(a[1] * s); r[2] = (__bf16)(a[2] * s); r[3] = (__bf16)(a[3] * s);
    r[4] = (__bf16)(b[0] * s); r[5] = (__bf16)(b[1] * s); r[6] = (__bf16)(b[2] * s); r[7] = (__bf16)(b[3] * s);
    return r;
}

template <int RB, int WAVES, int RING, int HALF>
__device__ __forceinline__ void attn_body(const AttnArgs& a, Smem<RB, WAVES, RING>& sm, int b, int s, int rt, int wave,
                                          int lane) {
    using G = Geo<RB, WAVES, RING>;
    constexpr int kRows = G::kRows;
    constexpr int kRing = RING;
    constexpr int kLoadsPerTile = G::kLoadsPerTile;
    const int g = lane >> 4;
    const int n = lane & 15;
    const int pair = wave >> 1;
    const ddtv_row rowd = a.rows[b];
    const int kv_len = rowd.kv_len, P = rowd.prefix;
    const int kv_lo = s * a.split_len;
    const int n_b = (kv_len + a.split_len - 1) / a.split_len;
    const int kv_hi = min(kv_len, kv_lo + a.split_len);
    const int ntiles = (kv_hi - kv_lo + kTile - 1) / kTile;
    const int64_t kv_base = rowd.kv_off;

    // query fragment (rb, t) of this half: dims 32(9*HALF + t) + 8g .. +7 of row
    // 16 rb + n of the pair, times scale*log2(e), as bf16
    const int row0 = rt * kRows + pair * 16 * RB + n;   // row of block rb: row0 + 16 rb
    bf16x8 qreg[RB][9];
    const uint32_t* mrow[RB];   // mask words of each row's node (read only in tiles that reach the tree)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int myrow = row0 + 16 * rb;
        const bool row_ok = myrow < a.R;
        const int64_t qrow = (int64_t)b * a.R + (row_ok ? myrow : 0);
        const f32x4* qa = reinterpret_cast<const f32x4*>(a.q_abs) + qrow * 128;
        const f32x4* qr = reinterpret_cast<const f32x4*>(a.q_rope) + qrow * 16;
        const float sc = row_ok ? a.scale_log2 : 0.f;
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int tg = 9 * HALF + t;
            const f32x4* src = (tg < 16) ? qa + 8 * tg + 2 * g : qr + 8 * (tg - 16) + 2 * g;
            qreg[rb][t] = to_bf16x8(src[0], src[1], sc);
        }
        mrow[rb] = a.bits + ((int64_t)b * a.Q + (row_ok ? myrow / a.H : 0)) * a.W;
    }

    // Per-lane byte offsets inside a tile buffer.
    //  score operand, cache row n, latent fragment tg = 4q + m: koff[m] + 256 q  (row 16+n: +16 KiB)
    //  score operand, cache row n, rope fragment 16 + m:         roff[m]          (row 16+n: +2 KiB)
    //  transpose read, rows (lane>>2) and 16+(lane>>2), dims of block c: toff[c & 7] + 256 (c >> 3) (+16 KiB)
    int koff[4], roff[2], toff[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) koff[m] = n * 1024 + ((((2 * m + (g >> 1)) ^ (n & 7)) << 1) + (g & 1)) * 16;
#pragma unroll
    for (int m = 0; m < 2; ++m)
        roff[m] = (kLatChunks + n * 8 + ((((2 * m + (g >> 1)) ^ ((n >> 1) & 3)) << 1) + (g & 1))) * 16;
    {
        const int vr = lane >> 2;
#pragma unroll
        for (int k = 0; k < 8; ++k) toff[k] = (vr * 64 + ((k ^ (vr & 7)) << 1)) * 16 + 8 * (lane & 3);
    }

    // all query loads were consumed above; from here the only vector-memory loads
    // in flight are tile prefetches (and mask words in tail tiles, which drain)
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k)
        if (k < ntiles) issue_tile<G>(sm.kv[k], a, kv_base, kv_lo + k * kTile, kv_len - 1, wave, lane);

    f32x4 oacc[RB][16];   // [rb][c]: output rows 16 rb + 4g + j, latent dim 16(16*HALF + c) + n
    float m_run[RB], l_lane[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int c = 0; c < 16; ++c) oacc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[rb] = -INFINITY;
        l_lane[rb] = 0.f;
    }

    for (int it = 0; it < ntiles; ++it) {
        const int t0 = kv_lo + it * kTile;
        // tile `it` must have landed (for every wave); up to 2 newer tiles may be in flight
        const int ahead = min(kRing - 2, ntiles - 1 - it);
        if (kRing >= 4 && ahead >= 2)
            vm_barrier<2 * kLoadsPerTile>();
        else if (kRing >= 3 && ahead >= 1)
            vm_barrier<kLoadsPerTile>();
        else
            vm_barrier<0>();
        // every wave is past tile it-1, so its buffer can be refilled
        if (it + kRing - 1 < ntiles)
            issue_tile<G>(sm.kv[(it + kRing - 1) % kRing], a, kv_base, t0 + (kRing - 1) * kTile, kv_len - 1, wave,
                          lane);
        const char* Kb = reinterpret_cast<const char*>(sm.kv[it % kRing]);

        // ---- partial S^T: cache blocks (rows n, 16 + n) x row blocks, over this half
        f32x4 sa[RB][2];   // [rb][kv block]
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sa[rb][0] = sa[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int tg = 9 * HALF + t;
            const char* p0 = (tg < 16) ? Kb + koff[tg & 3] + 256 * (tg >> 2) : Kb + roff[tg - 16];
            const bf16x8 k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const f32x4*>(p0));
            const bf16x8 k1 =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const f32x4*>(p0 + (tg < 16 ? 16384 : 2048)));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                sa[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[rb][t], sa[rb][0], 0, 0, 0);
                sa[rb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qreg[rb][t], sa[rb][1], 0, 0, 0);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            sm.sx[wave][2 * rb][lane] = sa[rb][0];
            sm.sx[wave][2 * rb + 1][lane] = sa[rb][1];
        }
        lds_barrier();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            sa[rb][0] += sm.sx[wave ^ 1][2 * rb][lane];
            sa[rb][1] += sm.sx[wave ^ 1][2 * rb + 1][lane];
        }

        // ---- online softmax (log2 units); lane holds row 16 rb + n, cache rows (e>>2)*16 + 4g + (e&3)
        const bool full = (t0 + kTile <= P) && (t0 + kTile <= kv_hi);
        bf16x8 pa[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float sv[8] = {sa[rb][0][0], sa[rb][0][1], sa[rb][0][2], sa[rb][0][3],
                           sa[rb][1][0], sa[rb][1][1], sa[rb][1][2], sa[rb][1][3]};
            if (!full) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = t0 + (e >> 2) * 16 + 4 * g + (e & 3);
                    bool vis = j < kv_hi;
                    if (vis && j >= P) vis = (mrow[rb][(j - P) >> 5] >> ((j - P) & 31)) & 1u;
                    sv[e] = vis ? sv[e] : -INFINITY;
                }
            }
            float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                               fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            tmax = row_max4(tmax);
            const bool raise = tmax > m_run[rb] + 8.f;
            if (__any(raise)) {
                const float m_new = raise ? tmax : m_run[rb];
                const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
                m_run[rb] = m_new;
                l_lane[rb] *= alpha;
                float aj[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, 4 * g + j, 64);
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    oacc[rb][c][0] *= aj[0];
                    oacc[rb][c][1] *= aj[1];
                    oacc[rb][c][2] *= aj[2];
                    oacc[rb][c][3] *= aj[3];
                }
            }
            const float m_use = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(sv[e] - m_use);
                l_lane[rb] += p;
                pa[rb][e] = (__bf16)p;
            }
        }

        // ---- O += P V over this half's 16 blocks of 16 latent dims: two transpose
        //      reads per block (cache rows 4g .. 4g+3 and 16+4g .. 16+4g+3 of dim
        //      16c' + n) feed both row blocks.  Four blocks per batch, one batch
        //      ahead of the MFMAs.
        {
            const uint32_t kb = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)Kb;
            uint32_t va[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) va[k] = kb + toff[k];
            s16x4 v0[8], v1[8];
            tr_batch<HALF, 0>(v0, va);
            tr_batch<HALF, 4>(v1, va);
            lgkm_wait_tied<8>(v0);
            pv_batch<0, RB>(oacc, pa, v0);
            tr_batch<HALF, 8>(v0, va);
            lgkm_wait_tied<8>(v1);
            pv_batch<4, RB>(oacc, pa, v1);
            tr_batch<HALF, 12>(v1, va);
            lgkm_wait_tied<8>(v0);
            pv_batch<8, RB>(oacc, pa, v0);
            lgkm_wait_tied<0>(v1);
            pv_batch<12, RB>(oacc, pa, v1);
        }
    }

    // ---- epilogue: lane holds rows 16 rb + 4g + j, latent dims 256*HALF + 16c + n
    const float kLn2 = 0.69314718055994530942f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float l_row = l_lane[rb] + wave_xor(l_lane[rb], 16);
        l_row += wave_xor(l_row, 32);
        const int myrow = row0 + 16 * rb;
        const int orow_base = rt * kRows + pair * 16 * RB + 16 * rb + 4 * g;
        if (n_b == 1) {
            const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ij = __shfl(inv, 4 * g + j, 64);
                const int orow = orow_base + j;
                if (orow < a.R) {
                    float* dst = a.out + ((int64_t)b * a.R + orow) * kDLat + 256 * HALF + n;
#pragma unroll
                    for (int c = 0; c < 16; ++c) dst[16 * c] = oacc[rb][c][j] * ij;
                }
            }
            if (HALF == 0 && a.lse && g == 0 && myrow < a.R)
                a.lse[(int64_t)b * a.R + myrow] = l_row > 0.f ? (m_run[rb] + log2f(l_row)) * kLn2 : -INFINITY;
        } else {
            const int64_t pbase = ((int64_t)b * a.n_split + s) * a.R;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int orow = orow_base + j;
                if (orow < a.R) {
                    float* dst = a.part_o + (pbase + orow) * kDLat + 256 * HALF + n;
#pragma unroll
                    for (int c = 0; c < 16; ++c) dst[16 * c] = oacc[rb][c][j];
                }
            }
            if (HALF == 0 && g == 0 && myrow < a.R) a.part_ml[pbase + myrow] = make_float2(m_run[rb], l_row);
        }
    }
}

template <int RB, int WAVES, int RING>
__global__ __launch_bounds__(WAVES * 64) void attn_mfma_bf16_kernel(AttnArgs a) {
    __shared__ Smem<RB, WAVES, RING> sm;
    const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
    const int rt = (int)(w % a.n_rt);
    const int s = (int)((w / a.n_rt) % a.n_split);
    const int b = (int)(w / ((int64_t)a.n_rt * a.n_split));
    if (s * a.split_len >= a.rows[b].kv_len) return;   // this batch row needs fewer splits
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wave & 1)
        attn_body<RB, WAVES, RING, 1>(a, sm, b, s, rt, wave, lane);
    else
        attn_body<RB, WAVES, RING, 0>(a, sm, b, s, rt, wave, lane);
}

}  // namespace

int bf16_rows_per_workgroup() { return GeoL::kRows; }

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL((attn_mfma_bf16_kernel<DDTV_BF16_RB, DDTV_BF16_WAVES, DDTV_BF16_RING>), dim3((unsigned)grid),
                       dim3(GeoL::kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ddtv
