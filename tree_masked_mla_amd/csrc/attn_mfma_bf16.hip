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
// Organisation: 8 waves = 4 wave pairs, 64 query rows per workgroup, one
// workgroup per CU.
//  * A wave pair owns 16 query rows of one batch row and KV split.  For the scores
//    the pair splits the 576-long contraction (wave h keeps query dims 288h ..
//    288h+287 of its rows in 36 VGPRs as bf16) and swaps partial sums through LDS;
//    for P.V it splits the 512 output dims (wave h accumulates dims 256h ..
//    256h+255).  No MFMA is duplicated.
//  * Scores are produced transposed, S^T = K Q^T: A = 16 cache rows x 32 dims read
//    from LDS (16 bytes per lane), B = the query fragment in VGPRs.  Each lane then
//    holds the scores of ONE query row for 8 cache positions -- the A-operand
//    layout of P.V -- so the probabilities never move between lanes.
//  * P.V needs, per lane, 8 consecutive cache positions of one latent dim: the
//    transpose read ds_read_b64_tr_b16 delivers exactly that from the row-major
//    tile (lane l reads row l>>2, dims 4(l&3)..+3 of a 16-dim block; inside each
//    16-lane group lane i receives element i&3 of the words read by lanes
//    4e + (i>>2)), so the tile is stored once.
//  * Ping-pong schedule.  The loop runs in half-tile slots separated by one
//    workgroup barrier each.  A wave alternates an MFMA slot (P.V of tile t-1, then
//    the partial scores of tile t) and a softmax slot (partner's partial scores,
//    mask, online softmax of tile t).  Waves 0-3 run one slot behind waves 4-7, so
//    each SIMD (which holds one wave of each group) always has one wave feeding the
//    matrix core while the other does its vector work.
//  * Operand reads are issued in batches as inline asm, with waits tied to their
//    results: the compiler's own scheduling waits for each LDS read right before
//    its MFMA, and its builtin transpose read also waits for every in-flight LDS
//    DMA (the tile prefetches).
//  * LDS: latent rows of 1024 B and rope rows of 128 B, XOR-swizzled in 32-byte
//    units so both the score reads and the transpose reads spread over the banks.
//    Tiles arrive with global_load_lds_dwordx4 into a ring of 4 buffers (144 KiB),
//    issued three to four slots before first use, each wave's share in its
//    softmax slot (issuing them costs a few hundred cycles, which an MFMA slot
//    would pay on its critical path); 16 KiB hold the partial scores.
//  * Row maxima cross lanes with v_permlane32_swap / v_permlane16_swap (no LDS).
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = (kWaves / 2) * 16;             // query rows per workgroup
constexpr int kRing = 4;                             // tile buffers
constexpr int kLatChunks = kTile * 64;               // 16-byte chunks of the latent region (32 KiB)
constexpr int kTileChunks = kLatChunks + kTile * 8;  // + rope region (4 KiB)
constexpr int kLatRows = kTile / kWaves;             // latent rows loaded per wave per tile
constexpr int kRopeLanes = kTile * 8 / kWaves;       // rope chunks loaded per wave per tile
constexpr int kLoadsPerTile = kLatRows + 1;          // global_load_lds per wave per tile
static_assert(kRopeLanes <= 64 && kRopeLanes % 8 == 0, "one rope instruction per wave");

#ifndef DDTV_BF16_GROUP_SHIFT
#define DDTV_BF16_GROUP_SHIFT 2   // group = wave >> 2: waves w and w+4 share a SIMD
#endif

struct Smem {
    f32x4 kv[kRing][kTileChunks];   // ring of cache tiles (36 KiB each)
    f32x4 sx[kWaves][2][64];        // partial scores swapped inside a wave pair
};

// End of a slot: this wave's LDS writes have landed, then the workgroup barrier.
// Vector-memory loads (tile prefetches) stay in flight.  The memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void slot_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Same, once this wave has at most N vector-memory loads outstanding (loads retire
// in order, so every older tile has landed).
template <int N>
__device__ __forceinline__ void slot_barrier_vm() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS reads issued as inline asm; the results are NOT ready when these return --
// see the tied waits below.
template <int OFF>
__device__ __forceinline__ void tr_read(s16x4& r, uint32_t addr) {
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void k_read(f32x4& r, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
}

// Wait until at most N LDS operations of this wave are outstanding; the values are
// tied through the asm so nothing reads them before the wait.  (The loop issues no
// scalar-memory loads, so the LDS counter is in program order.)
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(s16x4 (&v)[8]) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(f32x4 (&k)[6]) {
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5])
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

// O += P V for four 16-dim blocks (first C)
template <int C>
__device__ __forceinline__ void pv_batch(f32x4 (&oacc)[16], const bf16x8& pa, const s16x4 (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        oacc[C + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, cat8(v[2 * i], v[2 * i + 1]), oacc[C + i], 0, 0, 0);
}

// Score-operand reads for contraction step TG (TG = 9*HALF + local step): cache
// rows n (k0) and 16+n (k1).  Latent fragment TG < 16 sits at ka[TG & 3] +
// 256 (TG >> 2) (second row block +16 KiB); rope fragment TG >= 16 at
// ka[4 + TG - 16] (second row block +2 KiB).
template <int TG>
__device__ __forceinline__ void k_step(f32x4& k0, f32x4& k1, const uint32_t (&ka)[6]) {
    if constexpr (TG < 16) {
        k_read<256 * (TG >> 2)>(k0, ka[TG & 3]);
        k_read<256 * (TG >> 2) + 16384>(k1, ka[TG & 3]);
    } else {
        k_read<0>(k0, ka[4 + TG - 16]);
        k_read<2048>(k1, ka[4 + TG - 16]);
    }
}
template <int TG>
__device__ __forceinline__ void k_batch(f32x4 (&k)[6], const uint32_t (&ka)[6]) {
    k_step<TG>(k[0], k[1], ka);
    k_step<TG + 1>(k[2], k[3], ka);
    k_step<TG + 2>(k[4], k[5], ka);
}
template <int T>
__device__ __forceinline__ void qk_batch(f32x4 (&sa)[2], const bf16x8 (&q)[9], const f32x4 (&k)[6]) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        sa[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[2 * i]), q[T + i], sa[0], 0, 0, 0);
        sa[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[2 * i + 1]), q[T + i], sa[1], 0, 0, 0);
    }
}

// max over the 4 lanes holding one query row (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float row_max4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(x, fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(x, fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])));
}

// This wave's share of one cache tile: kLatRows latent rows and kRopeLanes rope chunks.
__device__ __forceinline__ void issue_tile(f32x4* buf, const AttnArgs& a, int64_t kv_base, int t0, int kv_last,
                                           int wave, int lane) {
    const char* ck = reinterpret_cast<const char*>(a.ckv);
    const char* kr = reinterpret_cast<const char*>(a.k_rope);
#pragma unroll
    for (int k = 0; k < kLatRows; ++k) {          // latent: one 1 KiB row per instruction
        const int r = wave * kLatRows + k;
        const int64_t row = kv_base + min(t0 + r, kv_last);
        const int c = (((lane >> 1) ^ (r & 7)) << 1) + (lane & 1);   // logical chunk stored at `lane`
        __builtin_amdgcn_global_load_lds(ck + row * 1024 + c * 16, (lds_void*)(buf + r * 64), 16, 0, 0);
    }
    {                                             // rope: kRopeLanes / 8 rows of 128 B
        const int slot = wave * kRopeLanes + min(lane, kRopeLanes - 1);
        const int r = slot >> 3, p = slot & 7;
        const int64_t row = kv_base + min(t0 + r, kv_last);
        const int c = (((p >> 1) ^ ((r >> 1) & 3)) << 1) + (p & 1);
        if (lane < kRopeLanes)
            __builtin_amdgcn_global_load_lds(kr + row * 128 + c * 16,
                                             (lds_void*)(buf + kLatChunks + wave * kRopeLanes), 16, 0, 0);
    }
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 a, f32x4 b, float s) {
    bf16x8 r;
    r[0] = (__bf16)(a[0] * s); r[1] = (__bf16)(a[1] * s); r[2] = (__bf16)(a[2] * s); r[3] = (__bf16)(a[3] * s);
    r[4] = (__bf16)(b[0] * s); r[5] = (__bf16)(b[1] * s); r[6] = (__bf16)(b[2] * s); r[7] = (__bf16)(b[3] * s);
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const f32x4* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) f32x4*)p;
}

// MFMA slot: O += P V of the tile at LDS address kb_pv over this half's 16 blocks
// of 16 latent dims (PV), then the partial S^T of the tile at kb_qk over this half
// of the contraction (QK), stored to this wave's swap area.
template <int HALF, bool PV, bool QK>
__device__ __forceinline__ void mfma_slot(f32x4 (&oacc)[16], f32x4 (&sa)[2], const bf16x8& pa, const bf16x8 (&qreg)[9],
                                          const uint32_t (&toff)[8], const uint32_t (&koff)[6], uint32_t kb_pv,
                                          uint32_t kb_qk, f32x4* sx_mine, int lane) {
    uint32_t ka[6];
    f32x4 k0[6], k1[6];
    if constexpr (QK) {
#pragma unroll
        for (int k = 0; k < 6; ++k) ka[k] = kb_qk + koff[k];
    }
    if constexpr (PV) {
        uint32_t va[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) va[k] = kb_pv + toff[k];
        s16x4 v0[8], v1[8];
        tr_batch<HALF, 0>(v0, va);
        tr_batch<HALF, 4>(v1, va);
        lgkm_wait_tied<8>(v0);
        pv_batch<0>(oacc, pa, v0);
        tr_batch<HALF, 8>(v0, va);
        lgkm_wait_tied<8>(v1);
        pv_batch<4>(oacc, pa, v1);
        tr_batch<HALF, 12>(v1, va);
        lgkm_wait_tied<8>(v0);
        pv_batch<8>(oacc, pa, v0);
        if constexpr (QK) {
            // the first score-operand batch goes out before the last P.V batch
            k_batch<9 * HALF + 0>(k0, ka);          // in flight: v1 (8) + k0 (6)
            lgkm_wait_tied<6>(v1);
            pv_batch<12>(oacc, pa, v1);
        } else {
            lgkm_wait_tied<0>(v1);
            pv_batch<12>(oacc, pa, v1);
        }
    } else if constexpr (QK) {
        k_batch<9 * HALF + 0>(k0, ka);
    }
    if constexpr (QK) {
        sa[0] = sa[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        k_batch<9 * HALF + 3>(k1, ka);
        lgkm_wait_tied<6>(k0);
        qk_batch<0>(sa, qreg, k0);
        k_batch<9 * HALF + 6>(k0, ka);
        lgkm_wait_tied<6>(k1);
        qk_batch<3>(sa, qreg, k1);
        lgkm_wait_tied<0>(k0);
        qk_batch<6>(sa, qreg, k0);
        sx_mine[lane] = sa[0];
        sx_mine[64 + lane] = sa[1];
    }
}

// Softmax slot for the tile starting at cache position t0 (log2 units): add the
// partner's partial scores, mask, online softmax; leaves the probabilities in pa.
// Lane (g, n) holds row n of the pair for cache rows (e>>2)*16 + 4g + (e&3).
__device__ __forceinline__ void softmax_slot(f32x4 (&oacc)[16], f32x4 (&sa)[2], bf16x8& pa, float& m_run,
                                             float& l_lane, const f32x4* sx_partner, int lane, int t0, int P,
                                             int kv_hi, const uint32_t* mrow) {
    const int g = lane >> 4;
    sa[0] += sx_partner[lane];
    sa[1] += sx_partner[64 + lane];
    float sv[8] = {sa[0][0], sa[0][1], sa[0][2], sa[0][3], sa[1][0], sa[1][1], sa[1][2], sa[1][3]};
    const bool full = (t0 + kTile <= P) && (t0 + kTile <= kv_hi);
    if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = t0 + (e >> 2) * 16 + 4 * g + (e & 3);
            bool vis = j < kv_hi;
            if (vis && j >= P) vis = (mrow[(j - P) >> 5] >> ((j - P) & 31)) & 1u;
            sv[e] = vis ? sv[e] : -INFINITY;
        }
    }
    float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
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
    for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(sv[e] - m_use);
        l_lane += p;
        pa[e] = (__bf16)p;
    }
}

template <int HALF>
__device__ __forceinline__ void attn_body(const AttnArgs& a, Smem& sm, int b, int s, int rt, int wave, int lane) {
    const int g = lane >> 4;
    const int n = lane & 15;
    const int pair = wave >> 1;
    const int grp = 1 - ((wave >> DDTV_BF16_GROUP_SHIFT) & 1);   // group 1 runs one slot behind
    const ddtv_row rowd = a.rows[b];
    const int kv_len = rowd.kv_len, P = rowd.prefix;
    const int kv_lo = s * a.split_len;
    const int n_b = (kv_len + a.split_len - 1) / a.split_len;
    const int kv_hi = min(kv_len, kv_lo + a.split_len);
    const int ntiles = (kv_hi - kv_lo + kTile - 1) / kTile;
    const int64_t kv_base = rowd.kv_off;

    // query fragment t of this half: dims 32(9*HALF + t) + 8g .. +7 of row
    // 16 pair + n, times scale*log2(e), as bf16
    const int myrow = rt * kRows + pair * 16 + n;
    const bool row_ok = myrow < a.R;
    bf16x8 qreg[9];
    {
        const int64_t qrow = (int64_t)b * a.R + (row_ok ? myrow : 0);
        const f32x4* qa = reinterpret_cast<const f32x4*>(a.q_abs) + qrow * 128;
        const f32x4* qr = reinterpret_cast<const f32x4*>(a.q_rope) + qrow * 16;
        const float sc = row_ok ? a.scale_log2 : 0.f;
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int tg = 9 * HALF + t;
            const f32x4* src = (tg < 16) ? qa + 8 * tg + 2 * g : qr + 8 * (tg - 16) + 2 * g;
            qreg[t] = to_bf16x8(src[0], src[1], sc);
        }
    }
    // mask words of this row's node (read only in tiles that reach the tree)
    const uint32_t* mrow = a.bits + ((int64_t)b * a.Q + (row_ok ? myrow / a.H : 0)) * a.W;

    // Per-lane byte offsets inside a tile buffer.
    //  score operand, cache row n, latent fragment tg = 4q + m: koff[m] + 256 q  (row 16+n: +16 KiB)
    //  score operand, cache row n, rope fragment 16 + m:         koff[4 + m]      (row 16+n: +2 KiB)
    //  transpose read, rows (lane>>2) and 16+(lane>>2), dims of block c: toff[c & 7] + 256 (c >> 3) (+16 KiB)
    uint32_t koff[6], toff[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) koff[m] = n * 1024 + ((((2 * m + (g >> 1)) ^ (n & 7)) << 1) + (g & 1)) * 16;
#pragma unroll
    for (int m = 0; m < 2; ++m)
        koff[4 + m] = (kLatChunks + n * 8 + ((((2 * m + (g >> 1)) ^ ((n >> 1) & 3)) << 1) + (g & 1))) * 16;
    {
        const int vr = lane >> 2;
#pragma unroll
        for (int k = 0; k < 8; ++k) toff[k] = (vr * 64 + ((k ^ (vr & 7)) << 1)) * 16 + 8 * (lane & 3);
    }
    const uint32_t ring0 = lds_addr(&sm.kv[0][0]);
    constexpr uint32_t kBufBytes = kTileChunks * 16;

    // all query loads were consumed above; from here the only vector-memory loads
    // in flight are tile prefetches (and mask words in tail tiles, which drain)
    if (ntiles > 0) issue_tile(sm.kv[0], a, kv_base, kv_lo, kv_len - 1, wave, lane);
    if (ntiles > 1) issue_tile(sm.kv[1], a, kv_base, kv_lo + kTile, kv_len - 1, wave, lane);
    if (ntiles > 1)
        slot_barrier_vm<kLoadsPerTile>();
    else
        slot_barrier_vm<0>();

    f32x4 oacc[16];   // [c]: output rows 4g + j of the pair, latent dim 16(16*HALF + c) + n
#pragma unroll
    for (int c = 0; c < 16; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;
    f32x4 sa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};   // scores of the current tile
    bf16x8 pa = {};   // probabilities of the previous tile, waiting for its P.V

    f32x4* sx_mine = &sm.sx[wave][0][0];
    const f32x4* sx_partner = &sm.sx[wave ^ 1][0][0];
    auto buf = [&](int t) { return ring0 + (uint32_t)(t & (kRing - 1)) * kBufBytes; };
    // Tile m goes into the buffer of tile m-4, whose last reader (group 1's P.V of
    // tile m-4) ran in slot 2m-5.  Each wave issues its share of a tile during its
    // softmax slot, where the issue cost is hidden behind the other group's MFMAs:
    // group 1 in slot 2m-4, group 0 in slot 2m-3.
    auto issue = [&](int m) {
        if (m < ntiles) issue_tile(sm.kv[m & (kRing - 1)], a, kv_base, kv_lo + m * kTile, kv_len - 1, wave, lane);
    };
    // End of an odd slot 2t-1: tile t must have landed for every wave (group 0
    // scores it in slot 2t); tile t+1 may still be in flight.
    auto end_odd_slot = [&](int t) {
        if (t + 1 < ntiles)
            slot_barrier_vm<kLoadsPerTile>();
        else
            slot_barrier_vm<0>();
    };

    // Slots: group 0 runs "MFMA slot t, softmax slot t" in slots 2t, 2t+1; group 1
    // runs the same one slot later.  The MFMA slot of tile t does the P.V of tile
    // t-1 and the partial scores of tile t; one slot after the last tile, the P.V
    // of the last tile.  Tiles 0 and 1 are issued before the loop.
    if (grp == 0) {
        for (int t = 0; t < ntiles; ++t) {
            if (t == 0)
                mfma_slot<HALF, false, true>(oacc, sa, pa, qreg, toff, koff, 0, buf(t), sx_mine, lane);
            else
                mfma_slot<HALF, true, true>(oacc, sa, pa, qreg, toff, koff, buf(t - 1), buf(t), sx_mine, lane);
            slot_barrier();                                                 // slot 2t
            issue(t + 2);
            softmax_slot(oacc, sa, pa, m_run, l_lane, sx_partner, lane, kv_lo + t * kTile, P, kv_hi, mrow);
            end_odd_slot(t + 1);                                            // slot 2t+1
        }
        mfma_slot<HALF, true, false>(oacc, sa, pa, qreg, toff, koff, buf(ntiles - 1), 0, sx_mine, lane);
        slot_barrier();                                                     // slot 2n
        slot_barrier();                                                     // slot 2n+1 (idle)
    } else {
        issue(2);
        slot_barrier();                                                     // slot 0 (idle)
        for (int t = 0; t < ntiles; ++t) {
            if (t == 0)
                mfma_slot<HALF, false, true>(oacc, sa, pa, qreg, toff, koff, 0, buf(t), sx_mine, lane);
            else
                mfma_slot<HALF, true, true>(oacc, sa, pa, qreg, toff, koff, buf(t - 1), buf(t), sx_mine, lane);
            end_odd_slot(t + 1);                                            // slot 2t+1
            issue(t + 3);
            softmax_slot(oacc, sa, pa, m_run, l_lane, sx_partner, lane, kv_lo + t * kTile, P, kv_hi, mrow);
            slot_barrier();                                                 // slot 2t+2
        }
        mfma_slot<HALF, true, false>(oacc, sa, pa, qreg, toff, koff, buf(ntiles - 1), 0, sx_mine, lane);
        slot_barrier();                                                     // slot 2n+1
    }

    // ---- epilogue: lane holds rows 4g + j of the pair, latent dims 256*HALF + 16c + n
    const float kLn2 = 0.69314718055994530942f;
    float l_row = l_lane + wave_xor(l_lane, 16);
    l_row += wave_xor(l_row, 32);
    const int orow_base = rt * kRows + pair * 16 + 4 * g;
    if (n_b == 1) {
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float ij = __shfl(inv, 4 * g + j, 64);
            const int orow = orow_base + j;
            if (orow < a.R) {
                float* dst = a.out + ((int64_t)b * a.R + orow) * kDLat + 256 * HALF + n;
#pragma unroll
                for (int c = 0; c < 16; ++c) dst[16 * c] = oacc[c][j] * ij;
            }
        }
        if (HALF == 0 && a.lse && g == 0 && row_ok)
            a.lse[(int64_t)b * a.R + myrow] = l_row > 0.f ? (m_run + log2f(l_row)) * kLn2 : -INFINITY;
    } else {
        const int64_t pbase = ((int64_t)b * a.n_split + s) * a.R;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int orow = orow_base + j;
            if (orow < a.R) {
                float* dst = a.part_o + (pbase + orow) * kDLat + 256 * HALF + n;
#pragma unroll
                for (int c = 0; c < 16; ++c) dst[16 * c] = oacc[c][j];
            }
        }
        if (HALF == 0 && g == 0 && row_ok) a.part_ml[pbase + myrow] = make_float2(m_run, l_row);
    }
}

__global__ __launch_bounds__(kThreads) void attn_mfma_bf16_kernel(AttnArgs a) {
    __shared__ Smem sm;
    const int64_t w = work_item(a);
    const int rt = (int)(w % a.n_rt);
    const int s = (int)((w / a.n_rt) % a.n_split);
    const int b = batch_row(a, (int)(w / ((int64_t)a.n_rt * a.n_split)));
    if (s * a.split_len >= a.rows[b].kv_len) return;   // this batch row needs fewer splits
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wave & 1)
        attn_body<1>(a, sm, b, s, rt, wave, lane);
    else
        attn_body<0>(a, sm, b, s, rt, wave, lane);
}

}  // namespace

int bf16_rows_per_workgroup() { return kRows; }

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(attn_mfma_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ddtv
