// S2..S6 for bf16 caches on the bf16 matrix cores with 32 query rows per wave
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Same definition and arithmetic as the other bf16 kernel (score = scale *
// (absorbed query . latent + rope query . rope key), softmax over visible
// positions, weighted latent sum -- "The Verify-Attn Kernel: A Single File
// Write ...", section "The Design Journey: From Concept to CUDA"): the cache is
// used as stored; the query, pre-multiplied by scale*log2(e), is rounded to bf16
// once; the probabilities are rounded to bf16 before the weighted sum; products
// accumulate in fp32 and the softmax statistics are fp32.
//
// Why 32 rows per wave: every MFMA here takes one operand (a 1 KiB fragment of the
// cache tile) from LDS and keeps the other in registers.  A 32x32x16 MFMA does
// twice the work of a 16x16x32 one for the same 1 KiB, so with 32 query rows per
// wave the LDS traffic per flop halves.
//
// Organisation: 4 waves (one per SIMD), 64 query rows per workgroup, one
// workgroup per CU.
//  * Waves 2p and 2p+1 (a pair) own query rows 32p .. 32p+31.  For the scores the
//    pair splits the 576-long contraction (wave half h keeps dims 288h .. 288h+287
//    of its 32 rows as bf16, 72 VGPRs) and swaps 32x32 partial sums through LDS;
//    for P.V it splits the 512 output dims (wave half h accumulates dims 256h ..
//    256h+255 of its 32 rows: 128 accumulators).
//  * Scores come out transposed, S^T = K Q^T: A = 32 cache rows x 16 dims (16
//    bytes per lane, one b128 read), B = the query fragment.  Lane l then holds the
//    scores of query row l % 32 at the 16 positions 8(v/4) + 4(l/32) + v%4 -- read
//    in that order they are the A operand of P.V for positions 0..15 (v < 8) and
//    16..31 (v >= 8), so probabilities never move between lanes; the value operand
//    takes its positions in the same order, two transpose reads
//    (ds_read_b64_tr_b16) of 4 cache rows each.
//  * A row's 16 + 16 scores sit in lanes l and l ^ 32: its maximum is one
//    v_permlane32_swap away.
//  * Loop per tile t: add the partner's partial scores of tile t; scores of tile
//    t+1 on the matrix cores next to the softmax of tile t on the vector ALU;
//    barrier; write the partial scores of t+1; P.V of tile t; barrier.
//  * LDS: a ring of 4 tiles (36 KiB each: latent rows of 1 KiB, rope rows of
//    128 B) filled by global_load_lds_dwordx4 three tiles ahead, plus 16 KiB of
//    partial scores: 160 KiB.  The 16-byte chunks of latent row r are permuted by
//    XOR with a 4-bit function of r & 15 chosen so that a score read (16 rows,
//    one chunk) and a transpose read (4 consecutive rows, two chunks) each touch
//    16 different bank groups; rope rows use r >> 1.
#include "ddtv_internal.hpp"

namespace ddtv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 64;                            // query rows per workgroup (2 pairs x 32)
constexpr int kRing = 4;                             // tile buffers
constexpr int kLatChunks = kTile * 64;               // 16-byte chunks of the latent region (32 KiB)
constexpr int kTileChunks = kLatChunks + kTile * 8;  // + rope region (4 KiB)
constexpr int kLatRowsPerWave = kTile / kWaves;      // latent rows each wave loads per tile
constexpr int kLoadsPerTile = kLatRowsPerWave + 1;   // + one rope instruction (8 rows)
constexpr int kChunks = 18;                          // 16-dim contraction chunks per wave (288 dims)
static_assert(kTile == 32 && kWaves * 8 == kTile, "one rope instruction of 8 rows per wave");

struct Smem {
    f32x4 kv[kRing][kTileChunks];   // ring of cache tiles
    f32x4 sx[kWaves][4][64];        // partial scores: wave, quarter of the 16 values, lane
};

// 4-bit permutation of a latent row's 16-byte chunks, by row r & 15: bits
// (r2, r0, r1, r3) -> (f0, f1, f2, f3).  Rows r .. r+15 map one chunk to 16
// different bank groups; rows 4k .. 4k+3 map chunks 2u, 2u+1 to 8.
__host__ __device__ __forceinline__ int lat_swz(int r) {
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (r & 8);
}
__host__ __device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ uint32_t lds_addr(const f32x4* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) f32x4*)p;
}

// Barrier once this wave's LDS accesses have landed (and, for the _vm form, at
// most N of its vector-memory loads are outstanding: loads retire in order, so
// every older tile has landed).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void barrier_vm() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS reads as inline asm: the results are NOT ready when these return; a tied
// wait below makes them so.  (The loop issues no scalar-memory loads, so the LDS
// counter counts these in program order.)
template <int OFF>
__device__ __forceinline__ void k_read(f32x4& r, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void tr_read(s16x4& r, uint32_t addr) {
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
}
template <int N>
__device__ __forceinline__ void wait_k6(f32x4 (&k)[6]) {
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5])
                 : "n"(N));
}
template <int N>
__device__ __forceinline__ void wait_v8(s16x4 (&v)[8]) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "n"(N));
}

// This wave's share of one cache tile: latent rows 8w .. 8w+7 (one 1 KiB row per
// instruction) and rope rows 8w .. 8w+7 (one instruction).  Rows past the last
// valid position re-read the last one (their scores are masked).
__device__ __forceinline__ void issue_tile(f32x4* buf, const AttnArgs& a, int64_t kv_base, int t0, int kv_last,
                                           int wave, int lane) {
    const char* ck = reinterpret_cast<const char*>(a.ckv);
    const char* kr = reinterpret_cast<const char*>(a.k_rope);
#pragma unroll
    for (int k = 0; k < kLatRowsPerWave; ++k) {
        const int r = wave * kLatRowsPerWave + k;
        const int64_t row = kv_base + min(t0 + r, kv_last);
        const int c = (lane & ~15) | ((lane & 15) ^ lat_swz(r & 15));   // chunk stored at `lane`
        __builtin_amdgcn_global_load_lds(ck + row * 1024 + c * 16, (lds_void*)(buf + r * 64), 16, 0, 0);
    }
    {
        const int r = wave * 8 + (lane >> 3);
        const int64_t row = kv_base + min(t0 + r, kv_last);
        const int c = (lane & 7) ^ rope_swz(r);
        __builtin_amdgcn_global_load_lds(kr + row * 128 + c * 16, (lds_void*)(buf + kLatChunks + wave * 64), 16, 0,
                                         0);
    }
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 a, f32x4 b, float s) {
    bf16x8 r;
    r[0] = (__bf16)(a[0] * s); r[1] = (__bf16)(a[1] * s); r[2] = (__bf16)(a[2] * s); r[3] = (__bf16)(a[3] * s);
    r[4] = (__bf16)(b[0] * s); r[5] = (__bf16)(b[1] * s); r[6] = (__bf16)(b[2] * s); r[7] = (__bf16)(b[3] * s);
    return r;
}

__device__ __forceinline__ bf16x8 cat8(s16x4 lo, s16x4 hi) {
    const bf16x4 b0 = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 b1 = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
}

// Score-operand read of contraction chunk C (of this wave's 18): cache row l % 32,
// 8 dims.  Latent chunk C at koff[C & 7] + 256 (C >> 3); rope chunk (half 1,
// C >= 14) at krope[C - 14].
template <int HALF, int C>
__device__ __forceinline__ void k_chunk(f32x4& k, uint32_t kb, const uint32_t (&koff)[8], const uint32_t (&krope)[4]) {
    if constexpr (HALF == 1 && C >= 14)
        k_read<0>(k, kb + krope[C - 14]);
    else
        k_read<256 * (C >> 3)>(k, kb + koff[C & 7]);
}

// Partial scores of one tile over this wave's 18 chunks, in two accumulators.
template <int HALF>
__device__ __forceinline__ f32x16 scores(uint32_t kb, const bf16x8 (&q)[kChunks], const uint32_t (&koff)[8],
                                         const uint32_t (&krope)[4]) {
    f32x16 s0 = {}, s1 = {};
    f32x4 k[6];
#define KB3(B, C0)                                                 \
    k_chunk<HALF, C0>(k[B + 0], kb, koff, krope);                 \
    k_chunk<HALF, C0 + 1>(k[B + 1], kb, koff, krope);             \
    k_chunk<HALF, C0 + 2>(k[B + 2], kb, koff, krope);
#define MM3(B, C0)                                                                                          \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k[B + 0]), q[C0 + 0], s0, 0, 0, 0); \
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k[B + 1]), q[C0 + 1], s1, 0, 0, 0); \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k[B + 2]), q[C0 + 2], s0, 0, 0, 0);
    KB3(0, 0)
    KB3(3, 3)
    wait_k6<3>(k);
    MM3(0, 0)
    KB3(0, 6)
    wait_k6<3>(k);
    MM3(3, 3)
    KB3(3, 9)
    wait_k6<3>(k);
    MM3(0, 6)
    KB3(0, 12)
    wait_k6<3>(k);
    MM3(3, 9)
    KB3(3, 15)
    wait_k6<3>(k);
    MM3(0, 12)
    wait_k6<0>(k);
    MM3(3, 15)
#undef KB3
#undef MM3
    return s0 + s1;
}

// O += P V for one 32x32 block, with the accumulators pinned to AGPRs (as a
// builtin the compiler moves all 128 of them through VGPRs every tile, because
// the running-max rescale multiplies them on the vector ALU).  The compiler sees
// no matrix instruction here, so code that reads the accumulators after the last
// of these waits first (acc_settle).
__device__ __forceinline__ void pv_mfma(f32x16& o, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}
// x *= f for one accumulator register, read and written in place (written as
// plain C++ the compiler keeps a VGPR copy of all 128 accumulators around the
// loop for this rarely taken path)
__device__ __forceinline__ float acc_scale(float x, float f) {
    float t, r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(x));
    t *= f;
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(r) : "v"(t));
    return r;
}
// Enough independent cycles for the last accumulation to land before vector
// instructions read its registers (a 32x32x16 bf16 product takes 8 passes).
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// O += P V of one tile: value fragments of position block KB (16 positions) for
// the 8 blocks of 32 dims of this half.  Transpose read j of dim block 4q + d at
// toff[2d + j] + 256 q (+ 16 KiB for the second position block).
template <int KB>
__device__ __forceinline__ void pv_block(f32x16 (&o)[8], const bf16x8& pa, uint32_t vb, const uint32_t (&toff)[8]) {
    constexpr int off = KB * 16384;
    s16x4 v[8], w[8];
    tr_read<off>(v[0], vb + toff[0]);
    tr_read<off>(v[1], vb + toff[1]);
    tr_read<off>(v[2], vb + toff[2]);
    tr_read<off>(v[3], vb + toff[3]);
    tr_read<off>(v[4], vb + toff[4]);
    tr_read<off>(v[5], vb + toff[5]);
    tr_read<off>(v[6], vb + toff[6]);
    tr_read<off>(v[7], vb + toff[7]);
    tr_read<off + 256>(w[0], vb + toff[0]);
    tr_read<off + 256>(w[1], vb + toff[1]);
    tr_read<off + 256>(w[2], vb + toff[2]);
    tr_read<off + 256>(w[3], vb + toff[3]);
    tr_read<off + 256>(w[4], vb + toff[4]);
    tr_read<off + 256>(w[5], vb + toff[5]);
    tr_read<off + 256>(w[6], vb + toff[6]);
    tr_read<off + 256>(w[7], vb + toff[7]);
    wait_v8<8>(v);
#pragma unroll
    for (int d = 0; d < 4; ++d) pv_mfma(o[d], pa, cat8(v[2 * d], v[2 * d + 1]));
    wait_v8<0>(w);
#pragma unroll
    for (int d = 0; d < 4; ++d) pv_mfma(o[4 + d], pa, cat8(w[2 * d], w[2 * d + 1]));
}

// Visibility of the 32 positions of a tile that starts at cache position t0, as
// bits: bit o for position t0 + o (tree positions through this row's mask words,
// prefix positions always; the split end is applied separately).
__device__ __forceinline__ uint32_t tile_window(const u32x8& mw, int t0, int P, int W) {
    const int base = t0 - P;   // wave-uniform
    if (base <= -kTile) return ~0u;
    if (base < 0) {
        const int sh = -base;   // 1 .. 31 prefix positions first
        return (mw[0] << sh) | ((1u << sh) - 1u);
    }
    const int w0 = base >> 5, sh = base & 31;
    const uint32_t lo = w0 < W ? mw[w0 & 7] : 0u;
    const uint32_t hi = w0 + 1 < W ? mw[(w0 + 1) & 7] : 0u;
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> sh);
}

// Softmax of one tile (log2 units): s holds row l % 32's scores at positions
// t0 + 8(v/4) + 4(l/32) + v%4.  Masks, updates the running max (lazily: only when
// a tile beats it by more than 2^8) and sum, rescales O on a raise, and returns
// the probabilities as the two A operands of P.V.
__device__ __forceinline__ void softmax(f32x16& s, f32x16 (&o)[8], bf16x8 (&pa)[2], float& m_run, float& l_lane,
                                        int lane, int t0, int P, int kv_hi, const u32x8& mw, int W) {
    const int hb = lane >> 5;
    const bool full = (t0 + kTile <= P) && (t0 + kTile <= kv_hi);
    if (!full) {
        const uint32_t win = tile_window(mw, t0, P, W);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int o = 8 * (v >> 2) + 4 * hb + (v & 3);
            const bool vis = (t0 + o < kv_hi) && ((win >> o) & 1u);
            s[v] = vis ? s[v] : -INFINITY;
        }
    }
    float tmax = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, s[v]);
    {
        auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(tmax, fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1])));
    }
    const bool raise = tmax > m_run + 8.f;
    if (__any(raise)) {
        const float m_new = raise ? tmax : m_run;
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_lane *= alpha;
        // O's lane holds rows 8(v/4) + 4(l/32) + v%4: fetch their factors
        float av[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) av[v] = __shfl(alpha, 8 * (v >> 2) + 4 * hb + (v & 3), 64);
        acc_settle();
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[d][v] = acc_scale(o[d][v], av[v]);
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(s[v] - m_use);
        l_lane += p;
        pa[v >> 3][v & 7] = (__bf16)p;
    }
}

template <int HALF>
__device__ __forceinline__ void attn_body(const AttnArgs& a, Smem& sm, int b, int s, int rt, int wave, int lane) {
    const int hb = lane >> 5;
    const int pair = wave >> 1;
    const ddtv_row rowd = a.rows[b];
    const int kv_len = rowd.kv_len, P = rowd.prefix;
    const int kv_lo = s * a.split_len;
    const int n_b = (kv_len + a.split_len - 1) / a.split_len;
    const int kv_hi = min(kv_len, kv_lo + a.split_len);
    const int ntiles = (kv_hi - kv_lo + kTile - 1) / kTile;
    const int64_t kv_base = rowd.kv_off;
    const uint32_t ring0 = lds_addr(&sm.kv[0][0]);
    constexpr uint32_t kBufBytes = kTileChunks * 16;
    auto buf = [&](int t) { return ring0 + (uint32_t)(t & (kRing - 1)) * kBufBytes; };

    // query fragment c: dims 288*HALF + 16c + 8(l/32) .. +7 of row 32 pair + l%32
    // (loaded first, converted once the first tiles are on their way)
    const int myrow = rt * kRows + pair * 32 + (lane & 31);
    const bool row_ok = myrow < a.R;
    f32x4 qf[2 * kChunks];
    {
        const int64_t qrow = (int64_t)b * a.R + (row_ok ? myrow : 0);
        const f32x4* qa = reinterpret_cast<const f32x4*>(a.q_abs) + qrow * 128;
        const f32x4* qr = reinterpret_cast<const f32x4*>(a.q_rope) + qrow * 16;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int d = 288 * HALF + 16 * c + 8 * hb;   // 0 .. 575
            const f32x4* src = d < kDLat ? qa + d / 4 : qr + (d - kDLat) / 4;
            qf[2 * c] = src[0];
            qf[2 * c + 1] = src[1];
        }
    }
    // mask words of this row's node (used in tiles that reach the tree)
    u32x8 mw;
    {
        const uint32_t* mrow = a.bits + ((int64_t)b * a.Q + (row_ok ? myrow / a.H : 0)) * a.W;
#pragma unroll
        for (int x = 0; x < kMaxW; ++x) mw[x] = x < a.W ? mrow[x] : 0u;
    }

    // the first three tiles
#pragma unroll
    for (int m = 0; m < 3; ++m)
        if (m < ntiles) issue_tile(sm.kv[m], a, kv_base, kv_lo + m * kTile, kv_len - 1, wave, lane);

    // times scale*log2(e), as bf16
    bf16x8 q[kChunks];
    {
        const float sc = row_ok ? a.scale_log2 : 0.f;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) q[c] = to_bf16x8(qf[2 * c], qf[2 * c + 1], sc);
    }
    // the mask words are waited for here, not inside the loop, where a wait would
    // also drain the tile prefetches
    asm volatile("" : "+v"(mw));

    // per-lane LDS byte offsets inside a tile buffer
    //  score operand, row p = l%32, latent chunk 8k + cr of this half: koff[cr] + 256 k
    //  score operand, rope chunk m (half 1): krope[m]
    //  transpose read of dim block 4q + d, half j: toff[2d + j] + 256 q
    uint32_t koff[8], krope[4], toff[8];
    {
        const int p = lane & 31;
        const int ch0 = 36 * HALF + hb;   // first 16-byte chunk of this lane's dims
#pragma unroll
        for (int cr = 0; cr < 8; ++cr) {
            const int ch = ch0 + 2 * cr;
            koff[cr] = (uint32_t)(p * 1024 + ((ch & ~15) | ((ch & 15) ^ lat_swz(p & 15))) * 16);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
            krope[m] = (uint32_t)((kLatChunks + p * 8 + ((2 * m + hb) ^ rope_swz(p))) * 16);
        // transpose reads: lane i of its 16-lane group reads row r0 + (i >> 2) at dims
        // d0 + 4(i & 3); the group's rows are 4(l/32) (+8 for the second read), its
        // dims 256*HALF + 32 d + 16((l/16) & 1)
        const int i = lane & 15;
        const int g1 = (lane >> 4) & 1;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = 4 * hb + 8 * j + (i >> 2);
                const int ch = 32 * HALF + 4 * d + 2 * g1 + ((i & 3) >> 1);
                toff[2 * d + j] =
                    (uint32_t)(row * 1024 + ((ch & ~15) | ((ch & 15) ^ lat_swz(row & 15))) * 16 + 8 * (i & 1));
            }
    }

    f32x16 o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        o[d] = f32x16{};
        asm volatile("" : "+a"(o[d]));
    }
    float m_run = -INFINITY, l_lane = 0.f;
    f32x4* sx_mine = &sm.sx[wave][0][0];
    const f32x4* sx_partner = &sm.sx[wave ^ 1][0][0];

    // tile 0's partial scores (tile 0 landed), then tile 1 landed for the loop
    if (ntiles > 2)
        barrier_vm<2 * kLoadsPerTile>();
    else if (ntiles > 1)
        barrier_vm<kLoadsPerTile>();
    else
        barrier_vm<0>();
    f32x16 sc_mine = scores<HALF>(buf(0), q, koff, krope);
#pragma unroll
    for (int x = 0; x < 4; ++x)
        sx_mine[x * 64 + lane] = f32x4{sc_mine[4 * x], sc_mine[4 * x + 1], sc_mine[4 * x + 2], sc_mine[4 * x + 3]};
    if (ntiles > 2)
        barrier_vm<kLoadsPerTile>();
    else
        barrier_vm<0>();

    for (int t = 0; t < ntiles; ++t) {
        // the partner's partial scores of tile t
        f32x16 st = sc_mine;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const f32x4 pp = sx_partner[x * 64 + lane];
            st[4 * x] += pp[0];
            st[4 * x + 1] += pp[1];
            st[4 * x + 2] += pp[2];
            st[4 * x + 3] += pp[3];
        }
        // tile t+3 into the buffer of tile t-1 (its last reader passed the barrier above)
        if (t + 3 < ntiles) issue_tile(sm.kv[(t + 3) & (kRing - 1)], a, kv_base, kv_lo + (t + 3) * kTile, kv_len - 1,
                                       wave, lane);
        // scores of tile t+1 next to the softmax of tile t
        if (t + 1 < ntiles) sc_mine = scores<HALF>(buf(t + 1), q, koff, krope);
        bf16x8 pa[2];
        softmax(st, o, pa, m_run, l_lane, lane, kv_lo + t * kTile, P, kv_hi, mw, a.W);
        barrier_lds();   // every wave has read its partner's scores of tile t
        if (t + 1 < ntiles) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
                sx_mine[x * 64 + lane] =
                    f32x4{sc_mine[4 * x], sc_mine[4 * x + 1], sc_mine[4 * x + 2], sc_mine[4 * x + 3]};
        }
        // P.V of tile t
        const uint32_t vb = buf(t);   // toff holds this half's dims
        pv_block<0>(o, pa[0], vb, toff);
        pv_block<1>(o, pa[1], vb, toff);
        // partial scores of t+1 visible; tile t+2 landed (tile t+3 may be in flight)
        if (t + 3 < ntiles)
            barrier_vm<kLoadsPerTile>();
        else
            barrier_vm<0>();
    }

    // ---- epilogue: lane holds rows 8(v/4) + 4(l/32) + v%4 of the pair, dim 256*HALF + 32 d + l%32
    const float kLn2 = 0.69314718055994530942f;
    float l_row = l_lane;
    {
        auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_row), __float_as_uint(l_row), false, false);
        l_row = __uint_as_float(x[0]) + __uint_as_float(x[1]);   // lanes l % 32 and l % 32 + 32, in that order
    }
    const int orow0 = rt * kRows + pair * 32;
    if (n_b == 1) {
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = 8 * (v >> 2) + 4 * hb + (v & 3);
            const float iv = __shfl(inv, r, 64);
            const int orow = orow0 + r;
            if (orow < a.R) {
                float* dst = a.out + ((int64_t)b * a.R + orow) * kDLat + 256 * HALF + (lane & 31);
#pragma unroll
                for (int d = 0; d < 8; ++d) dst[32 * d] = o[d][v] * iv;
            }
        }
        if (HALF == 0 && a.lse && hb == 0 && row_ok)
            a.lse[(int64_t)b * a.R + myrow] = l_row > 0.f ? (m_run + log2f(l_row)) * kLn2 : -INFINITY;
    } else {
        const int64_t pbase = ((int64_t)b * a.n_split + s) * a.R;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = 8 * (v >> 2) + 4 * hb + (v & 3);
            const int orow = orow0 + r;
            if (orow < a.R) {
                float* dst = a.part_o + (pbase + orow) * kDLat + 256 * HALF + (lane & 31);
#pragma unroll
                for (int d = 0; d < 8; ++d) dst[32 * d] = o[d][v];
            }
        }
        if (HALF == 0 && hb == 0 && row_ok) a.part_ml[pbase + myrow] = make_float2(m_run, l_row);
    }
}

__global__ __launch_bounds__(kThreads) void attn_mfma_bf16w_kernel(AttnArgs a) {
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

int bf16w_rows_per_workgroup() { return kRows; }

hipError_t launch_attn_mfma_bf16w(const AttnArgs& a, int64_t grid, hipStream_t stream) {
    (void)hipGetLastError();   // report only this launch's error
    hipLaunchKernelGGL(attn_mfma_bf16w_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ddtv
