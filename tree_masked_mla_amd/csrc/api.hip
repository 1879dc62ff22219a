// C ABI of libddtv: host-side argument checks, split planning and launches.
// Every check runs before the first HIP call, so argument errors are reported
// identically with or without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "ddtv_internal.hpp"
#include "neighbour.hpp"
#include "tail.hpp"

using namespace ddtv;

namespace {

constexpr int32_t kVersion = 800;   // 0.8.0: FP8 E4M3 caches

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct VisLayout {
    size_t bits, rows, status, order, total;
};

VisLayout vis_layout(int32_t B, int32_t Q) {
    VisLayout L{};
    const int W = (Q + 31) / 32;
    L.bits = 0;
    L.rows = round_up((size_t)B * Q * W * sizeof(uint32_t), 256);
    L.status = L.rows + round_up((size_t)B * sizeof(ddtv_row), 256);
    L.order = L.status + round_up((size_t)B * sizeof(int32_t), 256);
    L.total = L.order + round_up((size_t)B * sizeof(int32_t), 256);
    return L;
}

// Batch rows by cache length, longest first (equal lengths: lower row first).
// Under the spread order the grid visits rows in this order, so the longest
// rows start first and the short ones fill in at the end (longest-processing-
// time-first list scheduling).
std::vector<int> longest_first(const int32_t* prefix, int B) {
    std::vector<int> perm(B);
    for (int b = 0; b < B; ++b) perm[b] = b;
    if (prefix) std::stable_sort(perm.begin(), perm.end(), [&](int x, int y) { return prefix[x] > prefix[y]; });
    return perm;
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// A dispatch packet holds each grid dimension's work-item count in 32 bits, so
// `workgroups` workgroups of `threads` threads along one dimension must stay
// below 2^32.
bool grid_fits(int64_t workgroups, int threads) {
    return workgroups >= 0 && workgroups <= (int64_t)UINT32_MAX / threads;
}

constexpr int kMaxCusPerXcd = 64;              // planner's per-XCD CU table (MI355X: 32)
constexpr int32_t kMaxProjHeads = 1024;          // heads per projection call (grid z)
constexpr int64_t kMaxProjRows = (int64_t)1 << 28; // tokens per projection call: (rows / 64) x 512 threads < 2^32

bool dtype_ok(int d) { return d == DDTV_F32 || d == DDTV_BF16 || d == DDTV_FP8_E4M3; }

bool rope_ok(double theta) { return std::isfinite(theta) && theta > 0.0; }

// Rotary frequency of pair i (of 32): theta^(-2i/64), in float64.
void rope_frequencies(double theta, double* f) {
    for (int i = 0; i < kDRope / 2; ++i) f[i] = pow(theta, -(double)(2 * i) / (double)kDRope);
}

ddtv_status check_vis(const ddtv_vis* vis) {
    if (!vis || !vis->bits || !vis->rows) return DDTV_EINVAL;
    if (vis->B < 1 || vis->Q < 1 || vis->Q > kMaxQ || vis->W != (vis->Q + 31) / 32) return DDTV_EINVAL;
    if (vis->max_kv < vis->Q || vis->total_kv < (int64_t)vis->B * vis->Q) return DDTV_EINVAL;
    if (!aligned(vis->bits, 4) || !aligned(vis->rows, 8) || !aligned(vis->order, 4)) return DDTV_EINVAL;
    return DDTV_OK;
}

struct Plan {
    int path = DDTV_PATH_AUTO;
    bool bf16_mma = false;   // bf16 caches on the bf16 matrix cores
    bool halves = false;     // row-half mode of the matrix kernel (at most 32 query rows per batch row)
    int rows_per_wg = 0;
    int n_rt = 0;
    int split_len = 0;
    int absorb = 0;          // see splits_of
    int n_split = 1;
    int order = DDTV_ORDER_XCD_LOCAL;
    int64_t grid = 0;
    size_t ws_part_o = 0, ws_part_ml = 0, ws_bytes = 0;
};

// One XCD under in-order dispatch: its CUs' free times, kept sorted ascending;
// work items start in order on whichever CU frees first.  Consecutive items of
// equal cost are gathered into one run before they are placed.
struct XcdSchedule {
    double t[kMaxCusPerXcd];
    double tmp[kMaxCusPerXcd];
    int P;
    double pend_c;
    int64_t pend_k;
    void reset(int cus) {
        P = cus;
        for (int i = 0; i < P; ++i) t[i] = 0.0;
        pend_k = 0;
        pend_c = 0.0;
    }
    void add(double c, int64_t k) {
        if (k <= 0) return;
        if (pend_k > 0 && c == pend_c) {
            pend_k += k;
            return;
        }
        flush();
        pend_c = c;
        pend_k = k;
    }
    // a run of k items of cost c: each full round adds c to every CU, the
    // remaining r items go to the r CUs that free first
    void flush() {
        if (pend_k == 0) return;
        const double c = pend_c;
        const int64_t full = pend_k / P;
        const int r = (int)(pend_k % P);
        pend_k = 0;
        if (full)
            for (int i = 0; i < P; ++i) t[i] += (double)full * c;
        if (r == 0) return;
        int i = 0, j = r, o = 0;   // merge t[0..r) + c with t[r..P)
        while (i < r && j < P) tmp[o++] = (t[i] + c <= t[j]) ? t[i++] + c : t[j++];
        while (i < r) tmp[o++] = t[i++] + c;
        while (j < P) tmp[o++] = t[j++];
        for (int q = 0; q < P; ++q) t[q] = tmp[q];
    }
    double makespan() {
        flush();
        return t[P - 1];
    }
};

constexpr double kExitCost = 0.02;   // a work item past its row's last split: starts and exits
constexpr double kHalfTileCost = 0.65;  // a last tile of at most 16 rows on the fp32 matrix kernel (measured)

// Tile-times of a split of len cache rows: one per 32-row tile; with half tiles
// (fp32 matrix kernel, fp32 cache, usual mode) a last tile of at most 16 rows
// costs kHalfTileCost.
double tiles_of(int len, bool half) {
    const int full = len / kTile, r = len % kTile;
    return (double)full + (r == 0 ? 0.0 : (half && r <= kTile / 2) ? kHalfTileCost : 1.0);
}

// Total work of the grid spread evenly over all CUs, plus the merge pass: a
// lower bound on the makespan, and one that grows with the split count (each
// split adds its set-up and merge traffic).
double fluid_bound(const std::vector<int>& kv, int n_rt, int L, int absorb, int cus, double setup_tiles,
                   double merge_tiles_per_partial_row_split, int64_t R, bool half) {
    int n_split = 1;
    for (int k : kv) n_split = std::max(n_split, splits_of(k, L, absorb));
    half = half && L % kTile != 0;   // (the kernel's half-tile variant runs only then)
    const double full_tiles = tiles_of(L, half);
    double work = 0.0, merge = 0.0;
    for (int k : kv) {
        const int nb = splits_of(k, L, absorb);
        const int last = k - (nb - 1) * L;
        work += (double)n_rt * ((double)(nb - 1) * (setup_tiles + full_tiles) + setup_tiles +
                                tiles_of(last, half) + (double)(n_split - nb) * kExitCost);
        if (nb > 1) merge += merge_tiles_per_partial_row_split * (double)nb * (double)R;
    }
    return work / cus + merge;
}

// Estimated makespan (in tile-times) of the main kernel's grid plus the merge
// pass.  The grid holds B x n_split x n_rt work items (batch row slowest, query
// tile fastest); items past a short row's last split exit at once.  The
// dispatcher deals workgroup i to XCD i % 8, and each XCD starts its workgroups
// in order on whichever of its CUs frees first, one workgroup per CU at a time
// (every attention kernel uses most of a CU's LDS).  Workgroup i runs work item
// i (spread) or xcd_remap(i) (XCD-local: each XCD a contiguous block).  The n_rt
// query tiles of one (row, split) cost the same, so each XCD's list is
// simulated run by run.  `bound`: give up (returning at least bound) once the
// total work alone shows the plan cannot beat it.
double estimate(const std::vector<int>& kv, int n_rt, int L, int absorb, int cus, double setup_tiles,
                double merge_tiles_per_partial_row_split, int64_t R, bool half, bool spread,
                double bound = 1e300) {
    const int per_xcd = std::max(1, std::min(kMaxCusPerXcd, cus / kXcds));
    int n_split = 1;
    for (int k : kv) n_split = std::max(n_split, splits_of(k, L, absorb));
    const int64_t G = (int64_t)kv.size() * n_split * n_rt;
    half = half && L % kTile != 0;   // (the kernel's half-tile variant runs only then)
    double merge = 0.0;   // each partial row is written, then read by the merge pass
    for (int k : kv) {
        const int parts = splits_of(k, L, absorb);
        if (parts > 1) merge += merge_tiles_per_partial_row_split * (double)parts * (double)R;
    }
    auto cost = [&](int b, int s) {
        const int nb = splits_of(kv[b], L, absorb);
        const int len = s < nb - 1 ? L : s == nb - 1 ? kv[b] - s * L : 0;
        return len > 0 ? setup_tiles + tiles_of(len, half) : kExitCost;
    };
    const double fluid =
        fluid_bound(kv, n_rt, L, absorb, cus, setup_tiles, merge_tiles_per_partial_row_split, R, half);
    if (fluid >= bound) return fluid;
    if (G <= (int64_t)per_xcd * kXcds) {   // no XCD gets more items than CUs: all start at once
        int longest = 0;
        for (int k : kv) longest = std::max(longest, std::min(L, k));
        return setup_tiles + tiles_of(longest, half) + merge;
    }
    if ((int64_t)kv.size() * n_split * kXcds > ((int64_t)1 << 20)) return fluid;   // thousands per CU even out
    XcdSchedule X;
    double makespan = 0.0;
    if (spread) {
        // XCD x takes the items i of each (row, split) with i % 8 == x; with n_rt a
        // multiple of 8 every XCD gets the same list, so one stands for all
        const int base = n_rt / kXcds, extra = n_rt % kXcds;
        const int xcds = extra == 0 ? 1 : kXcds;
        for (int x = 0; x < xcds; ++x) {
            X.reset(per_xcd);
            if (base == 0) {   // fewer than 8 query tiles per (row, split): visit this XCD's items only
                for (int64_t i = x; i < G; i += kXcds) {
                    const int64_t g = i / n_rt;
                    X.add(cost((int)(g / n_split), (int)(g % n_split)), 1);
                }
            } else {
                for (int b = 0; b < (int)kv.size(); ++b)
                    for (int s = 0; s < n_split; ++s) {
                        const int64_t g0 = ((int64_t)b * n_split + s) * n_rt;
                        X.add(cost(b, s), base + ((((x - g0) % kXcds) + kXcds) % kXcds < extra ? 1 : 0));
                    }
            }
            makespan = std::max(makespan, X.makespan());
        }
    } else {
        const int64_t q = G / kXcds, r = G % kXcds;
        for (int x = 0; x < kXcds; ++x) {
            const int64_t lo = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
            const int64_t hi = lo + (x < r ? q + 1 : q);
            if (hi <= lo) continue;
            X.reset(per_xcd);
            for (int64_t g = lo / n_rt; g * n_rt < hi; ++g) {   // (row, split) runs overlapping the block
                const int64_t a0 = std::max(lo, g * n_rt), a1 = std::min(hi, (g + 1) * n_rt);
                X.add(cost((int)(g / n_split), (int)(g % n_split)), a1 - a0);
            }
            makespan = std::max(makespan, X.makespan());
        }
    }
    return makespan + merge;
}

ddtv_status make_plan_uncached(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts,
                               size_t ws_cap, Plan* p);

// Plans are pure functions of the shapes, the options, the device's CU count, the
// workspace limit and the per-row cache lengths; a verify loop over a fixed cache
// re-plans the same shapes every step, so the last few plans are kept (a search
// costs a few to a few tens of microseconds, a cached plan about two).
struct PlanKey {
    int32_t B, Q, W, max_kv, H, dtype, path, split, order, has_order, cus;
    int64_t total_kv;
    uint64_t prefix_hash;
    uint64_t ws_cap;
    bool operator==(const PlanKey& o) const { return memcmp(this, &o, sizeof *this) == 0; }
};

uint64_t hash_prefix(const ddtv_vis* vis) {
    uint64_t h = 1469598103934665603ull;   // FNV-1a over the prefix lengths
    if (!vis->prefix_host) return h;
    for (int b = 0; b < vis->B; ++b) {
        h ^= (uint32_t)vis->prefix_host[b];
        h *= 1099511628211ull;
    }
    return h;
}

// ws_cap: the largest workspace the caller can offer (SIZE_MAX: any); split
// candidates whose partials would not fit are skipped.
ddtv_status make_plan(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts, Plan* p,
                      size_t ws_cap = SIZE_MAX) {
    ddtv_status st = check_vis(vis);
    if (st) return st;
    PlanKey key;
    memset(&key, 0, sizeof key);
    key.B = vis->B;
    key.Q = vis->Q;
    key.W = vis->W;
    key.max_kv = vis->max_kv;
    key.total_kv = vis->total_kv;
    key.H = H;
    key.dtype = kv_dtype;
    key.path = opts ? opts->path : 0;
    key.split = opts ? opts->split_len : 0;
    key.order = opts ? opts->wg_order : 0;
    key.has_order = vis->order != nullptr;
    key.cus = cu_count();
    key.prefix_hash = hash_prefix(vis);
    key.ws_cap = ws_cap;
    static std::mutex mu;
    static PlanKey keys[8];
    static Plan plans[8];
    static int used = 0, next = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (keys[i] == key) {
                *p = plans[i];
                return DDTV_OK;
            }
    }
    st = make_plan_uncached(vis, H, kv_dtype, opts, ws_cap, p);
    if (st) return st;
    std::lock_guard<std::mutex> lock(mu);
    keys[next] = key;
    plans[next] = *p;
    next = (next + 1) % 8;
    if (used < 8) ++used;
    return DDTV_OK;
}

// Workspace bytes for `parts` partials per batch row of R query rows (0 when a
// single partial per row means the attention kernel writes the output itself).
size_t partial_bytes(int B, int64_t R, int parts) {
    if (parts <= 1) return 0;
    const size_t rows_total = (size_t)B * parts * (size_t)R;
    return round_up(rows_total * kDLat * sizeof(float), 256) + round_up(rows_total * sizeof(float2), 256);
}

ddtv_status make_plan_uncached(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts,
                               size_t ws_cap, Plan* p) {
    ddtv_status st = check_vis(vis);
    if (st) return st;
    if (H < 1 || H > 65536) return DDTV_EINVAL;
    if (!dtype_ok(kv_dtype)) return DDTV_EUNSUPPORTED;
    const int path_req = opts ? opts->path : DDTV_PATH_AUTO;
    if (path_req != DDTV_PATH_AUTO && path_req != DDTV_PATH_VALU && path_req != DDTV_PATH_MFMA &&
        path_req != DDTV_PATH_MFMA_F32)
        return DDTV_EUNSUPPORTED;
    const int split_req = opts ? opts->split_len : 0;
    if (split_req < 0 || (split_req % kSplitQuantum) != 0) return DDTV_EINVAL;
    const int order_req = opts ? opts->wg_order : DDTV_ORDER_AUTO;
    if (order_req != DDTV_ORDER_AUTO && order_req != DDTV_ORDER_XCD_LOCAL && order_req != DDTV_ORDER_SPREAD)
        return DDTV_EUNSUPPORTED;

    // Auto: the matrix cores once a batch row's query rows fill a 16-row MFMA tile.
    // All heads share the latent cache, so the H * Q rows of a batch row contract
    // against every cache tile together; the vector-ALU kernel is kept for the
    // cases with fewer rows than that.
    p->path = path_req != DDTV_PATH_AUTO ? path_req
                                         : ((int64_t)vis->Q * H < kValuRows ? DDTV_PATH_VALU : DDTV_PATH_MFMA);
    // fp32 and FP8 caches run the fp32 matrix-core kernel under either matrix path
    if (p->path == DDTV_PATH_MFMA_F32 && kv_dtype != DDTV_BF16) p->path = DDTV_PATH_MFMA;
    p->bf16_mma = p->path == DDTV_PATH_MFMA && kv_dtype == DDTV_BF16;
    const int64_t R = (int64_t)vis->Q * H;
    // Batch rows of at most 32 query rows run the fp32 matrix kernel in row-half
    // mode: two wave pairs share each 16-row group and split every cache tile.
    p->halves = p->path != DDTV_PATH_VALU && !p->bf16_mma && R <= 32;
    p->rows_per_wg = p->path == DDTV_PATH_VALU ? kValuRows
                     : p->bf16_mma             ? bf16_rows_per_workgroup()
                     : p->halves               ? 32
                                               : mfma_rows_per_workgroup(kv_dtype);
    if (R > (int64_t)INT32_MAX / 2) return DDTV_EUNSUPPORTED;
    p->n_rt = (int)((R + p->rows_per_wg - 1) / p->rows_per_wg);
    const int max_kv = vis->max_kv;
    const int single = (int)round_up((size_t)max_kv, kTile);

    std::vector<int> kv(vis->B), kv_sorted(vis->B);
    for (int b = 0; b < vis->B; ++b) kv[b] = vis->prefix_host ? vis->prefix_host[b] + vis->Q : max_kv;
    // the grid's batch-row order under the spread order (the row-order table, when present)
    if (vis->order) {
        const std::vector<int> perm = longest_first(vis->prefix_host, vis->B);
        for (int b = 0; b < vis->B; ++b) kv_sorted[b] = kv[perm[b]];
    } else {
        kv_sorted = kv;
    }
    const int cus = cu_count();
    // Tile-time units: one 32-row cache tile through one workgroup.  A partial
    // row costs 2 x 2 KiB of traffic in the merge (written, then read); for the
    // fp32 matrix kernel the write is counted in its set-up (it ends the
    // workgroup), which leaves the 2 KiB the merge pass reads (measured on the
    // 15-split, 1024-row plan: 7.8 us for 31.5 MB).
    // tile_us: rough time of one tile through one workgroup (fp32 MFMA and bf16
    // MFMA: 64 rows; VALU: 16 rows)
    const bool mfma = p->path != DDTV_PATH_VALU;
    // The fp32 matrix kernel on an fp32 cache (usual mode) runs a split's last tile
    // of at most 16 rows as half a tile (when the split length is an odd multiple
    // of 16), so split lengths 16 rows off the tile grid are candidates too; the
    // other kernels pay a whole tile for such a tile.
    const bool half = mfma && !p->bf16_mma && !p->halves && kv_dtype == DDTV_F32;
    // Row-half mode lets a row's last split take a remainder of up to 16 positions
    // (splits_of): decode rows one position past a split boundary then need no
    // workgroup for that position.  The other kernels end every split at split_len.
    p->absorb = p->halves ? kSplitQuantum : 0;
    const int absorb = p->absorb;
    const int cover = std::max(1, max_kv - absorb);   // what S equal pieces must cover
    const double setup = mfma ? 2.0 : 1.0;
    const double tile_us = p->bf16_mma ? 0.9 : (mfma ? 7.3 : 1.0);
    const double merge_per_row_split = ((half ? 2048.0 : 4096.0) / 4.0e12) * 1e6 / tile_us;   // ~4 TB/s effective
    // Simulated makespan at split length L under the requested order, or under the
    // better of the two.  The XCD-local order lets every query tile that reads a
    // cache tile find it in its XCD's L2, so the spread order has to be clearly
    // shorter to be chosen (it is when batch rows differ in length: XCD-local
    // then gives each XCD whole rows).
    auto cost_at = [&](int L, int* order, double bound) {
        if (order_req != DDTV_ORDER_AUTO) {
            *order = order_req;
            return order_req == DDTV_ORDER_SPREAD
                       ? estimate(kv_sorted, p->n_rt, L, absorb, cus, setup, merge_per_row_split, R, half, true, bound)
                       : estimate(kv, p->n_rt, L, absorb, cus, setup, merge_per_row_split, R, half, false, bound);
        }
        const double local = estimate(kv, p->n_rt, L, absorb, cus, setup, merge_per_row_split, R, half, false, bound);
        const double spread = estimate(kv_sorted, p->n_rt, L, absorb, cus, setup, merge_per_row_split, R, half, true,
                                       std::min(bound, local * 0.98));
        *order = spread < local * 0.98 ? DDTV_ORDER_SPREAD : DDTV_ORDER_XCD_LOCAL;
        return std::min(local, spread);
    };

    if (split_req > 0) {
        p->split_len = split_req;
        cost_at(split_req, &p->order, 1e300);
    } else {
        double best = 1e300;
        int bestL = single, bestOrder = DDTV_ORDER_XCD_LOCAL;
        const int64_t wg_cap = (int64_t)cus * 64;
        // Candidates: the longest row cut into S equal tile-aligned pieces, S = 1, 2, ...
        // (stop once the grid is far beyond the device or pieces get short).
        // With half tiles, the length 16 rows shorter than a tile-aligned candidate
        // is a candidate too, after it (so it has to beat it by 2 %), when its grid
        // starts in one round: there the estimate is the longest work item, while
        // the simulation of later rounds is not accurate enough to choose by
        // fractions of a tile.
        int prevLh = 0;
        auto try_half = [&](int S, int L) {
            if (!half) return;
            const int Lh = (int)round_up((size_t)((cover + S - 1) / S), kSplitQuantum);
            if (Lh == L || Lh == prevLh) return;
            prevLh = Lh;
            int64_t wh = 0;
            for (int b = 0; b < vis->B; ++b) wh += (int64_t)splits_of(kv[b], Lh, absorb) * p->n_rt;
            if (wh > cus || (S > 1 && partial_bytes(vis->B, R, splits_of(max_kv, Lh, absorb)) > ws_cap)) return;
            int order = DDTV_ORDER_XCD_LOCAL;
            const double e = cost_at(Lh, &order, best * 0.98);
            if (e < best * 0.98) {
                best = e;
                bestL = Lh;
                bestOrder = order;
            }
        };
        int prevL = 0, worse = 0;
        // (every S below 32, then steps of S / 32: the split lengths grow dense)
        for (int S = 1;; S += S < 32 ? 1 : S / 32) {
            const int L = (int)round_up((size_t)((cover + S - 1) / S), kTile);
            if (L < 4 * kTile && S > 1) break;
            if (L == prevL) {
                try_half(S, L);
                continue;
            }
            prevL = L;
            int64_t wgs = 0;
            for (int b = 0; b < vis->B; ++b) wgs += (int64_t)splits_of(kv[b], L, absorb) * p->n_rt;
            if (wgs > wg_cap && S > 1) break;
            const int parts_L = splits_of(max_kv, L, absorb);
            if (S > 1 && partial_bytes(vis->B, R, parts_L) > ws_cap) break;   // more splits only need more
            if (S > 1 && fluid_bound(kv, p->n_rt, L, absorb, cus, setup, merge_per_row_split, R, half) >= best * 0.98)
                break;   // its lower bound cannot beat the best by 2 %, nor can more splits'
            int order = DDTV_ORDER_XCD_LOCAL;
            const double e = cost_at(L, &order, best * 0.98);   // a plan must beat the best by 2 %
            if (e < best * 0.98) {   // prefer fewer splits unless clearly better
                best = e;
                bestL = L;
                bestOrder = order;
                worse = 0;
            } else if (wgs > 2 * (int64_t)cus && ++worse >= 8) {
                break;               // past a full device and no longer improving
            }
            try_half(S, L);
            if (S >= 4096) break;
        }
        p->split_len = bestL;
        p->order = bestOrder;
    }
    p->n_split = std::max(1, splits_of(max_kv, p->split_len, p->absorb));
    p->grid = (int64_t)vis->B * p->n_rt * p->n_split;
    if (!grid_fits(p->grid, 512)) return DDTV_EUNSUPPORTED;   // 512 = the largest attention workgroup
    const int parts = p->n_split;   // partials per batch row
    if (parts > 1 && !grid_fits(((int64_t)vis->B * R + 1) / 2, 256)) return DDTV_EUNSUPPORTED;   // merge
    p->ws_part_o = 0;
    p->ws_part_ml = parts > 1 ? round_up((size_t)vis->B * parts * (size_t)R * kDLat * sizeof(float), 256) : 0;
    p->ws_bytes = partial_bytes(vis->B, R, parts);
    return DDTV_OK;
}

// External-prefix (tree-tail) mode: the same trees seen without their prefix --
// each batch row's Q tree rows as a row of its own -- over a row table that a
// small kernel writes into the workspace.  Workspace: that table, the tree
// rows' lse, then the tail plan's own workspace.
struct TailLayout {
    size_t rows = 0, lse = 0, plan = 0, total = 0;
};

ddtv_vis tail_view(const ddtv_vis* vis, ddtv_row* rows) {
    ddtv_vis t = *vis;
    t.rows = rows;
    t.order = nullptr;
    t.prefix_host = nullptr;
    t.max_kv = vis->Q;
    t.total_kv = (int64_t)vis->B * vis->Q;
    return t;
}

ddtv_status tail_plan(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts, TailLayout* L,
                      Plan* p) {
    ddtv_status st = check_vis(vis);
    if (st) return st;
    if (H < 1 || H > 65536) return DDTV_EINVAL;
    const ddtv_vis t = tail_view(vis, vis->rows);   // geometry only: planning reads no device data
    st = make_plan(&t, H, kv_dtype, opts, p);
    if (st) return st;
    if (!grid_fits(((int64_t)vis->B * vis->Q * H + 1) / 2, 256)) return DDTV_EUNSUPPORTED;   // tail merge
    L->rows = 0;
    L->lse = round_up((size_t)vis->B * sizeof(ddtv_row), 256);
    L->plan = L->lse + round_up((size_t)vis->B * vis->Q * (size_t)H * sizeof(float), 256);
    L->total = L->plan + p->ws_bytes;
    return DDTV_OK;
}

ddtv_status check_verify_args(const float* q_abs, const float* q_rope, const void* ckv, const void* k_rope,
                              const float* out, const float* lse, float scale) {
    if (!q_abs || !q_rope || !ckv || !k_rope || !out) return DDTV_EINVAL;
    if (!aligned(q_abs, 16) || !aligned(q_rope, 16) || !aligned(ckv, 16) || !aligned(k_rope, 16) ||
        !aligned(out, 16) || (lse && !aligned(lse, 4)))
        return DDTV_EINVAL;
    if (!std::isfinite(scale)) return DDTV_EINVAL;
    return DDTV_OK;
}

// Enqueue S2..S7 under plan p; `workspace` holds p.ws_bytes of device memory.
ddtv_status launch_verify(const Plan& p, const float* q_abs, const float* q_rope, const void* ckv,
                          const void* k_rope, ddtv_dtype kv_dtype, int32_t H, const ddtv_vis* vis, float scale,
                          float* out, float* lse, void* workspace, hipStream_t stream, const ddtv_opts* opts) {
    AttnArgs a;
    a.q_abs = q_abs;
    a.q_rope = q_rope;
    a.ckv = ckv;
    a.k_rope = k_rope;
    a.bits = vis->bits;
    a.rows = vis->rows;
    a.out = out;
    a.lse = lse;
    a.part_o = p.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ws_part_o) : nullptr;
    a.part_ml = p.ws_bytes ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + p.ws_part_ml) : nullptr;
    a.B = vis->B;
    a.Q = vis->Q;
    a.H = H;
    a.W = vis->W;
    a.R = vis->Q * H;
    a.n_rt = p.n_rt;
    a.split_len = p.split_len;
    a.absorb = p.absorb;
    a.n_split = p.n_split;
    a.spread = p.order == DDTV_ORDER_SPREAD;
    a.halves = p.halves;
    a.order = a.spread ? vis->order : nullptr;   // XCD-local keeps rows in their natural order
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);

    if (opts && opts->attn_begin && hipEventRecord(opts->attn_begin, stream) != hipSuccess) return DDTV_EDEVICE;
    hipError_t e = p.bf16_mma ? launch_attn_mfma_bf16(a, p.grid, stream)
                   : (p.path == DDTV_PATH_VALU) ? launch_attn_valu(a, kv_dtype, p.grid, stream)
                                                : launch_attn_mfma(a, kv_dtype, p.grid, stream);
    if (e != hipSuccess) return DDTV_EDEVICE;
    if (opts && opts->attn_end && hipEventRecord(opts->attn_end, stream) != hipSuccess) return DDTV_EDEVICE;
    if (p.n_split > 1 && launch_merge(a, stream) != hipSuccess) return DDTV_EDEVICE;
    return DDTV_OK;
}

// ---------------------------------------------------------------------------
// Scratch of ddtv_verify_attn_noalloc: the split partials of callers that cannot
// allocate a workspace.  Every GPU the library runs on holds one copy until the
// process ends.  In host code `scratch` names a host-side stand-in, so kernels
// and copies get the device address looked up below, never the name itself.
constexpr size_t kScratchBytes = DDTV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* scratch_address() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

}  // namespace

extern "C" {

int32_t ddtv_version(void) { return kVersion; }

const char* ddtv_status_string(ddtv_status s) {
    switch (s) {
        case DDTV_OK: return "ok";
        case DDTV_EINVAL: return "invalid argument";
        case DDTV_ETREE: return "malformed tree (parent array)";
        case DDTV_EUNSUPPORTED: return "unsupported dtype, path or shape";
        case DDTV_EWORKSPACE: return "workspace or visibility buffer too small";
        case DDTV_EDEVICE: return "HIP device error";
    }
    return "unknown status";
}

size_t ddtv_vis_bytes(int32_t B, int32_t Q) {
    if (B < 1 || Q < 1 || Q > kMaxQ) return 0;
    return vis_layout(B, Q).total;
}

ddtv_status ddtv_build_visibility(const int32_t* parent, const int32_t* prefix_len, int32_t B, int32_t Q,
                                  void* vis_buf, size_t vis_buf_bytes, ddtv_vis* vis, hipStream_t stream) {
    if (!parent || !prefix_len || !vis_buf || !vis) return DDTV_EINVAL;
    if (B < 1 || Q < 1 || Q > kMaxQ) return DDTV_EINVAL;
    if (!aligned(parent, 4) || !aligned(vis_buf, 256)) return DDTV_EINVAL;
    int64_t total = 0;
    int32_t max_kv = 0;
    for (int b = 0; b < B; ++b) {
        if (prefix_len[b] < 0 || (int64_t)prefix_len[b] + Q > INT32_MAX) return DDTV_EINVAL;
        total += (int64_t)prefix_len[b] + Q;
        max_kv = std::max(max_kv, prefix_len[b] + Q);
    }
    const VisLayout L = vis_layout(B, Q);
    if (vis_buf_bytes < L.total) return DDTV_EWORKSPACE;

    char* base = static_cast<char*>(vis_buf);
    ddtv_vis v{};
    v.B = B;
    v.Q = Q;
    v.W = (Q + 31) / 32;
    v.max_kv = max_kv;
    v.total_kv = total;
    v.bits = reinterpret_cast<uint32_t*>(base + L.bits);
    v.rows = reinterpret_cast<ddtv_row*>(base + L.rows);
    v.status = reinterpret_cast<int32_t*>(base + L.status);
    v.order = reinterpret_cast<int32_t*>(base + L.order);
    v.prefix_host = prefix_len;
    const std::vector<int> perm = longest_first(prefix_len, B);

    int64_t off = 0;
    for (int b0 = 0; b0 < B; b0 += kVisChunk) {
        const int nb = std::min(kVisChunk, B - b0);
        VisChunk ch;
        memset(&ch, 0, sizeof ch);
        for (int k = 0; k < nb; ++k) {
            ch.kv_off[k] = off;
            ch.prefix[k] = prefix_len[b0 + k];
            ch.order[k] = perm[b0 + k];
            off += (int64_t)prefix_len[b0 + k] + Q;
        }
        if (launch_visibility(parent, b0, nb, Q, v.W, v.bits, v.rows, v.status, v.order, ch, stream) !=
            hipSuccess)
            return DDTV_EDEVICE;
    }
    *vis = v;
    return DDTV_OK;
}

ddtv_status ddtv_build_tree(const float* logp, const int32_t* tokens, int32_t B, int32_t D, int32_t K, int32_t Q,
                            int32_t* parent, int32_t* depth, int32_t* rank, int32_t* token, float* score,
                            hipStream_t stream) {
    if (!logp || !parent) return DDTV_EINVAL;
    if (!aligned(logp, 4) || !aligned(parent, 4) || !aligned(tokens, 4) || !aligned(depth, 4) ||
        !aligned(rank, 4) || !aligned(token, 4) || !aligned(score, 4))
        return DDTV_EINVAL;
    if (B < 1 || D < 1 || Q < 1 || Q > kMaxQ) return DDTV_EINVAL;
    if (K < 1 || K > kMaxTreeK) return DDTV_EUNSUPPORTED;
    if (!grid_fits(B, 64)) return DDTV_EUNSUPPORTED;
    // nodes of the full K-ary tree of depth D, counted until they reach Q
    int64_t nodes = 1, level = 1;
    for (int d = 1; d <= D && nodes < Q; ++d) {
        level = std::min<int64_t>(level * K, (int64_t)kMaxQ + 1);
        nodes += level;
    }
    if (nodes < Q) return DDTV_EINVAL;
    TreeArgs a;
    a.logp = logp;
    a.tokens = tokens;
    a.parent = parent;
    a.depth = depth;
    a.rank = rank;
    a.token = token;
    a.score = score;
    a.B = B;
    a.D = D;
    a.K = K;
    a.Q = Q;
    return launch_tree_build(a, stream) == hipSuccess ? DDTV_OK : DDTV_EDEVICE;
}

size_t ddtv_tail_workspace_bytes(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts) {
    TailLayout L;
    Plan p;
    return tail_plan(vis, H, kv_dtype, opts, &L, &p) == DDTV_OK ? L.total : 0;
}

ddtv_status ddtv_verify_attn_tail(const float* q_abs, const float* q_rope, const void* ckv, const void* k_rope,
                                  ddtv_dtype kv_dtype, int32_t H, const ddtv_vis* vis, float scale,
                                  const float* prefix_out, const float* prefix_lse, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream, const ddtv_opts* opts) {
    if (!prefix_out || !prefix_lse || !out) return DDTV_EINVAL;
    if (!aligned(prefix_out, 16) || !aligned(prefix_lse, 4)) return DDTV_EINVAL;
    TailLayout L;
    Plan p;
    ddtv_status st = tail_plan(vis, H, kv_dtype, opts, &L, &p);
    if (st) return st;
    if (!workspace || workspace_bytes < L.total) return DDTV_EWORKSPACE;
    if (!aligned(workspace, 256)) return DDTV_EINVAL;
    // tree-sparse route (one workgroup of 512 threads per node and 16 heads; the
    // grid's work-items must stay below 2^32)
    const int64_t sparse_items = (int64_t)vis->B * vis->Q * ((H + 15) / 16) * 512;
    if ((!opts || (opts->path == DDTV_PATH_AUTO && opts->split_len == 0)) && sparse_items <= (int64_t)UINT32_MAX) {
        // tree-sparse route: each node visits only its ancestors-or-self
        if (!q_abs || !q_rope || !ckv || !k_rope) return DDTV_EINVAL;
        if (!aligned(q_abs, 16) || !aligned(q_rope, 16) || !aligned(ckv, 16) || !aligned(k_rope, 16) ||
            !aligned(out, 16) || (lse && !aligned(lse, 4)))
            return DDTV_EINVAL;
        if (!std::isfinite(scale)) return DDTV_EINVAL;
        TailSparseArgs a;
        a.q_abs = q_abs;
        a.q_rope = q_rope;
        a.ckv = ckv;
        a.k_rope = k_rope;
        a.bits = vis->bits;
        a.rows = vis->rows;
        a.prefix_out = prefix_out;
        a.prefix_lse = prefix_lse;
        a.out = out;
        a.lse = lse;
        a.B = vis->B;
        a.Q = vis->Q;
        a.H = H;
        a.W = vis->W;
        a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
        if (opts && opts->attn_begin && hipEventRecord(opts->attn_begin, stream) != hipSuccess) return DDTV_EDEVICE;
        if (launch_tail_sparse(a, kv_dtype, stream) != hipSuccess) return DDTV_EDEVICE;
        if (opts && opts->attn_end && hipEventRecord(opts->attn_end, stream) != hipSuccess) return DDTV_EDEVICE;
        return DDTV_OK;
    }
    char* ws = static_cast<char*>(workspace);
    ddtv_row* rows = reinterpret_cast<ddtv_row*>(ws + L.rows);
    float* lse_tail = reinterpret_cast<float*>(ws + L.lse);
    const ddtv_vis t = tail_view(vis, rows);
    if (launch_tail_rows(vis->rows, rows, vis->B, vis->Q, stream) != hipSuccess) return DDTV_EDEVICE;
    st = ddtv_verify_attn_ex(q_abs, q_rope, ckv, k_rope, kv_dtype, H, &t, scale, out, lse_tail, ws + L.plan,
                             workspace_bytes - L.plan, stream, opts);
    if (st) return st;
    const int64_t n = (int64_t)vis->B * vis->Q * H;
    return launch_tail_merge(out, lse_tail, lse, prefix_out, prefix_lse, n, stream) == hipSuccess ? DDTV_OK
                                                                                                     : DDTV_EDEVICE;
}

ddtv_status ddtv_tree_accept(const float* logits, int32_t V, const int32_t* parent, const int32_t* token,
                             const ddtv_vis* vis, void* ckv, void* k_rope, ddtv_dtype kv_dtype, int32_t* pred,
                             int32_t* path, int32_t* out_tokens, int32_t* accept_len, hipStream_t stream) {
    if (!logits || !parent || !token || !pred || !path || !out_tokens || !accept_len) return DDTV_EINVAL;
    if (!aligned(logits, 4) || !aligned(parent, 4) || !aligned(token, 4) || !aligned(pred, 4) ||
        !aligned(path, 4) || !aligned(out_tokens, 4) || !aligned(accept_len, 4))
        return DDTV_EINVAL;
    ddtv_status st = check_vis(vis);
    if (st) return st;
    if (V < 1) return DDTV_EINVAL;
    if ((ckv == nullptr) != (k_rope == nullptr)) return DDTV_EINVAL;
    if (ckv) {
        if (!aligned(ckv, 16) || !aligned(k_rope, 16)) return DDTV_EINVAL;
        if (!dtype_ok(kv_dtype)) return DDTV_EUNSUPPORTED;
    }
    if (!grid_fits((int64_t)vis->B * vis->Q, 256)) return DDTV_EUNSUPPORTED;
    AcceptArgs a;
    a.logits = logits;
    a.parent = parent;
    a.token = token;
    a.rows = vis->rows;
    a.pred = pred;
    a.path = path;
    a.out_tokens = out_tokens;
    a.accept_len = accept_len;
    a.ckv = ckv;
    a.k_rope = k_rope;
    a.kv_elem = kv_dtype == DDTV_F32 ? 4 : (kv_dtype == DDTV_BF16 ? 2 : 1);
    a.B = vis->B;
    a.Q = vis->Q;
    a.V = V;
    return launch_tree_accept(a, stream) == hipSuccess ? DDTV_OK : DDTV_EDEVICE;
}

ddtv_status ddtv_read_status(const ddtv_vis* vis, int32_t* bad_row, int32_t* bad_node, hipStream_t stream) {
    if (bad_row) *bad_row = -1;
    if (bad_node) *bad_node = -1;
    if (!vis || !vis->status || vis->B < 1) return DDTV_EINVAL;
    std::vector<int32_t> st(vis->B);
    if (hipStreamSynchronize(stream) != hipSuccess) return DDTV_EDEVICE;
    if (hipMemcpy(st.data(), vis->status, sizeof(int32_t) * vis->B, hipMemcpyDeviceToHost) != hipSuccess)
        return DDTV_EDEVICE;
    for (int b = 0; b < vis->B; ++b) {
        if (st[b] >= 0) {
            if (bad_row) *bad_row = b;
            if (bad_node) *bad_node = st[b];
            return DDTV_ETREE;
        }
    }
    return DDTV_OK;
}

size_t ddtv_workspace_bytes_ex(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts) {
    Plan p;
    if (make_plan(vis, H, kv_dtype, opts, &p) != DDTV_OK) return 0;
    return p.ws_bytes;
}

size_t ddtv_workspace_bytes(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype) {
    return ddtv_workspace_bytes_ex(vis, H, kv_dtype, nullptr);
}

ddtv_status ddtv_plan_info(const ddtv_vis* vis, int32_t H, ddtv_dtype kv_dtype, const ddtv_opts* opts,
                           int32_t* path, int32_t* split_len, int32_t* n_split, int64_t* workgroups,
                           int32_t* wg_order) {
    Plan p;
    ddtv_status st = make_plan(vis, H, kv_dtype, opts, &p);
    if (st) return st;
    if (path) *path = p.path;
    if (split_len) *split_len = p.split_len;
    if (n_split) *n_split = p.n_split;
    if (workgroups) *workgroups = p.grid;
    if (wg_order) *wg_order = p.order;
    return DDTV_OK;
}

ddtv_status ddtv_verify_attn_ex(const float* q_abs, const float* q_rope, const void* ckv, const void* k_rope,
                                ddtv_dtype kv_dtype, int32_t H, const ddtv_vis* vis, float scale, float* out,
                                float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                const ddtv_opts* opts) {
    ddtv_status st = check_verify_args(q_abs, q_rope, ckv, k_rope, out, lse, scale);
    if (st) return st;
    Plan p;
    st = make_plan(vis, H, kv_dtype, opts, &p);
    if (st) return st;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return DDTV_EWORKSPACE;
        if (!aligned(workspace, 256)) return DDTV_EINVAL;
    }
    return launch_verify(p, q_abs, q_rope, ckv, k_rope, kv_dtype, H, vis, scale, out, lse, workspace, stream, opts);
}

ddtv_status ddtv_verify_attn_noalloc(const float* q_abs, const float* q_rope, const void* ckv, const void* k_rope,
                                     ddtv_dtype kv_dtype, int32_t H, const ddtv_vis* vis, float scale, float* out,
                                     float* lse, hipStream_t stream, const ddtv_opts* opts) {
    ddtv_status st = check_verify_args(q_abs, q_rope, ckv, k_rope, out, lse, scale);
    if (st) return st;
    Plan p;
    st = make_plan(vis, H, kv_dtype, opts, &p, kScratchBytes);
    if (st) return st;
    if (p.ws_bytes > kScratchBytes) return DDTV_EWORKSPACE;   // the plan's partials do not fit the scratch
    void* ws = nullptr;
    if (p.ws_bytes > 0 && !(ws = scratch_address())) return DDTV_EDEVICE;
    return launch_verify(p, q_abs, q_rope, ckv, k_rope, kv_dtype, H, vis, scale, out, lse, ws, stream, opts);
}

ddtv_status ddtv_prepare_query(const float* q, int32_t d_nope, int32_t H, const ddtv_vis* vis,
                               const int32_t* positions, double rope_theta, const float* w_kc, float* q_abs,
                               float* q_rope, hipStream_t stream) {
    if (!q || !w_kc || !q_abs || !q_rope) return DDTV_EINVAL;
    if (!aligned(q, 16) || !aligned(w_kc, 16) || !aligned(q_abs, 16) || !aligned(q_rope, 16) ||
        !aligned(positions, 4))
        return DDTV_EINVAL;
    ddtv_status st = check_vis(vis);
    if (st) return st;
    if (H < 1 || H > kMaxProjHeads || !rope_ok(rope_theta)) return DDTV_EINVAL;
    if (d_nope < 32 || d_nope > 512 || d_nope % 32 != 0) return DDTV_EUNSUPPORTED;
    if ((int64_t)vis->B * vis->Q > kMaxProjRows) return DDTV_EUNSUPPORTED;
    ProjArgs p{};
    p.M = (int64_t)vis->B * vis->Q;
    p.K = d_nope;
    p.N = kDLat;
    p.H = H;
    p.A = q;
    p.a_head = d_nope + kDRope;
    p.lda = (int64_t)H * p.a_head;
    p.B = w_kc;
    p.b_head = (int64_t)d_nope * kDLat;
    p.C = q_abs;
    p.c_head = kDLat;
    p.ldc = (int64_t)H * kDLat;
    p.rope_out = q_rope;
    p.positions = positions;
    p.bits = vis->bits;
    p.rows = vis->rows;
    p.Q = vis->Q;
    p.W = vis->W;
    rope_frequencies(rope_theta, p.inv_freq);
    return launch_proj(p, false, cu_count(), stream) == hipSuccess ? DDTV_OK : DDTV_EDEVICE;
}

ddtv_status ddtv_value_proj(const float* latent, int64_t M, int32_t H, int32_t d_v, const float* w_vc, float* v,
                            hipStream_t stream) {
    if (!latent || !w_vc || !v) return DDTV_EINVAL;
    if (!aligned(latent, 16) || !aligned(w_vc, 16) || !aligned(v, 4)) return DDTV_EINVAL;
    if (M < 0 || H < 1 || H > kMaxProjHeads) return DDTV_EINVAL;
    if (M > kMaxProjRows) return DDTV_EUNSUPPORTED;
    if (d_v < 1 || d_v > kDLat) return DDTV_EUNSUPPORTED;
    if (M == 0) return DDTV_OK;
    ProjArgs p{};
    p.M = M;
    p.K = kDLat;
    p.N = d_v;
    p.H = H;
    p.A = latent;
    p.a_head = kDLat;
    p.lda = (int64_t)H * kDLat;
    p.B = w_vc;
    p.b_head = (int64_t)d_v * kDLat;
    p.C = v;
    p.c_head = d_v;
    p.ldc = (int64_t)H * d_v;
    return launch_proj(p, true, cu_count(), stream) == hipSuccess ? DDTV_OK : DDTV_EDEVICE;
}

ddtv_status ddtv_append_kv(const float* latent, const float* k_pe, const ddtv_vis* vis, const int32_t* positions,
                           double rope_theta, void* ckv, void* k_rope, ddtv_dtype kv_dtype, hipStream_t stream) {
    if (!latent || !k_pe || !ckv || !k_rope) return DDTV_EINVAL;
    if (!aligned(latent, 16) || !aligned(k_pe, 4) || !aligned(ckv, 16) || !aligned(k_rope, 4) ||
        !aligned(positions, 4))
        return DDTV_EINVAL;
    ddtv_status st = check_vis(vis);
    if (st) return st;
    if (!rope_ok(rope_theta)) return DDTV_EINVAL;
    if (!dtype_ok(kv_dtype)) return DDTV_EUNSUPPORTED;
    if (!grid_fits((int64_t)vis->B * vis->Q, 64)) return DDTV_EUNSUPPORTED;
    AppendArgs p{};
    p.latent = latent;
    p.k_pe = k_pe;
    p.positions = positions;
    p.bits = vis->bits;
    p.rows = vis->rows;
    p.ckv = ckv;
    p.k_rope = k_rope;
    p.B = vis->B;
    p.Q = vis->Q;
    p.W = vis->W;
    p.dtype = kv_dtype;
    rope_frequencies(rope_theta, p.inv_freq);
    return launch_append_kv(p, stream) == hipSuccess ? DDTV_OK : DDTV_EDEVICE;
}

ddtv_status ddtv_verify_attn(const float* q_abs, const float* q_rope, const void* ckv, const void* k_rope,
                             ddtv_dtype kv_dtype, int32_t H, const ddtv_vis* vis, float scale, float* out,
                             float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return ddtv_verify_attn_ex(q_abs, q_rope, ckv, k_rope, kv_dtype, H, vis, scale, out, lse, workspace,
                               workspace_bytes, stream, nullptr);
}

}  // extern "C"
