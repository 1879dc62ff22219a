/*
 * CPU oracle of the steps around the verify attention: the query split with
 * NeoX rotary embedding and the w_kc absorb before it, the per-head w_vc value
 * projection after it, and the rotated key rows the tree nodes add to the cache
 * -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this code; the product library never does, and the two share no source.
 * Plain fp64 loops in index order, single-threaded.
 *
 * What it computes (pages: "The Query-Split Kernel: A Pivotal Edit in Building a
 * Native DDTree Inference Engine", sections "The Reasoning Chain" and "Input
 * Knowledge": the query projection of each (token, head) holds a nope part and a
 * rope part; the rope part gets NeoX rotary embedding with angles in float64;
 * the nope part is absorbed into latent space through w_kc; "The Verify-Attn
 * Kernel: A Single File Write ...", section "Design Decisions and Trade-Offs":
 * the attention returns the latent and a per-head GEMM with w_vc follows):
 *
 *   - q row (m, h) is d_nope + 64 floats: nope = q[0 .. d_nope), pe = q[d_nope ..);
 *   - q_abs[m][h][c] = sum_k nope[k] * w_kc[h][k][c]      (w_kc: [H][d_nope][512]);
 *   - q_rope[m][h]   = rope(pe, pos[m]);
 *   - rope(x, p): pair i (0 <= i < 32) is (x[i], x[i + 32]); with
 *     f_i = theta^(-2i/64) and a = p * f_i (float64),
 *         y[i]      = x[i] cos a - x[i + 32] sin a,
 *         y[i + 32] = x[i + 32] cos a + x[i] sin a
 *     (the rotate-half form: the two halves of the vector are the two coordinates
 *     of each rotated pair);
 *   - v[m][h][n] = sum_c o[m][h][c] * w_vc[h][n][c]        (w_vc: [H][d_v][512]);
 *   - a tree node's position is its batch row's prefix length plus its depth
 *     (root depth 0), the position it takes when its path is appended to the
 *     prefix; the node's new cache row holds its latent and its rotated rope key.
 */
#include <math.h>
#include <stdint.h>

enum { NREF_OK = 0, NREF_EINVAL = 1 };

#define N_LAT 512
#define N_ROPE 64
#define N_HALF 32

/* y = NeoX rotation of the 64-wide x at position pos (float64 throughout). */
void ddtvref_rope_neox(const float *x, int32_t pos, double theta, double *y) {
    for (int i = 0; i < N_HALF; ++i) {
        double f = pow(theta, -(double)(2 * i) / (double)N_ROPE);
        double a = (double)pos * f;
        double c = cos(a), s = sin(a);
        double x0 = (double)x[i], x1 = (double)x[i + N_HALF];
        y[i] = x0 * c - x1 * s;
        y[i + N_HALF] = x1 * c + x0 * s;
    }
}

/* Node positions prefix[b] + depth(i), depth by walking parent links to the root.
 * parent [B][Q] must be valid trees (parent[b][0] = -1, 0 <= parent[b][i] < i). */
int ddtvref_tree_positions(const int32_t *parent, const int32_t *prefix, int32_t B, int32_t Q,
                           int32_t *pos) {
    for (int32_t b = 0; b < B; ++b) {
        const int32_t *par = parent + (int64_t)b * Q;
        if (par[0] != -1) return NREF_EINVAL;
        for (int32_t i = 1; i < Q; ++i)
            if (par[i] < 0 || par[i] >= i) return NREF_EINVAL;
        for (int32_t i = 0; i < Q; ++i) {
            int32_t d = 0;
            for (int32_t cur = i; par[cur] != -1; cur = par[cur]) ++d;
            pos[(int64_t)b * Q + i] = prefix[b] + d;
        }
    }
    return NREF_OK;
}

/* Query split, rotation and absorb for M tokens of H heads.
 * q [M][H][d_nope + 64], pos [M], w_kc [H][d_nope][512] -> q_abs [M][H][512],
 * q_rope [M][H][64] (float64). */
int ddtvref_prepare_query(const float *q, int32_t M, int32_t H, int32_t d_nope, const int32_t *pos,
                          double theta, const float *w_kc, double *q_abs, double *q_rope) {
    if (M < 0 || H < 1 || d_nope < 1 || !(theta > 0.0)) return NREF_EINVAL;
    const int64_t row = d_nope + N_ROPE;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t h = 0; h < H; ++h) {
            const float *nope = q + (m * H + h) * row;
            const float *pe = nope + d_nope;
            double *qa = q_abs + (m * H + h) * N_LAT;
            for (int c = 0; c < N_LAT; ++c) {
                double acc = 0.0;
                for (int k = 0; k < d_nope; ++k)
                    acc += (double)nope[k] * (double)w_kc[(h * d_nope + k) * N_LAT + c];
                qa[c] = acc;
            }
            ddtvref_rope_neox(pe, pos[m], theta, q_rope + (m * H + h) * N_ROPE);
        }
    }
    return NREF_OK;
}

/* Per-head value projection: o [M][H][512], w_vc [H][d_v][512] -> v [M][H][d_v]. */
int ddtvref_value_proj(const float *o, int32_t M, int32_t H, int32_t d_v, const float *w_vc,
                       double *v) {
    if (M < 0 || H < 1 || d_v < 1) return NREF_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t h = 0; h < H; ++h) {
            const float *x = o + (m * H + h) * N_LAT;
            for (int64_t n = 0; n < d_v; ++n) {
                const float *w = w_vc + (h * d_v + n) * N_LAT;
                double acc = 0.0;
                for (int c = 0; c < N_LAT; ++c) acc += (double)x[c] * (double)w[c];
                v[(m * H + h) * d_v + n] = acc;
            }
        }
    }
    return NREF_OK;
}

/* The cache rows a batch of trees adds: node i of row b (position pos[b][i])
 * writes latent[b][i] and rope(k_pe[b][i], pos) at row kv_off[b] + prefix[b] + i,
 * kv_off[b] = sum over b' < b of (prefix[b'] + Q).  ckv [total][512] and
 * k_rope [total][64] are float64 here; rows the trees do not own are untouched. */
int ddtvref_append_kv(const float *latent, const float *k_pe, const int32_t *pos,
                      const int32_t *prefix, int32_t B, int32_t Q, double theta, double *ckv,
                      double *k_rope) {
    if (B < 1 || Q < 1 || !(theta > 0.0)) return NREF_EINVAL;
    int64_t off = 0;
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t i = 0; i < Q; ++i) {
            int64_t node = (int64_t)b * Q + i;
            int64_t r = off + prefix[b] + i;
            for (int c = 0; c < N_LAT; ++c) ckv[r * N_LAT + c] = (double)latent[node * N_LAT + c];
            ddtvref_rope_neox(k_pe + node * N_ROPE, pos[node], theta, k_rope + r * N_ROPE);
        }
        off += (int64_t)prefix[b] + Q;
    }
    return NREF_OK;
}
