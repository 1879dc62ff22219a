/*
 * ddtv_oracle.c -- CPU oracle for DDTree tree-verify MLA-absorb attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source, header, table or helper with the HIP
 * library.
 *
 * Plain, slow, single-threaded C.  Every floating-point step runs in double:
 * float inputs and bf16 bit patterns are widened exactly, sums run in index
 * order, exp/log come from libm.  Nothing is blocked, fused or reordered beyond
 * the definition below.
 *
 * What it computes (the plain definition of masked softmax attention in the
 * absorbed MLA form):
 *
 *   Pages: "The Verify-Attn Kernel: A Single File Write That Completed a Critical
 *   Piece of the DDTree Engine", sections "The Design Journey: From Concept to
 *   CUDA" (score = absorbed-query . cached latent + rope . rope; softmax over the
 *   visible positions with max subtraction; output is the weighted sum of
 *   latents) and "Design Decisions and Trade-Offs" (the kernel returns the
 *   512-d latent; the per-head value projection is a separate GEMM; prefix and
 *   tree tail can be attended separately and merged through log-sum-exp).
 *   "The Moment of Truth: Validating a Custom CUDA Attention Kernel for
 *   Speculative Decoding", section "The Design Journey: From Theory to Silicon"
 *   (same score and output contract).
 *
 *   Visibility: a tree node sees the whole shared prefix, its ancestors and
 *   itself -- "The Verify-Attn Kernel ...", sections "The Design Journey" and
 *   "Assumptions and the Path Forward" (every query sees at least its own
 *   position).  Tree nodes' KV rows sit right after the prefix, in node order --
 *   "The Architecture of an Inference Engine: ...", section "What the Message
 *   Actually Says" (new latents are written at cache positions starting at the
 *   prefix length).
 *
 * Readings taken where the pages are silent (all listed with reasons in the
 * design notes): parent[0] = -1 is the single root and parent[i] < i for i >= 1
 * (required, not repaired); masks are packed uint32, LSB first, tree columns
 * only, padding bits zero; the value is the 512-d latent only; an empty visible
 * set gives out = 0 and lse = -inf.
 *
 * Every function here is pinned by the CPU tests (closed forms, library
 * routines, invariants and brute force); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_OK 0
#define REF_EINVAL 1
#define REF_ETREE 2

#define D_LAT 512
#define D_ROPE 64

/* ----------------------------------------------------------------------------
 * Scalars
 * ------------------------------------------------------------------------- */

/* A bf16 value is the top 16 bits of a float32: widening is exact. */
static double bf16_value(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* An FP8 E4M3 value (the OCP 8-bit floating-point format, "fn" variant): sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals
 * m * 2^-9; no infinities; the all-ones magnitude 0x7F is NaN. */
double ddtvref_fp8_value(uint8_t b)
{
    int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

static double kv_value(const void *base, int kv_dtype, int64_t idx)
{
    if (kv_dtype == 0) return (double)((const float *)base)[idx];
    if (kv_dtype == 2) return ddtvref_fp8_value(((const uint8_t *)base)[idx]);
    return bf16_value(((const uint16_t *)base)[idx]);
}

int ddtvref_words(int Q) { return (Q + 31) / 32; }

/* ----------------------------------------------------------------------------
 * Tree validation and visibility (ancestor-or-self sets by explicit walk)
 * ------------------------------------------------------------------------- */

/* Node i of a tree is well formed iff (i == 0 and parent == -1) or
 * (i >= 1 and 0 <= parent < i). */
static int node_ok(const int32_t *par, int i)
{
    if (i == 0) return par[0] == -1;
    return par[i] >= 0 && par[i] < i;
}

/*
 * Build the visibility bits of B trees of Q nodes.
 *   parent  [B][Q]
 *   bits    [B][Q][W]  out; bit k of word w of node i is set iff node 32w+k is
 *                      i itself or an ancestor of i
 *   bad     [B]        out; lowest malformed node of row b, or -1
 * A malformed node sees only itself; the walk from any node stops at the first
 * malformed node it reaches (that node's bit included).
 * Returns REF_ETREE if any row is malformed, REF_OK otherwise.
 */
int ddtvref_build_visibility(const int32_t *parent, int B, int Q,
                             uint32_t *bits, int32_t *bad)
{
    if (B < 1 || Q < 1) return REF_EINVAL;
    const int W = ddtvref_words(Q);
    int rc = REF_OK;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (int64_t)b * Q;
        bad[b] = -1;
        for (int i = 0; i < Q; ++i) {
            if (!node_ok(par, i)) {
                bad[b] = i;
                rc = REF_ETREE;
                break;
            }
        }
        for (int i = 0; i < Q; ++i) {
            uint32_t *row = bits + ((int64_t)b * Q + i) * W;
            for (int w = 0; w < W; ++w) row[w] = 0u;
            int cur = i;
            for (;;) {
                row[cur / 32] |= 1u << (cur % 32);
                if (!node_ok(par, cur) || cur == 0) break;
                cur = par[cur];
            }
        }
    }
    return rc;
}

/* ----------------------------------------------------------------------------
 * Attention
 * ------------------------------------------------------------------------- */

/* Packed cache layout: batch row b occupies rows kv_off(b) .. kv_off(b)+P_b+Q-1,
 * with kv_off(b) = sum over b' < b of (P_b' + Q).  Node a of row b is at
 * kv_off(b) + P_b + a. */
static int64_t kv_offset(const int32_t *prefix, int Q, int b)
{
    int64_t off = 0;
    for (int i = 0; i < b; ++i) off += (int64_t)prefix[i] + Q;
    return off;
}

/* Visible flag of cache position j (0 <= j < P_b + Q) for node q of row b. */
static int visible(const uint32_t *bits, int Q, int P, int b, int q, int64_t j)
{
    if (j < P) return 1;
    const int W = ddtvref_words(Q);
    int64_t a = j - P;
    const uint32_t *row = bits + ((int64_t)b * Q + q) * W;
    return (row[a / 32] >> (a % 32)) & 1u;
}

/* Unscaled-then-scaled score of one query row against one cache row. */
static double score(const float *qa, const float *qr, const void *ckv, const void *krope,
                    int kv_dtype, int64_t row, double scale)
{
    double nope = 0.0, rope = 0.0;
    for (int d = 0; d < D_LAT; ++d)
        nope += (double)qa[d] * kv_value(ckv, kv_dtype, row * D_LAT + d);
    for (int t = 0; t < D_ROPE; ++t)
        rope += (double)qr[t] * kv_value(krope, kv_dtype, row * D_ROPE + t);
    return scale * (nope + rope);
}

/*
 * One query row (b, q, h):
 *   out[512] = sum_j p_j * ckv_j,  p_j = exp(s_j - m) / l,  lse = m + ln l,
 * over the visible positions j.  probs (optional, length P_b + Q) receives p_j
 * (0 for invisible positions); psum (optional) receives sum_j p_j.
 */
static void attend_row(const float *q_abs, const float *q_rope, const void *ckv,
                       const void *k_rope, int kv_dtype, int B, int Q, int H,
                       const int32_t *prefix, const uint32_t *bits, double scale,
                       int b, int q, int h, double *out, double *lse,
                       double *probs, double *psum)
{
    (void)B;
    const int P = prefix[b];
    const int64_t kv = (int64_t)P + Q;
    const int64_t base = kv_offset(prefix, Q, b);
    const float *qa = q_abs + (((int64_t)b * Q + q) * H + h) * D_LAT;
    const float *qr = q_rope + (((int64_t)b * Q + q) * H + h) * D_ROPE;

    double *s = (double *)malloc(sizeof(double) * (size_t)(kv > 0 ? kv : 1));
    double m = -INFINITY;
    for (int64_t j = 0; j < kv; ++j) {
        if (!visible(bits, Q, P, b, q, j)) continue;
        s[j] = score(qa, qr, ckv, k_rope, kv_dtype, base + j, scale);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int d = 0; d < D_LAT; ++d) out[d] = 0.0;
    if (m == -INFINITY) {               /* empty visible set */
        *lse = -INFINITY;
        if (probs) for (int64_t j = 0; j < kv; ++j) probs[j] = 0.0;
        if (psum) *psum = 0.0;
        free(s);
        return;
    }
    for (int64_t j = 0; j < kv; ++j) {
        if (!visible(bits, Q, P, b, q, j)) continue;
        s[j] = exp(s[j] - m);           /* reuse s[] for the unnormalised weight */
        l += s[j];
    }
    for (int64_t j = 0; j < kv; ++j) {
        if (!visible(bits, Q, P, b, q, j)) continue;
        const int64_t row = base + j;
        for (int d = 0; d < D_LAT; ++d)
            out[d] += s[j] * kv_value(ckv, kv_dtype, row * D_LAT + d);
    }
    for (int d = 0; d < D_LAT; ++d) out[d] /= l;
    *lse = m + log(l);
    if (probs || psum) {
        double acc = 0.0;
        for (int64_t j = 0; j < kv; ++j) {
            double p = visible(bits, Q, P, b, q, j) ? s[j] / l : 0.0;
            if (probs) probs[j] = p;
            acc += p;
        }
        if (psum) *psum = acc;
    }
    free(s);
}

static int check_shapes(int B, int Q, int H, const int32_t *prefix, int kv_dtype)
{
    if (B < 1 || Q < 1 || H < 1) return REF_EINVAL;
    if (kv_dtype < 0 || kv_dtype > 2) return REF_EINVAL;
    for (int b = 0; b < B; ++b)
        if (prefix[b] < 0) return REF_EINVAL;
    return REF_OK;
}

/*
 * Attention for a list of query rows.
 *   q_abs  float [B][Q][H][512], q_rope float [B][Q][H][64]
 *   ckv    [sum_b (P_b+Q)][512], k_rope [..][64]; float (kv_dtype 0), bf16 bits (1)
 *          or FP8 E4M3 bytes (2)
 *   prefix int32 [B], bits uint32 [B][Q][W]
 *   rows   flat row ids (b*Q + q)*H + h, n of them; NULL means every row in order
 *   out    double [n][512], lse double [n], psum double [n] (may be NULL)
 */
int ddtvref_verify_attn_rows(const float *q_abs, const float *q_rope, const void *ckv,
                             const void *k_rope, int kv_dtype, int B, int Q, int H,
                             const int32_t *prefix, const uint32_t *bits, double scale,
                             const int64_t *rows, int64_t n, double *out, double *lse,
                             double *psum)
{
    int rc = check_shapes(B, Q, H, prefix, kv_dtype);
    if (rc) return rc;
    const int64_t total = (int64_t)B * Q * H;
    if (!rows) n = total;
    for (int64_t k = 0; k < n; ++k) {
        int64_t r = rows ? rows[k] : k;
        if (r < 0 || r >= total) return REF_EINVAL;
        int h = (int)(r % H);
        int q = (int)((r / H) % Q);
        int b = (int)(r / ((int64_t)H * Q));
        attend_row(q_abs, q_rope, ckv, k_rope, kv_dtype, B, Q, H, prefix, bits, scale,
                   b, q, h, out + k * D_LAT, lse + k, NULL, psum ? psum + k : NULL);
    }
    return REF_OK;
}

/* Probabilities p_j (length P_b + Q, zero where invisible) of one query row. */
int ddtvref_row_probs(const float *q_abs, const float *q_rope, const void *ckv,
                      const void *k_rope, int kv_dtype, int B, int Q, int H,
                      const int32_t *prefix, const uint32_t *bits, double scale,
                      int64_t row, double *probs)
{
    int rc = check_shapes(B, Q, H, prefix, kv_dtype);
    if (rc) return rc;
    if (row < 0 || row >= (int64_t)B * Q * H) return REF_EINVAL;
    int h = (int)(row % H);
    int q = (int)((row / H) % Q);
    int b = (int)(row / ((int64_t)H * Q));
    double out[D_LAT], lse, psum;
    attend_row(q_abs, q_rope, ckv, k_rope, kv_dtype, B, Q, H, prefix, bits, scale,
               b, q, h, out, &lse, probs, &psum);
    return REF_OK;
}

/* ----------------------------------------------------------------------------
 * Split-KV partials and their log-sum-exp merge
 *
 * Pages: "The Verify-Attn Kernel ...", section "Design Decisions and
 * Trade-Offs", and "The Moment of Truth ...", section "The Design Journey:
 * From Theory to Silicon": attention over a long prefix and over the tree tail
 * can be computed separately and combined through log-sum-exp.
 * ------------------------------------------------------------------------- */

/*
 * Partial attention of one query vector (576 = 512 + 64 values, widened from
 * float) over an explicit list of cache rows:
 *   m = max_j s_j, l = sum_j exp(s_j - m), o[d] = sum_j exp(s_j - m) ckv_j[d]
 * (o is NOT divided by l).  An empty list gives m = -inf, l = 0, o = 0.
 */
int ddtvref_partial(const float *qa, const float *qr, const void *ckv, const void *k_rope,
                    int kv_dtype, const int64_t *idx, int64_t n, double scale,
                    double *m_out, double *l_out, double *o)
{
    if (kv_dtype < 0 || kv_dtype > 2) return REF_EINVAL;
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double m = -INFINITY;
    for (int64_t k = 0; k < n; ++k) {
        s[k] = score(qa, qr, ckv, k_rope, kv_dtype, idx[k], scale);
        if (s[k] > m) m = s[k];
    }
    for (int d = 0; d < D_LAT; ++d) o[d] = 0.0;
    double l = 0.0;
    if (m != -INFINITY) {
        for (int64_t k = 0; k < n; ++k) {
            double e = exp(s[k] - m);
            l += e;
            for (int d = 0; d < D_LAT; ++d) o[d] += e * kv_value(ckv, kv_dtype, idx[k] * D_LAT + d);
        }
    }
    *m_out = m;
    *l_out = l;
    free(s);
    return REF_OK;
}

/*
 * Merge S partials (m_s, l_s, o_s) of one query row:
 *   M = max_s m_s, L = sum_s exp(m_s - M) l_s,
 *   out = sum_s exp(m_s - M) o_s / L,  lse = M + ln L.
 * Partials with m_s = -inf carry no weight; if all are empty, out = 0, lse = -inf.
 */
int ddtvref_merge(int S, const double *m, const double *l, const double *o,
                  double *out, double *lse)
{
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
        if (m[s] > M) M = m[s];
    for (int d = 0; d < D_LAT; ++d) out[d] = 0.0;
    if (M == -INFINITY) {
        *lse = -INFINITY;
        return REF_OK;
    }
    double L = 0.0;
    for (int s = 0; s < S; ++s) {
        if (m[s] == -INFINITY) continue;
        double w = exp(m[s] - M);
        L += w * l[s];
        for (int d = 0; d < D_LAT; ++d) out[d] += w * o[(int64_t)s * D_LAT + d];
    }
    for (int d = 0; d < D_LAT; ++d) out[d] /= L;
    *lse = M + log(L);
    return REF_OK;
}
