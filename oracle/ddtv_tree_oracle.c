/*
 * CPU oracle of the best-first draft-tree builder -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this code; the product library never does, and the two share no source.
 *
 * What it computes ("The Moment of Truth: Validating a Custom CUDA Attention
 * Kernel for Speculative Decoding", section "Context: Building a Native DDTree
 * Inference Engine": a best-first tree builder that builds the draft tree in place
 * of a per-request CPU heap).  The pages give no more detail, so the reading
 * taken here is:
 *
 *   - the drafter supplies, for each batch row and each depth d = 1..D, its K best
 *     log-probabilities logp[d-1][0..K-1], sorted in descending order (one drafter
 *     pass gives a distribution per position), and optionally their token ids;
 *   - a tree node is a path of choices; its score is its parent's score plus the
 *     log-probability of its own choice, summed in float32; the root scores 0;
 *   - best first: repeatedly take the candidate with the highest score and make
 *     it the next tree node, until the tree has Q nodes.  Equal scores go to the
 *     candidate whose parent was taken first, then to the better-ranked choice:
 *     the order in which candidates appear when a taken node offers all K of its
 *     children at once;
 *   - taking node (depth d, choice r) offers its first child (depth d+1, choice 0)
 *     when d < D, and its next sibling (same parent, choice r+1) when d >= 1 and
 *     r+1 < K.  With log-probabilities sorted within each depth, a child never
 *     beats a better-ranked sibling under that order, so offering children one at
 *     a time takes the same nodes in the same order as offering all K at once,
 *     with at most two new candidates per step.
 *
 * The candidates are kept in a plain binary heap keyed by (score, parent, rank).
 * Outputs per node i (pop order): parent (-1 for the root), depth,
 * choice rank (-1 for the root), token (-1 for the root; tokens[depth-1][rank]
 * otherwise, or the rank when no token array is given) and score.
 */
#include <stdint.h>
#include <stdlib.h>

enum { TREF_OK = 0, TREF_EINVAL = 1 };

typedef struct {
    float score;
    int32_t parent;  /* tree index of the parent node, -1 for the root */
    int32_t depth;
    int32_t rank;
} Cand;

/* a before b in best-first order */
static int better(const Cand *a, const Cand *b) {
    if (a->score != b->score) return a->score > b->score;
    if (a->parent != b->parent) return a->parent < b->parent;
    return a->rank < b->rank;
}

static void heap_push(Cand *h, int *n, Cand c) {
    int i = (*n)++;
    h[i] = c;
    while (i > 0) {
        int p = (i - 1) / 2;
        if (!better(&h[i], &h[p])) break;
        Cand t = h[i]; h[i] = h[p]; h[p] = t;
        i = p;
    }
}

static Cand heap_pop(Cand *h, int *n) {
    Cand top = h[0];
    h[0] = h[--(*n)];
    int i = 0;
    for (;;) {
        int l = 2 * i + 1, r = l + 1, m = i;
        if (l < *n && better(&h[l], &h[m])) m = l;
        if (r < *n && better(&h[r], &h[m])) m = r;
        if (m == i) break;
        Cand t = h[i]; h[i] = h[m]; h[m] = t;
        i = m;
    }
    return top;
}

/* Number of nodes of the full K-ary tree of depth D, saturated at cap. */
int64_t ddtvref_tree_capacity(int32_t D, int32_t K, int64_t cap) {
    int64_t total = 1, level = 1;
    for (int d = 1; d <= D && total < cap; ++d) {
        level = (level > cap / (K > 0 ? K : 1)) ? cap : level * K;
        total += level;
        if (total > cap) total = cap;
    }
    return total;
}

/*
 * One batch row.  logp: [D][K] float, tokens: [D][K] int32 or NULL.  Outputs
 * [Q] each (any may be NULL).  Returns TREF_EINVAL for D < 1, K < 1, Q < 1 or a
 * Q larger than the full tree of depth D.
 */
int ddtvref_build_tree_row(const float *logp, const int32_t *tokens, int32_t D, int32_t K, int32_t Q,
                           int32_t *parent, int32_t *depth, int32_t *rank, int32_t *token, float *score) {
    if (D < 1 || K < 1 || Q < 1) return TREF_EINVAL;
    if (ddtvref_tree_capacity(D, K, (int64_t)Q) < Q) return TREF_EINVAL;
    Cand *heap = (Cand *)malloc(sizeof(Cand) * (size_t)(2 * Q + 2));
    float *node_score = (float *)malloc(sizeof(float) * (size_t)Q);
    if (!heap || !node_score) { free(heap); free(node_score); return TREF_EINVAL; }
    int n = 0;
    Cand root = {0.0f, -1, 0, -1};
    heap_push(heap, &n, root);
    for (int i = 0; i < Q; ++i) {
        if (n == 0) {   /* cannot happen once Q fits the full tree; guards the heap */
            free(heap);
            free(node_score);
            return TREF_EINVAL;
        }
        Cand c = heap_pop(heap, &n);
        node_score[i] = c.score;
        if (parent) parent[i] = c.parent;
        if (depth) depth[i] = c.depth;
        if (rank) rank[i] = c.rank;
        if (token) token[i] = c.depth == 0 ? -1 : (tokens ? tokens[(c.depth - 1) * K + c.rank] : c.rank);
        if (score) score[i] = c.score;
        if (c.depth < D) {                       /* first child */
            float s = c.score + logp[c.depth * K + 0];
            Cand ch = {s, i, c.depth + 1, 0};
            heap_push(heap, &n, ch);
        }
        if (c.depth >= 1 && c.rank + 1 < K) {   /* next sibling */
            float s = node_score[c.parent] + logp[(c.depth - 1) * K + c.rank + 1];
            Cand sb = {s, c.parent, c.depth, c.rank + 1};
            heap_push(heap, &n, sb);
        }
    }
    free(heap);
    free(node_score);
    return TREF_OK;
}
