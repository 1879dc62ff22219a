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
 *   - the drafter supplies, for each batch row and each depth d = 1..D, K choices
 *     with log-probabilities logp[d-1][0..K-1] in any order (one drafter pass
 *     gives a distribution per position), and optionally their token ids;
 *   - the choices of a depth are ranked by descending log-probability, equal
 *     values by their index k; a choice's rank is its place in that ranking;
 *   - a tree node is a path of choices; its score is its parent's score plus the
 *     log-probability of its own choice, summed in float32; the root scores 0;
 *   - best first: every child (depth d+1 <= D, each of the K choices) of every
 *     taken node is a candidate; repeatedly take the candidate with the highest
 *     score as the next tree node, until the tree has Q nodes.  Equal scores go
 *     to the candidate whose parent was taken first, then to the better-ranked
 *     choice.
 *
 * Written out plainly: a binary heap of candidates keyed by (score, parent,
 * rank); taking a node pushes all K of its children.  Outputs per node i (pop
 * order): parent (-1 for the root), depth, rank (-1 for the root), token (-1 for
 * the root; tokens[depth-1][k] for choice k, or k itself when no token array is
 * given) and score.
 */
#include <stdint.h>
#include <stdlib.h>

enum { TREF_OK = 0, TREF_EINVAL = 1 };

typedef struct {
    float score;
    int32_t parent;  /* tree index of the parent node, -1 for the root */
    int32_t depth;
    int32_t rank;    /* the choice's rank within its depth, -1 for the root */
    int32_t choice;  /* the choice's index k within its depth, -1 for the root */
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

/* The ranking of one depth's choices: descending value, equal values by index. */
typedef struct {
    float v;
    int32_t k;
} Choice;

static int choice_order(const void *pa, const void *pb) {
    const Choice *a = (const Choice *)pa, *b = (const Choice *)pb;
    if (a->v != b->v) return a->v > b->v ? -1 : 1;
    return a->k < b->k ? -1 : (a->k > b->k ? 1 : 0);
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
    /* a taken node's depth is below the number of nodes taken, so only the first
       min(D, Q) depths are ever read */
    const int Dr = D < Q ? D : Q;
    int32_t *rank_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)Dr * (size_t)K);
    Choice *sorted = (Choice *)malloc(sizeof(Choice) * (size_t)K);
    Cand *heap = (Cand *)malloc(sizeof(Cand) * ((size_t)Q * (size_t)K + 1));
    if (!rank_of || !sorted || !heap) {
        free(rank_of); free(sorted); free(heap);
        return TREF_EINVAL;
    }
    for (int d = 0; d < Dr; ++d) {
        for (int k = 0; k < K; ++k) {
            sorted[k].v = logp[d * K + k];
            sorted[k].k = k;
        }
        qsort(sorted, (size_t)K, sizeof(Choice), choice_order);
        for (int r = 0; r < K; ++r) rank_of[d * K + sorted[r].k] = r;
    }
    int n = 0;
    Cand root = {0.0f, -1, 0, -1, -1};
    heap_push(heap, &n, root);
    int rc = TREF_OK;
    for (int i = 0; i < Q; ++i) {
        if (n == 0) {   /* cannot happen once Q fits the full tree; guards the heap */
            rc = TREF_EINVAL;
            break;
        }
        Cand c = heap_pop(heap, &n);
        if (parent) parent[i] = c.parent;
        if (depth) depth[i] = c.depth;
        if (rank) rank[i] = c.rank;
        if (token) token[i] = c.depth == 0 ? -1 : (tokens ? tokens[(c.depth - 1) * K + c.choice] : c.choice);
        if (score) score[i] = c.score;
        if (c.depth < D) {   /* offer every child (c.depth <= i < Q, so c.depth < Dr) */
            for (int k = 0; k < K; ++k) {
                float s = c.score + logp[c.depth * K + k];
                Cand ch = {s, i, c.depth + 1, rank_of[c.depth * K + k], k};
                heap_push(heap, &n, ch);
            }
        }
    }
    free(rank_of);
    free(sorted);
    free(heap);
    return rc;
}
