/*
 * CPU oracle of the greedy tree-accept step and the KV compaction after it --
 * TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this code; the product library never does, and the two share no source.
 *
 * What it computes.  The pages describe a tree-accept step that walks the
 * verified tree greedily to find which draft tokens are accepted, taking the
 * longest valid prefix ("The Moment of Truth: Validating a Custom CUDA Attention
 * Kernel for Speculative Decoding", section "Context: Building a Native DDTree
 * Inference Engine"), and a KV cache compacted after acceptance to drop the
 * unaccepted branches ("The Architecture of an Inference Engine: Designing the
 * Model Structure for DDTree Speculative Decoding", section "Input Knowledge Required").
 * The reading taken here:
 *
 *   - the target model leaves, for every tree node i, logits over V tokens for
 *     the token that follows node i's path; its prediction pred[i] is their
 *     argmax (float32 comparisons, the lowest index among equal maxima);
 *   - the walk starts at the root (node 0); at node c it moves to the child of c
 *     (lowest node index first) whose draft token equals pred[c], and it stops
 *     at a node with no such child;
 *   - outputs: the accepted path (node indices, root first), its length minus
 *     one (k accepted draft tokens), and the k + 1 output tokens: the accepted
 *     nodes' draft tokens, then pred of the last accepted node (the bonus token);
 *   - compaction: node a's cache row sits at prefix + a (the tree rows follow the
 *     prefix in node order); after acceptance, the rows of path[1..k] move to
 *     prefix + 1 .. prefix + k, every other row keeping its content.
 */
#include <stdint.h>
#include <string.h>

enum { AREF_OK = 0, AREF_EINVAL = 1 };

/* pred[i] = argmax of logits[i][0..V-1] (float32; lowest index on ties) */
static int32_t argmax_row(const float *row, int32_t V) {
    int32_t best = 0;
    for (int32_t v = 1; v < V; ++v)
        if (row[v] > row[best]) best = v;
    return best;
}

/*
 * One batch row.  logits [Q][V], parent [Q] (a valid tree: parent[0] = -1,
 * 0 <= parent[i] < i), token [Q] (draft tokens; token[0] unused).  Outputs:
 * pred [Q], path [Q] (accepted nodes, then -1), out_tokens [Q] (k + 1 tokens,
 * then -1), *accept_len = k.
 */
int ddtvref_tree_accept_row(const float *logits, int32_t V, const int32_t *parent, const int32_t *token,
                            int32_t Q, int32_t *pred, int32_t *path, int32_t *out_tokens, int32_t *accept_len) {
    if (V < 1 || Q < 1 || parent[0] != -1) return AREF_EINVAL;
    for (int32_t i = 1; i < Q; ++i)
        if (parent[i] < 0 || parent[i] >= i) return AREF_EINVAL;
    for (int32_t i = 0; i < Q; ++i) pred[i] = argmax_row(logits + (int64_t)i * V, V);
    for (int32_t i = 0; i < Q; ++i) path[i] = out_tokens[i] = -1;
    int32_t cur = 0, k = 0;
    path[0] = 0;
    for (;;) {
        int32_t next = -1;
        for (int32_t c = cur + 1; c < Q; ++c)        /* children have larger indices */
            if (parent[c] == cur && token[c] == pred[cur]) {
                next = c;
                break;
            }
        if (next < 0) break;
        ++k;
        path[k] = next;
        out_tokens[k - 1] = token[next];
        cur = next;
    }
    out_tokens[k] = pred[cur];
    *accept_len = k;
    return AREF_OK;
}

/*
 * Compaction of one batch row's cache rows, out of place: dst starts as a copy
 * of src; then row prefix + j of dst receives row prefix + path[j] of src for
 * j = 1..k.  row_bytes bytes per row; rows are counted from the batch row's
 * first cache row.
 */
void ddtvref_compact_rows(const uint8_t *src, uint8_t *dst, int64_t n_rows, int64_t row_bytes, int32_t prefix,
                          const int32_t *path, int32_t k) {
    memcpy(dst, src, (size_t)(n_rows * row_bytes));
    for (int32_t j = 1; j <= k; ++j)
        memcpy(dst + (int64_t)(prefix + j) * row_bytes, src + (int64_t)(prefix + path[j]) * row_bytes,
               (size_t)row_bytes);
}
