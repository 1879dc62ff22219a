/*
 * ddtv.h -- DDTree tree-verify MLA-absorb attention for AMD Instinct MI355X (gfx950).
 *
 * The operation.  A draft tree of Q nodes (the root counts as a node) is verified
 * against one batch row of a multi-head latent attention (MLA) KV cache.  For
 * every (batch row b, tree node q, head h) the score against cache position j is
 *
 *     s_j = scale * ( q_abs[b,q,h,:] . ckv[j,:]  +  q_rope[b,q,h,:] . k_rope[j,:] )
 *
 * (512-d absorbed query against the 512-d cached latent, plus the 64-d rope
 * query against the 64-d rope key), a softmax runs over the positions the node
 * may see -- the whole shared prefix, its tree ancestors and itself -- and the
 * output is the softmax-weighted sum of the 512-d latents.  The per-head value
 * projection is NOT applied here; the caller runs it as a separate GEMM.
 *   Pages: "The Verify-Attn Kernel: A Single File Write That Completed a Critical
 *   Piece of the DDTree Engine", sections "The Design Journey: From Concept to
 *   CUDA" and "Design Decisions and Trade-Offs"; "The Moment of Truth:
 *   Validating a Custom CUDA Attention Kernel for Speculative Decoding",
 *   section "The Design Journey: From Theory to Silicon".
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless marked HOST.  The caller allocates and
 *     owns every buffer; the library never allocates, frees or synchronises,
 *     except ddtv_read_status (which synchronises the stream on purpose).
 *   - All device work is enqueued on `stream` and is asynchronous.
 *   - Argument checks happen on the host before any HIP call and return an error
 *     without touching the device.  Device-side launch failures map to
 *     DDTV_EDEVICE.  No exception crosses this interface.
 *   - Device pointers to float data must be 16-byte aligned.
 *   - Calls are re-entrant and thread-safe; calls on different streams may overlap
 *     (each with its own output and workspace buffers), except
 *     ddtv_verify_attn_noalloc, whose calls share one scratch per GPU.  The only
 *     state kept is a small cache of split plans (keyed by shapes, options, CU
 *     count, prefix lengths and workspace limit, guarded by a lock), the
 *     per-device CU count and the per-device address of that scratch; none of
 *     them changes results.
 */
#ifndef DDTV_H
#define DDTV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDTV_D_LATENT 512 /* latent (absorbed) width */
#define DDTV_D_ROPE 64    /* rope width */
#define DDTV_MAX_Q 256    /* largest supported tree (nodes incl. root) */

typedef enum {
    DDTV_OK = 0,
    DDTV_EINVAL = 1,       /* bad argument (null/misaligned pointer, bad size or scale) */
    DDTV_ETREE = 2,        /* a parent array is not a topologically ordered tree */
    DDTV_EUNSUPPORTED = 3, /* unsupported dtype, path or shape */
    DDTV_EWORKSPACE = 4,   /* workspace (or visibility buffer) too small */
    DDTV_EDEVICE = 5       /* a HIP call or kernel launch failed */
} ddtv_status;

/* Cache element types.  DDTV_FP8_E4M3 is the OCP 8-bit floating-point E4M3 format
 * ("fn" variant: sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
 * m * 2^-9, no infinities, 0x7F / 0xFF NaN; largest finite 448).  Cache values are
 * used as stored, with no scale: a per-tensor dequantisation scale s folds into
 * the caller's operands (q_abs * s_ckv and q_rope * s_krope before the call; out
 * * s_ckv after it). */
typedef enum { DDTV_F32 = 0, DDTV_BF16 = 1, DDTV_FP8_E4M3 = 2 } ddtv_dtype;

/* Per batch-row cache geometry, kept on the device (16 bytes). */
typedef struct {
    int64_t kv_off; /* first cache row of batch row b */
    int32_t prefix; /* P_b, shared-prefix length */
    int32_t kv_len; /* P_b + Q */
} ddtv_row;

/*
 * Visibility of a batch of trees (HOST struct, caller-owned; filled by
 * ddtv_build_visibility; plain data, so callers may also fill `bits` themselves).
 *
 * Tree node a of batch row b sits at cache row rows[b].kv_off + rows[b].prefix + a
 * (new KV rows are written right after the prefix, in node order -- "The
 * Architecture of an Inference Engine: Designing the Model Structure for DDTree
 * Speculative Decoding", section "What the Message Actually Says").  Batch rows
 * are packed back to back: kv_off(b) = sum over b' < b of (P_b' + Q).
 *
 * bits: word w, bit k (LSB first) of node i is set iff node 32w+k is i or an
 * ancestor of i.  Bits at positions >= Q are zero.  The prefix is implicit
 * (always visible) and has no bits.
 */
typedef struct {
    int32_t B, Q, W;     /* batch rows, tree nodes, mask words per node = ceil(Q/32) */
    int32_t max_kv;      /* max_b (P_b + Q) */
    int64_t total_kv;    /* sum_b (P_b + Q): cache rows spanned by the batch */
    uint32_t *bits;      /* DEVICE [B][Q][W] */
    ddtv_row *rows;      /* DEVICE [B] */
    int32_t *status;     /* DEVICE [B]: -1 if row b is a valid tree, else its lowest bad node */
    int32_t *order;      /* DEVICE [B] or NULL: the batch rows by cache length, longest first
                            (equal lengths: lower row first); a permutation of 0..B-1.  The
                            attention kernels start long rows first under the spread order. */
    const int32_t *prefix_host; /* HOST [B] or NULL: BORROWED from the build call; when set it
                                   must stay valid until the last verify call that plans with
                                   this struct returns (used only to balance KV splits) */
} ddtv_vis;

/* Bytes of device memory ddtv_build_visibility needs for B trees of Q nodes
 * (0 if B < 1 or Q outside 1..DDTV_MAX_Q). */
size_t ddtv_vis_bytes(int32_t B, int32_t Q);

/*
 * Draft-tree builder: the best-first tree of Q nodes from the drafter's per-depth
 * top-K log-probabilities, built on the device; its parent arrays feed
 * ddtv_build_visibility directly.
 *   Pages: "The Moment of Truth: Validating a Custom CUDA Attention Kernel for
 *   Speculative Decoding", section "Context: Building a Native DDTree Inference
 *   Engine" (a GPU best-first tree builder in place of a per-request CPU heap).
 *   The pages give no rule beyond "best first"; the one implemented is:
 *   - depth d = 1..D offers K choices, logp[b][d-1][0..K-1], in any order; a
 *     choice's rank is its place among them by descending log-probability,
 *     equal values by index k;
 *   - a node's score is its parent's score plus its choice's log-probability,
 *     summed in float32; the root (node 0) scores 0;
 *   - the next node is the untaken candidate with the highest score, over every
 *     child of every taken node; equal scores go to the candidate whose parent
 *     was taken first, then to the better rank.
 *   Node i's parent precedes it (parent[b][0] = -1), as ddtv_build_visibility requires.
 *
 *   logp    DEVICE float [B][D][K], finite
 *   tokens  DEVICE int32 [B][D][K] (token id of each choice) or NULL
 *   Q       nodes per tree including the root, 1..DDTV_MAX_Q; at most the
 *           1 + K + ... + K^D nodes that depth D allows
 *   K       1..64 choices per depth
 *   parent  DEVICE int32 [B][Q] out: parent node index, -1 for the root
 *   depth, rank, token  DEVICE int32 [B][Q] out or NULL: depth (root 0), choice
 *           rank (root -1), token id (root -1; tokens[b][d-1][k] for choice k, or
 *           k itself when tokens is NULL)
 *   score   DEVICE float [B][Q] out or NULL: cumulative log-probability
 * Nodes come out in the order they were taken, so scores are non-increasing when
 * every log-probability is <= 0.  Errors: DDTV_EINVAL (null logp or parent,
 * misaligned pointers, B < 1, D < 1, Q outside 1..DDTV_MAX_Q, Q beyond the depth-D
 * tree), DDTV_EUNSUPPORTED (K outside 1..64, B above 2^26), DDTV_EDEVICE.
 */
ddtv_status ddtv_build_tree(const float *logp, const int32_t *tokens, int32_t B, int32_t D, int32_t K,
                            int32_t Q, int32_t *parent, int32_t *depth, int32_t *rank, int32_t *token,
                            float *score, hipStream_t stream);

/*
 * S1: turn parent arrays into packed ancestor-or-self bit masks.
 *   Pages: "The Verify-Attn Kernel ...", section "The Design Journey" (each node
 *   sees the shared prefix and its tree ancestors); "The Architecture of an
 *   Inference Engine ...", section "Assumptions Embedded in the Design" (mask
 *   format left open; it is fixed here as packed bits).
 *
 *   parent     DEVICE int32 [B][Q].  parent[b][0] must be -1 (the root) and
 *              0 <= parent[b][i] < i for i >= 1 (parents precede children).
 *   prefix_len HOST int32 [B], each >= 0 (the host-tracked cache end).  Read
 *              during the call; its address is also stored in vis->prefix_host,
 *              so keep it alive while the struct is used for verify calls (or set
 *              vis->prefix_host to NULL afterwards).
 *   vis_buf    DEVICE buffer of at least ddtv_vis_bytes(B, Q) bytes, 256-byte
 *              aligned; bits, rows, status and order are carved out of it.
 *   vis        HOST struct filled on return (pointers into vis_buf).
 * Malformed trees are detected ON THE DEVICE: the call still returns DDTV_OK and
 * the lowest malformed node of each row is written to vis->status; a malformed
 * node sees only itself, and the ancestor chain of any node stops at the first
 * malformed node it meets (that node included), so attention stays defined.
 * Use ddtv_read_status to turn that into DDTV_ETREE.
 * Host-detected errors: DDTV_EINVAL (null pointers, B < 1, Q outside 1..256,
 * negative prefix, sum of KV rows >= 2^31 per row), DDTV_EWORKSPACE (vis_buf too
 * small).
 */
ddtv_status ddtv_build_visibility(const int32_t *parent, const int32_t *prefix_len,
                                  int32_t B, int32_t Q, void *vis_buf, size_t vis_buf_bytes,
                                  ddtv_vis *vis, hipStream_t stream);

/*
 * Synchronise `stream`, read vis->status and report the first malformed tree.
 *   bad_row, bad_node  HOST out (may be NULL): the lowest batch row with a
 *                      malformed tree and its lowest malformed node, or -1/-1.
 * Returns DDTV_OK, DDTV_ETREE, DDTV_EINVAL or DDTV_EDEVICE.  Not for hot loops.
 */
ddtv_status ddtv_read_status(const ddtv_vis *vis, int32_t *bad_row, int32_t *bad_node,
                             hipStream_t stream);

/* Execution path of the attention step. */
typedef enum {
    DDTV_PATH_AUTO = 0,     /* VALU when a batch row has fewer than 16 query rows (Q * H < 16),
                               MFMA otherwise: all heads share the latent cache, so the Q * H
                               rows of a batch row contract against each cache tile together */
    DDTV_PATH_VALU = 1,     /* vector-ALU kernel, fp32 arithmetic (any Q) */
    DDTV_PATH_MFMA = 2,     /* matrix-core kernel in the cache's precision (any Q): fp32 MFMA
                               for fp32 caches; bf16 MFMA with fp32 accumulation for bf16
                               caches (query and probabilities rounded to bf16); FP8 caches
                               take the fp32 MFMA kernel, widened exactly */
    DDTV_PATH_MFMA_F32 = 3  /* fp32 MFMA for any cache dtype (bf16 and FP8 widened exactly to
                               fp32): slower on bf16 caches, fp32-accurate */
} ddtv_path;

/* Order in which the main kernel's workgroups take their work items (batch row,
 * KV split, 64-row query tile).  MI355X deals workgroup i to XCD i % 8, and each
 * XCD has its own L2.  The order changes only which workgroup computes which
 * item: outputs are bit-identical under every order. */
typedef enum {
    DDTV_ORDER_AUTO = 0,       /* the planner picks the one with the shorter simulated schedule */
    DDTV_ORDER_XCD_LOCAL = 1,  /* consecutive work items on one XCD: the query tiles that read a
                                  cache tile share that XCD's L2; but each XCD then owns whole
                                  batch rows, which unbalances the XCDs when rows differ in length */
    DDTV_ORDER_SPREAD = 2      /* work item i on workgroup i: a batch row's query tiles go round
                                  all XCDs, which balances ragged batches, and batch rows start
                                  longest first (vis->order, when set); each XCD then reads every
                                  cache tile its query tiles need */
} ddtv_wg_order;

/* Optional controls for ddtv_verify_attn_ex (zero-initialise for defaults). */
typedef struct {
    int32_t path;          /* ddtv_path */
    int32_t split_len;     /* KV positions per split; 0 = automatic; else a multiple of 16 (cache
                              tiles hold 32 rows; the fp32 matrix kernel on an fp32 cache runs a
                              split's last tile of at most 16 rows as half a tile, the other
                              kernels mask the unused rows of a whole one).  In row-half mode (the
                              fp32 matrix kernel on batch rows of at most 32 query rows) a
                              row's last split also takes a remainder of up to 16 positions
                              rather than a split of its own: a row of n positions has
                              max(1, (n + L - 1 - 16) / L) splits there, ceil(n / L) elsewhere */
    hipEvent_t attn_begin; /* if non-NULL: recorded on `stream` right before the main kernel */
    hipEvent_t attn_end;   /* if non-NULL: recorded on `stream` right after it (before the merge) */
    int32_t wg_order;      /* ddtv_wg_order */
} ddtv_opts;

/* Workspace bytes ddtv_verify_attn(_ex) needs for this visibility, head count and
 * KV dtype (0 when no KV split is planned).  opts may be NULL. */
size_t ddtv_workspace_bytes(const ddtv_vis *vis, int32_t H, ddtv_dtype kv_dtype);
size_t ddtv_workspace_bytes_ex(const ddtv_vis *vis, int32_t H, ddtv_dtype kv_dtype,
                               const ddtv_opts *opts);

/*
 * S2..S7: masked absorbed-MLA attention of every (b, q, h) query row.
 *   Pages: "The Verify-Attn Kernel ...", sections "The Design Journey: From
 *   Concept to CUDA" (scores, max-subtracted softmax over visible positions,
 *   weighted latent sum), "Design Decisions and Trade-Offs" (latent output,
 *   separate value GEMM; long prefixes split and merged through log-sum-exp).
 *
 *   q_abs   DEVICE float [B][Q][H][512]  absorbed (nope) query, token-major
 *   q_rope  DEVICE float [B][Q][H][64]   rotated rope query
 *   ckv     DEVICE [vis->total_kv][512]  latent cache, float or bf16 per kv_dtype
 *   k_rope  DEVICE [vis->total_kv][64]   rotated rope keys, same dtype
 *   H       heads (>= 1); every head shares the one latent cache
 *   vis     HOST struct from ddtv_build_visibility (bits/rows must be complete on
 *           `stream` by the time the kernels run)
 *   scale   softmax scale applied to the summed dot product (finite)
 *   out     DEVICE float [B][Q][H][512]  softmax-weighted latent sum
 *   lse     DEVICE float [B][Q][H] or NULL: natural-log log-sum-exp of the scaled
 *           scores (-inf for a row that sees nothing)
 *   workspace, workspace_bytes  DEVICE scratch of at least ddtv_workspace_bytes()
 *           (may be NULL when that is 0), 256-byte aligned
 * A row that sees no position (possible only with a hand-made mask) gets out = 0
 * and lse = -inf.  Errors: DDTV_EINVAL, DDTV_EUNSUPPORTED, DDTV_EWORKSPACE,
 * DDTV_EDEVICE.
 */
ddtv_status ddtv_verify_attn(const float *q_abs, const float *q_rope, const void *ckv,
                             const void *k_rope, ddtv_dtype kv_dtype, int32_t H,
                             const ddtv_vis *vis, float scale, float *out, float *lse,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Same as ddtv_verify_attn with explicit controls (path, split length, timing
 * events).  opts may be NULL. */
ddtv_status ddtv_verify_attn_ex(const float *q_abs, const float *q_rope, const void *ckv,
                                const void *k_rope, ddtv_dtype kv_dtype, int32_t H,
                                const ddtv_vis *vis, float scale, float *out, float *lse,
                                void *workspace, size_t workspace_bytes, hipStream_t stream,
                                const ddtv_opts *opts);

/*
 * ddtv_verify_attn_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  It calls no hipMalloc, hipFree or other
 * allocating routine.  The split partials go to a scratch array that the library
 * holds in each GPU's memory (DDTV_NOALLOC_SCRATCH_BYTES per GPU, kept until the
 * process ends); the caller still passes inputs and outputs.
 *   Arguments, results and other errors: as ddtv_verify_attn_ex.  The automatic
 *   split choice only considers plans whose partials fit the scratch, so its
 *   plan may have fewer KV splits than ddtv_verify_attn_ex picks for the same
 *   call.  DDTV_EWORKSPACE: even the plan with the fewest splits (or the forced
 *   split length in opts) needs more than DDTV_NOALLOC_SCRATCH_BYTES; nothing is
 *   enqueued then.  DDTV_EDEVICE also covers a failed lookup of the scratch.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in time on
 *   one GPU (several streams or host threads) race on it and must be serialised
 *   by the caller.  Each call writes every partial it reads, so nothing carries
 *   over from the previous call.
 */
#define DDTV_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
ddtv_status ddtv_verify_attn_noalloc(const float *q_abs, const float *q_rope, const void *ckv,
                                     const void *k_rope, ddtv_dtype kv_dtype, int32_t H,
                                     const ddtv_vis *vis, float scale, float *out, float *lse,
                                     hipStream_t stream, const ddtv_opts *opts);

/*
 * External-prefix mode: the caller brings each query row's attention over the
 * shared prefix (from any prefix kernel); this call attends only the tree rows
 * and merges the two by log-sum-exp.
 *   Pages: "The Verify-Attn Kernel: A Single File Write ...", section "Design
 *   Decisions and Trade-Offs" (a prefix kernel for the long prefix, the masked
 *   kernel for the tree tail, merged by log-sum-exp).
 *   prefix_out  DEVICE float [B][Q][H][512], 16-byte aligned: softmax-weighted
 *               latent over the prefix rows only (normalised)
 *   prefix_lse  DEVICE float [B][Q][H]: its natural-log log-sum-exp; -inf for a
 *               batch row without prefix (prefix_out is then ignored)
 *   other arguments as for ddtv_verify_attn_ex; out/lse receive the merged result,
 *   which equals ddtv_verify_attn over prefix and tree when the prefix result is
 *   exact.  workspace: at least ddtv_tail_workspace_bytes(), 256-byte aligned
 *   (never NULL: the dense route keeps a row table and the tree rows' lse there).
 * Routes: with opts NULL, or path AUTO and split_len 0, one launch visits for
 * each node only its ancestors-or-self (fp32 arithmetic on any cache dtype,
 * cache values widened exactly) and merges the prefix result in the same pass;
 * a forced path or split length runs the attention kernels of ddtv_verify_attn_ex
 * over the tree rows, then a merge launch.
 * Errors: as ddtv_verify_attn_ex, plus DDTV_EINVAL for a null or misaligned prefix
 * result.
 */
size_t ddtv_tail_workspace_bytes(const ddtv_vis *vis, int32_t H, ddtv_dtype kv_dtype,
                                 const ddtv_opts *opts);
ddtv_status ddtv_verify_attn_tail(const float *q_abs, const float *q_rope, const void *ckv,
                                  const void *k_rope, ddtv_dtype kv_dtype, int32_t H,
                                  const ddtv_vis *vis, float scale, const float *prefix_out,
                                  const float *prefix_lse, float *out, float *lse,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream,
                                  const ddtv_opts *opts);

/* Describes the plan ddtv_verify_attn_ex would run (HOST out params, may be NULL):
 * path taken, KV positions per split, maximum splits per batch row, workgroups
 * of the main kernel, workgroup order (DDTV_ORDER_XCD_LOCAL or DDTV_ORDER_SPREAD).
 * Returns DDTV_EINVAL/DDTV_EUNSUPPORTED like the call would. */
ddtv_status ddtv_plan_info(const ddtv_vis *vis, int32_t H, ddtv_dtype kv_dtype,
                           const ddtv_opts *opts, int32_t *path, int32_t *split_len,
                           int32_t *n_split, int64_t *workgroups, int32_t *wg_order);

/*
 * Greedy tree acceptance after the verify step, then (optionally) the cache
 * compaction that drops the unaccepted branches.
 *   Pages: "The Moment of Truth: Validating a Custom CUDA Attention Kernel for
 *   Speculative Decoding", section "Context: Building a Native DDTree Inference
 *   Engine" (a greedy walk that decides which tree tokens are accepted); "The
 *   Architecture of an Inference Engine: Designing the Model Structure for DDTree
 *   Speculative Decoding", section "Input Knowledge Required" (the KV cache is
 *   compacted after acceptance).  The rule implemented:
 *   - pred[b][i] = argmax over v of logits[b][i][v] (float32; lowest index among
 *     equal maxima): the target's token after node i's path;
 *   - from the root, move to the lowest-index child whose draft token equals the
 *     current node's prediction; stop where there is none.  k = the number of
 *     moves (accepted draft tokens);
 *   - path[b][0..k] = the accepted nodes, root first, then -1;
 *     out_tokens[b][0..k] = the accepted nodes' draft tokens, then the last
 *     accepted node's prediction (the bonus token), then -1; accept_len[b] = k;
 *   - with ckv/k_rope: cache row prefix + path[j] of batch row b is copied to row
 *     prefix + j, j = 1..k, in place (rows at kv_off + prefix + node, as for the
 *     verify step); other rows are left as they are.
 *
 *   logits      DEVICE float [B][Q][V]; V >= 1
 *   parent      DEVICE int32 [B][Q], the trees that were verified (well formed:
 *               a malformed tree gives a walk over whatever its parents say)
 *   token       DEVICE int32 [B][Q] draft token of each node (token[b][0] unused)
 *   vis         HOST struct from ddtv_build_visibility for these trees (B, Q and
 *               the device row table give the cache geometry)
 *   ckv, k_rope DEVICE caches to compact (16-byte aligned), both or neither
 *   kv_dtype    their element type
 *   pred, path, out_tokens  DEVICE int32 [B][Q] out;  accept_len DEVICE int32 [B] out
 * Errors: DDTV_EINVAL (null or misaligned pointers, V < 1, one cache without the
 * other, a bad vis), DDTV_EUNSUPPORTED (dtype, more than 2^24 nodes), DDTV_EDEVICE.
 */
ddtv_status ddtv_tree_accept(const float *logits, int32_t V, const int32_t *parent,
                             const int32_t *token, const ddtv_vis *vis, void *ckv, void *k_rope,
                             ddtv_dtype kv_dtype, int32_t *pred, int32_t *path,
                             int32_t *out_tokens, int32_t *accept_len, hipStream_t stream);

/*
 * The steps around the attention (query preparation before it, the value
 * projection after it, the tree's new cache rows before both).
 *   Pages: "The Query-Split Kernel: A Pivotal Edit in Building a Native DDTree
 *   Inference Engine", sections "The Reasoning Chain" and "Input Knowledge" (the
 *   query projection of each token and head is a nope part followed by a rope
 *   part; the rope part gets NeoX rotary embedding with float64 angles; the nope
 *   part is absorbed into latent space through w_kc; the new key-value latents
 *   and rope keys are written to the cache); "The Verify-Attn Kernel ...",
 *   section "Design Decisions and Trade-Offs" (the attention returns the latent;
 *   a separate per-head GEMM with w_vc follows).
 *
 * Rotary embedding (NeoX, rotate-half form): pair i of a 64-wide vector x is
 * (x[i], x[i + 32]), i < 32; at position p it turns by a = p * theta^(-2i/64)
 * radians:  y[i] = x[i] cos a - x[i+32] sin a,  y[i+32] = x[i+32] cos a + x[i] sin a.
 * Frequencies, angles, sine, cosine and the rotation run in float64; results are
 * rounded once.  rope_theta: the rotary base (finite, > 0).
 *
 * Positions: node i of batch row b sits at position prefix[b] + depth(i) (root
 * depth 0), the position its token takes once its path is appended to the
 * prefix.  `positions` (DEVICE int32 [B][Q], or NULL) overrides this; when NULL
 * the depth is read from the ancestor-or-self masks of `vis` (depth + 1 bits).
 */

/*
 * Query preparation for the verify attention, in one launch: split, rotate, absorb.
 *   q       DEVICE float [B][Q][H][d_nope + 64]: the query projection of every
 *           tree node and head, nope part first (16-byte aligned)
 *   d_nope  width of the nope part: a multiple of 32 in 32..512
 *   vis     HOST struct from ddtv_build_visibility (B, Q and, when positions is
 *           NULL, the masks and row table; complete on `stream` when this runs)
 *   w_kc    DEVICE float [H][d_nope][512]: per-head absorb weights
 *   q_abs   DEVICE float [B][Q][H][512] out: q_abs[.., c] = sum_k nope[k] w_kc[h][k][c]
 *   q_rope  DEVICE float [B][Q][H][64] out: the rope part, rotated
 * The outputs are exactly the q_abs / q_rope operands of ddtv_verify_attn.
 * Errors: DDTV_EINVAL (null or misaligned pointers, H outside 1..1024, bad theta,
 * bad vis), DDTV_EUNSUPPORTED (d_nope, more than 2^28 nodes), DDTV_EDEVICE.
 */
ddtv_status ddtv_prepare_query(const float *q, int32_t d_nope, int32_t H, const ddtv_vis *vis,
                               const int32_t *positions, double rope_theta, const float *w_kc,
                               float *q_abs, float *q_rope, hipStream_t stream);

/*
 * Per-head value projection of the attention output (the separate GEMM after it).
 *   latent  DEVICE float [M][H][512]: ddtv_verify_attn's `out` (M = B * Q), 16-byte aligned
 *   w_vc    DEVICE float [H][d_v][512]: per-head value weights (16-byte aligned)
 *   v       DEVICE float [M][H][d_v] out: v[m][h][n] = sum_c latent[m][h][c] w_vc[h][n][c]
 *   d_v     1..512
 * M = 0 is a no-op.  Errors: DDTV_EINVAL (null or misaligned pointers, M < 0,
 * H outside 1..1024), DDTV_EUNSUPPORTED (d_v, M above 2^28), DDTV_EDEVICE.
 */
ddtv_status ddtv_value_proj(const float *latent, int64_t M, int32_t H, int32_t d_v, const float *w_vc,
                            float *v, hipStream_t stream);

/*
 * The tree nodes' new cache rows: node i of batch row b writes latent[b][i] and
 * its rope key rotated at its position to cache row kv_off(b) + prefix[b] + i
 * (the rows ddtv_verify_attn reads for the tree).  Other rows are untouched.
 *   latent  DEVICE float [B][Q][512] (16-byte aligned); k_pe DEVICE float [B][Q][64]
 *   vis, positions, rope_theta  as above
 *   ckv, k_rope  DEVICE caches ([total_kv][512], [total_kv][64]) of kv_dtype; ckv
 *           16-byte aligned.  Narrow caches receive the values rounded to nearest,
 *           ties to even: bf16 from the float32 value; FP8 E4M3 likewise, with
 *           magnitudes above 464 saturated to 448 (the largest finite code).
 *           Inputs must be finite (NaN and infinities are not encoded).
 * Errors: DDTV_EINVAL (null or misaligned pointers, bad theta, bad vis),
 * DDTV_EUNSUPPORTED (dtype, more than 2^26 nodes), DDTV_EDEVICE.
 */
ddtv_status ddtv_append_kv(const float *latent, const float *k_pe, const ddtv_vis *vis,
                           const int32_t *positions, double rope_theta, void *ckv, void *k_rope,
                           ddtv_dtype kv_dtype, hipStream_t stream);

/* Static description of a status code. */
const char *ddtv_status_string(ddtv_status s);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t ddtv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DDTV_H */
