/*
 * spec_verify.h -- C ABI of the EAGLE-2/3 tree-verification library for
 * AMD MI355X (gfx950).  ABI version 1.
 *
 * One verify step of speculative decoding with a draft tree is three calls,
 * issued in this order on one HIP stream:
 *
 *   spec_verify_tree_attn  attention of every tree node over the committed
 *                          prefix KV plus its own ancestors (tree mask);
 *   spec_accept_tree       the Leviathan acceptance rule walked down the tree;
 *   spec_kv_commit         gather the accepted path's KV rows behind the
 *                          prefix and advance the logical length.
 *
 * Pages the operations follow (cited by title and section):
 *   [LESSON] "推测解码与 EAGLE-3": section "不变量：Leviathan 拒绝采样"
 *            (the rule and one pass returning N+1 distributions), section
 *            "KV cache 回滚" (rollback; tree attention is one attention call
 *            with a mask that follows the tree), build steps 1-4;
 *   [GUIDE]  "EAGLE-1/2/3 拆解": section "一个可核对的经验性质" (a node is
 *            accepted only if its whole root path is), section on EAGLE-2's
 *            two stages (the tree mask starts as the identity);
 *   [TTT]    "EAGLE-3 完全拆解": section on the training-time attention mask
 *            (each token sees only its ancestors).
 *
 * Common conventions
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The
 *     library keeps no pointer after the stream work completes and allocates
 *     no device memory; scratch space comes from the caller's `workspace`,
 *     sized by the *_workspace_size functions for the same arguments and the
 *     same current device.  Its only host state is cached device properties
 *     (compute-unit count, occupancy) and an atomic launch counter, so calls
 *     from several host threads are safe; calls that share a workspace must
 *     be ordered on one stream.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *     asynchronous on it; outputs are valid once the caller synchronises.
 *   - A negative status is returned, before anything is launched, for any
 *     problem the host can see (NULL pointers, sizes, dtype, scalars,
 *     workspace size).  SPEC_E_HIP reports a failed launch.
 *   - Problems only the device can see are OR-ed into *dev_error (a device
 *     int32, may be NULL) as SPEC_DEVERR_* bits; the affected sequence is
 *     skipped (attention output rows left untouched; accept_len = -1).  The
 *     library never clears *dev_error; the caller zeroes it.
 *   - Trees: node 0 of sequence b is the pending root (the token emitted by
 *     the previous step, whose KV this verify pass produced); parents[b][0]
 *     = -1 and 0 <= parents[b][j] < j for 1 <= j < n_nodes[b] (topological
 *     ids).  Tree node j's K/V sit in cache row prefix_len[b] + j.
 *   - Limits: n_max <= 64, head_dim in {16, 32, 64, 128}, Hq % Hkv == 0.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 2
#define SPEC_MAX_NODES 64
#define SPEC_TREE_MAX_TOP_K 16  /* children per expanded node (tree construction) */
#define SPEC_TREE_MAX_DEPTH 16  /* levels of a constructed tree                   */

typedef int32_t spec_status_t;

enum {
  SPEC_OK = 0,
  SPEC_E_NULL = -1,        /* a required pointer is NULL                          */
  SPEC_E_SHAPE = -2,       /* a size argument is out of range, or a buffer that
                              must be 16-byte aligned is not                      */
  SPEC_E_DTYPE = -3,       /* unsupported dtype / head_dim combination            */
  SPEC_E_VALUE = -4,       /* bad scalar (temperature < 0 or NaN, scale <= 0)     */
  SPEC_E_WORKSPACE = -5,   /* workspace NULL, smaller than required, or (where it
                              must be) not 16-byte aligned                        */
  SPEC_E_HIP = -6,         /* a HIP runtime call or launch failed                 */
  SPEC_E_UNSUPPORTED = -7, /* the current device cannot run this configuration    */
  SPEC_E_SCRATCH = -8      /* the call needs more device scratch than the
                              library's fixed array holds (spec_accept_tree_noalloc) */
};

enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

/* How spec_accept_tree_ex launches the walk (its `launch` argument). */
enum { SPEC_LAUNCH_ORDINARY = 0, SPEC_LAUNCH_COOPERATIVE = 1 };

enum {
  SPEC_DEVERR_TREE = 1,       /* n_nodes outside [1, n_max], bad parents, depth > max_depth */
  SPEC_DEVERR_TOKEN = 2,      /* a draft token outside [0, V)                              */
  SPEC_DEVERR_NONFINITE = 4,  /* NaN/Inf in a logits or draft-probability entry read       */
  SPEC_DEVERR_CAPACITY = 8,   /* prefix_len < 0 or prefix_len + n_nodes > L_cap            */
  SPEC_DEVERR_SYNC = 16,      /* an inter-workgroup wait hit its bound (walk abandoned;
                                 spec_accept_tree outputs of the batch unspecified)        */
  SPEC_DEVERR_ALIGN = 32      /* a per-layer buffer of spec_kv_commit_layers(_paged) off
                                 16-byte alignment (nothing of the call committed)         */
};

/* One near-tie record of spec_accept_tree (kind 0: accept test, 1: sample,
 * 2: residual whose mass fell below 1e-12 of the previous one, so rounding
 * may decide whether it is zero, 3: top-p boundary of spec_accept_tree_ex
 * within 1e-8 of a kept or dropped token's mass above). */
typedef struct {
  int32_t b;      /* sequence                                             */
  int32_t node;   /* child tested (kinds 0, 2) or node visited (1, 3)     */
  int32_t kind;
  float u;        /* the uniform used (kind 3: top_p)                     */
  double margin;  /* |u - min(1, ratio)|; distance of u*W to the chosen
                     bucket's nearer edge divided by W; new / old
                     residual mass; or |mass above - top_p|               */
} spec_tie_t;

/*
 * spec_verify_tree_attn -- tree-masked attention ([LESSON] "KV cache 回滚";
 * [GUIDE] identity initial tree mask; [TTT] ancestors-only mask).
 *
 * For every sequence b, tree node i < n_nodes[b] and query head h:
 *   out[b][i][h] = softmax(scale * q[b][i][h] . K^T) V
 * over the keys/values of KV head h / (Hq/Hkv) in cache rows
 * [0, prefix_len[b]) (the committed prefix) and rows prefix_len[b] + j for
 * every j on the root-to-i path, i included -- exactly the last row of causal
 * attention over "prefix, then path(i)".
 *
 *   q          [B][n_max][Hq][head_dim], dtype; already position-encoded
 *   k_cache,   [B][Hkv][L_cap][head_dim], dtype; the caller has written the
 *   v_cache    tree's K/V into rows [prefix_len[b], prefix_len[b]+n_nodes[b])
 *   prefix_len [B] int32, n_nodes [B] int32, parents [B][n_max] int32
 *   scale      softmax scale (> 0; pass 1/sqrt(head_dim) for the usual one)
 *   dtype      SPEC_BF16 (any head_dim; the 128 case uses matrix cores) or
 *              SPEC_F32 (vector ALU only)
 *   out        [B][n_max][Hq][head_dim] float32; rows i >= n_nodes[b] and
 *              rows of failed sequences are not written
 *   workspace  >= spec_verify_tree_attn_workspace_size(...) bytes
 * The matrix-core path (SPEC_BF16, head_dim 128) moves 16-byte vectors: q,
 * k_cache, v_cache and out must then be 16-byte aligned (else SPEC_E_SHAPE),
 * and so must a workspace it uses (else SPEC_E_WORKSPACE).
 * Device errors: SPEC_DEVERR_TREE, SPEC_DEVERR_CAPACITY.
 */
spec_status_t spec_verify_tree_attn(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* parents,
    int32_t B, int32_t n_max, int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t L_cap,
    float scale, int32_t dtype, float* out,
    void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream);

size_t spec_verify_tree_attn_workspace_size(
    int32_t B, int32_t n_max, int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t L_cap,
    int32_t dtype);

/*
 * spec_verify_tree_attn_rope -- spec_verify_tree_attn with the rotary
 * position embedding of the queries fused in: q holds the queries before
 * rotation, and query row (b, i) is rotated at position prefix_len[b] +
 * depth(i) before the contraction (the draft candidates of one level share a
 * position: [GUIDE], the init_tree passage, where a level's position ids
 * start as zeros).  The rotation is the published rotary embedding: plane t
 * of the head dimension turns by pos * inv_freq[t].  The cache holds keys
 * already rotated (spec_tree_kv_write writes the tree's rows that way).
 *
 *   inv_freq    [head_dim/2] float32 device array (any frequency schedule,
 *               e.g. base^(-2t/head_dim) or a rescaled one)
 *   rope_style  1: plane t pairs dimensions t and t + head_dim/2 (the
 *               LLaMA-family layout); 2: dimensions 2t and 2t + 1
 * On the matrix-core path the rotated query is rounded to bf16, as a query
 * rotated by the caller would be; on the vector path it stays float32.
 * Other arguments, outputs and errors as spec_verify_tree_attn; a NULL
 * inv_freq is SPEC_E_NULL and another rope_style SPEC_E_VALUE.
 */
spec_status_t spec_verify_tree_attn_rope(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
    const int32_t* n_nodes, const int32_t* parents, int32_t B, int32_t n_max, int32_t Hq,
    int32_t Hkv, int32_t head_dim, int32_t L_cap, float scale, int32_t dtype,
    const float* inv_freq, int32_t rope_style, float* out, void* workspace,
    size_t workspace_bytes, int32_t* dev_error, void* stream);

/*
 * spec_tree_kv_write -- the verify pass's write of the tree's keys and values
 * into the cache, keys rotated ([LESSON] "KV cache 回滚": the verify pass
 * extends the cache by the tree's rows; positions as for
 * spec_verify_tree_attn_rope).  For every sequence b and node j <
 * n_nodes[b], cache row prefix_len[b] + j of every KV head receives
 * k_new[b][j][h] rotated at position prefix_len[b] + depth(j) (unrotated if
 * inv_freq is NULL) and v_new[b][j][h].  Other cache rows are not touched.
 *
 *   k_new, v_new      [B][n_max][Hkv][head_dim], dtype (must not overlap the
 *                     cache)
 *   k_cache, v_cache  [B][Hkv][L_cap][head_dim], dtype (in/out)
 *   prefix_len, n_nodes, parents   as for spec_verify_tree_attn
 *   head_dim          even, <= 1024
 *   inv_freq, rope_style           as for spec_verify_tree_attn_rope, or
 *                     inv_freq NULL (rope_style ignored)
 * bf16 results are rounded to nearest even.
 * Device errors: SPEC_DEVERR_TREE, SPEC_DEVERR_CAPACITY (the sequence is not
 * written).
 */
spec_status_t spec_tree_kv_write(const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const int32_t* prefix_len,
                                 const int32_t* n_nodes, const int32_t* parents, int32_t B,
                                 int32_t n_max, int32_t Hkv, int32_t head_dim, int32_t L_cap,
                                 int32_t dtype, const float* inv_freq, int32_t rope_style,
                                 int32_t* dev_error, void* stream);

/*
 * spec_accept_tree -- the acceptance walk ([LESSON] "不变量：Leviathan 拒绝
 * 采样" and build steps 1-3; [GUIDE] prefix property of tree acceptance).
 *
 * q_v = softmax(logits[b][v] / temperature), in float64.  Starting at the
 * root v = 0: the children c of v are tested in ascending id; child c (token
 * x) is accepted if draft_p[b][v][x] <= 0, else iff
 *   u_accept[b][c] < min(1, cur(x) / draft_p[b][v][x]),
 * where cur starts as q_v and, after each rejected child, becomes the
 * residual norm(max(0, cur - p_v)) (a zero-mass residual leaves cur as it
 * is).  On acceptance the walk descends to c.  When no child is accepted
 * (or v is a leaf) the terminal token is drawn from cur with u_sample[b][v]
 * by inverse CDF in ascending token id (smallest i whose running sum exceeds
 * u * total mass); at a leaf that is the bonus token from q_v.
 * temperature == 0 is greedy: a child is accepted iff its token is the
 * argmax of logits[b][v] (lowest id on ties), and the terminal token is that
 * argmax.  All vocab-wide arithmetic is float64.
 *
 *   tokens, parents        [B][n_max] int32 (tokens[b][0], the root, unused)
 *   n_nodes                [B] int32
 *   draft_p, logits        [B][n_max][V] float32; row v of draft_p is the
 *                          distribution v's children were drawn from; rows
 *                          are read only for nodes the walk visits
 *   max_depth              bound on tree depth; path/out_tokens hold
 *                          max_depth + 1 entries per sequence
 *   temperature            >= 0
 *   u_accept, u_sample     [B][n_max] float32 uniforms in [0, 1)
 *   accept_len  (out)      [B] int32: accepted drafts a (-1 on device error)
 *   path        (out)      [B][max_depth+1] int32: root..deepest accepted
 *                          node (a + 1 entries), then -1
 *   out_tokens  (out)      [B][max_depth+1] int32: the a accepted tokens,
 *                          then the terminal token, then -1
 *   n_out       (out)      [B] int32: a + 1 (0 on device error)
 *   final_dist  (out, nullable) [B][V] float32: normalised distribution the
 *                          terminal token was drawn from (one-hot at T = 0)
 *   tie_log     (out, nullable) up to tie_cap records of decisions with
 *                          |u - min(1, ratio)| < 1e-6 and samples whose
 *                          margin < 1e-9; *tie_count (device int32, required
 *                          when tie_log is given) is reset by the call and
 *                          counts all such events, logged or not
 *   workspace              >= spec_accept_tree_workspace_size(...) bytes of
 *                          device memory; needs no initialisation (the words
 *                          workgroups exchange through it carry a per-launch
 *                          tag, made of the host's launch id and a
 *                          per-sequence counter the walk advances in the
 *                          workspace, so replays of a call captured in a HIP
 *                          graph are tagged afresh too); calls sharing one
 *                          workspace must be ordered on one stream
 * Device errors: SPEC_DEVERR_TREE, _TOKEN, _NONFINITE, _SYNC.
 * The workgroups that share one sequence's vocabulary exchange partial sums
 * and must be resident together; the call sizes its launch so that they are
 * on an otherwise idle GPU and uses an ordinary launch (spec_accept_tree_ex
 * takes the launch mode as an argument).  Every wait is bounded: a walk whose
 * workgroups could not all be resident sets SPEC_DEVERR_SYNC instead of
 * hanging, and then every output of the call (all B sequences) is
 * unspecified.  The caller then discards them (they must not reach
 * spec_kv_commit), zeroes *dev_error and repeats the call on the same inputs,
 * which it has not changed, with launch = SPEC_LAUNCH_COOPERATIVE, where the
 * runtime guarantees residency.  A caller that shares the GPU with other
 * work can pass SPEC_LAUNCH_COOPERATIVE from the start (about 17 us more per
 * call).
 */
spec_status_t spec_accept_tree(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes,
    const float* draft_p, const float* logits,
    int32_t B, int32_t n_max, int32_t V, int32_t max_depth, float temperature,
    const float* u_accept, const float* u_sample,
    int32_t* accept_len, int32_t* path, int32_t* out_tokens, int32_t* n_out,
    float* final_dist, spec_tie_t* tie_log, int32_t tie_cap, int32_t* tie_count,
    void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream);

size_t spec_accept_tree_workspace_size(int32_t B, int32_t n_max, int32_t V);

/*
 * spec_accept_tree_noalloc -- spec_accept_tree without a workspace argument,
 * for callers that cannot allocate device memory around the call: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, outputs, arithmetic and device errors as
 * spec_accept_tree (the same kernels; outputs are bit-identical), minus
 * workspace / workspace_bytes.
 *
 * The words the workgroups exchange live in a fixed device array of the
 * library, SPEC_NOALLOC_SCRATCH_BYTES (1 MiB) per GPU, created with the
 * library's code object on each GPU it runs on and held until the process
 * ends; the call never allocates or frees memory (no hipMalloc, hipFree or
 * allocating library routine).  The array's device address is looked up once
 * per GPU, on the first call with that GPU current.  A batch needing more
 * than the array (spec_accept_tree_workspace_size(B, n_max, V) > 1 MiB, about
 * 500 sequences of a 128k vocabulary) returns SPEC_E_SCRATCH before any
 * launch.  The array keeps what the last call left in it; nothing in it needs
 * clearing (each exchange word carries its launch's tag).  Every call on one
 * GPU shares the array: calls that may overlap on one GPU (different streams
 * without ordering between them) race and must not be issued.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (1u << 20)
spec_status_t spec_accept_tree_noalloc(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes,
    const float* draft_p, const float* logits,
    int32_t B, int32_t n_max, int32_t V, int32_t max_depth, float temperature,
    const float* u_accept, const float* u_sample,
    int32_t* accept_len, int32_t* path, int32_t* out_tokens, int32_t* n_out,
    float* final_dist, spec_tie_t* tie_log, int32_t tie_cap, int32_t* tie_count,
    int32_t* dev_error, void* stream);

/*
 * spec_accept_tree_ex -- spec_accept_tree with variants of its inputs
 * ([GUIDE] "一次 eagenerate 调用的完整流转": temperature, top_p and top_k are
 * per-call sampling arguments, so a batch of requests carries them per
 * sequence; [GUIDE] "代码里能直接读到的三处改动": an EAGLE-3 draft head ranks
 * its own vocabulary and draft id i stands for target token i + d2t[i]).
 *
 *   temperatures  NULL (the scalar temperature applies), or [B] float32
 *                 device array: sequence b uses q = softmax(logits /
 *                 temperatures[b]), 0 meaning greedy for that sequence; a
 *                 negative or non-finite entry fails its sequence with
 *                 SPEC_DEVERR_NONFINITE
 *   top_k, top_p  NULL, or [B] int32 / float32 device arrays: sampling
 *                 filters on the verifier's q at T > 0 (greedy decoding is
 *                 unaffected).  Top-k keeps the tokens whose logit is at
 *                 least the k-th largest of the row (ties kept together);
 *                 top-p keeps a token when the tempered q-mass of the tokens
 *                 with strictly larger logits is below p; a token must pass
 *                 both, and q is renormalised over the kept tokens before
 *                 the acceptance tests, residuals and samples.  k <= 0 or
 *                 k >= V, and p <= 0 or p >= 1, turn a filter off for that
 *                 sequence; a NaN p fails it with SPEC_DEVERR_NONFINITE.
 *                 Boundaries within 1e-8 of p are logged (tie kind 3).
 *   d2t, Vd       NULL (draft_p rows hold V entries), or [Vd] int32 device
 *                 array with 1 <= Vd <= V: draft_p rows hold Vd entries over
 *                 the draft vocabulary, and the draft probability of target
 *                 token x is draft_p[..][i] for the i with i + d2t[i] = x, 0
 *                 if there is none.  A map that leaves [0, V) or sends two
 *                 draft ids to one token fails every sequence with
 *                 SPEC_DEVERR_TOKEN.  Tree tokens stay target ids.
 *   workspace     >= spec_accept_tree_ex_workspace_size(B, n_max, V, Vd,
 *                 filters) bytes (Vd = 0 without d2t; filters nonzero when
 *                 top_k or top_p is given); with d2t it also holds the
 *                 inverse map, which the call builds first, and with filters
 *                 the per-round histograms the workgroups exchange
 *   launch        SPEC_LAUNCH_ORDINARY: an ordinary launch, sized so that
 *                 all workgroups of a sequence are resident on an otherwise
 *                 idle GPU; SPEC_LAUNCH_COOPERATIVE: a cooperative launch,
 *                 for which the runtime guarantees residency (for a GPU
 *                 shared with other work, and the repeat after
 *                 SPEC_DEVERR_SYNC).  The outputs are the same bits either
 *                 way.  Any other value returns SPEC_E_VALUE.
 * Everything else as spec_accept_tree, which is this call with all four NULL
 * and launch = SPEC_LAUNCH_ORDINARY.
 */
spec_status_t spec_accept_tree_ex(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes,
    const float* draft_p, const float* logits,
    int32_t B, int32_t n_max, int32_t V, int32_t max_depth, float temperature,
    const float* temperatures, const int32_t* top_k, const float* top_p,
    const int32_t* d2t, int32_t Vd,
    const float* u_accept, const float* u_sample,
    int32_t* accept_len, int32_t* path, int32_t* out_tokens, int32_t* n_out,
    float* final_dist, spec_tie_t* tie_log, int32_t tie_cap, int32_t* tie_count,
    void* workspace, size_t workspace_bytes, int32_t launch, int32_t* dev_error,
    void* stream);

size_t spec_accept_tree_ex_workspace_size(int32_t B, int32_t n_max, int32_t V, int32_t Vd,
                                          int32_t filters);

/*
 * spec_kv_commit -- commit the accepted path ([LESSON] "KV cache 回滚" and
 * build step 4).  For every sequence with accept_len[b] = a >= 0 and every
 * KV head: cache row prefix_len[b] + i receives the pre-commit row
 * prefix_len[b] + path[b][i] for i = 0..a (K and V), then prefix_len[b]
 * becomes prefix_len[b] + a + 1 (the root and the a accepted drafts; the
 * terminal token is the next step's root).  A path equal to 0..a moves no
 * bytes (logical truncation).  Sequences with accept_len < 0 are untouched.
 * Not idempotent: call exactly once per step, after spec_accept_tree.
 *
 *   k_cache, v_cache [B][Hkv][L_cap][head_dim], dtype (in/out); 16-byte
 *                    aligned (rows move in 16-byte chunks), else SPEC_E_SHAPE
 *   prefix_len       [B] int32 (in/out)
 *   path, accept_len as written by spec_accept_tree with the same max_depth
 * Device errors: SPEC_DEVERR_TREE (path not increasing / out of range),
 * SPEC_DEVERR_CAPACITY.
 */
spec_status_t spec_kv_commit(
    void* k_cache, void* v_cache, int32_t* prefix_len,
    const int32_t* path, const int32_t* accept_len,
    int32_t B, int32_t Hkv, int32_t head_dim, int32_t L_cap, int32_t max_depth,
    int32_t dtype, int32_t* dev_error, void* stream);

/*
 * spec_kv_commit_layers -- spec_kv_commit for num_layers layers in one call,
 * in either rollback form of [LESSON] "KV cache 回滚":
 *   - in place (k_tree == NULL): the verify pass wrote tree node j's K/V of
 *     every layer into cache row prefix_len[b] + j; for every layer, cache
 *     row prefix_len[b] + i receives row prefix_len[b] + path[b][i]
 *     (spec_kv_commit, layer by layer);
 *   - scratch buffer (k_tree, v_tree given): the verify pass wrote the tree's
 *     K/V of layer l into k_tree[l], v_tree[l]; cache row prefix_len[b] + i
 *     receives scratch row path[b][i] for i = 0..a, the root included.
 * Then prefix_len[b] advances by a + 1, once.  Sequences with accept_len < 0
 * are untouched.  Not idempotent: call once per step, after spec_accept_tree
 * (and instead of spec_kv_commit).
 *
 *   k_layers, v_layers  device array [num_layers] of device pointers, each to
 *                       a [B][Hkv][L_cap][head_dim] cache of dtype (in/out)
 *   k_tree, v_tree      NULL for the in-place form, or device arrays
 *                       [num_layers] of device pointers, each to
 *                       [B][Hkv][n_max][head_dim] scratch rows of dtype
 *   num_layers          >= 1
 *   n_max               scratch rows per sequence (scratch form; otherwise
 *                       ignored)
 *   prefix_len, path, accept_len, B, Hkv, head_dim, L_cap, max_depth, dtype
 *                       as for spec_kv_commit
 * The pointer arrays are read by the kernels: they must stay valid until the
 * stream work completes.  Every pointer in them must be 16-byte aligned, as
 * for spec_kv_commit; the host cannot read device arrays, so the kernels
 * check: if any is not, no sequence of any layer is committed, no length
 * advances, and SPEC_DEVERR_ALIGN is set.
 * Device errors: as spec_kv_commit; in the scratch form also SPEC_DEVERR_TREE
 * for a path entry >= n_max; SPEC_DEVERR_ALIGN.  A failed sequence is left
 * untouched in every layer.
 */
spec_status_t spec_kv_commit_layers(
    void* const* k_layers, void* const* v_layers, const void* const* k_tree,
    const void* const* v_tree, int32_t num_layers, int32_t* prefix_len, const int32_t* path,
    const int32_t* accept_len, int32_t B, int32_t n_max, int32_t Hkv, int32_t head_dim,
    int32_t L_cap, int32_t max_depth, int32_t dtype, int32_t* dev_error, void* stream);

/*
 * Draft-tree construction (EAGLE-2), the step before verification
 * ([GUIDE] "一个可核对的经验性质": a node's value is the product of the
 * draft's confidences on its root path; the section on EAGLE-2's two stages:
 * Expansion runs the draft, level by level, only on the top_k most valuable
 * nodes of the level before, and Reranking sends the total_tokens most
 * valuable nodes of the whole tree to verification; the paragraph on the
 * papers' settings: 60/50/48 drafts, depth 6 (8 for EAGLE-3), 10 expanded
 * per level; section "代码里能直接读到的三处改动": an EAGLE-3 draft head
 * ranks its own vocabulary and draft id i is target token i + d2t[i]).
 *
 * Values are sums of float32 log-probabilities (log of the product of
 * confidences); confidences are the draft's softmax probabilities.  The
 * pool of one sequence holds, per level, the top_k children of each
 * expanded node: level 1 has the root's top_k children (all expanded), level
 * l >= 2 the top_k * top_k children of level l-1's expanded nodes, of which
 * the top_k are expanded.  Pool order is (level, draft row, child rank);
 * equal logits go to the lower draft id, equal values to the lower pool
 * index.  Pool ids: level 1 holds 0..top_k-1, level l >= 2 holds
 * top_k + (l-2)*top_k^2 + r*top_k + j for child rank j of draft row r.
 *
 * One tree per call sequence: spec_tree_expand for level 1, 2, ..., then
 * spec_tree_finalize, all on one stream with one state buffer.
 *
 * spec_tree_state_size -- bytes of the state buffer (device memory owned by
 *   the caller; 0 for arguments out of range).  It needs no initialisation:
 *   a level-1 call starts a new tree on it.  It holds the pool between
 *   calls, so trees in flight need one each.
 */
size_t spec_tree_state_size(int32_t B, int32_t top_k, int32_t depth);

/*
 * spec_tree_expand -- grow level `level` (1-based) of every sequence's tree.
 *
 *   draft_logits  [B][R][Vd], dtype SPEC_F32 or SPEC_BF16: R = 1 at level 1
 *                 (the draft's output at the root), R = top_k afterwards, row
 *                 r being the draft's output at the r-th node the previous
 *                 call returned in expanded_ids
 *   d2t           NULL, or [Vd] int32 offsets: a child's token is
 *                 id + d2t[id] (not range-checked here)
 *   B, Vd         1 <= B <= 65535; top_k <= Vd <= 2^24
 *   top_k, depth  1 <= top_k <= SPEC_TREE_MAX_TOP_K,
 *                 1 <= level <= depth <= SPEC_TREE_MAX_DEPTH (depth sizes
 *                 the state and must be the same in every call on it)
 *   state         >= spec_tree_state_size(B, top_k, depth) bytes
 *   expanded_tokens (out) [B][top_k] int32: tokens of the nodes chosen for
 *                 expansion, most valuable first (-1 for a failed sequence)
 *   expanded_ids  (out, nullable) [B][top_k] int32: their pool ids; the
 *                 parent of pool id p at level l >= 2 is the node of draft
 *                 row (p - top_k - (l-2)*top_k^2) / top_k of that level
 * Device errors: SPEC_DEVERR_NONFINITE (a NaN or +inf logit, or a row with
 * no finite logit), SPEC_DEVERR_TREE (level l >= 2 called when level l-1 was
 * not the last one grown on this state).  The sequence is then failed until
 * its next level-1 call: later levels return -1 tokens, finalize gives it
 * n_nodes = 0.
 */
spec_status_t spec_tree_expand(const void* draft_logits, int32_t dtype, const int32_t* d2t,
                               int32_t B, int32_t Vd, int32_t top_k, int32_t depth,
                               int32_t level, void* state, size_t state_bytes,
                               int32_t* expanded_tokens, int32_t* expanded_ids,
                               int32_t* dev_error, void* stream);

/*
 * spec_tree_finalize -- rerank: the total_tokens most valuable pool nodes
 * (nodes of value -inf excluded) follow the root, node 0, in pool order, so
 * parents precede children; the result is a tree in the format of
 * spec_verify_tree_attn and spec_accept_tree.
 *
 *   total_tokens  drafts to keep, 1 <= total_tokens < SPEC_MAX_NODES
 *   root_token    (nullable) [B] int32: written to tokens[b][0] (else -1)
 *   prefix_len    (nullable) [B] int32: positions = prefix_len + depth
 *                 (else depth)
 *   n_max         row stride of the outputs, total_tokens < n_max <= 64
 *   tokens, parents (out) [B][n_max] int32; parents[b][0] = -1
 *   n_nodes       (out) [B] int32: 1 + drafts kept (0 for a failed sequence)
 *   node_depth, positions, draft_row (out, nullable) [B][n_max] int32;
 *                 draft_row is the expansion row whose draft output holds the
 *                 node's children: 0 for the root, 1 + (l-1)*top_k + r for
 *                 the r-th node expanded at level l < levels grown, -1 for a
 *                 node without children
 *   anc_mask      (out, nullable) [B][n_max] uint64: bit i of row j set iff i
 *                 is j or an ancestor of j
 *   value         (out, nullable) [B][n_max] float32: sum of log-probabilities
 * Rows >= n_nodes[b] are not written.
 * The state must have had a level-1 call since it was allocated.
 * Device errors: SPEC_DEVERR_TREE (state not in a valid grown state).
 */
spec_status_t spec_tree_finalize(const void* state, size_t state_bytes, int32_t B,
                                 int32_t top_k, int32_t depth, int32_t total_tokens,
                                 const int32_t* root_token, const int32_t* prefix_len,
                                 int32_t n_max, int32_t* tokens, int32_t* parents,
                                 int32_t* n_nodes, int32_t* node_depth, int32_t* positions,
                                 uint64_t* anc_mask, int32_t* draft_row, float* value,
                                 int32_t* dev_error, void* stream);

/*
 * Paged caches.  [LESSON] "KV cache 回滚" names vLLM and TensorRT-LLM as the
 * systems that write the verify pass's KV to a temporary buffer and commit it
 * on acceptance; such servers keep the cache in fixed-size blocks.  The pages
 * do not give the layout; these calls take the usual one:
 *
 *   k_pool, v_pool  [num_blocks][Hkv][block_size][head_dim] per layer, dtype
 *   block_table     [B][max_blocks] int32 device array: logical row r of
 *                   sequence b is row r % block_size of physical block
 *                   block_table[b][r / block_size]
 *   block_size      a power of two in [16, 4096]
 *   max_blocks      logical blocks per sequence (the table's row length); the
 *                   logical capacity is max_blocks * block_size (the L_cap of
 *                   the contiguous calls)
 *   num_blocks      physical blocks in each pool
 *
 * Each call does exactly what its contiguous form does on the logical rows,
 * with the same kernels (bit-identical results for the same logical
 * contents).  A sequence that would read or write a row whose block id lies
 * outside [0, num_blocks) is not processed and sets SPEC_DEVERR_CAPACITY.
 * The blocks holding rows [prefix_len, prefix_len + n_nodes) of a sequence
 * must belong to that sequence alone (they are written); blocks of committed
 * prefix rows may be shared between sequences (they are only read).  Host
 * errors as the contiguous forms, plus SPEC_E_NULL for a NULL block_table and
 * SPEC_E_SHAPE for a bad block geometry.
 */

/* spec_verify_tree_attn_rope / spec_verify_tree_attn on a paged cache
 * (inv_freq NULL: no rotation, rope_style ignored).  workspace >=
 * spec_verify_tree_attn_workspace_size(B, n_max, Hq, Hkv, head_dim,
 * max_blocks * block_size, dtype). */
spec_status_t spec_verify_tree_attn_paged(
    const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
    int32_t max_blocks, int32_t block_size, int32_t num_blocks,
    const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* parents,
    int32_t B, int32_t n_max, int32_t Hq, int32_t Hkv, int32_t head_dim,
    float scale, int32_t dtype, const float* inv_freq, int32_t rope_style, float* out,
    void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream);

/* spec_tree_kv_write on a paged cache: node j's K (rotated when inv_freq is
 * given) and V go to logical row prefix_len + j. */
spec_status_t spec_tree_kv_write_paged(
    const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_table, int32_t max_blocks, int32_t block_size, int32_t num_blocks,
    const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* parents,
    int32_t B, int32_t n_max, int32_t Hkv, int32_t head_dim, int32_t dtype,
    const float* inv_freq, int32_t rope_style, int32_t* dev_error, void* stream);

/* spec_kv_commit_layers on paged caches: k_layers / v_layers point at each
 * layer's pool (one block table serves every layer); in place or from
 * scratch rows exactly as spec_kv_commit_layers, whose 16-byte alignment
 * rule and SPEC_DEVERR_ALIGN apply to the pools. */
spec_status_t spec_kv_commit_layers_paged(
    void* const* k_layers, void* const* v_layers, const void* const* k_tree,
    const void* const* v_tree, int32_t num_layers, const int32_t* block_table,
    int32_t max_blocks, int32_t block_size, int32_t num_blocks, int32_t* prefix_len,
    const int32_t* path, const int32_t* accept_len, int32_t B, int32_t n_max, int32_t Hkv,
    int32_t head_dim, int32_t max_depth, int32_t dtype, int32_t* dev_error, void* stream);

/* Static description of a status code (never NULL). */
const char* spec_status_string(spec_status_t status);

/* SPEC_ABI_VERSION of the loaded library. */
int32_t spec_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
