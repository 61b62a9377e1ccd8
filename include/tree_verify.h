/*
 * tree_verify.h -- C ABI of libtreeverify.so: tree-verification attention on MI355X (gfx950).
 *
 * One speculative-decoding step verifies a whole draft tree in a single target pass.  The
 * tree is flattened into N nodes (node 0 = root = the last accepted token) described by a
 * parent array.  Node i attends to every one of the L cached prefix positions and to tree
 * position L + j exactly when j is i or an ancestor of i, and carries position id
 * L + depth(i).  ("Tree attention mask for draft-tree verification", sections "TL;DR" and
 * "A strong answer"; "Tree Verification", section "Tree Attention".)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are plain host or device addresses as stated per argument; no entry point
 *    allocates, frees or synchronises.  Device work is enqueued on the caller's stream and
 *    is safe to capture in a HIP graph (sizes come from arguments, never from constants).
 *  - Errors are returned as tv_status; a human-readable detail of the last error on the
 *    calling thread is available from tv_last_error().  Nothing is written to outputs when
 *    an argument check fails.  N > TV_MAX_NODES (or D outside {64, 128}) is a shape the
 *    kernels do not implement: TV_ERR_UNSUPPORTED; N < 1 is TV_ERR_INVALID_ARG.
 *  - N (nodes per tree, root included) is 1..TV_MAX_NODES.  The ancestor bitmask of node i
 *    is one uint64 word with bit j set (LSB first) iff j is i or an ancestor of i.
 *  - Device-resident parent arrays must satisfy parent[0] == -1 and 0 <= parent[i] < i
 *    (any parent-before-child order is accepted; "Tree Verification", "Tree Attention").
 *    The kernels never read out of bounds or loop forever on a violation; tree_meta_from_parent
 *    flags the offending nodes (depth = pos = -1, bitmask = 0).
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_MAX_NODES 64
#define TV_ABI_VERSION 5

typedef enum {
  TV_OK = 0,
  TV_ERR_INVALID_ARG = 1,     /* null pointer, bad size, stride or dtype             */
  TV_ERR_INVALID_PATH = 2,    /* empty path or negative rank                          */
  TV_ERR_MISSING_PARENT = 3,  /* a path whose one-shorter prefix is not a node         */
  TV_ERR_CAPACITY = 4,        /* more nodes than the caller's arrays (or 64) can hold  */
  TV_ERR_UNSUPPORTED = 5,     /* a shape the kernels do not implement (e.g. D = 96)    */
  TV_ERR_WORKSPACE = 6,       /* workspace missing or smaller than required            */
  TV_ERR_HIP = 7              /* a HIP runtime call failed (launch, attribute query)   */
} tv_status;

typedef enum { TV_BF16 = 0, TV_F32 = 1 } tv_dtype;
typedef enum { TV_KV_CONTIGUOUS = 0, TV_KV_PAGED = 1 } tv_kv_layout;
typedef enum { TV_PATH_AUTO = 0, TV_PATH_VALU = 1, TV_PATH_MFMA = 2 } tv_path;

/*
 * tree_meta_build -- host metadata builder ("Tree attention mask for draft-tree
 * verification", section "A strong answer": rank-path candidates, node order, parent,
 * depth, the ancestor mask and position ids prefix + depth).
 *
 * Input (host memory, read only):
 *   ranks[path_off[p] .. path_off[p+1])  the drafter-rank tuple of candidate p, p < num_paths;
 *                                        path_off has num_paths + 1 entries, path_off[0] = 0.
 *   prefix_len                           L, the cached prefix length (>= 0).
 *   max_nodes                            capacity of the output arrays (>= 1).
 * Output (host memory, caller-owned, at least max_nodes entries each):
 *   parent[i], depth[i], pos[i] = prefix_len + depth[i], bitmask[i] (one uint64 per node);
 *   *num_nodes = N (root included).
 *   *bad_path  = input index of the offending path on TV_ERR_INVALID_PATH /
 *                TV_ERR_MISSING_PARENT, else -1.  (May be NULL.)
 * Node order: distinct paths sorted by (length, lexicographic ranks); duplicates collapse.
 * Errors: TV_ERR_INVALID_ARG (null pointers, num_paths < 0, bad offsets),
 *         TV_ERR_INVALID_PATH, TV_ERR_MISSING_PARENT (the first in sorted order),
 *         TV_ERR_CAPACITY (N > max_nodes or N > TV_MAX_NODES).  num_paths == 0 gives the
 *         root alone (N = 1): plain decoding.  Outputs are unspecified on error.
 */
tv_status tree_meta_build(const int32_t* ranks, const int64_t* path_off, int32_t num_paths,
                          int32_t prefix_len, int32_t max_nodes,
                          int32_t* parent, int32_t* depth, uint64_t* bitmask, int32_t* pos,
                          int32_t* num_nodes, int32_t* bad_path);

/*
 * tree_meta_build_batch -- tree_meta_build for B requests in one call, writing dense
 * [B, N] outputs ready for tree_verify_attn.
 *
 * Input (host): tree b owns candidates tree_off[b] .. tree_off[b+1]-1 of the CSR path list
 * (ranks/path_off as for tree_meta_build; tree_off has B + 1 entries, tree_off[0] = 0);
 * prefix_len[b] is its cached prefix length; N is the node count every output row holds.
 * Output (host, caller-owned): parent, depth, pos [B, N] int32 and bitmask [B, N] uint64;
 * num_nodes[b] = the tree's own node count.  A tree with fewer than N nodes is padded with
 * extra leaves under the root (parent 0) so that the row still satisfies the parent
 * convention; callers ignore outputs of nodes at or past num_nodes[b].
 * Errors: TV_ERR_INVALID_ARG (B < 0, N < 1, null pointers, tree_off or path_off not
 * starting at 0 or decreasing, a prefix length out of range -- *bad_tree names that tree)
 * and TV_ERR_UNSUPPORTED (N > TV_MAX_NODES): these checks cover the whole batch before
 * anything is written.  Then, per tree in order, the errors of tree_meta_build
 * (TV_ERR_INVALID_PATH, TV_ERR_MISSING_PARENT, TV_ERR_CAPACITY when a tree has more than
 * N nodes): *bad_tree names the first failing tree (may be NULL) and *bad_path the
 * offending path's index within it; rows of the trees before it hold their results, the
 * rest of the outputs are unspecified.  B == 0 is a no-op.
 */
tv_status tree_meta_build_batch(const int32_t* ranks, const int64_t* path_off,
                                const int64_t* tree_off, int32_t B,
                                const int32_t* prefix_len, int32_t N,
                                int32_t* parent, int32_t* depth, uint64_t* bitmask,
                                int32_t* pos, int32_t* num_nodes, int32_t* bad_tree,
                                int32_t* bad_path);

/*
 * tree_meta_from_parent -- the same metadata from device-resident parent arrays (the
 * faster kernel input is the parent array, expanded tile by tile inside the kernel: "Tree
 * attention mask for draft-tree verification", paragraph after the build listing).
 *
 * Device memory: parent[b * parent_sb + i] (int32; parent_sb = 0 shares one tree across
 * the batch), prefix_len[b] (int32; may be NULL, then pos = depth).
 * Device outputs, dense [B, N]: depth (int32), bitmask (uint64), pos (int32); any of the
 * three may be NULL to skip it.  Invalid nodes (see header comment) get -1 / 0 / -1.
 * Errors: TV_ERR_INVALID_ARG (B < 0, N < 1, parent NULL, parent_sb < 0),
 *         TV_ERR_UNSUPPORTED (N > 64), TV_ERR_HIP.  B == 0 is a no-op.
 */
tv_status tree_meta_from_parent(const int32_t* parent, int32_t parent_sb, int32_t B,
                                int32_t N, const int32_t* prefix_len, int32_t* depth,
                                uint64_t* bitmask, int32_t* pos, hipStream_t stream);

/*
 * Arguments of tree_verify_attn.  All tensor pointers are device memory (parent may also
 * be the device address of pinned host memory, see below); strides are in elements; the
 * last (D) dimension of q, k, v and out is contiguous.
 *
 *   q    [B, N, Hq, D]  at q + b*q_sb + i*q_sn + h*q_sh.
 *   k, v logical token t of request b, kv head g:
 *          contiguous: base + b*kv_sb + t*kv_st + g*kv_sh, t < prefix_len[b] + N;
 *          paged:      base + page*kv_sb + (t % page_size)*kv_st + g*kv_sh with
 *                      page = page_table[b*pages_per_seq + t / page_size].
 *        Tree node j's key/value is logical token prefix_len[b] + j, in node order
 *        ("Tree attention mask for draft-tree verification", section "What it costs").
 *        Tokens at or beyond prefix_len[b] + N are never read.
 *   parent [B, N] int32 at parent + b*parent_sb (parent_sb = 0: one shared tree).  Read
 *        once by every workgroup's prologue, so it may live in pinned host memory
 *        (hipHostMalloc; pass the address hipHostGetDevicePointer gives): a host that
 *        builds the trees every step then needs no copy.  It must stay unchanged until the
 *        pass has finished.
 *   prefix_len [B] int32, each in 0..max_prefix_len; max_prefix_len is a host-side upper
 *        bound used only to size the grid (no device sync).
 *   out  [B, N, Hq, D] (same dtype as q) at out + b*o_sb + i*o_sn + h*o_sh.
 *   lse  [B, N, Hq] fp32, contiguous, natural log of the sum of exp(scores); may be NULL.
 *   Query head h reads kv head h / (Hq / Hkv).  sm_scale = 0 means 1/sqrt(D).
 *   workspace: device scratch of tree_verify_attn_workspace_size() bytes (may be 0 bytes,
 *        then workspace may be NULL).  Contents need no initialisation.
 *   num_splits: 0 = automatic, else the number of key-range splits per (request, kv head).
 *   path: TV_PATH_AUTO picks the MFMA kernel for bf16 once N * (Hq / Hkv) >= 16, else the
 *        VALU kernel; the others force one (MFMA needs bf16).
 *   rope_theta: 0 = no rotary embedding (q and every key are used as given).  > 0 fuses
 *        the rotary embedding into the pass ("Tree attention mask for draft-tree
 *        verification", "What interviewers probe next" and "Common mistakes": node i sits
 *        at position L + depth(i), siblings share one): q and the tree keys
 *        (tokens L .. L+N-1) are given UNROTATED and are rotated inside the kernels at
 *        L + depth(i); prefix keys (t < L) are taken as already rotated at t.  Rotate-half
 *        form: features (m, m + D/2), m < D/2, turn by angle pos * rope_theta^(-2m/D)
 *        (angle reduced in fp64, cos/sin in fp32).  Nothing is written back: the tree rows
 *        stay unrotated in the cache until tree_kv_compact rotates the accepted ones.
 *   prefix_len_host: NULL, or a host array holding the same B prefix lengths as the device
 *        prefix_len (values are clamped to 0..max_prefix_len).  Read on the host only, by
 *        tree_verify_attn and tree_verify_attn_workspace_size, to plan the automatic split:
 *        the key chunk is sized to the batch's total work rather than to max_prefix_len,
 *        and when lengths differ (B <= 256, bf16 matrix-core path) the workgroups take the
 *        (request, key chunk) pieces longest first.  Results never depend on it: every split count covers
 *        max_prefix_len + N keys, and a hint that disagrees with the device values only
 *        costs balance.  The caller owns it; it is not retained after the call.
 *   meta_depth, meta_bitmask, meta_pos: NULL, or device arrays [B, N] (dense) that
 *        receive what tree_meta_from_parent writes for the same parent and prefix_len
 *        (depth, ancestor bitmask, prefix_len[b] + depth; -1 / 0 / -1 for invalid nodes).
 *        The pass expands the parent arrays in its prologue anyway; one workgroup per
 *        request writes them out, so a caller that wants both needs no second launch.
 */
typedef struct tv_attn_args {
  int32_t dtype;           /* tv_dtype of q, k, v and out                                  */
  int32_t B, N, Hq, Hkv, D;/* D in {64, 128}; 1 <= N <= 64; Hq % Hkv == 0                   */
  const void* q;
  int64_t q_sb, q_sn, q_sh;
  int32_t kv_layout;       /* tv_kv_layout                                                  */
  int32_t page_size;       /* paged only: tokens per page (>= 1)                           */
  const void* k;
  const void* v;
  int64_t kv_sb, kv_st, kv_sh;
  const int32_t* page_table;
  int32_t pages_per_seq;   /* paged only: row length of page_table                          */
  int32_t parent_sb;
  const int32_t* parent;
  const int32_t* prefix_len;
  int32_t max_prefix_len;
  float sm_scale;
  void* out;
  int64_t o_sb, o_sn, o_sh;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  int32_t num_splits;
  int32_t path;            /* tv_path                                                       */
  double rope_theta;       /* 0: none; > 0: fused rotary embedding at L + depth (above)     */
  const int32_t* prefix_len_host; /* optional HOST copy of prefix_len[B], or NULL (below)    */
  int32_t* meta_depth;     /* optional [B, N] outputs of the expanded tree (above), or NULL  */
  uint64_t* meta_bitmask;
  int32_t* meta_pos;
} tv_attn_args;

/*
 * tree_verify_attn_workspace_size -- bytes of device workspace the call needs for these
 * arguments (0 when one split covers every request).  Host only; depends on shapes,
 * strides, max_prefix_len, num_splits, path and prefix_len_host only (no other pointer
 * field is read), and the automatic split count on the current device's compute-unit
 * count.  Returns 0 for shapes tree_verify_attn would reject.
 */
size_t tree_verify_attn_workspace_size(const tv_attn_args* a);

/*
 * tree_verify_attn -- the verification attention pass.  For every request b, node i and
 * query head h: softmax over the allowed keys (all L prefix tokens, plus tree tokens of
 * i's ancestors and i itself) of sm_scale * <q, k>, applied to v; lse is the natural log
 * of the softmax denominator including its max ("Tree attention mask for draft-tree
 * verification", "A strong answer": full step mask = all-true prefix block beside the tree
 * mask; "Tree Verification", "Tree Attention").
 * Enqueues one attention kernel, plus one merge kernel when a request's keys are split,
 * on `stream`.  Errors: TV_ERR_INVALID_ARG, TV_ERR_UNSUPPORTED, TV_ERR_WORKSPACE,
 * TV_ERR_HIP (launch failure).  B == 0 is a no-op returning TV_OK.
 */
tv_status tree_verify_attn(const tv_attn_args* a, hipStream_t stream);

/*
 * tree_verify_attn_static -- for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  Exactly
 * tree_verify_attn (same checks, split plan, kernels and results; a->workspace and
 * a->workspace_bytes are ignored), except that the split workspace is a fixed array of
 * TV_STATIC_SCRATCH_BYTES that the library keeps on every device it runs on, from module
 * load until the process ends.  It calls no allocation routine.  A plan whose workspace
 * (tree_verify_attn_workspace_size) exceeds TV_STATIC_SCRATCH_BYTES is rejected with
 * TV_ERR_WORKSPACE before anything is enqueued (a smaller num_splits fits; one split
 * needs none).  All calls on one device share that device's array and it keeps the last
 * call's contents (nothing in it needs an initial value): calls whose work overlaps on one
 * device -- different streams, or host threads without ordering -- race on it.
 * Errors: those of tree_verify_attn, TV_ERR_WORKSPACE as above, TV_ERR_HIP if the array's
 * device address cannot be looked up, TV_ERR_UNSUPPORTED for a device index >= 64.
 */
#define TV_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)
tv_status tree_verify_attn_static(const tv_attn_args* a, hipStream_t stream);

/*
 * ---- After the pass: greedy acceptance and the accepted path's KV ----
 *
 * Arguments of tree_accept_greedy.  Device memory unless stated; strides in elements.
 *   dtype                 TV_BF16 or TV_F32 logits.
 *   B, N, V               requests (>= 0), tree nodes (1..TV_MAX_NODES), vocabulary (>= 1).
 *   logits [B, N, V]      the target's next-token logits at every node (vocabulary
 *                         contiguous); lg_sb, lg_sn strides of request and node (>= 0).
 *   tokens [B, N]         the draft token of every node (node 0, the root, is not read);
 *                         tokens_sb its request stride (0 = one row for all requests).
 *   parent [B, N]         the tree (parent_sb 0 = one tree for all requests); must satisfy
 *                         the parent-before-child convention above.
 * Outputs (caller-owned device memory, [B, N] int32 unless stated):
 *   target                the target's greedy token after each node: argmax over the
 *                         vocabulary, lowest index on ties, the first NaN if a row holds one.
 *   accepted              the accepted nodes, root first, then -1.
 *   emitted               the emitted tokens (accepted drafts, then the correction or bonus
 *                         token), then -1.
 *   num_accepted [B]      A = number of accepted nodes = number of emitted tokens, 1..depth+1.
 *   workspace             device scratch of at least tree_accept_greedy_workspace_size()
 *                         = B * N * ceil(V / 8192) * 8 bytes, 16-byte aligned (one key per
 *                         8192-entry slice of every row); caller-owned, contents need no
 *                         initialisation.
 */
typedef struct {
  int32_t dtype;           /* tv_dtype, held as a plain int so any value can be checked */
  int32_t B, N, V;
  const void* logits;
  int64_t lg_sb, lg_sn;
  const int32_t* tokens;
  int32_t tokens_sb;
  const int32_t* parent;
  int32_t parent_sb;
  int32_t* target;
  int32_t* accepted;
  int32_t* emitted;
  int32_t* num_accepted;
  void* workspace;
  size_t workspace_bytes;
} tv_accept_args;

/* Bytes of workspace tree_accept_greedy needs for these sizes (pointers are not read). */
size_t tree_accept_greedy_workspace_size(const tv_accept_args* a);

/*
 * tree_accept_greedy -- greedy verification of the tree ("Tree attention mask for
 * draft-tree verification", "A strong answer": the greedy walk; "Tree Verification",
 * "Accepting on a Tree").  Per node, the target's greedy token; then, per request, the
 * walk from the root: at the current node the greedy token is emitted and the first child
 * (in node order) whose draft token equals it is accepted and becomes the current node;
 * the walk stops when no child matches (correction) or at a leaf (bonus).  Enqueues, on
 * `stream`, the argmax kernel (one workgroup per 8192-entry slice of every row, HBM-bound on
 * the logits, each storing its best (value, index) as an order-preserving 64-bit key in the
 * workspace) and the walk kernel (one workgroup per request; it takes each row's largest
 * slice key).  Errors: TV_ERR_INVALID_ARG (null
 * pointers, sizes, strides < V for lg_sn, misaligned logits for the given dtype),
 * TV_ERR_WORKSPACE, TV_ERR_HIP.  B == 0 is a no-op.
 */
tv_status tree_accept_greedy(const tv_accept_args* a, hipStream_t stream);



/*
 * Arguments of tree_accept_stochastic.  Device memory unless stated; strides in elements.
 *   B, N, V               requests (>= 0), tree nodes (1..TV_MAX_NODES), vocabulary (>= 1).
 *   p [B, N, V]           float32: the target's next-token distribution after every node
 *                         (need not be normalised; every row the walk reads must be finite,
 *                         non-negative, with positive mass); p_sb, p_sn strides (>= 0).
 *   q [B, N, V]           float32: the drafter's distribution at every node, the one the
 *                         node's children were drawn from, i.i.d. (rows of leaves are not
 *                         read; same rules as p); q_sb, q_sn.
 *   tokens [B, N]         draft tokens in [0, V) (node 0's is not read); tokens_sb (0 = one
 *                         row for all requests).
 *   parent [B, N]         the tree, parent-before-child; parent_sb (0 = one tree for all).
 *   uniform [B, N]        float64 in [0, 1): uniform[c] drives child c's acceptance test,
 *                         uniform[0] the final draw (the root is never tested); uniform_sb
 *                         (0 = one row for all requests).
 * Outputs (caller-owned device memory, [B, N] int32 unless stated): accepted, emitted and
 *   num_accepted [B] exactly as tree_accept_greedy defines them.
 */
typedef struct {
  int32_t B, N, V;
  const float* p;
  int64_t p_sb, p_sn;
  const float* q;
  int64_t q_sb, q_sn;
  const int32_t* tokens;
  int32_t tokens_sb;
  const int32_t* parent;
  int32_t parent_sb;
  const double* uniform;
  int32_t uniform_sb;
  int32_t* accepted;
  int32_t* emitted;
  int32_t* num_accepted;
} tv_sample_args;

/*
 * tree_accept_stochastic -- lossless verification of the tree at temperature > 0
 * ("Implement a batched speculative sampling verifier", "A strong answer": the accept test
 * u * q < p, the residual max(0, p - q), the inverse-CDF draw and the p = q corner; "What
 * interviewers probe next": the tree is walked with the same rule, each sibling after a
 * rejection judged against the residual; "Tree Verification", "Accepting on a Tree").
 * Per request, from the root: r starts as the node's p; each child c in node order, token
 * x, is accepted when uniform[c] * q(x) * sum(r) < r(x); after a rejection r becomes
 * max(0, r / sum(r) - q) (unchanged if that has no mass).  The first accepted child
 * becomes the current node and its token is emitted; if none is (or at a leaf) one token
 * is drawn from r by inverse CDF with uniform[0] -- the first index whose running sum
 * exceeds uniform[0] * sum(r), the last index of positive weight if none does -- and the
 * walk stops.  All of this arithmetic is float64.  A child whose token lies outside
 * [0, V) is never accepted and leaves r unchanged; a final draw from a row with no mass
 * emits -1.  Enqueues one kernel on `stream` (one workgroup per request; one pass over a
 * node's p and q rows per test).  Needs no workspace.  Errors: TV_ERR_INVALID_ARG (null pointers, sizes, strides), TV_ERR_UNSUPPORTED
 * (N > 64), TV_ERR_HIP.  B == 0 is a no-op.
 */
tv_status tree_accept_stochastic(const tv_sample_args* a, hipStream_t stream);/*
 * Arguments of tree_kv_compact.  The KV cache as in tv_attn_args (contiguous or paged;
 * k and v are written in place) and, per request:
 *   prefix_len [B]        L before the verified tree (tree node i sits at logical L + i);
 *                         clamped on the device to [0, max_prefix_len], the host bound
 *                         the KV buffers are sized for (as in tv_attn_args).
 *   parent [B, N]         the tree (parent_sb 0 = shared), used to validate the list.
 *   accepted [B, N]       accepted nodes, root first (as tree_accept_greedy writes them).
 *   num_accepted [B]      A (entries past A are not read).
 * Outputs (device, optional -- may be NULL):
 *   new_len [B]           L + A, the cache length after the step.
 *   status [B]            0: moved; 1: the list is not a root path of the tree (A < 1 or
 *                         > N, accepted[0] != 0, an entry out of range, or an entry that is
 *                         not a child of the one before it) -- nothing of that request moves.
 *   rope_theta            0: rows move unchanged.  > 0: the companion of tree_verify_attn's
 *                         fused rotary embedding -- the tree keys are unrotated in the cache,
 *                         and accepted node a_j's key is written to L + j rotated at
 *                         position L + j (= L + depth(a_j)), rows already in place included,
 *                         so every cached key is then rotated at its position.  Values move
 *                         unchanged.
 */
typedef struct {
  int32_t dtype;           /* tv_dtype, held as a plain int so any value can be checked */
  int32_t B, N, Hkv, D;
  int32_t kv_layout;       /* tv_kv_layout */
  void* k;
  void* v;
  int64_t kv_sb, kv_st, kv_sh;
  const int32_t* page_table;
  int32_t page_size, pages_per_seq;
  const int32_t* prefix_len;
  int32_t max_prefix_len;
  const int32_t* parent;
  int32_t parent_sb;
  const int32_t* accepted;
  const int32_t* num_accepted;
  int32_t* new_len;
  int32_t* status;
  double rope_theta;
} tv_compact_args;

/*
 * tree_kv_compact -- move the accepted path's KV rows to consecutive positions ("Tree
 * attention mask for draft-tree verification", "What it costs": the tree's cache rows sit
 * in node order, and before the next step the accepted ones are packed together;
 * "Tree Verification", "The Cost Side": cache rows of rejected branches are discarded).  For every request and kv head, the K and V rows of accepted node a_j move from
 * logical position L + a_j to L + j, j < A; rows at or past L + A are left as they are
 * (the new cache length excludes them).  All source rows of a (request, kv head) are read
 * before any is written, so overlapping moves are safe.  One workgroup per (kv head,
 * request) on `stream`.  Errors: TV_ERR_INVALID_ARG (as tree_verify_attn's KV checks),
 * TV_ERR_UNSUPPORTED (D not 64 or 128), TV_ERR_HIP.  B == 0 is a no-op.
 */
tv_status tree_kv_compact(const tv_compact_args* a, hipStream_t stream);

/*
 * Tree-budget policy (host arithmetic only; every pointer below is host memory, caller
 * owned; nothing is allocated on the device and no stream is used).
 *
 * Acceptance model ("Tree attention mask for draft-tree verification", "What it buys"):
 * rank_prob[r] is the probability that the target's greedy token is the drafter's rank-r
 * candidate (each in [0, 1], sum <= 1, 1 <= num_ranks <= 4096; ranks >= num_ranks have
 * probability 0).  The probability of reaching a node is the product of rank_prob over
 * the ranks on its path from the root.
 */

/*
 * tree_expected_tokens -- expected tokens per step of one tree under greedy verification:
 * 1 + the sum over non-root nodes of their reach probability ("What it buys").
 *   parent[n]  parent convention of the header comment (n >= 1, no upper limit here);
 *   rank[n]    node i's drafter rank among its siblings (>= 0, distinct among siblings;
 *              rank[0] is not read);
 *   reach[n]   optional output (may be NULL): each node's reach probability, 1 at the root;
 *   *expected  output.
 * Errors: TV_ERR_INVALID_ARG (NULL, n < 1, a parent violation, negative or repeated
 * sibling rank, probabilities outside [0, 1] or summing above 1).
 */
tv_status tree_expected_tokens(const int32_t* parent, const int32_t* rank, int32_t n,
                               const double* rank_prob, int32_t num_ranks, double* reach,
                               double* expected);

/*
 * tree_ridge_tokens -- tokens per step at which a decode step turns from bandwidth- to
 * compute-bound ("What it costs": dense flops over HBM bandwidth, for two-byte weights):
 * *ridge = peak_flops * bytes_per_weight / (2 * hbm_bytes_per_s).  All inputs finite, > 0.
 */
tv_status tree_ridge_tokens(double peak_flops, double hbm_bytes_per_s, double bytes_per_weight,
                            double* ridge);

/*
 * tree_budget_nodes -- the tree size a batch can afford: the largest N with
 * batch * N <= ridge_tokens, clamped to [1, max_nodes] ("What it costs": break-even batch =
 * ridge / N; trees shrink toward a chain, and at the ridge to the root alone, as the batch
 * grows).  Errors: TV_ERR_INVALID_ARG (batch < 1, max_nodes < 1, ridge negative or not
 * finite, nodes NULL).
 */
tv_status tree_budget_nodes(int32_t batch, double ridge_tokens, int32_t max_nodes,
                            int32_t* nodes);

/*
 * tree_best_static -- the tree of at most `nodes` nodes (root included, 1..TV_MAX_NODES)
 * and depth <= max_depth (1..63) with the most expected tokens ("Tree Verification", "The
 * Cost Side": a node is worth its path product, so spend nodes where the acceptance mass
 * is).  Since a path's product never exceeds its parent's, the nodes - 1 rank paths of
 * largest product form a tree; ties go to the shorter, then the lexicographically smaller
 * path; paths of product 0 are never taken (so fewer paths may come back).
 * Output (host, caller-owned): the chosen rank paths in the CSR form tree_meta_build reads
 * -- ranks[path_off[p] .. path_off[p+1]) -- in (length, lexicographic) order, i.e. the
 * builder's node order; path_off needs nodes entries, ranks ranks_cap entries
 * ((nodes - 1) * max_depth always suffices); *num_paths = paths returned; *expected (may
 * be NULL) = their expected tokens per step.
 * Errors: TV_ERR_INVALID_ARG (NULL outputs, bad probabilities or depth),
 *         TV_ERR_CAPACITY (nodes outside 1..64, or ranks_cap too small).
 */
tv_status tree_best_static(const double* rank_prob, int32_t num_ranks, int32_t nodes,
                           int32_t max_depth, int32_t* ranks, int64_t ranks_cap,
                           int64_t* path_off, int32_t* num_paths, double* expected);

/*
 * tree_budget_plan -- tree_budget_nodes (max_nodes clamped to TV_MAX_NODES) followed by
 * tree_best_static of that size: the static tree a batch of `batch` requests should
 * verify.  *nodes (may be NULL) receives the size; other outputs as tree_best_static.
 */
tv_status tree_budget_plan(int32_t batch, double ridge_tokens, int32_t max_nodes,
                           const double* rank_prob, int32_t num_ranks, int32_t max_depth,
                           int32_t* nodes, int32_t* ranks, int64_t ranks_cap, int64_t* path_off,
                           int32_t* num_paths, double* expected);

/* Static string naming a status code. */
const char* tv_status_string(tv_status s);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* tv_last_error(void);

/*
 * tv_pinned_device_address -- the device address of pinned host memory (hipHostMalloc), as
 * hipHostGetDevicePointer gives it: what tree_verify_attn's parent field takes when the
 * host writes the parent arrays every step and the pass reads them in place.  Host only.
 * Errors: TV_ERR_INVALID_ARG (NULL argument), TV_ERR_HIP (not pinned host memory; *device
 * is then NULL).
 */
tv_status tv_pinned_device_address(const void* host, const void** device);

/* TV_ABI_VERSION of the loaded library. */
int32_t tv_abi_version(void);

/* sizeof(tv_attn_args) as compiled into the library, for bindings to check their mirror. */
size_t tv_attn_args_sizeof(void);

/* sizeof(tv_accept_args), sizeof(tv_sample_args) and sizeof(tv_compact_args), likewise. */
size_t tv_accept_args_sizeof(void);
size_t tv_sample_args_sizeof(void);
size_t tv_compact_args_sizeof(void);

#ifdef __cplusplus
}
#endif
#endif /* TREE_VERIFY_H */
