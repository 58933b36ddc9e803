/*
 * gdn_tree.h -- C ABI of the MI355X (gfx950) library for rollback-free tree
 * verification of Gated DeltaNet (GDN) layers.
 *
 * The operation (Trees from Marginals, technical summary, Methodology,
 * "3. Rollback-Free Tree Verification for GDN"):  a speculative proposal tree
 * of N nodes, sorted topologically, is scored against one GDN layer's
 * recurrent state S0 in a single pass.  Every node i receives the output the
 * GDN delta rule produces when it runs from S0 along the root-to-i path,
 *
 *     S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t                              (after node t's own update),
 *
 * without ever advancing or rolling back S0.  The section casts this as a
 * masked triangular solve (I + X) U = beta V over the tree with interaction
 * matrices X, Y that follow the ancestor relation; the state is committed
 * later, once, for the accepted node only (the same section's delayed state
 * commitment).  The state S here maps a key to a value (d_v x d_k), the
 * transpose of the section's d_k x d_v orientation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to a dense, row-major
 *    (C-contiguous) array, 16-byte aligned, in the layout given at each
 *    argument.  Sizes are element counts.  The caller owns every buffer,
 *    including the workspace; the library never allocates device memory and
 *    never synchronises on the verify/commit path.
 *  - Value head h reads key head h / (H_v / H_k) (consecutive grouping);
 *    g and beta are per value head.  No query scaling is applied.
 *  - parent[b][i] is in [-1, i-1]; -1 means "child of the prefix state"
 *    (several such roots, a forest, are allowed).
 *  - Supported sizes: B >= 0, 0 <= N <= 256, H_k >= 1, H_v % H_k == 0,
 *    d_k, d_v in {64, 128}.  B == 0 or N == 0 is a no-op returning GDN_OK.
 *  - All O(1) argument checks (null pointers, dims, dtype, alignment,
 *    workspace size, commit without verify) are made on the host before any
 *    HIP call and return a status; no C++ exception crosses this ABI.
 *  - Data-dependent checks (parent order, accepted range) happen on the
 *    device: each batch element's verdict is written to the workspace and
 *    reported by gdn_ctx_status().  With the environment variable
 *    GDN_VALIDATE=1 set when the context is created, they are also made
 *    synchronously on the host before launching.  Outputs of a batch element
 *    whose tree or accepted node is invalid are unspecified (but every
 *    access stays in bounds).
 *  - Non-finite inputs propagate; they are not checked.
 *  - Range: results are stated for beta in [0, 1] and |k_i|^2 <= 2 (Gated
 *    DeltaNet normalises k to unit length and takes beta in (0, 1)).  There
 *    beta_a |k_a . k_b| <= 2, so the fp32 intermediates of the tree solve
 *    grow by at most 3x per root-path node and stay finite.  Outside it they
 *    can overflow on long root paths even where strong decay keeps the true
 *    result finite.
 *  - GDN_FORCE_SIMPLE=1 (read when a context is created) routes that
 *    context's verify to the per-node walk kernels instead of the MFMA path
 *    (for A/B comparison; results agree within the stated tolerance).
 *  - Calls are asynchronous on `stream` (NULL = the default stream) and
 *    complete in stream order.
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,      /* a required pointer is NULL                           */
    GDN_ERR_SHAPE = 2,     /* unsupported or inconsistent dims                     */
    GDN_ERR_DTYPE = 3,     /* unknown dtype code                                   */
    GDN_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned              */
    GDN_ERR_WORKSPACE = 5, /* workspace missing or smaller than required           */
    GDN_ERR_TREE = 6,      /* some parent[b][i] outside [-1, i-1]                  */
    GDN_ERR_ACCEPT = 7,    /* some accepted[b] outside [-1, N-1]                   */
    GDN_ERR_STATE = 8,     /* a commit without a prior gdn_tree_verify             */
    GDN_ERR_HIP = 9        /* a HIP runtime call or kernel launch failed           */
} gdn_status;

/* Element type of q, k and v.  g, beta, S0, o and S_new are always fp32. */
typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

typedef struct {
    int32_t B;         /* sequences in the batch                   */
    int32_t N;         /* tree nodes per sequence                  */
    int32_t H_k;       /* key/query heads                          */
    int32_t H_v;       /* value heads (a multiple of H_k)          */
    int32_t d_k;       /* key dimension                            */
    int32_t d_v;       /* value dimension                          */
    int32_t qkv_dtype; /* gdn_dtype of q, k, v                     */
} gdn_tree_dims;

/* Opaque host-side handle tying a verify to its delayed commit. */
typedef struct gdn_ctx gdn_ctx;

/* Bytes of device workspace a context for `dims` needs (a multiple of 256;
 * holds the per-sequence tree / accepted verdicts and, for N > 128, the
 * verify's intermediate between its two launches: per (sequence, value head)
 * the values of the tree-shaped operator on the ancestor pairs and gamma, per
 * sequence where each pair goes, about 4 (24 N + N) H_v B + 4 N B bytes).
 * 0 if dims is NULL. */
size_t gdn_tree_workspace_bytes(const gdn_tree_dims* dims);

/* Creates a context for `dims` over a caller-owned device workspace of at
 * least gdn_tree_workspace_bytes(dims) bytes (256-byte aligned).  The
 * workspace must outlive the context.  *out receives the handle. */
gdn_status gdn_ctx_create(const gdn_tree_dims* dims, void* workspace, size_t workspace_bytes,
                          gdn_ctx** out);

/* Frees the host handle (not the workspace).  NULL is accepted. */
gdn_status gdn_ctx_destroy(gdn_ctx* ctx);

/* Verifies the whole tree in one pass (the section's rollback-free tree
 * verification).
 *   q, k    [B][N][H_k][d_k]  bf16 or fp32 (dims.qkv_dtype)
 *   v       [B][N][H_v][d_v]  bf16 or fp32
 *   g       [B][N][H_v]       fp32 log-decay, alpha = exp(g)
 *   beta    [B][N][H_v]       fp32 write strength
 *   parent  [B][N]            int32, topological (see conventions)
 *   S0      [B][H_v][d_v][d_k] fp32 prefix state; READ ONLY: never advanced,
 *                             never rolled back
 *   o       [B][N][H_v][d_v]  fp32 output, written: o[b][i][h] = S_i q_i
 * The context records k, v, g, beta, parent and S0 (borrowed, not copied)
 * for the matching gdn_commit_path; the caller must leave them unchanged
 * until that commit has run in stream order.  A new verify on the same
 * context replaces the pending record. */
gdn_status gdn_tree_verify(gdn_ctx* ctx, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const int32_t* parent,
                           const float* S0, float* o, hipStream_t stream);

/* Per-branch recurrent verification, the baseline the fused verification is
 * compared with (Trees from Marginals technical summary, Experimental
 * Results: 7.1x at tree size 128; wispaper.ai page, "Systems Innovation:
 * Fused GDN Verification").  Same arguments, outputs, context record and
 * status as gdn_tree_verify; each root-to-leaf branch is run as its own
 * sequence from a fresh copy of S0, token by token, so nodes shared by
 * several branches are recomputed once per branch.  Results equal
 * gdn_tree_verify's up to rounding.  Far slower; for comparison only. */
gdn_status gdn_tree_verify_branches(gdn_ctx* ctx, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const int32_t* parent,
                                    const float* S0, float* o, hipStream_t stream);

/* Delayed state commitment for the accepted node (same section): for each
 * sequence b, S_new[b] is the state the recurrence reaches at accepted[b]
 * when run from S0 along the root-to-accepted path of the tree recorded by
 * the last gdn_tree_verify on ctx; accepted[b] == -1 gives S_new[b] = S0[b].
 *   accepted [B]              int32 device array, in [-1, N-1]
 *   S_new    [B][H_v][d_v][d_k] fp32, written; may be exactly S0 (in place),
 *                             must not partially overlap any input
 * Returns GDN_ERR_STATE if no verify was recorded on ctx. */
gdn_status gdn_commit_path(gdn_ctx* ctx, const int32_t* accepted, float* S_new,
                           hipStream_t stream);

/* The delayed commit fused into the next verify (same section: the state is
 * committed at the next decoding step, once the accepted branch is known).
 * Equivalent to gdn_commit_path(ctx, accepted, S_next) followed by
 * gdn_tree_verify(ctx, q, k, v, g, beta, parent, S_next, o): S_next[b] is
 * the state at accepted[b] of the tree recorded on ctx, and o is the new
 * tree's output on that state.  For bf16 q/k/v and N <= 128 one kernel
 * forms S_next on chip, writes it once and verifies on it without reading
 * it back; other cases run the two steps in turn.
 *   accepted        [B] int32, in [-1, N-1], for the recorded tree
 *   q .. parent, o  the new tree, as in gdn_tree_verify (same dims)
 *   S_next          [B][H_v][d_v][d_k] fp32, written; may be exactly the
 *                   recorded S0 (in place), must not partially overlap any
 *                   input
 * Afterwards ctx records the new tree with S0 = S_next (for the next
 * commit), and gdn_ctx_status reports both the accepted-node verdicts and
 * the new tree's.  Returns GDN_ERR_STATE if no verify was recorded on ctx;
 * a failed argument check leaves the record unchanged. */
gdn_status gdn_commit_verify(gdn_ctx* ctx, const int32_t* accepted, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, const int32_t* parent,
                             float* S_next, float* o, hipStream_t stream);

/* Ancestor sets of every node (the "ancestor relationships" the interaction
 * matrices follow, same section): anc[b][i] is a bit row of ceil(N/32)
 * uint32 words with bit s set iff s lies on the root-to-i path (i included);
 * depth[b][i] is that path's length (a root has depth 1).
 *   parent [B][N] int32;  anc [B][N][ceil(N/32)] uint32;  depth [B][N] int32
 *   tree_status [B] int32, written: 0, or GDN_ERR_TREE for a sequence whose
 *               parent array is invalid (its anc/depth rows are then
 *               unspecified).  May be NULL.
 * Only B and N of dims are used.  Asynchronous on stream. */
gdn_status gdn_tree_ancestors(const gdn_tree_dims* dims, const int32_t* parent, uint32_t* anc,
                              int32_t* depth, int32_t* tree_status, hipStream_t stream);

/* Accepted-node selection: the step between a verify and the delayed
 * commit, which commits the state once the accepted branch is known (same
 * section).  The pages do not print the acceptance rule; this is greedy
 * matching from the root, the rule of lossless greedy speculative decoding:
 * starting at the prefix, move to the lowest-index child whose drafted token
 * equals the verifier's choice after the current node, until no child
 * matches.  accepted[b] is the last node reached (-1 if none) and can be
 * passed straight to gdn_commit_path; accept_len[b] is its depth, the number
 * of drafted tokens accepted.
 *   parent       [B][N]   int32, topological (an invalid entry is flagged
 *                         and read as -1)
 *   draft_token  [B][N]   int32, the token each node drafts
 *   target_token [B][N+1] int32, the verifier's choice after the prefix
 *                         (index 0) and after each node i (index i + 1)
 *   accepted     [B]      int32, written
 *   accept_len   [B]      int32, written; may be NULL
 *   tree_status  [B]      int32, written: 0 or GDN_ERR_TREE; may be NULL
 * Only B and N of dims are used; N == 0 gives accepted = -1.  Asynchronous
 * on stream. */
gdn_status gdn_accept_path(const gdn_tree_dims* dims, const int32_t* parent, const int32_t* draft_token,
                           const int32_t* target_token, int32_t* accepted, int32_t* accept_len,
                           int32_t* tree_status, hipStream_t stream);

/* Draft-tree construction upstream of verification (Trees from Marginals,
 * technical summary, Methodology, "2. Tree Construction"): a best-first
 * search over candidate continuations that pops the w best candidates of
 * the heap at a time and expands them together, so N nodes take about
 * ceil(N / w) sequential steps.  Candidate r of the prefix scores
 * root_logp[b][r]; once node j exists, its candidate r scores
 * score[j] + node_logp[b][j][r] (fp32).  Ties go to the lower parent (the
 * prefix first), then to the lower rank.  The popped candidates become nodes
 * in pop order, so the parent array is topological; a step's nodes are
 * expanded only when the step ends, and a node at depth max_depth (the
 * prefix's children have depth 1) is not expanded.
 *   root_logp  [B][n_cand]     fp32, each row non-increasing (best first)
 *   node_logp  [B][N][n_cand]  fp32, row j = candidates of the node that
 *                              becomes node j; each row non-increasing
 *   parent     [B][N]          int32, written
 *   cand_rank  [B][N]          int32, written: each node's rank among its
 *                              parent's candidates; may be NULL
 *   score      [B][N]          fp32, written: each node's score; may be NULL
 *   steps      [B]             int32, written: expansion steps taken; may be NULL
 *   build_status [B]           int32, written: 0, GDN_ERR_SHAPE (a row is
 *                              not non-increasing), or GDN_ERR_TREE (the heap
 *                              ran dry before N nodes); outputs of such a
 *                              sequence are unspecified; may be NULL
 * n_cand in [1, 32], w >= 1, max_depth >= 1; log-probabilities must be
 * finite.  Only B and N of dims are used.  Asynchronous on stream. */
gdn_status gdn_tree_build(const gdn_tree_dims* dims, int32_t n_cand, int32_t w, int32_t max_depth,
                          const float* root_logp, const float* node_logp, int32_t* parent, int32_t* cand_rank,
                          float* score, int32_t* steps, int32_t* build_status, hipStream_t stream);

/* Synchronises `stream` and reports the device-side verdicts of the last
 * verify (GDN_ERR_TREE if any sequence had an invalid parent array;
 * GDN_ERR_HIP if a bounded wait inside a verify kernel timed out, which
 * means a defect of the kernel, not of the inputs) and, after a commit, of
 * the last commit (GDN_ERR_ACCEPT if any accepted[b] was out of range).
 * GDN_OK otherwise. */
gdn_status gdn_ctx_status(gdn_ctx* ctx, hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation:
 * gdn_tree_verify without a context or a caller workspace.  Same inputs,
 * output and kernels as gdn_tree_verify; the per-sequence verdicts those
 * kernels write (the scratch memory a context takes from its workspace) go
 * to a fixed array in the library's own device memory, GDN_STATIC_MAX_B
 * words on each GPU, held until the process ends.  The call allocates
 * nothing and does not synchronise.  It arms no commit and reports no
 * verdicts (use a context for those).  B above GDN_STATIC_MAX_B is
 * GDN_ERR_SHAPE.  Calls that overlap on one GPU race on that array; calls
 * ordered on a stream do not.  GDN_VALIDATE and GDN_FORCE_SIMPLE do not
 * apply. */
#define GDN_STATIC_MAX_B 65536
gdn_status gdn_tree_verify_static(const gdn_tree_dims* dims, const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, const int32_t* parent, const float* S0,
                                  float* o, hipStream_t stream);

/* Static English name of a status code. */
const char* gdn_status_string(gdn_status status);

/* Detail message of the last error returned on the calling thread ("" if
 * none).  Valid until the next call on that thread. */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
