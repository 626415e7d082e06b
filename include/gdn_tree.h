/*
 * gdn_tree.h -- C ABI of libgdntree.so: rollback-free tree verification and
 * state commit for Gated DeltaNet (GDN) layers on AMD MI355X (gfx950).
 *
 * The operations follow the DFlash-TfM summary page, section "Verifica
 * dell'Albero Senza Rollback per GDN" (rollback-free tree verification for
 * GDN):
 *   - the GDN state update S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
 *     + beta_t k_t v_t^T, with S of shape d_k x d_v;
 *   - the draft tree is topologically sorted;
 *   - outputs for every tree node are computed from the committed state
 *     without updating it, through ancestor interaction matrices X, Y and
 *     the system (I + X) U = beta V;
 *   - the state is committed later, along the accepted branch only, so no
 *     rollback is ever needed.
 * The output of node i is o_i = S_i^T q_i, where S_i is the state after the
 * update of node i along its root-to-node path (the pages do not print the
 * readout; this is the reading adopted).  No scaling of q is applied.
 *
 * Conventions shared by every entry point
 *   - All array arguments are caller-owned DEVICE pointers, C-contiguous,
 *     16-byte aligned.  The library allocates no device memory and never
 *     frees caller memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Host-detected errors are returned synchronously as a
 *     negative gdn_status and launch nothing.
 *   - Device-detected tree faults are written, without any host sync, to
 *     the optional int32 array status[batch] (may be NULL): status[b] is
 *     OVERWRITTEN with the OR of the GDN_FAULT_* flags found for batch
 *     element b, 0 when none.
 *   - Shapes: 1 <= batch, 1 <= H, 1 <= n <= GDN_MAX_NODES, and
 *     d_k, d_v multiples of 8 in [8, GDN_MAX_DIM].  n is uniform over the
 *     batch; the trees may differ per sequence.
 *   - Functions are stateless and thread-safe.  Calls that overlap on the
 *     same output memory race.
 *
 * Tensor layouts (row-major):
 *   q, k    [batch][n][H][d_k]    bf16 or fp32 (qkv_dtype)
 *   v       [batch][n][H][d_v]    same dtype as q, k
 *   alpha   [batch][n][H]         fp32, the decay alpha_t
 *   beta    [batch][n][H]         fp32, the write strength beta_t
 *   parent  [batch][n]            int32; -1 = child of the committed state;
 *                                 valid trees have -1 <= parent[i] < i
 *   S0, S   [batch][H][d_k][d_v]  fp32 state
 *   out     [batch][n][H][d_v]    fp32
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_TREE_ABI_VERSION 8
#define GDN_MAX_NODES 128
#define GDN_MAX_DIM 128
#define GDN_MAX_CANDIDATES 32   /* child candidates per node, gdn_tree_build */

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size          */
    GDN_ERR_UNSUPPORTED = -2, /* shape or dtype outside the supported set   */
    GDN_ERR_HIP = -3          /* the HIP runtime refused a launch           */
} gdn_status;

/* element types: q/k/v take F32 or BF16; the pseudo-values of
   gdn_tree_commit_verify take F32 or F16 */
typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1, GDN_DTYPE_F16 = 2 } gdn_dtype;

/* device-detected fault flags (status[b]) */
#define GDN_FAULT_BAD_PARENT 1 /* some parent[i] outside [-1, i)             */
#define GDN_FAULT_BAD_PATH 2   /* path not a root-connected increasing chain,
                                  an id outside [0, n), or a length outside
                                  [0, max_path]                             */

/*
 * Tree verify (the rollback-free verification of the section above).
 * For every batch element b, head h and node i, writes
 *   out[b][i][h][:] = S_i^T q[b][i][h][:]
 * where S_i is S0[b][h] advanced by the GDN update along root..i.
 * S0 is READ-ONLY: verify never writes the committed state.
 * `out` must not alias any input.  A batch element whose parent row is
 * malformed gets GDN_FAULT_BAD_PARENT and all its out rows set to NaN.
 * Arithmetic: products and sums in fp32 (bf16 inputs are widened exactly).
 */
gdn_status gdn_tree_verify(const void *q, const void *k, const void *v,
                           gdn_dtype qkv_dtype, const float *alpha,
                           const float *beta, const int32_t *parent,
                           const float *S0, float *out, int batch, int n,
                           int H, int d_k, int d_v, int32_t *status,
                           void *stream);

/*
 * Single-branch recurrent verification (the baseline of the experimental
 * results section of the DFlash-TfM page: the fused tree kernel is compared
 * with verifying one branch at a time by the recurrence).  Same arguments,
 * layouts, fault behaviour and result as gdn_tree_verify (up to rounding
 * order): every root-to-leaf branch is run from S0 as its own chain by the
 * GDN update, and each node's output S_i^T q_i is written by the branches
 * through it.  S0 is read once per branch and shared prefixes are
 * recomputed per branch.  Meant for measurement, not for serving.
 */
gdn_status gdn_branch_verify(const void *q, const void *k, const void *v,
                             gdn_dtype qkv_dtype, const float *alpha,
                             const float *beta, const int32_t *parent,
                             const float *S0, float *out, int batch, int n,
                             int H, int d_k, int d_v, int32_t *status,
                             void *stream);

/*
 * State commit along the accepted branch (the delayed commitment of the
 * section above).  For each batch element b with m = path_len[b]:
 *   S[b][h] <- GDN update applied for t = path[b][0], ..., path[b][m-1]
 * in place, for every head h.  path is [batch][max_path] int32, root first;
 * path_len is [batch] int32.  k, v, alpha, beta, parent are the tensors of
 * the verify call that produced the tree.  m = 0 is a no-op.  A batch
 * element whose path is invalid (see GDN_FAULT_BAD_PATH) gets that flag and
 * its S is left bit-unchanged.  Commit is not idempotent: do not replay it.
 */
gdn_status gdn_tree_commit(float *S, const int32_t *path,
                           const int32_t *path_len, int max_path,
                           const void *k, const void *v, gdn_dtype qkv_dtype,
                           const float *alpha, const float *beta,
                           const int32_t *parent, int batch, int n, int H,
                           int d_k, int d_v, int32_t *status, void *stream);

/*
 * Commit of the previous step's accepted branch fused with the verify of
 * the next tree (the commitment is deferred to the next iteration in the
 * section above, so the two meet in one call).  Same result as
 *   gdn_tree_commit(S, path, path_len, max_path, k_prev, v_prev, qkv_dtype,
 *                   alpha_prev, beta_prev, parent_prev, batch, n_prev, H,
 *                   d_k, d_v, ...);
 *   gdn_tree_verify(q, k, v, qkv_dtype, alpha, beta, parent, S, out, batch,
 *                   n, H, d_k, d_v, ...);
 * on the same stream: S is advanced in place along path (the previous tree,
 * n_prev nodes, tensors k_prev, v_prev, alpha_prev, beta_prev, parent_prev
 * in the layouts above with n_prev rows), then the tree (q, k, v, alpha,
 * beta, parent, n nodes) is verified from the committed S, which the call
 * reads from HBM once and writes once.  status[b] receives the OR of both
 * halves' flags: GDN_FAULT_BAD_PATH leaves S[b] bit-unchanged and the
 * verify runs from it; GDN_FAULT_BAD_PARENT (of the new tree) sets that
 * element's out rows to NaN and does not undo its commit.  path_len[b] = 0
 * commits nothing.
 *
 * Pseudo-values (optional).  The verify solves for u_i = beta_i (v_i -
 * alpha_i S_p^T k_i) of every node (S_p: the state at i's parent), and the
 * state after a path is e^{g} S + sum_s e^{g - g_s} k_s u_s^T.  u_out
 * [batch][n][H][d_v], when not NULL, receives the new tree's u (NaN rows
 * for a malformed tree).  u_prev [batch][n_prev][H][d_v], when not NULL,
 * must be the u_out that the call verifying the previous tree wrote from
 * this same S: the commit then applies that sum directly instead of
 * solving again (faster; same result up to rounding).  Other u_prev values
 * give that sum, not the commit.  With u_prev, a previous tree whose parent
 * row is malformed (its verify wrote NaN pseudo-values) counts as a bad
 * path: GDN_FAULT_BAD_PATH, S[b] left bit-unchanged.  The first call of a decode loop passes
 * path_len = 0 and u_prev = NULL.  u_dtype (read only when u_prev or u_out
 * is given) is the element type of both: GDN_DTYPE_F32, or GDN_DTYPE_F16
 * for half the bytes, u rounded to the nearest fp16 when written (relative
 * error at most 2^-11 for |u| in [2^-14, 65504]; larger |u| overflows, so
 * F16 is for pseudo-values in that range).  The committed state then
 * differs from the solving commit by at most 2^-11 sum_s e^{g - g_s}
 * |k_s| |u_s|^T elementwise (plus rounding).  u_out needs bf16 and
 * d_k = d_v = 128 (else GDN_ERR_UNSUPPORTED).  u_prev is used when n <= 64.
 * For 64 < n <= 128 the commit solves for the pseudo-values itself and
 * u_prev is ignored (one launch).  Other shapes (fp32 q/k/v, d != 128) take
 * a commit launch then a verify launch and ignore u_prev.
 *
 * out and u_out must not alias any input, S must not alias any other
 * argument; the previous-tree tensors may be the same tensors as the new
 * ones.  1 <= n_prev <= GDN_MAX_NODES, 1 <= max_path.
 */
gdn_status gdn_tree_commit_verify(float *S, const int32_t *path,
                                  const int32_t *path_len, int max_path,
                                  const void *k_prev, const void *v_prev,
                                  const float *alpha_prev,
                                  const float *beta_prev,
                                  const int32_t *parent_prev,
                                  const void *u_prev, int n_prev,
                                  const void *q, const void *k, const void *v,
                                  gdn_dtype qkv_dtype, const float *alpha,
                                  const float *beta, const int32_t *parent,
                                  float *out, void *u_out, gdn_dtype u_dtype,
                                  int batch, int n, int H, int d_k, int d_v,
                                  int32_t *status, void *stream);

/*
 * Width-w best-first draft-tree construction (the DFlash-TfM page's tree
 * construction section: top-w candidates are taken off the candidate heap
 * and expanded together, ceil(B/w) rounds for a budget of B nodes).
 * cand_logp [batch][n][K] fp32 and cand_tok [batch][n][K] int32: row i holds
 * the K child candidates that the i-th inserted node proposes (log-probs,
 * -inf or NaN for an absent slot, token ids); node ids are insertion order.
 * Node 0 is the root (score 0, depth 0, token root_tok[b], or -1 when
 * root_tok is NULL).  An inserted node proposes its candidates with score
 * = its score + log-prob (one fp32 addition) unless the child would be
 * deeper than max_depth; each round takes up to `width` candidates, best
 * first (higher score, then lower node id, then lower slot), and the new
 * nodes propose from the next round on.  Writes parent/token/score
 * [batch][n] (a topologically sorted tree, ready for gdn_tree_verify) and,
 * when not NULL, n_built[b]: fewer than n when the candidates run out, the
 * unused rows then hold parent -1, token -1, score -inf.  The score order
 * decides integers, so it is fp32 exactly as stated; results are bit-exact.
 * 1 <= n <= GDN_MAX_NODES, 1 <= K <= GDN_MAX_CANDIDATES, width >= 1,
 * max_depth >= 0.
 */
gdn_status gdn_tree_build(const float *cand_logp, const int32_t *cand_tok,
                          const int32_t *root_tok, int32_t *parent,
                          int32_t *token, float *score, int32_t *n_built,
                          int batch, int n, int K, int width, int max_depth,
                          void *stream);

/*
 * Greedy acceptance walk: finds the accepted branch whose commitment the
 * section above defers to the next iteration.  draft_tok [batch][n] holds
 * each node's draft token id, verify_tok [batch][n] the verifier's greedy
 * token id after the node's root-to-node prefix.  Node 0 (the tree's root)
 * is accepted; from an accepted node p the walk moves to the lowest-id child
 * c with draft_tok[c] == verify_tok[p] and stops when no child matches.
 * Roots other than node 0 are never reached.  Writes accepted[b] (the last
 * accepted node: feed it to gdn_tree_path), and, when not NULL,
 * accept_len[b] (accepted nodes, depth + 1) and bonus_tok[b] (the
 * verifier's token at the last accepted node).  A malformed parent row gives
 * GDN_FAULT_BAD_PARENT, accepted -1, length 0, token -1.  Integer work,
 * bit-exact.  The pages do not spell out the acceptance rule; this greedy
 * match is the reading adopted.
 */
gdn_status gdn_tree_accept(const int32_t *parent, const int32_t *draft_tok,
                           const int32_t *verify_tok, int32_t *accepted,
                           int32_t *accept_len, int32_t *bonus_tok, int batch,
                           int n, int32_t *status, void *stream);

/*
 * Accepted path (the section above commits the state along the accepted
 * branch only, once that branch is known; this call turns the accepted node
 * into that branch, the input of gdn_tree_commit and of the commit half of
 * gdn_tree_commit_verify): path[b][0..m) = root .. accepted[b] (root
 * first), the rest of the row -1, path_len[b] = m.  The walk goes up from accepted[b]; a
 * parent outside [-1, node) stops it with GDN_FAULT_BAD_PARENT; an accepted
 * id outside [0, n) or m > max_path gives GDN_FAULT_BAD_PATH.  A faulted row
 * is all -1 with path_len 0.  Integer work, bit-exact.  1 <= max_path.
 */
gdn_status gdn_tree_path(const int32_t *parent, const int32_t *accepted,
                         int32_t *path, int32_t *path_len, int batch, int n,
                         int max_path, int32_t *status, void *stream);

/*
 * Tree indexing (the section above takes the draft tree topologically sorted
 * and builds X and Y from the ancestor relations between its nodes: X over
 * strict ancestors, Y over ancestors and the node itself; this call exposes
 * the indexing that the verify kernels compute on chip, for inspection and
 * tests): depth[b][i] (root = 0) and the ancestor-or-self bitmask
 * anc[b][i][ceil(n/32)] (bit s%32 of word s/32 is set iff s == i or s is an
 * ancestor of i).  A malformed tree gives GDN_FAULT_BAD_PARENT, depth -1
 * and anc 0 for every node of that batch element.  Bit-exact.
 */
gdn_status gdn_tree_index(const int32_t *parent, int32_t *depth,
                          uint32_t *anc, int batch, int n, int32_t *status,
                          void *stream);

/* human-readable text for a gdn_status value (never NULL) */
const char *gdn_status_string(int status);

/* GDN_TREE_ABI_VERSION of the loaded library */
int gdn_tree_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
