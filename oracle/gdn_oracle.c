/*
 * fp64 CPU oracle for Gated DeltaNet tree verification and commit.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or constant table with the HIP
 * library: the fault flag values below are restated from the documented
 * meaning of the status array, not included.
 *
 * What it computes is the plain definition, not the method's fast form:
 *
 *   GDN update (DFlash-TfM page, "Verifica dell'Albero Senza Rollback per
 *   GDN", the state-update formula):
 *       S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   with alpha_t multiplying only the (I - beta k k^T) S term, the write
 *   beta k v^T undecayed (as printed).  S is d_k x d_v.
 *
 *   Tree verify: the tree is topologically sorted (same section, first
 *   bullet of the solution), so every node's root-to-node path is known; the
 *   output of node i is o_i = S_i^T q_i where S_i is the state after running
 *   the update along that path from the committed state S0.  S0 is never
 *   written (same section: outputs are computed without updating the
 *   recurrent state).  The readout o = S^T q is the reading adopted for the
 *   output, which the pages do not print.
 *
 *   Commit: the same update run along the accepted branch, root first (same
 *   section: commitment is deferred until the accepted branch is known).
 *
 *   Tree indexing: depth and the ancestor-or-self set of each node.
 *
 *   Acceptance walk: the greedy walk from the root that makes the accepted
 *   branch known (see oracle_accept for the reading adopted).
 *
 * Every sum runs in a fixed order (row index ascending).  The memoised
 * verify computes the state of node i from the stored state of parent(i)
 * with exactly the same operations in the same order as the literal walk, so
 * the two agree bit for bit.  OpenMP splits over independent
 * (sequence, head) pairs only.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* fault flags written to status[b]; 0 = no fault */
enum { ORACLE_BAD_PARENT = 1, ORACLE_BAD_PATH = 2 };

/* parent[i] must lie in [-1, i): the topological order is an input contract */
static int tree_ok(const int32_t *parent, int n)
{
    for (int i = 0; i < n; ++i)
        if (parent[i] < -1 || parent[i] >= i)
            return 0;
    return 1;
}

/* one GDN update of S (d_k x d_v, row-major) by (k, v, alpha, beta).
 * w = S^T k is formed first from the old S, then every entry is replaced. */
static void gdn_update(double *S, int dk, int dv, const double *kt,
                       const double *vt, double a, double b, double *w)
{
    for (int c = 0; c < dv; ++c)
        w[c] = 0.0;
    for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c)
            w[c] += S[(size_t)r * dv + c] * kt[r];
    for (int r = 0; r < dk; ++r) {
        const double bk = b * kt[r];
        for (int c = 0; c < dv; ++c) {
            double *s = &S[(size_t)r * dv + c];
            *s = a * (*s - bk * w[c]) + bk * vt[c];
        }
    }
}

/* o = S^T q */
static void gdn_readout(const double *S, int dk, int dv, const double *qt,
                        double *o)
{
    for (int c = 0; c < dv; ++c)
        o[c] = 0.0;
    for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c)
            o[c] += S[(size_t)r * dv + c] * qt[r];
}

static int default_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Verify.  q,k [batch][n][H][dk], v [batch][n][H][dv], alpha/beta
 * [batch][n][H], parent [batch][n], S0 [batch][H][dk][dv], out
 * [batch][n][H][dv].  memo = 0: literal per-node path walk; memo != 0:
 * state of i from the stored state of parent(i).  status [batch] (may be
 * NULL) receives ORACLE_BAD_PARENT for a malformed tree, whose out rows are
 * all NaN.  Returns the number of threads used.
 */
int oracle_verify(const double *q, const double *k, const double *v,
                  const double *alpha, const double *beta,
                  const int32_t *parent, const double *S0, double *out,
                  int batch, int n, int H, int dk, int dv, int memo,
                  int nthreads, int32_t *status)
{
    const int nt = default_threads(nthreads);
    for (int b = 0; b < batch; ++b) {
        int ok = tree_ok(parent + (size_t)b * n, n);
        if (status)
            status[b] = ok ? 0 : ORACLE_BAD_PARENT;
        if (!ok)
            for (size_t e = 0; e < (size_t)n * H * dv; ++e)
                out[(size_t)b * n * H * dv + e] = NAN;
    }
    const long pairs = (long)batch * H;
#pragma omp parallel num_threads(nt)
    {
        const size_t ss = (size_t)dk * dv;
        double *S = malloc(ss * sizeof(double));
        double *w = malloc((size_t)dv * sizeof(double));
        double *states = memo ? malloc((size_t)n * ss * sizeof(double)) : NULL;
        int *path = malloc((size_t)n * sizeof(int));
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < pairs; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H);
            const int32_t *par = parent + (size_t)b * n;
            if (!tree_ok(par, n))
                continue;
            const double *s0 = S0 + ((size_t)b * H + h) * ss;
            for (int i = 0; i < n; ++i) {
                const size_t row = ((size_t)b * n + i) * H + h;
                const double *kt = k + row * dk, *vt = v + row * dv;
                double *cur;
                if (memo) {
                    cur = states + (size_t)i * ss;
                    const double *from = par[i] < 0 ? s0 : states + (size_t)par[i] * ss;
                    memcpy(cur, from, ss * sizeof(double));
                    gdn_update(cur, dk, dv, kt, vt, alpha[row], beta[row], w);
                } else {
                    int m = 0;
                    for (int t = i; t >= 0; t = par[t])
                        path[m++] = t;
                    memcpy(S, s0, ss * sizeof(double));
                    for (int j = m - 1; j >= 0; --j) {
                        const size_t rt = ((size_t)b * n + path[j]) * H + h;
                        gdn_update(S, dk, dv, k + rt * dk, v + rt * dv,
                                   alpha[rt], beta[rt], w);
                    }
                    cur = S;
                }
                gdn_readout(cur, dk, dv, q + row * dk, out + row * dv);
            }
        }
        free(S);
        free(w);
        free(states);
        free(path);
    }
    return nt;
}

/* path [batch][max_path] root first; validity: 0 <= m <= max_path, ids in
 * [0, n), parent[path[0]] == -1, parent[path[j]] == path[j-1] and
 * path[j-1] < path[j].  Returns 1 if the path of batch element b is valid. */
static int path_ok(const int32_t *par, int n, const int32_t *path, int m,
                   int max_path)
{
    if (m < 0 || m > max_path)
        return 0;
    for (int j = 0; j < m; ++j) {
        const int id = path[j];
        if (id < 0 || id >= n)
            return 0;
        const int want = j == 0 ? -1 : path[j - 1];
        if (par[id] != want)
            return 0;
        if (j > 0 && path[j - 1] >= id)
            return 0;
    }
    return 1;
}

/*
 * Commit: S [batch][H][dk][dv] updated in place along path[b][0..m).  A
 * batch element with an invalid path keeps its S untouched and gets
 * ORACLE_BAD_PATH in status.  m = 0 is a no-op.
 */
int oracle_commit(double *S, const int32_t *path, const int32_t *path_len,
                  int max_path, const double *k, const double *v,
                  const double *alpha, const double *beta,
                  const int32_t *parent, int batch, int n, int H, int dk,
                  int dv, int nthreads, int32_t *status)
{
    const int nt = default_threads(nthreads);
    int *ok = malloc((size_t)batch * sizeof(int));
    for (int b = 0; b < batch; ++b) {
        ok[b] = path_ok(parent + (size_t)b * n, n, path + (size_t)b * max_path,
                        path_len[b], max_path);
        if (status)
            status[b] = ok[b] ? 0 : ORACLE_BAD_PATH;
    }
    const long pairs = (long)batch * H;
#pragma omp parallel num_threads(nt)
    {
        double *w = malloc((size_t)dv * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < pairs; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H);
            if (!ok[b])
                continue;
            double *s = S + ((size_t)b * H + h) * (size_t)dk * dv;
            for (int j = 0; j < path_len[b]; ++j) {
                const size_t rt = ((size_t)b * n + path[(size_t)b * max_path + j]) * H + h;
                gdn_update(s, dk, dv, k + rt * dk, v + rt * dv, alpha[rt],
                           beta[rt], w);
            }
        }
        free(w);
    }
    free(ok);
    return nt;
}

/*
 * Accepted path: root -> accepted[b], written to path[b][0..m), the rest of
 * the row -1.  The walk goes up from the accepted node; a parent outside
 * [-1, node) stops it with ORACLE_BAD_PARENT; an accepted id outside [0, n)
 * or a walk longer than max_path gives ORACLE_BAD_PATH.  On a fault the row
 * is all -1 and path_len[b] = 0.
 */
void oracle_path(const int32_t *parent, const int32_t *accepted,
                 int32_t *path, int32_t *path_len, int batch, int n,
                 int max_path, int32_t *status)
{
    int *tmp = malloc((size_t)(n > 0 ? n : 1) * sizeof(int));
    for (int b = 0; b < batch; ++b) {
        const int32_t *par = parent + (size_t)b * n;
        int32_t *row = path + (size_t)b * max_path;
        int flag = 0, m = 0;
        int a = accepted[b];
        if (a < 0 || a >= n) {
            flag = ORACLE_BAD_PATH;
        } else {
            int cur = a;
            while (cur != -1) {
                tmp[m++] = cur;
                const int p = par[cur];
                if (p < -1 || p >= cur) {
                    flag = ORACLE_BAD_PARENT;
                    break;
                }
                cur = p;
            }
            if (!flag && m > max_path)
                flag = ORACLE_BAD_PATH;
        }
        for (int j = 0; j < max_path; ++j)
            row[j] = -1;
        if (!flag)
            for (int j = 0; j < m; ++j)
                row[j] = tmp[m - 1 - j];
        path_len[b] = flag ? 0 : m;
        if (status)
            status[b] = flag;
    }
    free(tmp);
}

/*
 * Tree indexing: depth [batch][n] (root = 0) and the ancestor-or-self bitmask
 * anc [batch][n][ceil(n/32)] (bit s%32 of word s/32 set iff s is i or an
 * ancestor of i).  A malformed tree gives depth -1, anc 0 for all its nodes
 * and ORACLE_BAD_PARENT.
 */
void oracle_index(const int32_t *parent, int32_t *depth, uint32_t *anc,
                  int batch, int n, int32_t *status)
{
    const int W = (n + 31) / 32;
    for (int b = 0; b < batch; ++b) {
        const int32_t *par = parent + (size_t)b * n;
        int32_t *dep = depth + (size_t)b * n;
        uint32_t *a = anc + (size_t)b * n * W;
        const int ok = tree_ok(par, n);
        if (status)
            status[b] = ok ? 0 : ORACLE_BAD_PARENT;
        memset(a, 0, (size_t)n * W * sizeof(uint32_t));
        for (int i = 0; i < n; ++i) {
            if (!ok) {
                dep[i] = -1;
                continue;
            }
            dep[i] = 0;
            for (int t = i; t >= 0; t = par[t]) {
                a[(size_t)i * W + t / 32] |= 1u << (t % 32);
                if (t != i)
                    dep[i] += 1;
            }
        }
    }
}

/*
 * Greedy acceptance walk (the step that makes the accepted branch known;
 * DFlash-TfM page, "Verifica dell'Albero Senza Rollback per GDN": the
 * commitment waits for the accepted branch).  Reading adopted: node 0 is the
 * tree's root and is always accepted; from an accepted node p the walk moves
 * to the child c whose draft token equals the verifier's greedy token at p
 * (draft[c] == verify[p]), the lowest such id when several siblings match,
 * and stops when no child matches.  Roots other than node 0 are never
 * reached.  Outputs: the last accepted node, the number of accepted nodes
 * (its depth + 1) and the verifier's token at it (the token the step emits
 * after the accepted draft).  A malformed parent row gives accepted -1,
 * length 0, token -1 and ORACLE_BAD_PARENT.
 */
void oracle_accept(const int32_t *parent, const int32_t *draft, const int32_t *verify,
                   int32_t *accepted, int32_t *accept_len, int32_t *bonus, int batch, int n,
                   int32_t *status)
{
    for (int b = 0; b < batch; ++b) {
        const int32_t *par = parent + (size_t)b * n;
        const int32_t *dr = draft + (size_t)b * n;
        const int32_t *vf = verify + (size_t)b * n;
        if (!tree_ok(par, n)) {
            accepted[b] = -1;
            accept_len[b] = 0;
            bonus[b] = -1;
            if (status)
                status[b] = ORACLE_BAD_PARENT;
            continue;
        }
        int cur = 0, len = 1;
        for (;;) {
            int next = -1;
            for (int c = cur + 1; c < n; ++c)
                if (par[c] == cur && dr[c] == vf[cur]) {
                    next = c;
                    break;
                }
            if (next < 0)
                break;
            cur = next;
            ++len;
        }
        accepted[b] = cur;
        accept_len[b] = len;
        bonus[b] = vf[cur];
        if (status)
            status[b] = 0;
    }
}

/*
 * Pseudo-values of the tree (the u of the chunked form; DFlash-TfM page,
 * "Verifica dell'Albero Senza Rollback per GDN", the system (I + X) U = ...).
 * Written out from the update itself: with S_p the state at the parent of
 * node i (S0 for a root),
 *     S_i = alpha_i (I - beta_i k_i k_i^T) S_p + beta_i k_i v_i^T
 *         = alpha_i S_p + k_i u_i^T,   u_i = beta_i (v_i - alpha_i S_p^T k_i),
 * so the committed state after a path is e^{g_a} S0 + sum_s e^{g_a - g_s}
 * k_s u_s^T.  U [batch][n][H][dv].  A malformed tree gives NaN rows and
 * ORACLE_BAD_PARENT.  States are formed by the same memoised walk as the
 * verify (state of i from the stored state of parent(i)).
 */
int oracle_pseudo(const double *k, const double *v, const double *alpha,
                  const double *beta, const int32_t *parent, const double *S0,
                  double *U, int batch, int n, int H, int dk, int dv, int nthreads,
                  int32_t *status)
{
    const int nt = default_threads(nthreads);
    for (int b = 0; b < batch; ++b) {
        int ok = tree_ok(parent + (size_t)b * n, n);
        if (status)
            status[b] = ok ? 0 : ORACLE_BAD_PARENT;
        if (!ok)
            for (size_t e = 0; e < (size_t)n * H * dv; ++e)
                U[(size_t)b * n * H * dv + e] = NAN;
    }
    const long pairs = (long)batch * H;
#pragma omp parallel num_threads(nt)
    {
        const size_t ss = (size_t)dk * dv;
        double *st = malloc((size_t)n * ss * sizeof(double));
        double *w = malloc((size_t)dv * sizeof(double));
#pragma omp for schedule(dynamic)
        for (long bh = 0; bh < pairs; ++bh) {
            const int b = (int)(bh / H), h = (int)(bh % H);
            const int32_t *par = parent + (size_t)b * n;
            if (!tree_ok(par, n))
                continue;
            const double *s0 = S0 + (size_t)bh * ss;
            for (int i = 0; i < n; ++i) {
                const size_t row = ((size_t)b * n + i) * H + h;
                const double *kt = k + row * dk, *vt = v + row * dv;
                const double a = alpha[row], be = beta[row];
                const double *Sp = par[i] < 0 ? s0 : st + (size_t)par[i] * ss;
                /* w = S_p^T k, then u = beta (v - alpha w) */
                for (int c = 0; c < dv; ++c)
                    w[c] = 0.0;
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c)
                        w[c] += Sp[(size_t)r * dv + c] * kt[r];
                for (int c = 0; c < dv; ++c)
                    U[row * dv + c] = be * (vt[c] - a * w[c]);
                /* the node's state, for its children */
                double *Si = st + (size_t)i * ss;
                memcpy(Si, Sp, ss * sizeof(double));
                gdn_update(Si, dk, dv, kt, vt, a, be, w);
            }
        }
        free(st);
        free(w);
    }
    return nt;
}
