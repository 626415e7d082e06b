// Fused commit + verify for bf16 q/k/v, d_k = d_v = 128, n <= 64 (gfx950).
//
// The commitment of an accepted branch is deferred to the next iteration
// (DFlash-TfM page, section on rollback-free tree verification for GDN), so
// one call advances S along the previous tree's accepted path and verifies
// the next tree from the result.  One workgroup per (sequence, head): the
// state slab of each wave (128 x 32 fp32, four result tiles) is read from
// HBM once, committed in registers (path_commit.hpp), written back once, and
// is then the B operand of Q S and K S for the verify (tree_verify.hpp)
// without another trip through memory.  The write-back of the committed
// state is issued before the verify's tree matrices are built, so it drains
// while the workgroup computes.
//
// Load order: the state slab first (the commit needs it), then the path
// rows, then the new tree's Q/K while the first path chunk is prepared, then
// V while the committed state is written back.  LDS (79 KB, two workgroups
// per CU): the Q/K tiles are staged during the commit; the commit's chunk
// tiles, the new V tile and the solve blocks take turns in one region.
#include "internal.hpp"
#include "path_commit.hpp"
#include "tree_verify.hpp"

namespace gdn {
namespace {

using namespace tv;

struct CommitPart {
    pc::ChunkTiles ct;
    pc::PathIds pi;
};

struct Smem {
    union {
        QKTiles t;
        float o[kN][kD + 4];
    } a;
    union {
        CommitPart cp;
        uint16_t v[kN][kQK];
        SolveBlocks s;
    } b;
    Topo tp;
    int commit_ok;
};

__global__ __launch_bounds__(kThreads, 2) void commit_verify_mfma_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k_prev, const uint16_t *__restrict__ v_prev,
    const float *__restrict__ alpha_prev, const float *__restrict__ beta_prev,
    const int32_t *__restrict__ parent_prev, int n_prev, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, float *__restrict__ out, int n, int H,
    int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const Lane c = lane_coords();
    const Seq s = seq_coords(blockIdx.x, n, H);
    const int mlen = path_len[s.b];
    float *slab = S + (size_t)blockIdx.x * kD * kD;

    // ---- 1. previous path (wave 1), state slab, new tree gates
    f32x16 st[4];
    if (c.w == 1) {
        const bool ok = pc::validate_and_keep(sm.b.cp.pi, parent_prev + (size_t)s.b * n_prev,
                                              path + (size_t)s.b * max_path, mlen, max_path,
                                              n_prev, c.l);
        if (c.l == 0) sm.commit_ok = ok;
    }
    load_state(st, slab, c.col, c.h);
    const Gates gt = load_gates(c, s, parent, alpha, beta);
    if (c.w == 3) topology(c, s, gt, sm.tp, status, false);
    lds_barrier();
    const bool commit_ok = sm.commit_ok;
    if (c.tid == 0 && s.hd == 0 && status)
        status[s.b] = (commit_ok ? 0 : kFaultBadPath) | (sm.tp.bad ? kFaultBadParent : 0);

    // ---- 2. commit along the previous path, chunk by chunk, in registers.
    //         The new tree's Q/K rows are requested right after the first
    //         chunk's rows, so they arrive while the chunk is prepared.
    const bool commit = commit_ok && mlen > 0;
    if (commit) {
        bf16x8 ident[2];
        pc::key_identity(ident, c.m, c.h);
        {
            const pc::ChunkRows cr = pc::load_chunk(sm.b.cp.pi.pid, 0, mlen, s.b, s.hd, n_prev, H,
                                                    k_prev, v_prev, alpha_prev, beta_prev, c.tid);
            uint4 rq[4], rk[4];
            load_rows(c, s, q, rq);
            load_rows(c, s, k, rk);
            pc::build_chunk(sm.b.cp.ct, cr, 0, mlen, c.tid, c.w, c.l);
            store_rows_permuted(c, rq, sm.a.t.q);
            store_rows_permuted(c, rk, sm.a.t.k);
            pc::apply_chunk(sm.b.cp.ct, st, ident, c.m, c.h, c.col);
            lds_barrier();   // the chunk tiles are restaged (or become the V tile)
        }
        for (int c0 = pc::kC; c0 < mlen; c0 += pc::kC) {
            pc::prepare_chunk(sm.b.cp.ct, sm.b.cp.pi.pid, c0, mlen, s.b, s.hd, n_prev, H, k_prev,
                              v_prev, alpha_prev, beta_prev, c.tid, c.w, c.l);
            pc::apply_chunk(sm.b.cp.ct, st, ident, c.m, c.h, c.col);
            lds_barrier();
        }
    } else {
        uint4 rq[4], rk[4];
        load_rows(c, s, q, rq);
        load_rows(c, s, k, rk);
        store_rows_permuted(c, rq, sm.a.t.q);
        store_rows_permuted(c, rk, sm.a.t.k);
    }

    // ---- 3. new V rows in flight while the committed state is written back
    uint4 rv[4];
    load_rows(c, s, v, rv);
    if (commit) store_state(st, slab, c.col, c.h);
    store_rows(c, rv, sm.b.v);
    lds_barrier();

    // ---- 4. verify the new tree from the committed state (held in st)
    f32x16 gc, ga;
    if (c.w < 3) gram(c, sm.a.t, gc, ga);
    uint32_t vpk[2][8];
    v_to_regs(c, sm.b.v, vpk);
    lds_barrier();
    if (sm.tp.bad) {
        store_nan(c, s, out);
        return;
    }
    if (c.w < 3) mask(c, sm.tp, gc, ga, sm.b.s);
    lds_barrier();
    inverse(c, sm.b.s);
    f32x16 P[2], R[2];
    contract(c, sm.a.t, st, P, R);
    lds_barrier();
    f32x16 o0, o1;
    solve_output(c, sm.tp, sm.b.s, P, R, vpk, o0, o1);
    store_output(c, s, sm.a.o, o0, o1, out);
}

}  // namespace

bool commit_verify_mfma_supports(const CommitVerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.c.dtype == GDN_DTYPE_BF16 && a.c.dk == kD && a.c.dv == kD && a.v.n <= kN &&
           a.v.H <= 4096;
}

hipError_t launch_commit_verify_mfma(const CommitVerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(commit_verify_mfma_kernel, dim3((unsigned)(a.v.batch * a.v.H)),
                       dim3(kThreads), 0, s, a.c.S, a.c.path, a.c.path_len, a.c.max_path,
                       (const uint16_t *)a.c.k, (const uint16_t *)a.c.v, a.c.alpha, a.c.beta,
                       a.c.parent, a.c.n, (const uint16_t *)a.v.q, (const uint16_t *)a.v.k,
                       (const uint16_t *)a.v.v, a.v.alpha, a.v.beta, a.v.parent, a.v.out, a.v.n,
                       a.v.H, a.v.status);
    return hipGetLastError();
}

}  // namespace gdn
