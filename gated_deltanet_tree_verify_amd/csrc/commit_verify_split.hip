// d_v-split fused commit + verify for small launches: bf16 q/k/v, d_k = d_v =
// 128, new trees of at most 32 nodes, previous paths that fit one commit
// chunk (16 slots when the commit solves for the pseudo-values, 32 when they
// are carried), one three-wave workgroup per (sequence, head, quarter of d_v)
// (gfx950).
//
// The commitment of an accepted branch is deferred to the next iteration
// (DFlash-TfM page, section on rollback-free tree verification for GDN): one
// call advances S along the previous tree's accepted path and verifies the
// next tree from the result.  The commit, like the verify, is column by
// column in d_v (R = K_p S, U = T beta (V_p - e^g R) or U given, S <- e^{g_l}
// S + K_p^T W), so a quarter's workgroup commits and verifies its own 32
// columns of the state; the path's chunk (keys, gates, its T) and the new
// tree's matrices are formed by every quarter.  Why split: see
// tree_split.hpp.
//   wave 0: the path ids and the previous tree's parent row (validation),
//           the chunk's keys and gates, then the chunk (path_commit.hpp);
//   wave 1: the new tree's K rows, the quarter's state columns and v values,
//           then the chunk's values (or carried pseudo-values) in its
//           columns.  Solving commit: Q S and K S from the slab before the
//           commit while the chunk is built; R_p = K_p S and the Grams of the
//           path keys against the new tree's queries and keys; the commit
//           once the chunk's T is in, Q S' and K S' by the commit's rank-m
//           correction.  Carried: the commit as soon as the chunk's keys are
//           in, then Q S' and K S'.  Then the committed columns written back,
//           the solve and the output rows;
//   wave 2: the new tree's gates and Q rows, the topology, the Gram tile,
//           masks and T = (I + X)^{-1}, its substitution beside the chunk's.
#include "internal.hpp"
#include "path_commit.hpp"
#include "tree_split.hpp"

namespace gdn {
namespace {

using namespace tile;
using ts::kQuarters;

constexpr int kThreads = 192;       // three waves
constexpr int kMaxPathIds = 128;    // a valid path has at most n_prev <= 128 nodes

struct Smem {
    ts::Tree t;
    union {
        pc::EarlyChunk16 e;   // the commit solves: the path's keys, X and T (16 slots)
        pc::KeyChunk32 kc;    // pseudo-values carried: the path's keys (32 slots)
    } ch;
    pc::Chunk16Aux cx;
    int pid[kMaxPathIds];     // previous path ids
    int commit_ok;
};

// Q S' and K S' from P = Q S and R = K S (S the slab before the commit):
// the commit is S' = e^{g_l} S + K_p^T W with W_j = e^{g_l - g_j} u_j, so
// Q S' = e^{g_l} Q S + (Q K_p^T) W and likewise for K.  Gq, Gk are the
// transposed Grams K_p Q^T and K_p K^T (rows = path slots crow(r, h)),
// i.e. register for register the A operands of Q K_p^T and K K_p^T; W
// enters split hi / lo as in the update of the slab (pc::apply_update).
template <int NR>
__device__ __forceinline__ void correct(f32x16 &P, f32x16 &R, const f32x16 &Gq,
                                        const f32x16 &Gk, const f32x16 &U, const float *wdec,
                                        float gl, int h) {
    constexpr int KS = NR / 16;   // k-steps over path slots that can be nonzero
    P = P * gl;
    R = R * gl;
    const SplitTile gq = split_tile(Gq), gk = split_tile(Gk);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        float wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = wdec[crow(8 * kk + j, h)] * U[8 * kk + j];
        bf16x8 wh, wl;
        split8(wv, wh, wl);
        P = mfma(gq.hi[kk], wh, P);
        P = mfma(gq.hi[kk], wl, P);
        P = mfma(gq.lo[kk], wh, P);
        R = mfma(gk.hi[kk], wh, R);
        R = mfma(gk.hi[kk], wl, R);
        R = mfma(gk.lo[kk], wh, R);
    }
}

// kU: the previous tree's pseudo-values u_prev are given (the commit is the
// rank-m update, no solve); kUout: the new tree's pseudo-values go to u_out;
// kUh: u_prev and u_out hold fp16 values (fp32 otherwise)
template <bool kU, bool kUout, bool kUh>
__global__ __launch_bounds__(kThreads) void commit_verify_split_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k_prev, const uint16_t *__restrict__ v_prev,
    const float *__restrict__ alpha_prev, const float *__restrict__ beta_prev,
    const int32_t *__restrict__ parent_prev, const void *__restrict__ u_prev, int n_prev,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ alpha,
    const float *__restrict__ beta, const int32_t *__restrict__ parent,
    float *__restrict__ out, void *__restrict__ u_out, int n, int H,
    int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = threadIdx.x & 63, m = l & 31, h = l >> 5;
    const int bh = blockIdx.x / kQuarters, quarter = blockIdx.x % kQuarters;
    const int col = 32 * quarter + m;
    const tv::Seq s = tv::seq_coords(bh, n, H);
    const int mlen = path_len[s.b];
    float *slab = S + (size_t)bh * tv::kD * tv::kD;
    // previous tree, this (sequence, head): node 0's row and gate entry
    const size_t prow0 = ((size_t)s.b * n_prev * H + s.hd) * tv::kD;
    const size_t pgate0 = (size_t)s.b * n_prev * H + s.hd;
    const uint32_t pbytes = (uint32_t)((size_t)n_prev * H * tv::kD * 2);
    constexpr int kC0 = kU ? 32 : pc::kC16;   // slots of the one chunk

    // ---- 1. loads and what needs only them
    uint4 x[8];
    f32x16 st[4];
    uint32_t vpk[8];
    pc::PathLanes pl{-1, -1, -2, -2};
    pc::KeyRows16 r16;
    pc::KeyRows32 k32;
    bool path_ok = false;
    if (w == 0) {
        // path ids and the previous tree's parent row (nodes l and 64 + l):
        // the parents of the path nodes come out of it by lane shuffles
        int pp0 = -1, pp1 = -1;
        const int32_t *prow = path + (size_t)s.b * max_path;
        const int lim = min(min(mlen, max_path), kMaxPathIds);
        if (l < lim) pl.id0 = prow[l];
        if (64 + l < lim) pl.id1 = prow[64 + l];
        const int32_t *ppar = parent_prev + (size_t)s.b * n_prev;
        if (l < n_prev) pp0 = ppar[l];
        if (64 + l < n_prev) pp1 = ppar[64 + l];
        pl.par0 = pc::parent_of(pl.id0, pp0, pp1, n_prev);
        pl.par1 = pc::parent_of(pl.id1, pp0, pp1, n_prev);
        if (pl.id0 >= 0) sm.pid[l] = pl.id0;
        if (pl.id1 >= 0) sm.pid[64 + l] = pl.id1;
        // the chunk's key rows and gates (slots past the chunk read zero)
        const int mc0 = min(kC0, mlen);
        if constexpr (kU) {
            const int rj = l >> 1, rid = pc::slot_id(pl, rj);
            k32 = pc::load_keys32(rid, rj < mc0 && rid >= 0 && rid < n_prev, pl.id0,
                                  l < mc0 && pl.id0 >= 0 && pl.id0 < n_prev, k_prev + prow0,
                                  alpha_prev + pgate0, H * tv::kD, H, pbytes, l);
        } else {
            const int rj = l >> 2, rid = pc::slot_id(pl, rj);
            r16 = pc::load_keys16(rid, rj < mc0 && rid >= 0 && rid < n_prev, pl.id0,
                                  l < mc0 && pl.id0 >= 0 && pl.id0 < n_prev, k_prev + prow0,
                                  alpha_prev + pgate0, beta_prev + pgate0, H * tv::kD, H, pbytes,
                                  l);
        }
        // with u_prev, a malformed previous tree counts as a bad path: the
        // call that verified it wrote NaN pseudo-values
        path_ok = pc::path_valid(pl, mlen, max_path, n_prev, l) &&
                  (!kU || pc::tree_valid(pp0, pp1, n_prev, l));
        if (l == 0) sm.commit_ok = path_ok && mlen > 0;
        // zero rows for the chunk operands' padded slots
        for (int i = l; i < pc::kKP; i += ts::kLanes) sm.cx.zk[i] = 0;
        if (l < pc::kBL) sm.cx.zt[l] = 0;
    } else if (w == 1) {
        ts::load_rows32(s, k, l, x);
        load_state(st, slab, col, h);
        ts::load_v_col(s, v, col, h, vpk);
        ts::store_rows32(sm.t.k, l, x);
    } else {
        ts::load_rows32(s, q, l, x);
        ts::topology(sm.t, s, parent, alpha, beta, l);
        ts::store_rows32(sm.t.q, l, x);
    }
    lds_barrier();   // path ids and validity, Q and K rows, the topology
    const bool tree_ok = !sm.t.bad;
    const bool commit = sm.commit_ok;

    // ---- 2. the chunk's keys (and X) (wave 0); the chunk's values, then Q S
    //         and K S from the slab before the commit (wave 1); the new tree's
    //         Gram and masks (wave 2)
    pc::ChunkWords U0;
    f32x16 P, R;
    if (w == 0) {
        if (l == 0 && quarter == 0 && s.hd == 0 && status)
            status[s.b] = (path_ok ? 0 : kFaultBadPath) | (tree_ok ? 0 : kFaultBadParent);
        if (commit) {
            if constexpr (kU) pc::build_keys32(sm.ch.kc, sm.cx, k32, min(32, mlen), l);
            else pc::build16_x(sm.ch.e, sm.cx, r16.k, r16.la, r16.bt, min(pc::kC16, mlen), l);
        }
    } else if (w == 1) {
        // (unconditional: with no valid slots every load reads past the end
        // of its buffer resource and returns zero)
        const int mc0 = (mlen > 0 && mlen <= kMaxPathIds) ? min(kC0, mlen) : 0;
        if constexpr (kU) {
            constexpr size_t ues = kUh ? 2 : 4;   // bytes per pseudo-value
            const void *u_head = static_cast<const char *>(u_prev) + prow0 * ues;
            const uint32_t ubytes = (uint32_t)((size_t)n_prev * H * tv::kD * ues);
            U0 = pc::load_u_chunk<kUh>(u_head, ubytes, sm.pid, 0, mc0, H * tv::kD, col, h);
        } else {
            U0 = pc::load_v_chunk16(v_prev + prow0, pbytes, sm.pid, 0, mc0, H * tv::kD, col, h);
        }
        // (the solving commit's chunk takes longer to build than the
        // contraction: Q S and K S from the slab before the commit, corrected
        // after it; with pseudo-values carried the chunk is ready at once and
        // the contraction follows the commit)
        if (!kU && tree_ok) ts::contract(sm.t, st, m, h, P, R);
    } else if (tree_ok) {
        ts::gram_mask(sm.t, m, h);
    }
    lds_barrier();   // the chunk's keys (and X); the tree's X and Y

    // ---- 3. the solving commit: the chunk's T (wave 0); R_p = K_p S and the
    //         Grams of the path keys against the new tree's queries and keys
    //         (wave 1); the substitution of the tree's diagonal sub-blocks
    //         (wave 2).  Pseudo-values carried: the commit and the contraction
    //         (wave 1), the tree's whole inverse (wave 2).
    f32x16 Rp, Gq, Gk;
    if (w == 0) {
        if constexpr (!kU) {
            if (commit) pc::build16_t(sm.ch.e, l);
        }
    } else if (w == 1 && kU) {
        // pseudo-values carried: the commit, the committed columns written
        // back, then Q S' and K S'
        if (commit) {
            bf16x8 ident[2];
            pc::key_identity(ident, m, h);
            pc::apply_known_u(sm.ch.kc, sm.cx, pc::u_values<kUh>(U0), st, ident, m, h);
            store_state(st, slab, col, h);
        }
        if (tree_ok) ts::contract(sm.t, st, m, h, P, R);
    } else if (w == 1) {
        if (commit) {
            const uint16_t *kp_row;
            if constexpr (kU) kp_row = sm.ch.kc.kp[m];
            else kp_row = m < pc::kC16 ? sm.ch.e.kp[m] : sm.cx.zk;
            if constexpr (!kU) {
                // two accumulators (two short MFMA chains)
                f32x16 Ra = {}, Rb = {};
                pc::rp_tile(kp_row, st[0], 0, Ra, h);
                pc::rp_tile(kp_row, st[1], 1, Rb, h);
                pc::rp_tile(kp_row, st[2], 2, Ra, h);
                pc::rp_tile(kp_row, st[3], 3, Rb, h);
                Rp = Ra + Rb;
            }
            if (tree_ok) {
                // transposed: lane (node i = m, h) holds k_p,s.q_i and k_p,s.k_i
                // for path slot s = crow(r, h)
                Gq = Gk = f32x16{};
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const bf16x8 a = lds8(kp_row + 16 * kk + 8 * h);
                    Gq = mfma(a, lds8(&sm.t.q[m][16 * kk + 8 * h]), Gq);
                    Gk = mfma(a, lds8(&sm.t.k[m][16 * kk + 8 * h]), Gk);
                }
            }
        }
    } else if (tree_ok) {
        if constexpr (kU) ts::inverse(sm.t, l);
        else ts::inverse_subst(sm.t, l);
    }
    lds_barrier();   // the chunk's T; the tree's sub-block inverses (all of T when carried)

    // ---- 4. the solving commit of the quarter's columns, then Q S' and K S'
    //         from Q S and K S (wave 1); the rest of the tree's inverse (wave 2)
    if (w == 1 && !kU) {
        if (commit) {
            bf16x8 ident[2];
            pc::key_identity(ident, m, h);
            const pc::ChunkView cv = pc::early_view(sm.ch.e, sm.cx, m);
            const f32x16 U = pc::chunk_u<pc::kC16>(cv, pc::widen_bf16(U0), Rp, h);
            pc::apply_update<pc::kC16>(cv, U, st, ident, h);
            if (tree_ok) correct<pc::kC16>(P, R, Gq, Gk, U, cv.wdec, cv.glast, h);
            store_state(st, slab, col, h);
        }
    } else if (w == 2 && !kU && tree_ok) {
        ts::inverse_finish(sm.t, l);
    }
    lds_barrier();   // the tree's T
    if (w != 1) return;

    // ---- 4. the solve and the output rows of the quarter's columns
    if (!tree_ok) {
        f32x16 nan;
#pragma unroll
        for (int r = 0; r < 16; ++r) nan[r] = __builtin_nanf("");
        ts::store_col(s, out, col, h, nan);
        if constexpr (kUout) {
            if constexpr (kUh) ts::store_col_f16(s, static_cast<uint16_t *>(u_out), col, h, nan);
            else ts::store_col(s, static_cast<float *>(u_out), col, h, nan);
        }
        return;
    }
    f32x16 u, o;
    ts::solve(sm.t, vpk, P, R, m, h, u, o);
    ts::store_col(s, out, col, h, o);
    if constexpr (kUout) {
        if constexpr (kUh) ts::store_col_f16(s, static_cast<uint16_t *>(u_out), col, h, u);
        else ts::store_col(s, static_cast<float *>(u_out), col, h, u);
    }
}

template <bool kU, bool kUout, bool kUh>
hipError_t launch_cvs(const CommitVerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((commit_verify_split_kernel<kU, kUout, kUh>),
                       dim3((unsigned)(a.v.batch * a.v.H * kQuarters)), dim3(kThreads), 0, s,
                       a.c.S, a.c.path, a.c.path_len, a.c.max_path, (const uint16_t *)a.c.k,
                       (const uint16_t *)a.c.v, a.c.alpha, a.c.beta, a.c.parent, a.u_prev,
                       a.c.n, (const uint16_t *)a.v.q, (const uint16_t *)a.v.k,
                       (const uint16_t *)a.v.v, a.v.alpha, a.v.beta, a.v.parent, a.v.out,
                       a.u_out, a.v.n, a.v.H, a.v.status);
    return hipGetLastError();
}

template <bool kU, bool kUout>
hipError_t launch_cvs_u(const CommitVerifyArgs &a, hipStream_t s) {
    if constexpr (kU || kUout) {
        if (a.u_half) return launch_cvs<kU, kUout, true>(a, s);
    }
    return launch_cvs<kU, kUout, false>(a, s);
}

}  // namespace

bool commit_verify_split_supports(const CommitVerifyArgs &a) {
    // small launches (as for the split verify) whose previous paths fit the
    // one chunk
    return a.c.dtype == GDN_DTYPE_BF16 && a.c.dk == tv::kD && a.c.dv == tv::kD &&
           a.v.n <= ts::kN1 && a.c.n <= kMaxPathIds && a.v.H <= 4096 &&
           a.c.max_path <= (a.u_prev ? 32 : pc::kC16) &&
           (long long)a.v.batch * a.v.H * kQuarters <= 2LL * device_cu_count();
}

hipError_t launch_commit_verify_split(const CommitVerifyArgs &a, hipStream_t s) {
    if (a.u_prev) return a.u_out ? launch_cvs_u<true, true>(a, s) : launch_cvs_u<true, false>(a, s);
    return a.u_out ? launch_cvs_u<false, true>(a, s) : launch_cvs_u<false, false>(a, s);
}

}  // namespace gdn
