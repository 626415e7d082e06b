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
//           columns; the commit once the chunk is built, the committed
//           columns written back, P and R, the solve and the output rows;
//   wave 2: the new tree's gates and Q rows, the topology, the Gram tile,
//           masks and T = (I + X)^{-1}.
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

    // ---- 2. the chunk (wave 0), its values (wave 1), the new tree's Gram
    //         and masks (wave 2)
    pc::ChunkWords U0;
    if (w == 0) {
        if (l == 0 && quarter == 0 && s.hd == 0 && status)
            status[s.b] = (path_ok ? 0 : kFaultBadPath) | (tree_ok ? 0 : kFaultBadParent);
        if (commit) {
            if constexpr (kU) {
                pc::build_keys32(sm.ch.kc, sm.cx, k32, min(32, mlen), l);
            } else {
                pc::build16_x(sm.ch.e, sm.cx, r16.k, r16.la, r16.bt, min(pc::kC16, mlen), l);
                ts::wave_lds_sync();
                pc::build16_t(sm.ch.e, l);
            }
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
    } else if (tree_ok) {
        ts::gram_mask(sm.t, m, h);
    }
    lds_barrier();   // the chunk, X and Y

    // ---- 3. the commit of the quarter's columns and P / R (wave 1), T (wave 2)
    f32x16 P, R;
    if (w == 1) {
        if (commit) {
            bf16x8 ident[2];
            pc::key_identity(ident, m, h);
            if constexpr (kU) {
                pc::apply_known_u(sm.ch.kc, sm.cx, pc::u_values<kUh>(U0), st, ident, m, h);
            } else {
                // R = K_p S over the four tiles in two accumulators, then
                // U = T RHS and the update
                const pc::ChunkView cv = pc::early_view(sm.ch.e, sm.cx, m);
                f32x16 Ra = {}, Rb = {};
                pc::rp_tile(cv.kp_row, st[0], 0, Ra, h);
                pc::rp_tile(cv.kp_row, st[1], 1, Rb, h);
                pc::rp_tile(cv.kp_row, st[2], 2, Ra, h);
                pc::rp_tile(cv.kp_row, st[3], 3, Rb, h);
                pc::finish_rows_v<pc::kC16>(cv, pc::widen_bf16(U0), Ra + Rb, st, ident, h);
            }
            store_state(st, slab, col, h);
        }
        if (tree_ok) ts::contract(sm.t, st, m, h, P, R);
    } else if (w == 2 && tree_ok) {
        ts::inverse(sm.t, l);
    }
    lds_barrier();   // T
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
