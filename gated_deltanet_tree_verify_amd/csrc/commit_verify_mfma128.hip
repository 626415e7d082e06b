// Fused commit + verify for bf16 q/k/v, d_k = d_v = 128 and new trees of
// 65..128 nodes (gfx950), two workgroups per CU.
//
// The commitment of an accepted branch is deferred to the next iteration
// (DFlash-TfM page, section on rollback-free tree verification for GDN), so
// one call advances S along the previous tree's accepted path and verifies
// the next tree from the result.  One workgroup per (sequence, head), four
// waves, wave w owning d_v columns [32 w, 32 w + 32).  The commit is the
// chunked solving commit of path_commit.hpp (R = K_p S, U = T RHS,
// S <- e^{g_last} S + K_p^T W per chunk of path slots); the verify is the
// two-halves 65..128-node verify of tree_verify128h.hpp, run on the
// committed slab, which never leaves the registers in between.
//
// Schedule.  Wave 3 reads the path ids and the previous tree's parent row,
// validates the path, builds the new tree's topology and (paths of at most
// 16 nodes) lays out the 16-slot chunk, while every wave requests its state
// slab and lays out the new tree's Q / K rows 0..63.  The commit's chunk
// and path ids sit in the LDS of the solve blocks, which the verify writes
// only after the commit; longer paths go in 32-slot chunks, each later
// chunk's rows requested while the one before it is applied.  The committed
// slab is written back at once and stays in registers as the B operand of
// Q S and K S.  The new tree's pseudo-values (u_out) leave through LDS as
// whole rows next to the outputs.
#include <stddef.h>

#include "internal.hpp"
#include "tree_verify128h.hpp"

namespace gdn {
namespace {

using namespace tile;
using tv::kD;
using tv::kThreads;
using tv::Lane;
using tv::Seq;
using tvh::kMaxPathIds;

// NaN rows of an fp16 [batch][n][H][128] tensor, 128-node layout (this
// lane's entries)
__device__ __forceinline__ void store_nan_half128(const Lane &c, const Seq &s, uint16_t *dst) {
    uint16_t *row = dst + s.base + c.col;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * t + crow(r, c.h);
            if (i < s.n) row[(size_t)i * s.rstride] = 0x7e00;   // quiet NaN
        }
}

// kLong: paths may be longer than 16 nodes (the host takes this instance
// whenever max_path exceeds 16); kUout: the new tree's pseudo-values are
// written to u_out, fp16 with kUh (else fp32)
template <bool kLong, bool kUout, bool kUh>
__global__ __launch_bounds__(kThreads, 2) void commit_verify_mfma128_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k_prev, const uint16_t *__restrict__ v_prev,
    const float *__restrict__ alpha_prev, const float *__restrict__ beta_prev,
    const int32_t *__restrict__ parent_prev, int n_prev, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, float *__restrict__ out, void *__restrict__ u_out, int n,
    int H, int32_t *__restrict__ status) {
    __shared__ tvh::Smem sm;
    const Lane c = tv::lane_coords();
    const Seq s = tv::seq_coords(blockIdx.x, n, H);
    float *slab = S + (size_t)blockIdx.x * kD * kD;
    tvh::CommitAux &ax = sm.b.cm.ax;
    const int mlen = path_len[s.b];
    // previous tree, this (sequence, head): node 0's row and gate entry
    const size_t prow0 = ((size_t)s.b * n_prev * H + s.hd) * kD;
    const size_t pgate0 = (size_t)s.b * n_prev * H + s.hd;
    const uint32_t pbytes = (uint32_t)((size_t)n_prev * H * kD * 2);

    // ---- 1. wave 3: the previous path's ids, the previous tree's parents
    //         and the new tree's gates; every wave: its state slab and the
    //         new tree's Q / K rows 0..63
    pc::PathLanes pl{-1, -1, -2, -2};
    int pp0 = -1, pp1 = -1;
    tv128::Gates2 gt;
    if (c.w == 3) {
        const int32_t *prow = path + (size_t)s.b * max_path;
        const int32_t *ppar = parent_prev + (size_t)s.b * n_prev;
        const int lim = min(min(mlen, max_path), kMaxPathIds);
        if (c.l < lim) pl.id0 = prow[c.l];
        if (64 + c.l < lim) pl.id1 = prow[64 + c.l];
        if (c.l < n_prev) pp0 = ppar[c.l];
        if (64 + c.l < n_prev) pp1 = ppar[64 + c.l];
        gt = tv128::load_gates2(c, s, parent, alpha, beta);
    }
    f32x16 st[4];
    load_state(st, slab, c.col, c.h);
    uint4 rq[4], rk[4];
    tv::load_rows(c, s, q, rq);
    tv::load_rows<0>(c, s, k, rk);   // cached: rows 0..63 of K are read again for the cross blocks
    if (c.w == 3) {
        pl.par0 = pc::parent_of(pl.id0, pp0, pp1, n_prev);
        pl.par1 = pc::parent_of(pl.id1, pp0, pp1, n_prev);
        if (pl.id0 >= 0) ax.pid[c.l] = pl.id0;
        if (pl.id1 >= 0) ax.pid[64 + c.l] = pl.id1;
        pc::KeyRows16 r16;
        if constexpr (!kLong) {
            const int mc0 = min(pc::kC16, mlen);
            const int rj = c.l >> 2;
            const int rid = pc::slot_id(pl, rj);
            r16 = pc::load_keys16(rid, rj < mc0 && rid >= 0 && rid < n_prev, pl.id0,
                                  c.l < mc0 && pl.id0 >= 0 && pl.id0 < n_prev, k_prev + prow0,
                                  alpha_prev + pgate0, beta_prev + pgate0, H * kD, H, pbytes,
                                  c.l);
        }
        tv128::topology(c, s, gt, sm.tp, status, false, false);
        for (int i = c.l; i < pc::kKP; i += 64) ax.cx.zk[i] = 0;
        if (c.l < pc::kBL) ax.cx.zt[c.l] = 0;
        // validate the path (status: the path's flag and the new tree's)
        const bool ok = pc::path_valid(pl, mlen, max_path, n_prev, c.l);
        if (c.l == 0) {
            ax.commit_ok = ok;
            if (s.hd == 0 && status)
                status[s.b] = (ok ? 0 : kFaultBadPath) | (sm.tp.bad ? kFaultBadParent : 0);
        }
        if constexpr (!kLong) {
            if (ok && mlen > 0) {
                pc::build16_x(sm.b.cm.e, ax.cx, r16.k, r16.la, r16.bt, min(pc::kC16, mlen), c.l);
                pc::build16_t(sm.b.cm.e, c.l);
            }
        }
    }
    tv::store_rows_permuted(c, rq, sm.a.t.q);
    tv::store_rows_permuted(c, rk, sm.a.t.k);
    lds_barrier();
    const bool commit = ax.commit_ok && mlen > 0;

    // ---- 2. the commit on this wave's slab, written back at once
    if (commit) {
        bf16x8 ident[2];
        pc::key_identity(ident, c.m, c.h);
        if constexpr (kLong) {
            pc::ChunkRows rows = pc::load_chunk(ax.pid, 0, mlen, s.b, s.hd, n_prev, H, k_prev,
                                                v_prev, alpha_prev, beta_prev, c.tid);
            for (int c0 = 0; c0 < mlen; c0 += pc::kC) {
                pc::build_chunk(sm.b.cm.ct, rows, c0, mlen, c.tid, c.w, c.l);
                if (c0 + pc::kC < mlen)
                    rows = pc::load_chunk(ax.pid, c0 + pc::kC, mlen, s.b, s.hd, n_prev, H, k_prev,
                                          v_prev, alpha_prev, beta_prev, c.tid);
                pc::apply_chunk(sm.b.cm.ct, st, ident, c.m, c.h, c.col);
                lds_barrier();   // the chunk tiles are restaged next
            }
        } else {
            const pc::ChunkWords V0 = pc::load_v_chunk16(
                v_prev + prow0, pbytes, ax.pid, 0, min(pc::kC16, mlen), H * kD, c.col, c.h);
            const pc::ChunkView cv = pc::early_view(sm.b.cm.e, ax.cx, c.m);
            f32x16 Ra = {}, Rb = {};
            pc::rp_tile(cv.kp_row, st[0], 0, Ra, c.h);
            pc::rp_tile(cv.kp_row, st[1], 1, Rb, c.h);
            pc::rp_tile(cv.kp_row, st[2], 2, Ra, c.h);
            pc::rp_tile(cv.kp_row, st[3], 3, Rb, c.h);
            pc::finish_rows_v<pc::kC16>(cv, pc::widen_bf16(V0), Ra + Rb, st, ident, c.h);
            lds_barrier();   // every wave has read the chunk
        }
        store_state(st, slab, c.col, c.h);
    }
    if (sm.tp.bad) {
        tv128::store_nan(c, s, out);
        if constexpr (kUout) {
            if constexpr (kUh) store_nan_half128(c, s, static_cast<uint16_t *>(u_out));
            else tv128::store_nan(c, s, static_cast<float *>(u_out));
        }
        return;
    }

    // ---- 3. the verify from the committed slab
    tvh::verify_halves<kUout, kUh>(tvh::fresh_lane(), s, sm, st, q, k, v, out, u_out);
}

template <bool kLong, bool kUout, bool kUh>
hipError_t launch_cv128(const CommitVerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((commit_verify_mfma128_kernel<kLong, kUout, kUh>),
                       dim3((unsigned)(a.v.batch * a.v.H)), dim3(kThreads), 0, s, a.c.S, a.c.path,
                       a.c.path_len, a.c.max_path, (const uint16_t *)a.c.k,
                       (const uint16_t *)a.c.v, a.c.alpha, a.c.beta, a.c.parent, a.c.n,
                       (const uint16_t *)a.v.q, (const uint16_t *)a.v.k, (const uint16_t *)a.v.v,
                       a.v.alpha, a.v.beta, a.v.parent, a.v.out, a.u_out, a.v.n, a.v.H,
                       a.v.status);
    return hipGetLastError();
}

template <bool kLong>
hipError_t launch_cv128_u(const CommitVerifyArgs &a, hipStream_t s) {
    if (!a.u_out) return launch_cv128<kLong, false, false>(a, s);
    return a.u_half ? launch_cv128<kLong, true, true>(a, s)
                    : launch_cv128<kLong, true, false>(a, s);
}

}  // namespace

bool commit_verify_mfma128_supports(const CommitVerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.c.dtype == GDN_DTYPE_BF16 && a.c.dk == kD && a.c.dv == kD && a.v.n > 64 &&
           a.v.n <= tv128::kN && a.c.n <= tv128::kN && a.v.H <= 4096;
}

hipError_t launch_commit_verify_mfma128(const CommitVerifyArgs &a, hipStream_t s) {
    if (a.c.max_path > pc::kC16) return launch_cv128_u<true>(a, s);
    return launch_cv128_u<false>(a, s);
}

}  // namespace gdn
