// Fused commit + verify for bf16 q/k/v, d_k = d_v = 128, n <= 64 (gfx950).
//
// The commitment of an accepted branch is deferred to the next iteration
// (DFlash-TfM page, section on rollback-free tree verification for GDN), so
// one call advances S along the previous tree's accepted path and verifies
// the next tree from the result.  One workgroup per (sequence, head): the
// state slab of each wave (128 x 32 fp32, four result tiles) is read from
// HBM once, committed in registers (path_commit.hpp), written back once, and
// is then the B operand of Q S and K S for the verify (tree_verify.hpp)
// without another trip through memory.
//
// Schedule.  The only verify work that needs the state is Q S, K S and what
// follows; the Gram matrices, masks and block inverses of the new tree need
// only q, k and the parents.  So waves 0-2 request the q and k rows first
// (wave 3 meanwhile reads the gates, the previous path's ids together with
// the previous tree's parent row, which validates the path, then the first
// chunk's rows and gates, and builds the topology), every wave its first state tiles once q and k are in, then
// the rest of its slab (one tile per tree-matrix phase) and last its v rows;
// the tree matrices are built while the state streams in.
//   * Pseudo-values carried (u_prev): while waves 0-2 compute the masks,
//     wave 3 validates the path and lays out the first 32-slot key chunk
//     over the T rows of the solve blocks, which the inverse writes only in
//     its last step; every wave applies the chunk (a rank-m update, no
//     solve) between the inverse's Z / L steps and that last step.
//   * Otherwise (the commit solves for the pseudo-values) the first 16-slot
//     chunk goes to the same place: wave 3 lays out its keys and builds its
//     Gram and X during the masks, wave 0 its T = (I + X)^{-1} while wave 3
//     substitutes the tree's blocks, and every wave holds its own columns of
//     the chunk's value rows in registers; every wave applies it at the same
//     point (R = K_p S, U = T RHS, then the update).
// Longer paths continue chunk by chunk over the inverse scratch, after the
// inverse's last step.  The verify then finishes from the committed slab,
// writing the slab back tile by tile as the contraction consumes it (when
// every path fits the first chunk, the inverse's last step waits until the
// contraction is done: the contraction does not need T), and the solve's
// first 32-row block is stored while the second is solved.
//
// The new tree's v rows are needed only by the solve, so they are requested
// behind the state and wait in registers; once the contraction has read the
// K tile, the V tile passes through its place into each lane's columns.
//
// LDS (80 KB, two workgroups per CU): Q/K tiles (then the V tile, then the
// output staging), the solve blocks, whose inverse scratch or T rows hold
// the commit chunk in turn, and the topology / chunk gate arrays.
#include <stddef.h>

#include "internal.hpp"
#include "path_commit.hpp"
#include "tree_verify.hpp"

namespace gdn {
namespace {

using namespace tv;

constexpr int kMaxPathIds = 128;   // a valid path has at most n_prev <= 128 nodes

struct Smem {
    union {
        QKTiles t;
        float o[kN][kD + 4];
    } a;
    union {
        SolveBlocks s;
        pc::Chunk16 ch;      // over d / tinv, dead once the inverse has finished
        pc::KeyChunk32 kc;   // same place, for the later key chunks of a long path
        struct {
            unsigned char skip[offsetof(SolveBlocks, th)];
            pc::KeyChunk32 kc;   // the first key chunk, over the T rows (th / tl),
                                 // which the inverse writes only in its last step
        } kt;
        struct {
            unsigned char skip[offsetof(SolveBlocks, th)];
            pc::EarlyChunk16 ch;   // the first chunk of a solving commit, same place
        } kt16;
    } b;
    Topo tp;
    pc::Chunk16Aux cx;
    int pid[kMaxPathIds];    // previous path ids
    int commit_ok;
};

static_assert(sizeof(pc::Chunk16) <= offsetof(SolveBlocks, th) &&
                  sizeof(pc::KeyChunk32) <= offsetof(SolveBlocks, th),
              "the commit chunk must fit in the inverse scratch of the solve blocks");
static_assert(offsetof(SolveBlocks, th) + sizeof(pc::KeyChunk32) <= offsetof(SolveBlocks, xh) &&
                  offsetof(SolveBlocks, th) + sizeof(pc::EarlyChunk16) <= offsetof(SolveBlocks, xh),
              "the first commit chunk must stay inside the T rows, clear of what the mask writes");
static_assert(sizeof(Smem) <= 81920, "two workgroups per CU");

// 64 node rows of a bf16 [batch][n][H][128] tensor loaded by waves 0-2 alone
// (192 threads, 16-byte chunks e = tid + 192 it, six per thread, the last
// partly empty); rows past n read as zero
__device__ __forceinline__ void load_rows3(const Lane &c, const Seq &s, const uint16_t *src,
                                           uint4 (&x)[6]) {
    const uint32_t bytes = (uint32_t)(s.n * s.rstride * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + s.base, bytes);
#pragma unroll
    for (int it = 0; it < 6; ++it) {
        const int e = c.tid + 192 * it, row = e >> 4, c8 = (e & 15) * 8;
        x[it] = load16(rs, e < 1024 ? (uint32_t)((row * s.rstride + c8) * 2) : bytes);
    }
}

__device__ __forceinline__ void store_rows3_permuted(const Lane &c, const uint4 (&x)[6],
                                                     uint16_t (*dst)[kQK]) {
#pragma unroll
    for (int it = 0; it < 6; ++it) {
        const int e = c.tid + 192 * it, row = e >> 4, c8 = (e & 15) * 8;
        if (e < 1024) store_row8_permuted(dst[row], c8, x[it]);
    }
}

// kU: the previous tree's pseudo-values u_prev are given, so the commit is
// the rank-m update S <- e^{g_a} S + sum_s e^{g_a - g_s} k_s u_s^T with no
// solve; otherwise the commit solves for them chunk by chunk.  kUout: the
// new tree's pseudo-values are written to u_out.  kLong: paths may be longer
// than the first chunk (32 slots with pseudo-values given, else 16), so the
// later chunks are applied too; without it a longer path is never read
// (the host takes the kLong instance whenever max_path exceeds the first
// chunk), and the kernel carries no code and no registers for them.  kUh:
// u_prev and u_out hold fp16 values (fp32 otherwise).  kOne: the new
// trees have at most 32 nodes, so only the first 32-row block is contracted
// and solved.
template <bool kU, bool kUout, bool kLong, bool kUh, bool kOne>
__global__ __launch_bounds__(kThreads, 2) void commit_verify_mfma_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k_prev, const uint16_t *__restrict__ v_prev,
    const float *__restrict__ alpha_prev, const float *__restrict__ beta_prev,
    const int32_t *__restrict__ parent_prev, const void *__restrict__ u_prev, int n_prev,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ alpha,
    const float *__restrict__ beta, const int32_t *__restrict__ parent,
    float *__restrict__ out, void *__restrict__ u_out, int n, int H, int ncu,
    int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const Lane c = lane_coords();
    const Seq s = seq_coords(blockIdx.x, n, H);
    const int mlen = path_len[s.b];
    float *slab = S + (size_t)blockIdx.x * kD * kD;
    // previous tree, this (sequence, head): node 0's row and gate entry
    const size_t prow0 = ((size_t)s.b * n_prev * H + s.hd) * kD;
    const size_t pgate0 = (size_t)s.b * n_prev * H + s.hd;
    const uint32_t pbytes = (uint32_t)((size_t)n_prev * H * kD * 2);
    const int32_t *ppar = parent_prev + (size_t)s.b * n_prev;

    // ---- 1. loads: wave 3 first takes the new tree's gates, the path ids
    //         and the previous parents, every wave its q/k/v rows, then its
    //         state slab; wave 3 requests the first chunk rows in between
    Gates gt{-1, 1.f, 0.f, false};
    pc::PathLanes pl{-1, -1, -2, -2};
    // the previous tree's parent row (nodes l and 64 + l), read whole and
    // independently of the path ids: the parents of the path nodes come out
    // of it by lane shuffles, and with u_prev the whole tree is checked
    int pp0 = -1, pp1 = -1;
    if (c.w == 3) {
        gt = load_gates(c, s, parent, alpha, beta);
        const int32_t *prow = path + (size_t)s.b * max_path;
        const int lim = min(min(mlen, max_path), kMaxPathIds);
        if (c.l < lim) pl.id0 = prow[c.l];
        if (64 + c.l < lim) pl.id1 = prow[64 + c.l];
        if (c.l < n_prev) pp0 = ppar[c.l];
        if (64 + c.l < n_prev) pp1 = ppar[64 + c.l];
    }
    uint4 rq[6], rk[6], rv[4];
    if (c.w < 3) {
        load_rows3(c, s, q, rq);
        load_rows3(c, s, k, rk);
    }
    // the state slab is requested one 32-row tile at a time, between the
    // tree-matrix phases: a wave that issues a whole 64 KiB slab stalls
    // until the memory system has accepted all of it
    f32x16 st[4];
    pc::KeyRows16 r16;
    pc::KeyRows32 k32;
    if (c.w == 3) {
        // parents of the path ids (ids out of range fail validation by
        // themselves) and the first chunk's rows and gates
        pl.par0 = pc::parent_of(pl.id0, pp0, pp1, n_prev);
        pl.par1 = pc::parent_of(pl.id1, pp0, pp1, n_prev);
        // ids for every wave's u or v loads
        if (pl.id0 >= 0) sm.pid[c.l] = pl.id0;
        if (pl.id1 >= 0) sm.pid[64 + c.l] = pl.id1;
        if constexpr (kU) {
            // the first chunk's keys and gates
            const int mc0 = min(32, mlen);
            const int rj = c.l >> 1;
            const int rid = pc::slot_id(pl, rj);
            k32 = pc::load_keys32(rid, rj < mc0 && rid >= 0 && rid < n_prev, pl.id0,
                                  c.l < mc0 && pl.id0 >= 0 && pl.id0 < n_prev, k_prev + prow0,
                                  alpha_prev + pgate0, H * kD, H, pbytes, c.l);
        } else {
            const int mc0 = min(pc::kC16, mlen);
            const int rj = c.l >> 2;
            const int rid = pc::slot_id(pl, rj);
            r16 = pc::load_keys16(rid, rj < mc0 && rid >= 0 && rid < n_prev, pl.id0,
                                  c.l < mc0 && pl.id0 >= 0 && pl.id0 < n_prev, k_prev + prow0,
                                  alpha_prev + pgate0, beta_prev + pgate0, H * kD, H, pbytes,
                                  c.l);
        }
        topology(c, s, gt, sm.tp, status, false);
        // zero rows for the padded slots of the commit chunk operands
        for (int i = c.l; i < pc::kKP; i += 64) sm.cx.zk[i] = 0;
        if (c.l < pc::kBL) sm.cx.zt[c.l] = 0;
    }
    if (c.w < 3) {
        store_rows3_permuted(c, rq, sm.a.t.q);
        store_rows3_permuted(c, rk, sm.a.t.k);
    }
    // the state once q and k are in: every workgroup's Gram operands are
    // fetched before any of the bulk behind them
    load_state_tile(st[0], 0, slab, c.col, c.h);
    lds_barrier();
    load_state_tile(st[1], 1, slab, c.col, c.h);

    // the first chunk's pseudo-values (this wave's columns), in flight
    // during the tree matrices
    constexpr size_t ues = kUh ? 2 : 4;   // bytes per pseudo-value
    const void *u_head = static_cast<const char *>(u_prev) + prow0 * ues;
    const uint32_t ubytes = (uint32_t)((size_t)n_prev * H * kD * ues);
    // (unconditional: with no valid slots every load reads past the end of
    // its buffer resource and returns zero, so no merge of loaded and zero
    // values forces a wait for these loads here)
    const int mc0 = (mlen > 0 && mlen <= kMaxPathIds) ? min(kU ? 32 : pc::kC16, mlen) : 0;
    pc::ChunkWords U0;
    if constexpr (kU)
        U0 = pc::load_u_chunk<kUh>(u_head, ubytes, sm.pid, 0, mc0, H * kD, c.col, c.h);
    else   // the first chunk's values, in this wave's columns
        U0 = pc::load_v_chunk16(v_prev + prow0, pbytes, sm.pid, 0, mc0, H * kD, c.col, c.h);

    // ---- 2. the new tree's Gram, masks and block inverses (no state needed)
    f32x16 gc, ga;
    if (c.w < 3) gram(c, sm.a.t, gc, ga);
    load_state_tile(st[2], 2, slab, c.col, c.h);
    const bool tree_ok = !sm.tp.bad;
    // wave 3: the previous path's validity (and the fault flags)
    auto validate = [&]() -> bool {
        // with u_prev, a malformed previous tree counts as a bad path: the
        // call that verified it wrote NaN pseudo-values
        const bool ok = pc::path_valid(pl, mlen, max_path, n_prev, c.l) &&
                        (!kU || pc::tree_valid(pp0, pp1, n_prev, c.l));
        if (c.l == 0) {
            sm.commit_ok = ok;
            if (s.hd == 0 && status)
                status[s.b] = (ok ? 0 : kFaultBadPath) | (tree_ok ? 0 : kFaultBadParent);
        }
        return ok;
    };
    bool commit;
    bf16x8 ident[2];
    pc::key_identity(ident, c.m, c.h);
    if constexpr (kU) {
        // ---- 3. wave 3 validates the path and lays out the first key chunk
        //         (over the T rows) while the others mask; the chunk is applied
        //         between the inverse's Z / L steps and its last step
        if (c.w == 3) {
            if (validate() && mlen > 0)
                pc::build_keys32(sm.b.kt.kc, sm.cx, k32, min(32, mlen), c.l);
        } else if (tree_ok) {
            mask(c, sm.tp, gc, ga, sm.b.s);
        }
        load_state_tile(st[3], 3, slab, c.col, c.h);
        // v is needed only by the solve: its rows are requested behind the
        // last state tile and wait in registers (the V tile passes through
        // LDS after the contraction); with the later chunks they are
        // requested after those, which need the registers
        if constexpr (!kLong) load_rows(c, s, v, rv);
        lds_barrier();
        commit = sm.commit_ok && mlen > 0;
        if (tree_ok) {
            inverse_subst(c, sm.b.s);
            inverse_zl(c, sm.b.s);
        }
        if (commit)
            pc::apply_known_u(sm.b.kt.kc, sm.cx, pc::u_values<kUh>(U0), st, ident, c.m, c.h);
        if constexpr (kLong) {
            // the later chunks need the inverse scratch: the inverse's last
            // step first (it starts with a barrier: the first chunk is read)
            if (tree_ok) inverse_split(c, sm.b.s);
            lds_barrier();   // the inverse scratch is free from here on
        }
        if (kLong && commit) {
            for (int c0 = 32; c0 < mlen; c0 += 32) {
                const int mc = min(32, mlen - c0);
                const pc::ChunkWords Uc =
                    pc::load_u_chunk<kUh>(u_head, ubytes, sm.pid, c0, mc, H * kD, c.col, c.h);
                if (c.w == 3) {
                    const int rj = c.l >> 1;
                    const pc::KeyRows32 kr = pc::load_keys32(
                        pc::slot_id(pl, c0 + rj), rj < mc, pc::slot_id(pl, c0 + (c.l & 31)), c.l < mc,
                        k_prev + prow0, alpha_prev + pgate0, H * kD, H, pbytes, c.l);
                    pc::build_keys32(sm.b.kc, sm.cx, kr, mc, c.l);
                }
                lds_barrier();
                pc::apply_known_u(sm.b.kc, sm.cx, pc::u_values<kUh>(Uc), st, ident, c.m, c.h);
                lds_barrier();   // every wave is done with this chunk
            }
        }
    } else {
        // ---- 3. the first 16-slot chunk (over the T rows): wave 3 validates
        //         the path and builds the chunk's keys and X while the others
        //         mask, wave 0 its T while wave 3 substitutes the tree's
        //         diagonal blocks; every wave applies it, its values from
        //         registers, between the inverse's Z / L steps and its last step
        if (c.w == 3) {
            if (validate() && mlen > 0)
                pc::build16_x(sm.b.kt16.ch, sm.cx, r16.k, r16.la, r16.bt, min(pc::kC16, mlen),
                              c.l);
        } else if (tree_ok) {
            mask(c, sm.tp, gc, ga, sm.b.s);
        }
        load_state_tile(st[3], 3, slab, c.col, c.h);
        // v is needed only by the solve: its rows are requested behind the
        // last state tile and wait in registers (the V tile passes through
        // LDS after the contraction); with the later chunks they are
        // requested after those, which need the registers
        if constexpr (!kLong) load_rows(c, s, v, rv);
        lds_barrier();
        commit = sm.commit_ok && mlen > 0;
        if (commit && c.w == 0) pc::build16_t(sm.b.kt16.ch, c.l);
        if (tree_ok) {
            inverse_subst(c, sm.b.s);
            inverse_zl(c, sm.b.s);   // starts with a barrier: T is in place
        } else {
            lds_barrier();
        }
        if (commit) {
            // R = K_p S over the four tiles in two accumulators (two short
            // MFMA chains), then U = T RHS and the update
            const pc::ChunkView cv = pc::early_view(sm.b.kt16.ch, sm.cx, c.m);
            f32x16 Ra = {}, Rb = {};
            pc::rp_tile(cv.kp_row, st[0], 0, Ra, c.h);
            pc::rp_tile(cv.kp_row, st[1], 1, Rb, c.h);
            pc::rp_tile(cv.kp_row, st[2], 2, Ra, c.h);
            pc::rp_tile(cv.kp_row, st[3], 3, Rb, c.h);
            pc::finish_rows_v<pc::kC16>(cv, pc::widen_bf16(U0), Ra + Rb, st, ident, c.h);
        }
        if constexpr (kLong) {
            if (tree_ok) inverse_split(c, sm.b.s);   // starts with a barrier: the chunk is read
            lds_barrier();                           // the inverse scratch is free from here on
        }
        if (kLong && commit) {
            // later chunks: wave 3 loads and prepares each over the inverse
            // scratch, every wave applies it
            for (int c0 = pc::kC16; c0 < mlen; c0 += pc::kC16) {
                if (c.w == 3) {
                    const int mc = min(pc::kC16, mlen - c0);
                    const int rj = c.l >> 2;
                    const pc::Rows16 rr = pc::load_rows16(
                        pc::slot_id(pl, c0 + rj), rj < mc, pc::slot_id(pl, c0 + (c.l & 15)), c.l < mc,
                        k_prev + prow0, v_prev + prow0, alpha_prev + pgate0, beta_prev + pgate0,
                        H * kD, H, pbytes, c.l);
                    pc::build16(sm.b.ch, sm.cx, rr, mc, c.l);
                }
                lds_barrier();
                pc::apply16(sm.b.ch, sm.cx, st, ident, c.m, c.h, c.col);
                lds_barrier();   // every wave is done with this chunk
            }
        }
    }

    if constexpr (kLong) load_rows(c, s, v, rv);

    // ---- 4. verify from the committed slab, writing the slab back as the
    //         contraction consumes it
    if (!tree_ok) {
        if (commit) store_state(st, slab, c.col, c.h);
        store_nan(c, s, out);
        if constexpr (kUout) {
            if constexpr (kUh) store_nan_f16(c, s, static_cast<uint16_t *>(u_out));
            else store_nan(c, s, static_cast<float *>(u_out));
        }
        return;
    }
    f32x16 P[2], R[2];
    // Every state load has landed by now (the commit consumed the tiles),
    // but the compiler cannot see that on the no-commit path and would wait
    // on the memory counter inside the contraction, i.e. for the slab
    // stores issued there.  One explicit wait here settles it.
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    contract<kOne ? 1 : 2>(c, sm.a.t, st, P, R, commit ? slab : nullptr);
    // Without the later chunks, the inverse's last step (the T rows, over
    // the first chunk) comes only now: the contraction needs the committed
    // slab but not T, so no wave waits for that step's barriers before
    // contracting.  It starts with a barrier (every wave has applied the
    // chunk); the barrier after it publishes T and frees the K tile.
    if constexpr (!kLong) inverse_split(c, sm.b.s);
    // the V tile through the K tile's place (free once every wave has
    // finished the contraction) into this lane's columns
    lds_barrier();
    store_rows(c, rv, sm.a.t.k);
    lds_barrier();
    uint32_t vpk[2][8];
    v_to_regs(c, sm.a.t.k, vpk);
    // the first block's staging rows overlap the K tile only when the
    // pseudo-values are staged beside the outputs
    if constexpr (kUout) lds_barrier();
    // the first block's rows leave while the second block is solved
    SolveCarry cy;
    f32x16 u0, o0, u1, o1;
    solve_block0(c, sm.tp, sm.b.s, P, R, vpk, u0, o0, cy);
    store_block<kUout, kUh>(c, s, sm.a.o, o0, out, u0, u_out, 0);
    if constexpr (kOne) return;
    solve_block1(c, sm.b.s, P, cy, u1, o1);
    lds_barrier();   // every thread has read the first block from the staging area
    store_block<kUout, kUh>(c, s, sm.a.o, o1, out, u1, u_out, 32);
}

}  // namespace

bool commit_verify_mfma_supports(const CommitVerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.c.dtype == GDN_DTYPE_BF16 && a.c.dk == kD && a.c.dv == kD && a.v.n <= kN &&
           a.v.H <= 4096;
}

namespace {

template <bool kU, bool kUout, bool kLong, bool kUh, bool kOne>
hipError_t launch_cv1(const CommitVerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((commit_verify_mfma_kernel<kU, kUout, kLong, kUh, kOne>),
                       dim3((unsigned)(a.v.batch * a.v.H)), dim3(kThreads), 0, s, a.c.S,
                       a.c.path, a.c.path_len, a.c.max_path, (const uint16_t *)a.c.k,
                       (const uint16_t *)a.c.v, a.c.alpha, a.c.beta, a.c.parent, a.u_prev,
                       a.c.n, (const uint16_t *)a.v.q, (const uint16_t *)a.v.k,
                       (const uint16_t *)a.v.v, a.v.alpha, a.v.beta, a.v.parent, a.v.out,
                       a.u_out, a.v.n, a.v.H, device_cu_count(), a.v.status);
    return hipGetLastError();
}

template <bool kU, bool kUout, bool kLong, bool kUh>
hipError_t launch_cv(const CommitVerifyArgs &a, hipStream_t s) {
    if (a.v.n <= 32) return launch_cv1<kU, kUout, kLong, kUh, true>(a, s);
    return launch_cv1<kU, kUout, kLong, kUh, false>(a, s);
}

template <bool kU, bool kUout, bool kLong>
hipError_t launch_cv_u(const CommitVerifyArgs &a, hipStream_t s) {
    if constexpr (kU || kUout) {
        if (a.u_half) return launch_cv<kU, kUout, kLong, true>(a, s);
    }
    return launch_cv<kU, kUout, kLong, false>(a, s);
}

template <bool kU, bool kUout>
hipError_t launch_cv_len(const CommitVerifyArgs &a, hipStream_t s) {
    // paths longer than the first chunk need the chunk loop
    if (a.c.max_path > (kU ? 32 : pc::kC16)) return launch_cv_u<kU, kUout, true>(a, s);
    return launch_cv_u<kU, kUout, false>(a, s);
}

}  // namespace

hipError_t launch_commit_verify_mfma(const CommitVerifyArgs &a, hipStream_t s) {
    if (a.u_prev) return a.u_out ? launch_cv_len<true, true>(a, s) : launch_cv_len<true, false>(a, s);
    return a.u_out ? launch_cv_len<false, true>(a, s) : launch_cv_len<false, false>(a, s);
}

}  // namespace gdn
