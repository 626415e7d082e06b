// Fused commit + verify for bf16 q/k/v, d_k = d_v = 128 and new trees of
// 65..128 nodes (gfx950).
//
// The commitment of an accepted branch is deferred to the next iteration
// (DFlash-TfM page, section on rollback-free tree verification for GDN), so
// one call advances S along the previous tree's accepted path and verifies
// the next tree from the result.  One workgroup per (sequence, head), four
// waves, wave w owning d_v columns [32 w, 32 w + 32); the verify is the
// 65..128-node one (tree_verify128.hpp: two 64-node halves, the cross blocks
// of the second half against the first), the commit the chunked solving
// commit of path_commit.hpp (R = K_p S, U = T RHS, S <- e^{g_last} S +
// K_p^T W per chunk of path slots).
//
// Schedule.  Wave 3 reads the path ids and the previous tree's parent row,
// validates the path and builds the topology while waves 0-2 lay out the Q
// and K tiles; every wave requests its whole state slab, which the commit
// needs before any of it is contracted for the verify.
//   * Paths of at most 16 nodes (the usual decode case): wave 3 also lays
//     out the 16-slot chunk (keys, X, T) during the loads, between the V
//     tile and the cross blocks, and every wave applies it right after the
//     cross blocks, so the commit costs the verify's chain one application.
//   * Longer paths: 32-slot chunks in the cross blocks' place before those
//     are formed, each later chunk's rows requested while the one before it
//     is applied.
// The committed slab is written back at once (the memory pipe is otherwise
// idle while the tree matrices are formed) and stays in registers as the B
// operand of Q S and K S; the verify then runs as in the 65..128-node verify
// kernel.  The new tree's pseudo-values (u_out) leave through LDS as whole
// rows next to the outputs.
//
// LDS (one workgroup per CU): the Q/K tiles (then the output and
// pseudo-value staging rows), one region that holds the V tile (and the
// short chunk past it), then each half's solve blocks plus the cross blocks,
// the topology and the commit's path ids and decay weights.
#include <stddef.h>

#include "internal.hpp"
#include "path_commit.hpp"
#include "tree_verify128.hpp"

namespace gdn {
namespace {

using namespace tv128;

constexpr int kMaxPathIds = 128;   // a valid path has at most n_prev <= 128 nodes

// what the commit keeps in LDS besides its chunk tiles
struct CommitAux {
    pc::Chunk16Aux cx;        // decay weights of the 16-slot chunk, zero rows
    int pid[kMaxPathIds];     // previous path ids
    int commit_ok;
};

struct Smem {
    union {
        QKTiles t;
        struct {
            float o[64][kD + 4];   // one half's output rows, once Q and K are dead
            float u[64][kD + 4];   // and its pseudo-value rows
        } st;
    } a;
    union {
        uint16_t v[kN][kQK];
        struct {
            SolveBlocks s;
            Cross x;
        } sx;
        struct {   // long paths: 32-slot chunks in the cross blocks' place
            unsigned char skip[sizeof(SolveBlocks)];
            pc::ChunkTiles ct;
        } lc;
        struct {   // paths of at most 16 nodes: one chunk past the V tile, in
                   // the solve blocks' place (written only after the commit)
            unsigned char skip[sizeof(uint16_t) * kN * kQK];
            pc::EarlyChunk16 e;
        } ec;
    } b;
    Topo tp;
    CommitAux ax;
};

static_assert(sizeof(Smem) <= 163840, "one workgroup per CU");
static_assert(sizeof(uint16_t) * kN * kQK <= sizeof(SolveBlocks),
              "the V tile must not reach the cross blocks");
static_assert(sizeof(uint16_t) * kN * kQK + sizeof(pc::EarlyChunk16) <= sizeof(SolveBlocks),
              "the short chunk lies between the V tile and the cross blocks");
static_assert(sizeof(pc::ChunkTiles) <= sizeof(Cross), "the long chunks lie in the cross blocks");

// one half's output rows (and, with kUout, pseudo-value rows, fp32 or with
// kUh fp16 rounded to nearest) through the LDS staging rows as whole rows;
// a barrier of the caller must separate the staging area's previous readers
template <bool kUout, bool kUh>
__device__ __forceinline__ void store_half(const Lane &c, const Seq &s, int hf,
                                           const f32x16 (&o)[2], const f32x16 (&u)[2], Smem &sm,
                                           float *out, void *u_out) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sm.a.st.o[32 * t + crow(r, c.h)][c.col] = o[t][r];
            if constexpr (kUout) sm.a.st.u[32 * t + crow(r, c.h)][c.col] = u[t][r];
        }
    tv::lds_barrier();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 5, c4 = (e & 31) * 4;
        const int i = 64 * hf + row;
        if (i < s.n) {
            store16(out + s.base + (size_t)i * s.rstride + c4,
                    *reinterpret_cast<const float4 *>(&sm.a.st.o[row][c4]));
            if constexpr (kUout && !kUh)
                store16(static_cast<float *>(u_out) + s.base + (size_t)i * s.rstride + c4,
                        *reinterpret_cast<const float4 *>(&sm.a.st.u[row][c4]));
        }
    }
    if constexpr (kUout && kUh) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = c.tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
            const int i = 64 * hf + row;
            const float4 x0 = *reinterpret_cast<const float4 *>(&sm.a.st.u[row][c8]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&sm.a.st.u[row][c8 + 4]);
            const uint4 hv = make_uint4(
                (uint32_t)f16_bits(x0.x) | ((uint32_t)f16_bits(x0.y) << 16),
                (uint32_t)f16_bits(x0.z) | ((uint32_t)f16_bits(x0.w) << 16),
                (uint32_t)f16_bits(x1.x) | ((uint32_t)f16_bits(x1.y) << 16),
                (uint32_t)f16_bits(x1.z) | ((uint32_t)f16_bits(x1.w) << 16));
            if (i < s.n)
                store16h(static_cast<uint16_t *>(u_out) + s.base + (size_t)i * s.rstride + c8,
                         hv);
        }
    }
}

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
__global__ __launch_bounds__(kThreads, 1) void commit_verify_mfma128_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k_prev, const uint16_t *__restrict__ v_prev,
    const float *__restrict__ alpha_prev, const float *__restrict__ beta_prev,
    const int32_t *__restrict__ parent_prev, int n_prev, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, float *__restrict__ out, void *__restrict__ u_out, int n,
    int H, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const Lane c = tv::lane_coords();
    const Seq s = tv::seq_coords(blockIdx.x, n, H);
    float *slab = S + (size_t)blockIdx.x * kD * kD;
    CommitAux &ax = sm.ax;
    const int mlen = path_len[s.b];
    // previous tree, this (sequence, head): node 0's row and gate entry
    const size_t prow0 = ((size_t)s.b * n_prev * H + s.hd) * kD;
    const size_t pgate0 = (size_t)s.b * n_prev * H + s.hd;
    const uint32_t pbytes = (uint32_t)((size_t)n_prev * H * kD * 2);
    const int32_t *ppar = parent_prev + (size_t)s.b * n_prev;

    // ---- 1. the Q and K tiles (waves 0-2); wave 3 reads the previous path
    //         and the previous tree's parents, validates the path, builds the
    //         topology and (short paths) the chunk; every wave its share of
    //         the V rows, then its state slab
    pc::PathLanes pl{-1, -1, -2, -2};
    {
        uint4 x[8];
        if (c.w < 3) {
            uint4 y[11];
            tv128::load_rows3(c, s, q, y);
            tv128::store_rows3_permuted(c, y, sm.a.t.q);
            tv128::load_rows3(c, s, k, y);
            tv128::store_rows3_permuted(c, y, sm.a.t.k);
            tv128::load_rows(c, s, v, x);
        } else {
            const int32_t *prow = path + (size_t)s.b * max_path;
            const int lim = min(min(mlen, max_path), kMaxPathIds);
            if (c.l < lim) pl.id0 = prow[c.l];
            if (64 + c.l < lim) pl.id1 = prow[64 + c.l];
            int pp0 = -1, pp1 = -1;
            if (c.l < n_prev) pp0 = ppar[c.l];
            if (64 + c.l < n_prev) pp1 = ppar[64 + c.l];
            tv128::load_rows(c, s, v, x);
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
                                      c.l < mc0 && pl.id0 >= 0 && pl.id0 < n_prev,
                                      k_prev + prow0, alpha_prev + pgate0, beta_prev + pgate0,
                                      H * kD, H, pbytes, c.l);
            }
            tv128::topology(c, s, parent, alpha, beta, sm.tp, status, false, false);
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
                    pc::build16_x(sm.b.ec.e, ax.cx, r16.k, r16.la, r16.bt, min(pc::kC16, mlen),
                                  c.l);
                    pc::build16_t(sm.b.ec.e, c.l);
                }
            }
        }
        tv128::store_rows(c, x, sm.b.v);
    }
    f32x16 st[4];
    if constexpr (!kLong) {
#pragma unroll
        for (int t = 0; t < 4; ++t) load_state_tile(st[t], t, slab, c.col, c.h);
    }
    lds_barrier();
    const bool commit = ax.commit_ok && mlen > 0;
    bf16x8 ident[2];
    pc::key_identity(ident, c.m, c.h);

    // ---- 2. long paths: the commit, 32-slot chunks (the first chunk's rows
    //         requested ahead of the state, each later chunk's while the one
    //         before it is applied)
    pc::ChunkWords V0;
    if constexpr (kLong) {
        pc::ChunkRows rows{};
        if (commit)
            rows = pc::load_chunk(ax.pid, 0, mlen, s.b, s.hd, n_prev, H, k_prev, v_prev,
                                  alpha_prev, beta_prev, c.tid);
#pragma unroll
        for (int t = 0; t < 4; ++t) load_state_tile(st[t], t, slab, c.col, c.h);
        if (commit) {
            for (int c0 = 0; c0 < mlen; c0 += pc::kC) {
                pc::build_chunk(sm.b.lc.ct, rows, c0, mlen, c.tid, c.w, c.l);
                if (c0 + pc::kC < mlen)
                    rows = pc::load_chunk(ax.pid, c0 + pc::kC, mlen, s.b, s.hd, n_prev, H,
                                          k_prev, v_prev, alpha_prev, beta_prev, c.tid);
                pc::apply_chunk(sm.b.lc.ct, st, ident, c.m, c.h, c.col);
                lds_barrier();   // the chunk tiles are restaged next
            }
            store_state(st, slab, c.col, c.h);
        }
    } else {
        // the chunk's values in this wave's columns (zero when there is no
        // commit: with no valid slots every load reads past the end of its
        // buffer resource)
        V0 = pc::load_v_chunk16(v_prev + prow0, pbytes, ax.pid, 0,
                                commit ? min(pc::kC16, mlen) : 0, H * kD, c.col, c.h);
    }

    // ---- 3. cross blocks (one per wave), V -> registers; short paths: the
    //         commit (the chunk lies clear of both, in the solve blocks'
    //         place, which is written only after the barrier that follows)
    tv128::cross_block(c, sm.a.t, sm.tp, sm.b.sx.x);
    uint32_t vpk[4][8];
    tv128::v_to_regs(c, sm.b.v, vpk);
    if constexpr (!kLong) {
        if (commit) {
            const pc::ChunkView cv = pc::early_view(sm.b.ec.e, ax.cx, c.m);
            f32x16 Ra = {}, Rb = {};
            pc::rp_tile(cv.kp_row, st[0], 0, Ra, c.h);
            pc::rp_tile(cv.kp_row, st[1], 1, Rb, c.h);
            pc::rp_tile(cv.kp_row, st[2], 2, Ra, c.h);
            pc::rp_tile(cv.kp_row, st[3], 3, Rb, c.h);
            pc::finish_rows_v<pc::kC16>(cv, pc::widen_bf16(V0), Ra + Rb, st, ident, c.h);
            store_state(st, slab, c.col, c.h);
        }
    }
    lds_barrier();
    if (sm.tp.bad) {
        tv128::store_nan(c, s, out);
        if constexpr (kUout) {
            if constexpr (kUh) store_nan_half128(c, s, static_cast<uint16_t *>(u_out));
            else tv128::store_nan(c, s, static_cast<float *>(u_out));
        }
        return;
    }

    // ---- 4. half 0: blocks, inverse, solve, outputs; half 1's block values
    //         wait in registers until its solve blocks are free; each state
    //         tile goes into both halves' P / R
    f32x16 P0[2] = {}, R0[2] = {}, P1[2] = {}, R1[2] = {};
    tv128::contract_tile(c, sm.a.t, 0, st[0], P0, R0, P1, R1);
    float y1[16], x1[16];
    if (c.w < 3) {
        float y0[16], x0[16];
        tv128::half_values(c, sm.a.t, sm.tp, 0, y0, x0);
        tv128::half_values(c, sm.a.t, sm.tp, 1, y1, x1);
        tv128::half_store(c, y0, x0, sm.b.sx.s);
    }
    lds_barrier();
    tv128::contract_tile(c, sm.a.t, 1, st[1], P0, R0, P1, R1);
    tv::inverse(c, sm.b.sx.s);
    tv128::contract_tile(c, sm.a.t, 2, st[2], P0, R0, P1, R1);
    lds_barrier();
    tv128::contract_tile(c, sm.a.t, 3, st[3], P0, R0, P1, R1);
    f32x16 u01[2];
    {
        f32x16 rhs[2], o[2];
        tv128::rhs_and_decay(c, sm.tp, 0, P0, R0, vpk, rhs);
        tv128::solve_half(c, sm.b.sx.s, rhs, P0, u01, o);
        lds_barrier();   // every wave has read its last Q / K rows
        store_half<kUout, kUh>(c, s, 0, o, u01, sm, out, u_out);
    }
    lds_barrier();   // every wave is done with half 0's solve blocks and staging rows

    // ---- 5. half 1, with the cross terms of half 0's pseudo-values
    if (c.w < 3) tv128::half_store(c, y1, x1, sm.b.sx.s);
    lds_barrier();
    tv::inverse(c, sm.b.sx.s);
    lds_barrier();
    {
        f32x16 rhs[2], u[2], o[2];
        tv128::rhs_and_decay(c, sm.tp, 1, P1, R1, vpk, rhs);
        const Cross &cr = sm.b.sx.x;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const SplitTile ub = split_tile(u01[b]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                rhs[t] = mm3<kBL>(cr.xh[t][b], cr.xl[t][b], ub, rhs[t], c.m, c.h);
                P1[t] = mm3<kBL>(cr.yh[t][b], cr.yl[t][b], ub, P1[t], c.m, c.h);
            }
        }
        tv128::solve_half(c, sm.b.sx.s, rhs, P1, u, o);
        store_half<kUout, kUh>(c, s, 1, o, u, sm, out, u_out);
    }
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
           a.v.n <= kN && a.c.n <= kN && a.v.H <= 4096;
}

hipError_t launch_commit_verify_mfma128(const CommitVerifyArgs &a, hipStream_t s) {
    if (a.c.max_path > pc::kC16) return launch_cv128_u<true>(a, s);
    return launch_cv128_u<false>(a, s);
}

}  // namespace gdn
