// The 65..128-node MFMA tree verify (bf16 q/k/v, d_k = d_v = 128, gfx950)
// scheduled for two workgroups per CU; shared by the verify kernel and the
// fused commit-verify kernel.
//
// Same system as tree_verify128.hpp (the whole tree one chunk of the delta
// rule, solved as two halves of 64 nodes; DFlash-TfM page, section on
// rollback-free tree verification for GDN), scheduled so that a workgroup
// fits in half of a CU's LDS: only the current half's 64 Q / K rows are in
// LDS at a time.
//   half 0: the 64-node verify on nodes 0..63 (Gram blocks, inverse,
//           P_01 / R_01, solve, output rows), keeping U_01 and the state
//           slab in registers;
//   half 1: Q / K rows 64..127 replace rows 0..63; P_23 / R_23 from the
//           kept slab; the four cross blocks X_{23,01}, Y_{23,01} take the
//           key rows 0..63 as operand fragments straight from global memory
//           (one 32-row block per wave); the right-hand side and P_23 take
//           the cross terms of U_01; then half 1's blocks, inverse, solve
//           and output rows.
// LDS (80 KB): the 64-row Q / K tiles (later a half's output staging), one
// region for a half's solve blocks, the cross blocks, a half's pseudo-value
// staging or, before the verify starts, the fused kernel's commit chunk; the
// topology.  With two resident workgroups per CU each stage's latency is
// hidden behind the other workgroup's work, which one workgroup per CU (the
// whole tree's Q / K tiles and all blocks resident) cannot do.
#pragma once

#include "path_commit.hpp"
#include "tree_verify128.hpp"

namespace gdn {
namespace tvh {

using namespace tile;
using tv::kBL;
using tv::kD;
using tv::kThreads;
using tv::Lane;
using tv::Seq;
using tv::SolveBlocks;

constexpr int kMaxPathIds = 128;   // a valid path has at most n_prev <= 128 nodes

// what the fused kernel's commit keeps in LDS besides its chunk tiles
struct CommitAux {
    pc::Chunk16Aux cx;        // decay weights of the 16-slot chunk, zero rows
    int pid[kMaxPathIds];     // previous path ids
    int commit_ok;
};

struct Smem {
    union {
        tv::QKTiles t;        // the current half's Q and K rows, d_k permuted
        float o[64][kD + 4];  // a half's output rows
    } a;
    union {
        SolveBlocks s;        // the current half's blocks
        tv128::Cross x;       // X_{23,01}, Y_{23,01}
        float u[64][kD + 4];  // a half's pseudo-value rows
        struct {
            CommitAux ax;
            union {
                pc::ChunkTiles ct;     // 32-slot chunks (long paths)
                pc::EarlyChunk16 e;    // one 16-slot chunk (paths of at most 16 nodes)
            };
        } cm;
    } b;
    tv128::Topo tp;
};

static_assert(sizeof(Smem) <= 81920, "two workgroups per CU");

// local row block la of the tiles against key fragments ks (8 k-steps of one
// 32-row key block): lane (node row 32 la + m, h) holds k_s.q_i and k_s.k_i
__device__ __forceinline__ void gram_frags(const Lane &c, const tv::QKTiles &t, int la,
                                           const bf16x8 (&ks)[8], f32x16 &gc, f32x16 &ga) {
    gc = f32x16{};
    ga = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 qi = lds8(&t.q[32 * la + c.m][16 * kk + 8 * c.h]);
        const bf16x8 ki = lds8(&t.k[32 * la + c.m][16 * kk + 8 * c.h]);
        gc = mfma(ks[kk], qi, gc);
        ga = mfma(ks[kk], ki, ga);
    }
}

// the same with the key block lb of the tiles
__device__ __forceinline__ void gram_tiles(const Lane &c, const tv::QKTiles &t, int la, int lb,
                                           f32x16 &gc, f32x16 &ga) {
    bf16x8 ks[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ks[kk] = lds8(&t.k[32 * lb + c.m][16 * kk + 8 * c.h]);
    gram_frags(c, t, la, ks, gc, ga);
}

// key rows 32 kb + m of the sequence as the A-operand fragments the tiles'
// permuted layout implies: for k-step kk, half h supplies d_k indices
// 16 kk + 4 h + {0..3} and 16 kk + 8 + 4 h + {0..3} (two 8-byte loads).
// Rows 0..63 always exist here (n > 64).
__device__ __forceinline__ void load_key_frags(const Lane &c, const Seq &s, const uint16_t *k,
                                               int kb, bf16x8 (&ks)[8]) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(k + s.base, (uint32_t)(s.n * s.rstride * 2));
    const int row = (int)((32 * kb + c.m) * s.rstride * 2);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const u32x2 a = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, row + 2 * (16 * kk + 4 * c.h), 0, 0));
        const u32x2 b = __builtin_bit_cast(
            u32x2,
            __builtin_amdgcn_raw_buffer_load_b64(rs, row + 2 * (16 * kk + 8 + 4 * c.h), 0, 0));
        ks[kk] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
    }
}

// v values of this lane's column for rows 32 t + crow(r, h) of the rows
// starting at s.base (rows at or past s.n read as zero), as bf16 pairs:
// 2-byte loads straight into the result layout, no LDS round trip
__device__ __forceinline__ void load_v_direct(const Lane &c, const Seq &s, const uint16_t *v,
                                              uint32_t (&vpk)[2][8]) {
    // the whole offset goes in the lane offset, which the range check covers
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(v + s.base, (uint32_t)(s.n * s.rstride * 2));
    const int rb = (int)(2 * s.rstride);
    const int vo = 2 * c.col + 4 * c.h * rb;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int r0 = 32 * t + crow(r, 0);
            const uint32_t a = __builtin_amdgcn_raw_buffer_load_b16(rs, vo + r0 * rb, 0, kNT);
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b16(rs, vo + (r0 + 1) * rb, 0, kNT);
            vpk[t][r / 2] = a | (b << 16);
        }
}

// state tile q's share of P = Q S and R = K S for this wave's columns over
// the tiles' 64 rows, the tile given already split into bf16 hi + lo
// (split_tile): the products and their order are tv::contract_tile's, so
// the sums are the same bit for bit; the split is done once for both halves
__device__ __forceinline__ void contract_split_tile(const Lane &c, const tv::QKTiles &t,
                                                    const SplitTile &sq, int q, f32x16 (&P)[2],
                                                    f32x16 (&R)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const bf16x8 aq = lds8(&t.q[32 * tt + c.m][32 * q + 16 * kk + 8 * c.h]);
            const bf16x8 ak = lds8(&t.k[32 * tt + c.m][32 * q + 16 * kk + 8 * c.h]);
            P[tt] = mfma(aq, sq.hi[kk], P[tt]);
            P[tt] = mfma(aq, sq.lo[kk], P[tt]);
            R[tt] = mfma(ak, sq.hi[kk], R[tt]);
            R[tt] = mfma(ak, sq.lo[kk], R[tt]);
        }
}

// one half's output rows (and, with kUout, its pseudo-value rows, fp32 or
// with kUh fp16 rounded to nearest) as whole rows: the result tiles into the
// LDS staging rows (outputs over the Q / K tiles, pseudo-values over the
// solve blocks), then 16-byte row chunks.  A barrier of the caller must
// separate the staging areas' previous readers from this call.
template <bool kUout, bool kUh>
__device__ __forceinline__ void store_half(const Lane &c, const Seq &s, int hf,
                                           const f32x16 (&o)[2], const f32x16 (&u)[2], Smem &sm,
                                           float *out, void *u_out) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sm.a.o[32 * t + crow(r, c.h)][c.col] = o[t][r];
            if constexpr (kUout) sm.b.u[32 * t + crow(r, c.h)][c.col] = u[t][r];
        }
    lds_barrier();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 5, c4 = (e & 31) * 4;
        const int i = 64 * hf + row;
        if (i < s.n) {
            store16(out + s.base + (size_t)i * s.rstride + c4,
                    *reinterpret_cast<const float4 *>(&sm.a.o[row][c4]));
            if constexpr (kUout && !kUh)
                store16(static_cast<float *>(u_out) + s.base + (size_t)i * s.rstride + c4,
                        *reinterpret_cast<const float4 *>(&sm.b.u[row][c4]));
        }
    }
    if constexpr (kUout && kUh) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = c.tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
            const int i = 64 * hf + row;
            const float4 x0 = *reinterpret_cast<const float4 *>(&sm.b.u[row][c8]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&sm.b.u[row][c8 + 4]);
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

// The verify from the point where the Q / K rows 0..63 lie in the tiles, the
// topology is built (and the tree is well formed) and every wave holds its
// slab st (the state the tree is verified from).  Writes the output rows
// (and with kUout the pseudo-values) of all nodes < n.
// the lane coordinates recomputed from an opaque copy of the thread index:
// addresses of the second half are then formed anew instead of being kept
// live from the first half
__device__ __forceinline__ Lane fresh_lane() {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    Lane c;
    c.tid = (int)t;
    c.w = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    c.l = c.tid & 63;
    c.m = c.l & 31;
    c.h = c.l >> 5;
    c.col = 32 * c.w + c.m;
    return c;
}

template <bool kUout, bool kUh>
__device__ __forceinline__ void verify_halves(const Lane &c, const Seq &s, Smem &sm,
                                              const f32x16 (&st)[4],
                                              const uint16_t *__restrict__ q,
                                              const uint16_t *__restrict__ k,
                                              const uint16_t *__restrict__ v,
                                              float *__restrict__ out, void *__restrict__ u_out) {
    Seq s1 = s;   // rows 64.. of the same (sequence, head)
    s1.base += 64 * s.rstride;
    s1.n = s.n - 64;
    // waves 0-2 take the blocks (0,0), (1,0), (1,1) of a half
    const int la = c.w == 0 ? 0 : 1, lb = c.w == 2 ? 1 : 0;

    // ---- half 0: blocks, inverse, P_01 / R_01 (the slab kept, split), solve
    if (c.w < 3) {
        f32x16 gc, ga;
        gram_tiles(c, sm.a.t, la, lb, gc, ga);
        float y[16], x[16];
        tv128::mask(c, sm.tp, la, lb, gc, ga, y, x);
        tv128::half_store(c, y, x, sm.b.s);
    }
    uint4 rv[4];   // V rows 0..63, needed after the contraction
    tv::load_rows(c, s, v, rv);
    lds_barrier();
    tv::inverse_subst(c, sm.b.s);
    tv::inverse_zl(c, sm.b.s);
    f32x16 P[2] = {}, R[2] = {};
    SplitTile ss[4];   // the slab as bf16 hi + lo, kept for half 1
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        ss[q] = split_tile(st[q]);
        contract_split_tile(c, sm.a.t, ss[q], q, P, R);
    }
    tv::inverse_split(c, sm.b.s);   // starts with a barrier: the tiles are read
    tv::store_rows(c, rv, sm.a.t.k);   // the V rows over the K tile
    lds_barrier();
    uint32_t vpk[2][8];
    tv::v_to_regs(c, sm.a.t.k, vpk);
    f32x16 u01[2], o[2];
    {
        f32x16 rhs[2];
        tv128::rhs_and_decay(c, sm.tp, 0, P, R, vpk, rhs);
        tv128::solve_half(c, sm.b.s, rhs, P, u01, o);
    }
    // ---- half 1's Q / K rows requested before half 0's stores, the key
    //      fragments of the cross blocks right after them: both arrive while
    //      the stores drain, not on the critical path behind them (issued
    //      later, the compiler schedules the fragments into the contraction
    //      and the cross blocks wait for them)
    const Lane c1 = fresh_lane();
    uint4 rq[4], rk[4];
    tv::load_rows(c1, s1, q, rq);
    tv::load_rows(c1, s1, k, rk);
    lds_barrier();   // every wave has read its V values and the solve blocks
    store_half<kUout, kUh>(c, s, 0, o, u01, sm, out, u_out);
    bf16x8 kf[8];
    load_key_frags(c1, s, k, c1.w & 1, kf);
    lds_barrier();   // every thread has stored its staged rows
    tv::store_rows_permuted(c1, rq, sm.a.t.q);
    tv::store_rows_permuted(c1, rk, sm.a.t.k);
    lds_barrier();

    // ---- P_23 / R_23 (the split slab's last use), then the cross blocks: wave
    //      w = 2 a + b forms (2 + a, b) from key fragments of rows 32 b..
    P[0] = P[1] = R[0] = R[1] = f32x16{};
#pragma unroll
    for (int q = 0; q < 4; ++q) contract_split_tile(c1, sm.a.t, ss[q], q, P, R);
    load_v_direct(c1, s1, v, vpk);
    {
        f32x16 gc, ga;
        gram_frags(c1, sm.a.t, c1.w >> 1, kf, gc, ga);
        float y[16], x[16];
        tv128::mask(c1, sm.tp, 2 + (c1.w >> 1), c1.w & 1, gc, ga, y, x);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = -x[r];
        tv128::store_split(c1, y, sm.b.x.yh[c1.w >> 1][c1.w & 1], sm.b.x.yl[c1.w >> 1][c1.w & 1]);
        tv128::store_split(c1, x, sm.b.x.xh[c1.w >> 1][c1.w & 1], sm.b.x.xl[c1.w >> 1][c1.w & 1]);
    }
    lds_barrier();   // cross blocks in

    // ---- half 1's right-hand side and P with the cross terms of U_01
    f32x16 rhs[2];
    tv128::rhs_and_decay(c1, sm.tp, 1, P, R, vpk, rhs);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const SplitTile ub = split_tile(u01[b]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            rhs[t] = mm3<kBL>(sm.b.x.xh[t][b], sm.b.x.xl[t][b], ub, rhs[t], c1.m, c1.h);
            P[t] = mm3<kBL>(sm.b.x.yh[t][b], sm.b.x.yl[t][b], ub, P[t], c1.m, c1.h);
        }
    }
    lds_barrier();   // every wave is done with the cross blocks

    // ---- half 1's blocks, inverse, solve, output rows
    if (c1.w < 3) {
        f32x16 gc, ga;
        gram_tiles(c1, sm.a.t, la, lb, gc, ga);
        float y[16], x[16];
        tv128::mask(c1, sm.tp, 2 + la, 2 + lb, gc, ga, y, x);
        tv128::half_store(c1, y, x, sm.b.s);
    }
    lds_barrier();
    tv::inverse(c1, sm.b.s);
    lds_barrier();
    f32x16 u[2];
    tv128::solve_half(c1, sm.b.s, rhs, P, u, o);
    if constexpr (kUout) lds_barrier();   // the pseudo-values are staged over the solve blocks
    store_half<kUout, kUh>(c1, s, 1, o, u, sm, out, u_out);
}

}  // namespace tvh
}  // namespace gdn
