// MFMA tree-verify kernel for bf16 q/k/v, d_k = d_v = 128 and trees of
// 65..128 nodes, two workgroups per CU (gfx950).
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
// region for a half's solve blocks or the cross blocks, the topology.  With
// two resident workgroups per CU each stage's latency is hidden behind the
// other workgroup's work, which one workgroup per CU (the whole tree's Q / K
// tiles and all blocks resident) cannot do.
#include "internal.hpp"
#include "tree_verify128.hpp"

namespace gdn {
namespace {

using namespace tile;
using tv::kBL;
using tv::kD;
using tv::kThreads;
using tv::Lane;
using tv::Seq;
using tv::SolveBlocks;

struct Smem {
    union {
        tv::QKTiles t;        // the current half's Q and K rows, d_k permuted
        float o[64][kD + 4];  // a half's output rows
    } a;
    union {
        SolveBlocks s;        // the current half's blocks
        tv128::Cross x;       // X_{23,01}, Y_{23,01}
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
// These rows were read in half 0, so they normally come from L2.
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

__global__ __launch_bounds__(kThreads, 2) void verify_mfma_n128_halves_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status, bool status_or) {
    __shared__ Smem sm;
    const Lane c = tv::lane_coords();
    const Seq s = tv::seq_coords(blockIdx.x, n, H);
    Seq s1 = s;   // rows 64.. of the same (sequence, head)
    s1.base += 64 * s.rstride;
    s1.n = n - 64;
    const float *slab = S0 + (size_t)blockIdx.x * kD * kD;
    // waves 0-2 take the blocks (0,0), (1,0), (1,1) of a half
    const int la = c.w == 0 ? 0 : 1, lb = c.w == 2 ? 1 : 0;

    // ---- 1. gates (wave 3), rows 0..63 of Q and K, the slab, rows 0..63 of
    //         V; the topology while they are in flight
    tv128::Gates2 gt;
    if (c.w == 3) gt = tv128::load_gates2(c, s, parent, alpha, beta);
    uint4 rq[4], rk[4], rv[4];
    tv::load_rows(c, s, q, rq);
    tv::load_rows(c, s, k, rk);
    if (c.w == 3) tv128::topology(c, s, gt, sm.tp, status, s.hd == 0, status_or);
    tv::store_rows_permuted(c, rq, sm.a.t.q);
    tv::store_rows_permuted(c, rk, sm.a.t.k);
    f32x16 st[4];
    load_state(st, slab, c.col, c.h);
    tv::load_rows(c, s, v, rv);
    lds_barrier();
    if (sm.tp.bad) {
        tv128::store_nan(c, s, out);
        return;
    }

    // ---- 2. half 0: blocks, inverse, P_01 / R_01 (the slab stays), solve
    if (c.w < 3) {
        f32x16 gc, ga;
        gram_tiles(c, sm.a.t, la, lb, gc, ga);
        float y[16], x[16];
        tv128::mask(c, sm.tp, la, lb, gc, ga, y, x);
        tv128::half_store(c, y, x, sm.b.s);
    }
    lds_barrier();
    tv::inverse_subst(c, sm.b.s);
    tv::inverse_zl(c, sm.b.s);
    f32x16 P[2], R[2];
    tv::contract(c, sm.a.t, st, P, R);
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
    lds_barrier();   // every wave has read its V values
    tv128::store_out_staged(c, s, 0, o, sm.a.o, out);

    // ---- 3. half 1's Q / K rows over half 0's
    tv::load_rows(c, s1, q, rq);
    tv::load_rows(c, s1, k, rk);
    lds_barrier();   // every thread has stored its staged output rows
    tv::store_rows_permuted(c, rq, sm.a.t.q);
    tv::store_rows_permuted(c, rk, sm.a.t.k);
    lds_barrier();

    // ---- 4. P_23 / R_23 (the slab's last use), then the cross blocks: wave
    //         w = 2 a + b forms (2 + a, b) from key fragments of rows 32 b..
    tv::contract(c, sm.a.t, st, P, R);
    load_v_direct(c, s1, v, vpk);
    bf16x8 kf[8];
    load_key_frags(c, s, k, c.w & 1, kf);
    {
        f32x16 gc, ga;
        gram_frags(c, sm.a.t, c.w >> 1, kf, gc, ga);
        float y[16], x[16];
        tv128::mask(c, sm.tp, 2 + (c.w >> 1), c.w & 1, gc, ga, y, x);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = -x[r];
        tv128::store_split(c, y, sm.b.x.yh[c.w >> 1][c.w & 1], sm.b.x.yl[c.w >> 1][c.w & 1]);
        tv128::store_split(c, x, sm.b.x.xh[c.w >> 1][c.w & 1], sm.b.x.xl[c.w >> 1][c.w & 1]);
    }
    lds_barrier();   // cross blocks in

    // ---- 5. half 1's right-hand side and P with the cross terms of U_01
    f32x16 rhs[2];
    tv128::rhs_and_decay(c, sm.tp, 1, P, R, vpk, rhs);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const SplitTile ub = split_tile(u01[b]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            rhs[t] = mm3<kBL>(sm.b.x.xh[t][b], sm.b.x.xl[t][b], ub, rhs[t], c.m, c.h);
            P[t] = mm3<kBL>(sm.b.x.yh[t][b], sm.b.x.yl[t][b], ub, P[t], c.m, c.h);
        }
    }
    lds_barrier();   // every wave is done with the cross blocks

    // ---- 6. half 1's blocks, inverse, solve, output rows
    if (c.w < 3) {
        f32x16 gc, ga;
        gram_tiles(c, sm.a.t, la, lb, gc, ga);
        float y[16], x[16];
        tv128::mask(c, sm.tp, 2 + la, 2 + lb, gc, ga, y, x);
        tv128::half_store(c, y, x, sm.b.s);
    }
    lds_barrier();
    tv::inverse(c, sm.b.s);
    lds_barrier();
    f32x16 u[2];
    tv128::solve_half(c, sm.b.s, rhs, P, u, o);
    tv128::store_out_staged(c, s, 1, o, sm.a.o, out);
}

}  // namespace

bool verify_mfma128h_supports(const VerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n > 64 &&
           a.n <= tv128::kN && a.H <= 4096;
}

hipError_t launch_verify_mfma128h(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_mfma_n128_halves_kernel, dim3((unsigned)(a.batch * a.H)),
                       dim3(kThreads), 0, s, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H,
                       a.status, a.status_or);
    return hipGetLastError();
}

}  // namespace gdn
