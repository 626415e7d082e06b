// MFMA tree-verify kernel for bf16 q/k/v, d_k = d_v = 128 and trees of
// 65..128 nodes (gfx950).  One workgroup per (sequence, head), four waves,
// wave w owning d_v columns [32 w, 32 w + 32); the stages and the two-half
// solve are in tree_verify128.hpp.  LDS: the 128-row Q/K tiles (68 KB), one
// region that holds the V tile and then the 64-node solve blocks of each
// half in turn plus the four cross blocks (82 KB), and the topology (5.5 KB):
// one workgroup per CU.  Each half's output rows are staged over the Q/K
// tiles once the last contraction has read them.  The state slab is requested one 32-row tile at a
// time between the phases that do not need it.  With one wave per SIMD
// nothing hides a stage's latency, so independent work is paired: each wave
// forms its first- and second-half block values together (the second half's
// wait in registers until its solve blocks are free), and each state tile is
// contracted into both halves' P / R as soon as it has landed, ahead of the
// stage that follows, so only the last tile's share waits for the last tile.
#include "internal.hpp"
#include "tree_verify128.hpp"

namespace gdn {
namespace {

using namespace tv128;

struct Smem {
    union {
        QKTiles t;
        float o[64][kD + 4];   // one half's output rows, once Q and K are dead
    } a;
    union {
        uint16_t v[kN][kQK];
        struct {
            SolveBlocks s;
            Cross x;
        } sx;
    } b;
    Topo tp;
};

static_assert(sizeof(Smem) <= 163840, "one workgroup per CU");
static_assert(sizeof(uint16_t) * kN * kQK <= sizeof(SolveBlocks),
              "the V tile must not reach the cross blocks");

__global__ __launch_bounds__(kThreads, 1) void verify_mfma_n128_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status, bool status_or) {
    __shared__ Smem sm;
    const Lane c = tv::lane_coords();
    const Seq s = tv::seq_coords(blockIdx.x, n, H);
    const float *slab = S0 + (size_t)blockIdx.x * kD * kD;

    // ---- 1. the Q and K tiles (waves 0-2) while wave 3 builds the topology
    //         under its share of the V rows; then the V tile
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
            tv128::load_rows(c, s, v, x);
            tv128::topology(c, s, parent, alpha, beta, sm.tp, status, s.hd == 0, status_or);
        }
        tv128::store_rows(c, x, sm.b.v);
    }
    f32x16 st[4];
    load_state_tile(st[0], 0, slab, c.col, c.h);
    lds_barrier();

    // ---- 2. cross blocks (one per wave), V -> registers
    tv128::cross_block(c, sm.a.t, sm.tp, sm.b.sx.x);
    uint32_t vpk[4][8];
    tv128::v_to_regs(c, sm.b.v, vpk);
    load_state_tile(st[1], 1, slab, c.col, c.h);
    lds_barrier();
    if (sm.tp.bad) {
        tv128::store_nan(c, s, out);
        return;
    }

    // ---- 3. half 0: blocks, inverse, solve, outputs; half 1's block values
    //         wait in registers until its solve blocks are free, and each
    //         state tile goes into both halves' P / R once it has landed
    f32x16 P0[2] = {}, R0[2] = {}, P1[2] = {}, R1[2] = {};
    tv128::contract_tile(c, sm.a.t, 0, st[0], P0, R0, P1, R1);
    float y1[16], x1[16];
    if (c.w < 3) {
        float y0[16], x0[16];
        tv128::half_values(c, sm.a.t, sm.tp, 0, y0, x0);
        tv128::half_values(c, sm.a.t, sm.tp, 1, y1, x1);
        tv128::half_store(c, y0, x0, sm.b.sx.s);
    }
    load_state_tile(st[2], 2, slab, c.col, c.h);
    lds_barrier();
    tv128::contract_tile(c, sm.a.t, 1, st[1], P0, R0, P1, R1);
    tv::inverse(c, sm.b.sx.s);
    load_state_tile(st[3], 3, slab, c.col, c.h);
    tv128::contract_tile(c, sm.a.t, 2, st[2], P0, R0, P1, R1);
    lds_barrier();
    tv128::contract_tile(c, sm.a.t, 3, st[3], P0, R0, P1, R1);
    f32x16 u01[2];
    {
        f32x16 rhs[2], o[2];
        tv128::rhs_and_decay(c, sm.tp, 0, P0, R0, vpk, rhs);
        tv128::solve_half(c, sm.b.sx.s, rhs, P0, u01, o);
        lds_barrier();   // every wave has read its last Q / K rows
        tv128::store_out_staged(c, s, 0, o, sm.a.o, out);
    }
    lds_barrier();   // every wave is done with half 0's solve blocks

    // ---- 4. half 1, with the cross terms of half 0's pseudo-values
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
        tv128::store_out_staged(c, s, 1, o, sm.a.o, out);
    }
}

}  // namespace

bool verify_mfma128_supports(const VerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n > 64 && a.n <= kN &&
           a.H <= 4096;
}

hipError_t launch_verify_mfma128(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_mfma_n128_kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads),
                       0, s, (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, a.status,
                       a.status_or);
    return hipGetLastError();
}

}  // namespace gdn
