// MFMA tree-verify kernel for bf16 q/k/v, d_k = d_v = 128, n <= 64 (gfx950).
//
// One workgroup per (sequence, head); the stages (topology, transposed Gram
// tiles, mask and decay, tiled block inverse, Q S0 / K S0, solve, output)
// are in tree_verify.hpp, where the method is described.  This kernel adds
// the load schedule: Q/K tiles first (16-byte row chunks into LDS), then
// the S0 slab, then the v rows, which only the solve needs: they wait in
// registers and pass through the K tile's place once the contraction has
// read it, so the tree matrices never wait for them.  A wave that issues
// the 64 KiB slab stalls until the memory system has accepted it, so the
// two workgroups resident on a CU (dispatch rounds r and r + 1) take
// opposite orders: one streams its state first and builds the tree
// matrices afterwards, the other builds them while its neighbour streams,
// then streams its own.  LDS: 79 KB, two workgroups per CU; the output rows
// are staged over the dead Q/K tiles.
#include "internal.hpp"
#include "tree_verify.hpp"

namespace gdn {
namespace {

using namespace tv;

struct Smem {
    union {
        QKTiles t;
        float o[kN][kD + 4];
    } a;
    union {
        SolveBlocks s;
    } b;
    Topo tp;
};

// kOne: the trees have at most 32 nodes, so only the first 32-row block is
// contracted and solved (the host picks the instance)
template <bool kOne>
__global__ __launch_bounds__(kThreads, 2) void verify_mfma_n64_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int ncu, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const Lane c = lane_coords();
    const Seq s = seq_coords(blockIdx.x, n, H);

    // ---- 1. gates first (wave 3), then the Q and K tiles; topology while
    //         the tiles are in flight
    const Gates gt = load_gates(c, s, parent, alpha, beta);
    uint4 rq[4], rk[4], rv[4];
    load_rows(c, s, q, rq);
    load_rows(c, s, k, rk);
    if (c.w == 3) topology(c, s, gt, sm.tp, status, true);
    store_rows_permuted(c, rq, sm.a.t.q);
    store_rows_permuted(c, rk, sm.a.t.k);
    lds_barrier();

    const bool state_first = ((blockIdx.x / ncu) & 1) == 0;
    const float *slab = S0 + (size_t)blockIdx.x * kD * kD;
    f32x16 st[4];
    if (state_first) {
        load_state(st, slab, c.col, c.h);
        load_rows(c, s, v, rv);
    }

    // ---- 2. transposed Gram tiles (waves 0-2)
    f32x16 gc, ga;
    if (c.w < 3) gram(c, sm.a.t, gc, ga);
    lds_barrier();
    if (sm.tp.bad) {
        store_nan(c, s, out);
        return;
    }

    // ---- 3. X and Y blocks, 4. block inverses
    if (c.w < 3) mask(c, sm.tp, gc, ga, sm.b.s);
    lds_barrier();
    inverse_subst(c, sm.b.s);
    inverse_zl(c, sm.b.s);

    // ---- 5. P = Q S0, R = K S0 (the contraction does not need T, so the
    //         inverse's last step and its barrier come after it)
    if (!state_first) {
        load_state(st, slab, c.col, c.h);
        load_rows(c, s, v, rv);
    }
    f32x16 P[2], R[2];
    contract<kOne ? 1 : 2>(c, sm.a.t, st, P, R);
    inverse_split(c, sm.b.s);
    // the V tile through the K tile's place into this lane's columns (the
    // first block's staging rows lie in the Q tile's place)
    lds_barrier();
    store_rows(c, rv, sm.a.t.k);
    lds_barrier();
    uint32_t vpk[2][8];
    v_to_regs(c, sm.a.t.k, vpk);

    // ---- 6. solve and output, 7. whole-row stores
    // the first block's rows leave while the second block is solved
    SolveCarry cy;
    f32x16 u0, o0, u1, o1;
    solve_block0(c, sm.tp, sm.b.s, P, R, vpk, u0, o0, cy);
    store_block<false>(c, s, sm.a.o, o0, out, u0, nullptr, 0);
    if constexpr (kOne) return;
    solve_block1(c, sm.b.s, P, cy, u1, o1);
    lds_barrier();   // every thread has read the first block from the staging area
    store_block<false>(c, s, sm.a.o, o1, out, u1, nullptr, 32);
}

}  // namespace

bool verify_mfma_supports(const VerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n <= kN && a.H <= 4096;
}

hipError_t launch_verify_mfma(const VerifyArgs &a, hipStream_t s) {
    auto kernel = a.n <= 32 ? verify_mfma_n64_kernel<true> : verify_mfma_n64_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0, s,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, device_cu_count(),
                       a.status);
    return hipGetLastError();
}

}  // namespace gdn
