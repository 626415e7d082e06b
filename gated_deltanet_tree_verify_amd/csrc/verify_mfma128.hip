// MFMA tree-verify kernel for bf16 q/k/v, d_k = d_v = 128 and trees of
// 65..128 nodes, two workgroups per CU (gfx950).  One workgroup per
// (sequence, head), four waves, wave w owning d_v columns [32 w, 32 w + 32);
// the schedule of the two 64-node halves is in tree_verify128h.hpp.  This
// kernel adds the loads: wave 3 requests the gates and builds the topology
// while every wave's Q / K rows 0..63 and its state slab are in flight.
#include "internal.hpp"
#include "tree_verify128h.hpp"

namespace gdn {
namespace {

using namespace tile;
using tv::kD;
using tv::kThreads;
using tv::Lane;
using tv::Seq;

__global__ __launch_bounds__(kThreads, 2) void verify_mfma_n128_halves_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status, bool status_or) {
    __shared__ tvh::Smem sm;
    const Lane c = tv::lane_coords();
    const Seq s = tv::seq_coords(blockIdx.x, n, H);
    const float *slab = S0 + (size_t)blockIdx.x * kD * kD;

    tv128::Gates2 gt;
    if (c.w == 3) gt = tv128::load_gates2(c, s, parent, alpha, beta);
    uint4 rq[4], rk[4];
    tv::load_rows(c, s, q, rq);
    tv::load_rows<0>(c, s, k, rk);   // cached: rows 0..63 of K are read again for the cross blocks
    if (c.w == 3) tv128::topology(c, s, gt, sm.tp, status, s.hd == 0, status_or);
    tv::store_rows_permuted(c, rq, sm.a.t.q);
    tv::store_rows_permuted(c, rk, sm.a.t.k);
    f32x16 st[4];
    load_state(st, slab, c.col, c.h);
    lds_barrier();
    if (sm.tp.bad) {
        tv128::store_nan(c, s, out);
        return;
    }
    tvh::verify_halves<false, false>(c, s, sm, st, q, k, v, out, nullptr);
}

}  // namespace

bool verify_mfma128_supports(const VerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n > 64 &&
           a.n <= tv128::kN && a.H <= 4096;
}

hipError_t launch_verify_mfma128(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_mfma_n128_halves_kernel, dim3((unsigned)(a.batch * a.H)),
                       dim3(kThreads), 0, s, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H,
                       a.status, a.status_or);
    return hipGetLastError();
}

}  // namespace gdn
