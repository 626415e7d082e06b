// d_v-split tree verify for small launches: bf16 q/k/v, d_k = d_v = 128,
// trees of at most 32 nodes, one two-wave workgroup per (sequence, head,
// quarter of d_v) (gfx950).  The stages and the reason for the split are in
// tree_split.hpp.
//   wave 0: the gates and Q rows, the topology, the Gram tile, masks and
//           T = (I + X)^{-1};
//   wave 1: the K rows, then the quarter's state columns and v values (its
//           stall on issuing them is off wave 0's path), P and R while wave 0
//           builds T, then the solve and the output rows.
#include "internal.hpp"
#include "tree_split.hpp"

namespace gdn {
namespace {

using namespace tile;
using ts::kQuarters;

constexpr int kThreads = 128;   // two waves

__global__ __launch_bounds__(kThreads) void verify_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status, bool status_or) {
    __shared__ ts::Tree sm;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = threadIdx.x & 63, m = l & 31, h = l >> 5;
    const int bh = blockIdx.x / kQuarters, quarter = blockIdx.x % kQuarters;
    const int col = 32 * quarter + m;
    const tv::Seq s = tv::seq_coords(bh, n, H);

    uint4 x[8];
    ts::load_rows32(s, w == 0 ? q : k, l, x);
    f32x16 st[4];
    uint32_t vpk[8];
    if (w == 0) {
        const bool bad = ts::topology(sm, s, parent, alpha, beta, l);
        if (l == 0 && quarter == 0 && s.hd == 0 && status) {
            const int f = bad ? kFaultBadParent : 0;
            status[s.b] = status_or ? (status[s.b] | f) : f;
        }
        ts::store_rows32(sm.q, l, x);
    } else {
        load_state(st, S0 + (size_t)bh * tv::kD * tv::kD, col, h);
        ts::load_v_col(s, v, col, h, vpk);
        ts::store_rows32(sm.k, l, x);
    }
    lds_barrier();   // Q and K rows, the topology
    if (sm.bad) {
        if (w == 1) {
            f32x16 nan;
#pragma unroll
            for (int r = 0; r < 16; ++r) nan[r] = __builtin_nanf("");
            ts::store_col(s, out, col, h, nan);
        }
        return;
    }
    if (w == 0) {
        ts::gram_mask(sm, m, h);
        ts::wave_lds_sync();
        ts::inverse(sm, l);
        lds_barrier();   // T and Y are in; wave 1 solves
        return;
    }
    f32x16 P, R, u, o;
    ts::contract(sm, st, m, h, P, R);
    lds_barrier();   // T and Y are in
    ts::solve(sm, vpk, P, R, m, h, u, o);
    ts::store_col(s, out, col, h, o);
}

}  // namespace

bool verify_split_supports(const VerifyArgs &a) {
    // small launches only (at most two split workgroups per CU): measured at
    // 32 nodes and 32 heads against one workgroup per (sequence, head),
    // batch 1 and 2 take 7.0 us instead of 9.4, batch 4 9.2 instead of 9.9,
    // batch 8 would take 13.9 instead of 10.5
    return a.dtype == GDN_DTYPE_BF16 && a.dk == tv::kD && a.dv == tv::kD && a.n <= ts::kN1 &&
           a.H <= 4096 && (long long)a.batch * a.H * kQuarters <= 2LL * device_cu_count();
}

hipError_t launch_verify_split(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_split_kernel, dim3((unsigned)(a.batch * a.H * kQuarters)),
                       dim3(kThreads), 0, s, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H,
                       a.status, a.status_or);
    return hipGetLastError();
}

}  // namespace gdn
