// d_v-split state commit for small launches: bf16 k/v, d_k = d_v = 128,
// paths of at most 16 nodes, one two-wave workgroup per (sequence, head,
// quarter of d_v) (gfx950).
//
// The commit along the accepted branch (DFlash-TfM page, section on
// rollback-free tree verification for GDN) in the chunked form of
// path_commit.hpp, R = K_p S, U = T beta (V_p - e^g R), S <- e^{g_l} S +
// K_p^T W, is column by column in d_v: a quarter's workgroup commits its 32
// columns of the state and forms the path's chunk (keys, gates, X, T) itself.
// With one workgroup per (sequence, head), a launch far below the CU count
// has each CU read and write a whole 64 KiB slab (see tree_split.hpp).
//   wave 0: the path ids and the tree's parent row (validation), the chunk's
//           keys and gates, then the chunk's X and T;
//   wave 1: the quarter's state columns, then the chunk's values in its
//           columns, R_p = K_p S once the keys are in, the update and the
//           committed columns written back.
#include "internal.hpp"
#include "path_commit.hpp"
#include "tree_split.hpp"

namespace gdn {
namespace {

using namespace tile;
using ts::kQuarters;

constexpr int kThreads = 128;       // two waves
constexpr int kMaxPathIds = 128;    // a valid path has at most n <= 128 nodes

struct Smem {
    pc::EarlyChunk16 ch;   // the path's keys, X and T
    pc::Chunk16Aux cx;
    int pid[kMaxPathIds];  // path ids (slots < 16 used)
    int ok;
};

__global__ __launch_bounds__(kThreads) void commit_split_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, int n, int H, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = threadIdx.x & 63, m = l & 31, h = l >> 5;
    const int bh = blockIdx.x / kQuarters, quarter = blockIdx.x % kQuarters;
    const int b = bh / H, hd = bh % H;
    const int col = 32 * quarter + m;
    const int mlen = path_len[b];
    float *slab = S + (size_t)bh * tv::kD * tv::kD;
    // node 0's row and gate entry of this (sequence, head)
    const size_t row0 = ((size_t)b * n * H + hd) * tv::kD;
    const size_t gate0 = (size_t)b * n * H + hd;
    const uint32_t bytes = (uint32_t)((size_t)n * H * tv::kD * 2);

    // ---- 1. wave 0: ids, parents (the tree's parent row, nodes l and
    //         64 + l), the chunk's keys and gates, validation; wave 1: the
    //         quarter's state columns
    f32x16 st[4];
    pc::KeyRows16 r16;
    if (w == 0) {
        pc::PathLanes pl{-1, -1, -2, -2};
        int pp0 = -1, pp1 = -1;
        const int32_t *prow = path + (size_t)b * max_path;
        const int lim = min(min(mlen, max_path), pc::kC16);
        if (l < lim) pl.id0 = prow[l];
        const int32_t *par = parent + (size_t)b * n;
        if (l < n) pp0 = par[l];
        if (64 + l < n) pp1 = par[64 + l];
        pl.par0 = pc::parent_of(pl.id0, pp0, pp1, n);
        if (l < pc::kC16 && pl.id0 >= 0) sm.pid[l] = pl.id0;
        const int mc = min(pc::kC16, mlen);
        const int rj = l >> 2, rid = pc::slot_id(pl, rj);
        r16 = pc::load_keys16(rid, rj < mc && rid >= 0 && rid < n, pl.id0,
                              l < mc && pl.id0 >= 0 && pl.id0 < n, k + row0, alpha + gate0,
                              beta + gate0, H * tv::kD, H, bytes, l);
        const bool ok = pc::path_valid(pl, mlen, max_path, n, l) && mlen <= pc::kC16;
        if (l == 0) {
            sm.ok = ok && mlen > 0;
            if (hd == 0 && quarter == 0 && status) status[b] = ok ? 0 : kFaultBadPath;
        }
        for (int i = l; i < pc::kKP; i += ts::kLanes) sm.cx.zk[i] = 0;
        if (l < pc::kBL) sm.cx.zt[l] = 0;
    } else {
        load_state(st, slab, col, h);
    }
    lds_barrier();   // the path ids and validity
    if (!sm.ok) return;

    // ---- 2. the chunk's keys and X (wave 0), its values in this quarter's
    //         columns (wave 1)
    pc::ChunkWords V0;
    if (w == 0) {
        pc::build16_x(sm.ch, sm.cx, r16.k, r16.la, r16.bt, min(pc::kC16, mlen), l);
    } else {
        V0 = pc::load_v_chunk16(v + row0, bytes, sm.pid, 0, min(pc::kC16, mlen), H * tv::kD, col,
                                h);
    }
    lds_barrier();   // the chunk's keys and X

    // ---- 3. the chunk's T (wave 0), R_p = K_p S (wave 1)
    f32x16 Rp;
    const pc::ChunkView cv = pc::early_view(sm.ch, sm.cx, m);
    if (w == 0) {
        pc::build16_t(sm.ch, l);
    } else {
        // two accumulators (two short MFMA chains)
        f32x16 Ra = {}, Rb = {};
        pc::rp_tile(cv.kp_row, st[0], 0, Ra, h);
        pc::rp_tile(cv.kp_row, st[1], 1, Rb, h);
        pc::rp_tile(cv.kp_row, st[2], 2, Ra, h);
        pc::rp_tile(cv.kp_row, st[3], 3, Rb, h);
        Rp = Ra + Rb;
    }
    lds_barrier();   // the chunk's T
    if (w == 0) return;

    // ---- 4. U = T RHS, the update, the committed columns written back
    bf16x8 ident[2];
    pc::key_identity(ident, m, h);
    pc::finish_rows_v<pc::kC16>(cv, pc::widen_bf16(V0), Rp, st, ident, h);
    store_state(st, slab, col, h);
}

}  // namespace

bool commit_split_supports(const CommitArgs &a) {
    // small launches (as for the split verify) whose paths fit the one chunk
    return a.dtype == GDN_DTYPE_BF16 && a.dk == tv::kD && a.dv == tv::kD && a.H <= 4096 &&
           a.n <= kMaxPathIds && a.max_path <= pc::kC16 &&
           (long long)a.batch * a.H * kQuarters <= 2LL * device_cu_count();
}

hipError_t launch_commit_split(const CommitArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(commit_split_kernel, dim3((unsigned)(a.batch * a.H * kQuarters)),
                       dim3(kThreads), 0, s, a.S, a.path, a.path_len, a.max_path,
                       (const uint16_t *)a.k, (const uint16_t *)a.v, a.alpha, a.beta, a.parent,
                       a.n, a.H, a.status);
    return hipGetLastError();
}

}  // namespace gdn
