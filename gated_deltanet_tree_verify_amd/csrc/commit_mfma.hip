// MFMA state commit along the accepted branch, bf16 k/v, d_k = d_v = 128.
// One workgroup per (sequence, head); the chunked commit stages are in
// path_commit.hpp, where the method is described.  The state is read once
// and written once.
#include "internal.hpp"
#include "path_commit.hpp"

namespace gdn {
namespace {

using namespace pc;

struct Smem {
    ChunkTiles ct;
    PathIds pi;
};

__global__ __launch_bounds__(kThreads, 2) void commit_mfma_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, int n, int H, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    // the wave index is uniform: keep it scalar so role branches stay scalar
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int m = l & 31, h = l >> 5;
    const int bh = blockIdx.x, b = bh / H, hd = bh % H;
    const int col = 32 * w + m;
    const int32_t *prow = path + (size_t)b * max_path;
    const int mlen = path_len[b];

    if (w == 0) {
        const bool ok = validate_and_keep(sm.pi, parent + (size_t)b * n, prow, mlen, max_path, n, l);
        if (l == 0) {
            sm.pi.ok = ok;
            if (hd == 0 && status) status[b] = ok ? 0 : kFaultBadPath;
        }
    }
    lds_barrier();
    if (!sm.pi.ok || mlen == 0) return;

    // state slab: four result tiles of this lane's column
    float *slab = S + (size_t)bh * kD * kD;
    f32x16 st[4];
    load_state(st, slab, col, h);
    bf16x8 ident[2];
    key_identity(ident, m, h);
    for (int c0 = 0; c0 < mlen; c0 += kC) {
        prepare_chunk(sm.ct, sm.pi.pid, c0, mlen, b, hd, n, H, k, v, alpha, beta, tid, w, l);
        apply_chunk(sm.ct, st, ident, m, h, col);
        lds_barrier();   // the chunk tiles are restaged next
    }
    store_state(st, slab, col, h);
}

}  // namespace

bool commit_mfma_supports(const CommitArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.H <= 4096;
}

hipError_t launch_commit_mfma(const CommitArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(commit_mfma_kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0, s,
                       a.S, a.path, a.path_len, a.max_path, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.n, a.H, a.status);
    return hipGetLastError();
}

}  // namespace gdn
