// MFMA state commit along the accepted branch, bf16 k/v, d_k = d_v = 128.
// One workgroup per (sequence, head); the chunked commit stages are in
// path_commit.hpp, where the method is described.  The state is read once
// and written once.  Two kernels: 32-slot chunks for any path length, and
// one 16-slot chunk prepared while the state streams in for paths of at
// most 16 nodes (chosen by max_path).
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
    // the first chunk's rows are requested ahead of the state, which only its
    // application needs; each later chunk's rows while the one before it is
    // applied.  State: 4-byte accesses, one tile at a time (measured faster
    // here than the whole-slab 8-byte ones).
    ChunkRows rows = load_chunk(sm.pi.pid, 0, mlen, b, hd, n, H, k, v, alpha, beta, tid);
#pragma unroll
    for (int q = 0; q < 4; ++q) load_state_tile(st[q], q, slab, col, h);
    bf16x8 ident[2];
    key_identity(ident, m, h);
    for (int c0 = 0; c0 < mlen; c0 += kC) {
        build_chunk(sm.ct, rows, c0, mlen, tid, w, l);
        if (c0 + kC < mlen)
            rows = load_chunk(sm.pi.pid, c0 + kC, mlen, b, hd, n, H, k, v, alpha, beta, tid);
        apply_chunk(sm.ct, st, ident, m, h, col);
        lds_barrier();   // the chunk tiles are restaged next
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) store_state_tile(st[q], q, slab, col, h);
}

// Paths of at most 16 nodes (max_path <= 16, the usual case: a tree of
// depth d gives paths of at most d + 1 nodes): one 16-slot chunk, prepared by
// wave 0 alone while the other waves stream the state.  Wave 0 reads the
// path ids, then in one round the parents that validate them and the
// chunk's key / value rows and gates, then its own state tiles, which land
// while it builds the chunk (Gram, X, T = (I + X)^{-1}); waves 1-3 request
// theirs at once.  Every wave then applies the chunk (R = K_p S,
// U = T RHS, the update) and writes its slab back.
struct SmemShort {
    Chunk16 ch;
    Chunk16Aux cx;
    int ok;
};

__global__ __launch_bounds__(kThreads, 2) void commit_mfma_short_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, int n, int H, int32_t *__restrict__ status) {
    __shared__ SmemShort sm;
    // the wave index is uniform: keep it scalar so role branches stay scalar
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int m = l & 31, h = l >> 5;
    const int bh = blockIdx.x, b = bh / H, hd = bh % H;
    const int col = 32 * w + m;
    const int mlen = path_len[b];
    float *slab = S + (size_t)bh * kD * kD;
    f32x16 st[4];
    if (w == 0) {
        // node 0's row and gate entry of this (sequence, head)
        const size_t row0 = ((size_t)b * n * H + hd) * kD;
        const size_t gate0 = (size_t)b * n * H + hd;
        const uint32_t bytes = (uint32_t)((size_t)n * H * kD * 2);
        const int32_t *prow = path + (size_t)b * max_path;
        const int32_t *par = parent + (size_t)b * n;
        PathLanes pl{-1, -1, -2, -2};
        const int lim = min(min(mlen, max_path), kC16);
        if (l < lim) pl.id0 = prow[l];
        if (pl.id0 >= 0 && pl.id0 < n) pl.par0 = par[pl.id0];
        const int mc = min(kC16, mlen);
        const int rj = l >> 2;
        const int rid = slot_id(pl, rj);
        const Rows16 r16 = load_rows16(rid, rj < mc && rid >= 0 && rid < n, pl.id0,
                                       l < mc && pl.id0 >= 0 && pl.id0 < n, k + row0, v + row0,
                                       alpha + gate0, beta + gate0, H * kD, H, bytes, l);
        load_state(st, slab, col, h);
        for (int i = l; i < kKP; i += 64) sm.cx.zk[i] = 0;
        if (l < kBL) sm.cx.zt[l] = 0;
        const bool ok = path_valid(pl, mlen, max_path, n, l) && mlen <= kC16;
        if (l == 0) {
            sm.ok = ok;
            if (hd == 0 && status) status[b] = ok ? 0 : kFaultBadPath;
        }
        if (ok && mlen > 0) build16(sm.ch, sm.cx, r16, mc, l);
    } else {
        load_state(st, slab, col, h);
    }
    lds_barrier();
    if (!sm.ok || mlen == 0) return;
    bf16x8 ident[2];
    key_identity(ident, m, h);
    apply16(sm.ch, sm.cx, st, ident, m, h, col);
    store_state(st, slab, col, h);
}

}  // namespace

bool commit_mfma_supports(const CommitArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.H <= 4096;
}

hipError_t launch_commit_mfma(const CommitArgs &a, hipStream_t s) {
    auto kern = a.max_path <= kC16 ? commit_mfma_short_kernel : commit_mfma_kernel;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0, s,
                       a.S, a.path, a.path_len, a.max_path, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.n, a.H, a.status);
    return hipGetLastError();
}

}  // namespace gdn
