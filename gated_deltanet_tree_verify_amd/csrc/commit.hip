// State commit along the accepted branch (DFlash-TfM page, section on
// rollback-free tree verification for GDN: commitment is deferred until the
// accepted branch is known, so verify never has to roll anything back).
//
// For every (sequence, head) the state S (d_k x d_v fp32) is advanced in
// place by the GDN update for each node of the path, root first:
//     w = S^T k_t;   S <- alpha_t (S - beta_t k_t w^T) + beta_t k_t v_t^T.
// Each column of S evolves independently, so a workgroup owns a tile of 64
// columns and all d_k rows of it, split over four row groups of threads;
// w for a column is the sum of four partial dot products exchanged in LDS.
// The tile stays in registers for the whole path: S is read once and
// written once, which is the HBM floor for an in-place commit.  The path's
// rows (k, this tile's v, alpha, beta) are staged in LDS 8 nodes at a
// time, all of a chunk's loads in flight together, so the steps wait on no
// global load.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTileV = 64;
constexpr int kGroups = kThreads / kTileV;               // row groups
constexpr int kRowsMax = GDN_MAX_DIM / kGroups;          // rows per thread (<= 32)
constexpr int kChunk = 8;                                // path nodes staged at a time
constexpr int kKLoads = kChunk * GDN_MAX_DIM / kThreads; // k values per thread and chunk
constexpr int kVLoads = kChunk * kTileV / kThreads;      // v values per thread and chunk

// A path is valid when 0 <= m <= max_path, every id is in [0, n), the first
// node is a root (parent -1) and every later node's parent is the previous
// node, with ids strictly increasing (topological order).  Checked by one
// wave, one path slot per lane: two rounds of reads rather than a chain.
__device__ bool path_valid_wave(const int32_t *par, const int32_t *path, int m, int max_path,
                                int n, int lane) {
    if (m < 0 || m > max_path) return false;
    bool bad = false;
    for (int j0 = 0; j0 < m; j0 += 64) {
        const int j = j0 + lane;
        if (j < m) {
            const int id = path[j];
            const int prev = j == 0 ? -1 : path[j - 1];
            if (id < 0 || id >= n || (j > 0 && prev >= id)) bad = true;
            else if (par[id] != prev) bad = true;
        }
    }
    return __ballot(bad) == 0ull;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void commit_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, int n, int H, int dk, int dv,
    int32_t *__restrict__ status) {
    __shared__ float s_k[kChunk][GDN_MAX_DIM];
    __shared__ float s_v[kChunk][kTileV];
    __shared__ float s_a[kChunk], s_b[kChunk];
    __shared__ int s_id[kChunk];
    __shared__ float s_part[kGroups][kTileV];
    __shared__ int s_ok;

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int c0 = blockIdx.y * kTileV;
    const int cl = tid % kTileV, grp = tid / kTileV;
    const int c = c0 + cl;
    const int rows = (dk + kGroups - 1) / kGroups;
    const int r0 = grp * rows;
    const int32_t *prow = path + (size_t)b * max_path;

    if (tid < 64) {
        const bool ok = path_valid_wave(parent + (size_t)b * n, prow, path_len[b], max_path, n, tid);
        if (tid == 0) {
            s_ok = ok;
            if (h == 0 && blockIdx.y == 0 && status) status[b] = ok ? 0 : kFaultBadPath;
        }
    }
    __syncthreads();
    if (!s_ok) return;
    const int m = path_len[b];
    if (m == 0) return;

    float *st = S + (size_t)bh * dk * dv;
    float reg[kRowsMax];
#pragma unroll
    for (int j = 0; j < kRowsMax; ++j) {
        const int r = r0 + j;
        reg[j] = (j < rows && r < dk && c < dv) ? st[(size_t)r * dv + c] : 0.f;
    }

    const size_t row0 = (size_t)b * n * H + h;   // gate row of node 0 (node stride H)
    for (int t0 = 0; t0 < m; t0 += kChunk) {
        const int mc = min(kChunk, m - t0);
        __syncthreads();   // the previous chunk is consumed
        if (tid < mc) s_id[tid] = prow[t0 + tid];
        __syncthreads();
        // every load of the chunk issued before any is stored
        float kx[kKLoads], vx[kVLoads];
#pragma unroll
        for (int it = 0; it < kKLoads; ++it) {
            const int e = tid + kThreads * it, t = e / dk, d = e - t * dk;
            const int id = s_id[min(t, kChunk - 1)];   // read only when t < mc
            kx[it] = (t < mc) ? to_f32(k[(row0 + (size_t)id * H) * dk + d]) : 0.f;
        }
#pragma unroll
        for (int it = 0; it < kVLoads; ++it) {
            const int e = tid + kThreads * it, t = e / kTileV, cc = e - t * kTileV;
            vx[it] = (t < mc && c0 + cc < dv)
                         ? to_f32(v[(row0 + (size_t)s_id[t] * H) * dv + c0 + cc]) : 0.f;
        }
        if (tid < mc) {
            const size_t row = row0 + (size_t)s_id[tid] * H;
            s_a[tid] = alpha[row];
            s_b[tid] = beta[row];
        }
#pragma unroll
        for (int it = 0; it < kKLoads; ++it) {
            const int e = tid + kThreads * it, t = e / dk, d = e - t * dk;
            if (t < mc) s_k[t][d] = kx[it];
        }
#pragma unroll
        for (int it = 0; it < kVLoads; ++it) {
            const int e = tid + kThreads * it;
            s_v[e / kTileV][e % kTileV] = vx[it];
        }
        __syncthreads();
        for (int t = 0; t < mc; ++t) {
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < kRowsMax; ++j)
                if (j < rows && r0 + j < dk) part = fmaf(reg[j], s_k[t][r0 + j], part);
            s_part[grp][cl] = part;
            __syncthreads();
            float w = 0.f;
#pragma unroll
            for (int g = 0; g < kGroups; ++g) w += s_part[g][cl];
            const float vc = s_v[t][cl], a = s_a[t], be = s_b[t];
#pragma unroll
            for (int j = 0; j < kRowsMax; ++j) {
                if (j < rows && r0 + j < dk) {
                    const float bk = be * s_k[t][r0 + j];
                    reg[j] = a * (reg[j] - bk * w) + bk * vc;
                }
            }
            __syncthreads();   // s_part is rewritten by the next step
        }
    }

#pragma unroll
    for (int j = 0; j < kRowsMax; ++j) {
        const int r = r0 + j;
        if (j < rows && r < dk && c < dv) st[(size_t)r * dv + c] = reg[j];
    }
}

}  // namespace

hipError_t launch_commit(const CommitArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.batch * a.H), (unsigned)((a.dv + kTileV - 1) / kTileV));
    if (a.dtype == GDN_DTYPE_BF16) {
        hipLaunchKernelGGL(commit_kernel<uint16_t>, grid, dim3(kThreads), 0, s, a.S, a.path,
                           a.path_len, a.max_path, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           a.alpha, a.beta, a.parent, a.n, a.H, a.dk, a.dv, a.status);
    } else {
        hipLaunchKernelGGL(commit_kernel<float>, grid, dim3(kThreads), 0, s, a.S, a.path,
                           a.path_len, a.max_path, (const float *)a.k, (const float *)a.v,
                           a.alpha, a.beta, a.parent, a.n, a.H, a.dk, a.dv, a.status);
    }
    return hipGetLastError();
}

}  // namespace gdn
