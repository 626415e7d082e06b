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
// written once, which is the HBM floor for an in-place commit.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTileV = 64;
constexpr int kGroups = kThreads / kTileV;               // row groups
constexpr int kRowsMax = GDN_MAX_DIM / kGroups;          // rows per thread (<= 32)

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
    __shared__ float s_k[GDN_MAX_DIM];
    __shared__ float s_v[kTileV];
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

    for (int t = 0; t < m; ++t) {
        const int node = prow[t];
        const size_t row = ((size_t)b * n + node) * H + h;
        for (int d = tid; d < dk; d += kThreads) s_k[d] = to_f32(k[row * dk + d]);
        if (tid < kTileV) s_v[tid] = (c0 + tid < dv) ? to_f32(v[row * dv + c0 + tid]) : 0.f;
        const float a = alpha[row], be = beta[row];
        __syncthreads();
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < kRowsMax; ++j)
            if (j < rows && r0 + j < dk) part = fmaf(reg[j], s_k[r0 + j], part);
        s_part[grp][cl] = part;
        __syncthreads();
        float w = 0.f;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) w += s_part[g][cl];
        const float vc = s_v[cl];
#pragma unroll
        for (int j = 0; j < kRowsMax; ++j) {
            if (j < rows && r0 + j < dk) {
                const float bk = be * s_k[r0 + j];
                reg[j] = a * (reg[j] - bk * w) + bk * vc;
            }
        }
        __syncthreads();   // s_k / s_v / s_part are rewritten by the next step
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
