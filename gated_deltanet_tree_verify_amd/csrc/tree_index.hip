// Integer tree kernels: accepted-path extraction and tree indexing (depth,
// ancestor-or-self bitmasks).  The draft tree is topologically sorted
// (DFlash-TfM page, rollback-free GDN verification section), so every walk
// toward the root visits strictly decreasing ids and ends in at most n
// steps; a parent outside [-1, node) is reported instead of followed.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kWords = (GDN_MAX_NODES + 31) / 32;

// one thread per sequence: walk up from the accepted node, then write the
// path root first and pad the row with -1
__global__ __launch_bounds__(256) void path_kernel(const int32_t *__restrict__ parent,
                                                   const int32_t *__restrict__ accepted,
                                                   int32_t *__restrict__ path,
                                                   int32_t *__restrict__ path_len, int batch,
                                                   int n, int max_path,
                                                   int32_t *__restrict__ status) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int32_t *par = parent + (size_t)b * n;
    int32_t *row = path + (size_t)b * max_path;
    const int a = accepted[b];
    int flag = 0, m = 0;
    if (a < 0 || a >= n) {
        flag = kFaultBadPath;
    } else {
        for (int cur = a; cur != -1;) {
            ++m;
            const int p = par[cur];
            if (!parent_ok(p, cur)) { flag = kFaultBadParent; break; }
            cur = p;
        }
        if (!flag && m > max_path) flag = kFaultBadPath;
    }
    if (flag) m = 0;
    for (int j = m; j < max_path; ++j) row[j] = -1;
    for (int cur = a, j = m - 1; j >= 0; --j) {   // fill from the accepted node up
        row[j] = cur;
        cur = par[cur];
    }
    path_len[b] = m;
    if (status) status[b] = flag;
}

// one workgroup per sequence, one thread per node
__global__ __launch_bounds__(GDN_MAX_NODES) void index_kernel(const int32_t *__restrict__ parent,
                                                              int32_t *__restrict__ depth,
                                                              uint32_t *__restrict__ anc, int n,
                                                              int32_t *__restrict__ status) {
    const int b = blockIdx.x, i = threadIdx.x;
    const int32_t *par = parent + (size_t)b * n;
    const int W = (n + 31) / 32;
    const int bad = __syncthreads_or(i < n && !parent_ok(par[i], i));
    if (i == 0 && status) status[b] = bad ? kFaultBadParent : 0;
    if (i >= n) return;
    uint32_t bits[kWords];
#pragma unroll
    for (int w = 0; w < kWords; ++w) bits[w] = 0u;
    int d = -1;
    if (!bad) {
        d = 0;
        for (int t = i; t >= 0; t = par[t]) {
#pragma unroll
            for (int w = 0; w < kWords; ++w)
                if (w == t / 32) bits[w] |= 1u << (t % 32);
            if (t != i) ++d;
        }
    }
    depth[(size_t)b * n + i] = d;
    for (int w = 0; w < W; ++w) anc[((size_t)b * n + i) * W + w] = bits[w];
}

}  // namespace

hipError_t launch_path(const int32_t *parent, const int32_t *accepted, int32_t *path,
                       int32_t *path_len, int batch, int n, int max_path, int32_t *status,
                       hipStream_t s) {
    const int threads = 256;
    hipLaunchKernelGGL(path_kernel, dim3((batch + threads - 1) / threads), dim3(threads), 0, s,
                       parent, accepted, path, path_len, batch, n, max_path, status);
    return hipGetLastError();
}

hipError_t launch_index(const int32_t *parent, int32_t *depth, uint32_t *anc, int batch, int n,
                        int32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(index_kernel, dim3(batch), dim3(GDN_MAX_NODES), 0, s, parent, depth, anc,
                       n, status);
    return hipGetLastError();
}

}  // namespace gdn
