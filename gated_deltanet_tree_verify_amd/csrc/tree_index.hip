// Integer tree kernels: the greedy acceptance walk, accepted-path
// extraction and tree indexing (depth, ancestor-or-self bitmasks).  The draft tree is topologically sorted
// (DFlash-TfM page, rollback-free GDN verification section), so every walk
// toward the root visits strictly decreasing ids and ends in at most n
// steps; a parent outside [-1, node) is reported instead of followed.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kWords = (GDN_MAX_NODES + 31) / 32;

// one wave per sequence: the parents sit in registers (nodes l and 64 + l
// per lane), so the walk up from the accepted node is a chain of lane
// shuffles rather than of dependent global loads; the path is then written
// root first and the row padded with -1
__device__ __forceinline__ int par_of(const int (&par)[2], int node) {
    const int a = __shfl(par[0], node & 63), b = __shfl(par[1], node & 63);
    return node < 64 ? a : b;
}

__global__ __launch_bounds__(64) void path_kernel(const int32_t *__restrict__ parent,
                                                  const int32_t *__restrict__ accepted,
                                                  int32_t *__restrict__ path,
                                                  int32_t *__restrict__ path_len, int n,
                                                  int max_path, int32_t *__restrict__ status) {
    const int b = blockIdx.x, l = threadIdx.x;
    const int32_t *prow = parent + (size_t)b * n;
    int32_t *row = path + (size_t)b * max_path;
    int par[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) par[u] = 64 * u + l < n ? prow[64 * u + l] : -1;
    const int a = accepted[b];
    int flag = 0, m = 0;
    if (a < 0 || a >= n) {
        flag = kFaultBadPath;
    } else {
        // every lane follows the same (uniform) chain; ids strictly decrease
        for (int cur = a; cur != -1;) {
            ++m;
            const int p = par_of(par, cur);
            if (!parent_ok(p, cur)) { flag = kFaultBadParent; break; }
            cur = p;
        }
        if (!flag && m > max_path) flag = kFaultBadPath;
    }
    if (flag) m = 0;
    for (int j = m + l; j < max_path; j += 64) row[j] = -1;
    for (int cur = a, j = m - 1; j >= 0; --j) {   // fill from the accepted node up
        if (l == 0) row[j] = cur;
        cur = par_of(par, cur);
    }
    if (l == 0) {
        path_len[b] = m;
        if (status) status[b] = flag;
    }
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

// Greedy acceptance walk, one wave per sequence.  Node 0 is accepted; from
// an accepted node p the walk moves to the lowest-id child c with
// draft[c] == verify[p] and stops when there is none.  Each lane holds
// nodes l and 64 + l; a step is one ballot over "child of the current node
// with the matching token", so a walk costs (accepted length) ballots.
__global__ __launch_bounds__(64) void accept_kernel(const int32_t *__restrict__ parent,
                                                    const int32_t *__restrict__ draft,
                                                    const int32_t *__restrict__ verify,
                                                    int32_t *__restrict__ accepted,
                                                    int32_t *__restrict__ accept_len,
                                                    int32_t *__restrict__ bonus, int n,
                                                    int32_t *__restrict__ status) {
    const int b = blockIdx.x, l = threadIdx.x;
    const size_t base = (size_t)b * n;
    int par[2], dr[2], vf[2];
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + l;
        const bool live = i < n;
        par[u] = live ? parent[base + i] : -2;
        dr[u] = live ? draft[base + i] : 0;
        vf[u] = live ? verify[base + i] : 0;
        if (live && !parent_ok(par[u], i)) bad = true;
    }
    if (__ballot(bad) != 0ull) {
        if (l == 0) {
            accepted[b] = -1;
            if (accept_len) accept_len[b] = 0;
            if (bonus) bonus[b] = -1;
            if (status) status[b] = kFaultBadParent;
        }
        return;
    }
    int cur = 0, len = 1;
    for (;;) {
        // the verifier's token at the current node, from the lane that holds it
        const int want = __shfl(cur < 64 ? vf[0] : vf[1], cur & 63);
        const unsigned long long m0 = __ballot(par[0] == cur && dr[0] == want);
        const unsigned long long m1 = __ballot(par[1] == cur && dr[1] == want);
        if ((m0 | m1) == 0ull) break;
        cur = m0 ? __builtin_ctzll(m0) : 64 + __builtin_ctzll(m1);
        ++len;
    }
    // every lane takes part in the shuffle (cur is uniform: it comes from ballots)
    const int last = __shfl(cur < 64 ? vf[0] : vf[1], cur & 63);
    if (l == 0) {
        accepted[b] = cur;
        if (accept_len) accept_len[b] = len;
        if (bonus) bonus[b] = last;
        if (status) status[b] = 0;
    }
}

}  // namespace

hipError_t launch_path(const int32_t *parent, const int32_t *accepted, int32_t *path,
                       int32_t *path_len, int batch, int n, int max_path, int32_t *status,
                       hipStream_t s) {
    hipLaunchKernelGGL(path_kernel, dim3((unsigned)batch), dim3(64), 0, s, parent, accepted, path,
                       path_len, n, max_path, status);
    return hipGetLastError();
}

hipError_t launch_index(const int32_t *parent, int32_t *depth, uint32_t *anc, int batch, int n,
                        int32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(index_kernel, dim3(batch), dim3(GDN_MAX_NODES), 0, s, parent, depth, anc,
                       n, status);
    return hipGetLastError();
}

hipError_t launch_accept(const int32_t *parent, const int32_t *draft, const int32_t *verify,
                         int32_t *accepted, int32_t *accept_len, int32_t *bonus, int batch, int n,
                         int32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(accept_kernel, dim3((unsigned)batch), dim3(64), 0, s, parent, draft, verify,
                       accepted, accept_len, bonus, n, status);
    return hipGetLastError();
}

}  // namespace gdn
