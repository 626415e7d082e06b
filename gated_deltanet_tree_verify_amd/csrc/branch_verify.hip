// Single-branch recurrent verification: the baseline that the tree verify
// is measured against (DFlash-TfM page, experimental results: the fused
// tree kernel against recurrent verification of one branch at a time).
//
// Every root-to-leaf branch of the draft tree is run as its own chain by the
// GDN recurrence from S0,
//     w = S^T k_t;   S <- alpha_t (S - beta_t k_t w^T) + beta_t k_t v_t^T;   o_t = S^T q_t,
// and each node's output is written by every branch through it (the values
// agree bit for bit: a node's arithmetic depends only on its path prefix).
// Nodes on shared prefixes are recomputed once per branch and S0 is read
// once per branch, which is what the tree formulation avoids.
//
// d_k = d_v = 128 (the kernel that is timed): see branch_verify_d128_kernel.
// Other head sizes: one workgroup per (sequence, head, leaf, 64-column tile
// of S); the tile stays in registers for the whole branch, each thread
// holding one column and a quarter of the rows, and the two reductions per
// node (w and o) go through LDS.  Leaves are taken in id order; workgroups
// past the tree's leaf count exit at once.
#include "device_common.hpp"
#include "internal.hpp"
#include "mfma_tile.hpp"

namespace gdn {
namespace {

using namespace tile;

constexpr int kThreads = 256;
constexpr int kTileV = 64;
constexpr int kGroups = kThreads / kTileV;        // row groups
constexpr int kRowsMax = GDN_MAX_DIM / kGroups;   // rows per thread (<= 32)
constexpr int kMaxN = GDN_MAX_NODES;

template <typename T>
__global__ __launch_bounds__(kThreads) void branch_verify_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int dk, int dv, int32_t *__restrict__ status) {
    __shared__ int s_haschild[kMaxN];
    __shared__ int s_path[kMaxN];
    __shared__ int s_len, s_bad, s_leaf;
    __shared__ float s_k[GDN_MAX_DIM], s_q[GDN_MAX_DIM];
    __shared__ float s_v[kTileV];
    __shared__ float s_part[kGroups][kTileV];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int leaf_rank = blockIdx.y;
    const int c0 = blockIdx.z * kTileV;
    const int cl = tid % kTileV, grp = tid / kTileV;
    const int c = c0 + cl;
    const int rows = (dk + kGroups - 1) / kGroups;
    const int r0 = grp * rows;
    const int32_t *par = parent + (size_t)b * n;

    // ---- tree check and the leaf this workgroup runs
    for (int i = tid; i < n; i += kThreads) s_haschild[i] = 0;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
        const int p = par[i];
        if (!parent_ok(p, i)) s_bad = 1;            // benign race: every writer stores 1
        else if (p >= 0) s_haschild[p] = 1;
    }
    __syncthreads();
    if (s_bad) {
        if (leaf_rank == 0) {
            if (h == 0 && blockIdx.z == 0 && tid == 0 && status) status[b] = kFaultBadParent;
            for (int e = tid; e < n * kTileV; e += kThreads) {
                const int i = e / kTileV, cc = c0 + e % kTileV;
                if (cc < dv) out[(((size_t)b * n + i) * H + h) * dv + cc] = __builtin_nanf("");
            }
        }
        return;
    }
    if (tid == 0) {
        if (h == 0 && leaf_rank == 0 && blockIdx.z == 0 && status) status[b] = 0;
        // the leaf_rank-th leaf in id order, and its root-to-leaf path
        int seen = 0, leaf = -1;
        for (int i = 0; i < n && leaf < 0; ++i)
            if (!s_haschild[i] && seen++ == leaf_rank) leaf = i;
        int len = 0;
        if (leaf >= 0) {
            for (int j = leaf; j >= 0; j = par[j]) ++len;
            int j = leaf;
            for (int t = len - 1; t >= 0; --t, j = par[j]) s_path[t] = j;
        }
        s_leaf = leaf;
        s_len = len;
    }
    __syncthreads();
    if (s_leaf < 0) return;
    const int m = s_len;

    // ---- this thread's rows of column c of S0
    const float *st0 = S0 + (size_t)bh * dk * dv;
    float reg[kRowsMax];
#pragma unroll
    for (int j = 0; j < kRowsMax; ++j) {
        const int r = r0 + j;
        reg[j] = (j < rows && r < dk && c < dv) ? st0[(size_t)r * dv + c] : 0.f;
    }

    for (int t = 0; t < m; ++t) {
        const int node = s_path[t];
        const size_t row = ((size_t)b * n + node) * H + h;
        for (int d = tid; d < dk; d += kThreads) {
            s_k[d] = to_f32(k[row * dk + d]);
            s_q[d] = to_f32(q[row * dk + d]);
        }
        if (tid < kTileV) s_v[tid] = (c0 + tid < dv) ? to_f32(v[row * dv + c0 + tid]) : 0.f;
        const float a = alpha[row], be = beta[row];
        __syncthreads();
        // w = S^T k for this column
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
        // update, then o = S^T q
        float po = 0.f;
#pragma unroll
        for (int j = 0; j < kRowsMax; ++j) {
            if (j < rows && r0 + j < dk) {
                const float bk = be * s_k[r0 + j];
                reg[j] = a * (reg[j] - bk * w) + bk * vc;
                po = fmaf(reg[j], s_q[r0 + j], po);
            }
        }
        __syncthreads();   // every thread has read s_part for w
        s_part[grp][cl] = po;
        __syncthreads();
        if (grp == 0 && c < dv) {
            float o = 0.f;
#pragma unroll
            for (int g = 0; g < kGroups; ++g) o += s_part[g][cl];
            out[row * dv + c] = o;
        }
        __syncthreads();   // s_k, s_q, s_v, s_part are rewritten by the next node
    }
}

// ---- d_k = d_v = 128: register-resident state, one wave per 32 columns.
// Each wave holds rows crow(r, h) + 32 q of its lane's column (the 32x32
// result-tile layout), so S^T k and S^T q are a lane's 64 products plus one
// exchange with the lane holding the other half of the column; waves run
// their branch with no barrier between nodes.  A workgroup takes leaf ranks
// y, y + G, y + 2G, ... of its (sequence, head), G = gridDim.y.
constexpr int kD = 128;

template <typename T>
__device__ __forceinline__ float ld_f32(const T *p, int i) {
    return to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void branch_verify_d128_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status) {
    __shared__ int s_par[kMaxN];
    __shared__ unsigned long long s_leafmask[2];
    __shared__ int s_bad;
    __shared__ float s_k[4][kD], s_bk[4][kD], s_q[4][kD];   // per wave: k, beta k, q of the node
    __shared__ int s_path[4][kMaxN];                         // per wave: the branch, root first

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int m = l & 31, h = l >> 5, col = 32 * w + m;
    const int bh = blockIdx.x, b = bh / H, hd = bh % H;
    const int32_t *par = parent + (size_t)b * n;

    // ---- wave 0: parents, validity and the leaf set (a leaf has no child)
    if (w == 0) {
        int p[2];
        bool bad = false;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = 64 * u + l;
            p[u] = i < n ? par[i] : -1;
            if (i < n) {
                s_par[i] = p[u];
                if (!parent_ok(p[u], i)) bad = true;
            }
        }
        const bool any_bad = __ballot(bad) != 0ull;
        // has-child flags through LDS (one wave: its accesses complete in order)
        __shared__ int s_child[kMaxN];
#pragma unroll
        for (int u = 0; u < 2; ++u) s_child[64 * u + l] = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = 64 * u + l;
            if (i < n && !any_bad && p[u] >= 0) s_child[p[u]] = 1;
        }
        const unsigned long long m0 = __ballot(l < n && !s_child[l]);
        const unsigned long long m1 = __ballot(64 + l < n && !s_child[64 + l]);
        if (l == 0) {
            s_bad = any_bad;
            s_leafmask[0] = m0;
            s_leafmask[1] = m1;
            if (hd == 0 && blockIdx.y == 0 && status) status[b] = any_bad ? kFaultBadParent : 0;
        }
    }
    __syncthreads();
    if (s_bad) {
        if (blockIdx.y == 0) {
            float *orow = out + ((size_t)b * n * H + hd) * kD + col;
            for (int i = h; i < n; i += 2) orow[(size_t)i * H * kD] = __builtin_nanf("");
        }
        return;
    }
    const unsigned long long lm0 = s_leafmask[0], lm1 = s_leafmask[1];
    const int nleaves = __popcll(lm0) + __popcll(lm1);
    const float *slab = S0 + (size_t)bh * kD * kD;
    const size_t node0 = (size_t)b * n * H + hd;   // (node 0, head) row index

    for (int rank = blockIdx.y; rank < nleaves; rank += gridDim.y) {
        // leaf of this rank (id order): the rank-th set bit of the mask
        int leaf;
        {
            const int c0 = __popcll(lm0);
            unsigned long long mm = rank < c0 ? lm0 : lm1;
            int rr = rank < c0 ? rank : rank - c0;
            for (; rr > 0; --rr) mm &= mm - 1;
            leaf = __builtin_ctzll(mm) + (rank < c0 ? 0 : 64);
        }
        // the branch root..leaf into this wave's path slots (lane 0 walks up;
        // one wave's LDS accesses complete in order)
        int depth = 0;
        for (int j = leaf; s_par[j] >= 0; j = s_par[j]) ++depth;
        if (l == 0)
            for (int j = leaf, t = depth; t >= 0; j = s_par[j], --t) s_path[w][t] = j;

        // node inputs of this lane: gates, k and q entries l and 64 + l, v at col
        struct NodeIn {
            float a, be, k0, k1, q0, q1, vc;
        };
        auto fetch = [&](int t) {
            const size_t row = node0 + (size_t)s_path[w][t] * H;
            const T *kr = k + row * kD, *qr = q + row * kD;
            return NodeIn{alpha[row],      beta[row],        ld_f32(kr, l),
                          ld_f32(kr, 64 + l), ld_f32(qr, l), ld_f32(qr, 64 + l),
                          ld_f32(v + row * kD, col)};
        };
        f32x16 st[4];
        NodeIn nx = fetch(0);
        load_state(st, slab, col, h);
        for (int t = 0; t <= depth; ++t) {
            const NodeIn cur = nx;
            if (t < depth) nx = fetch(t + 1);   // the next node's inputs are in flight meanwhile
            const size_t row = node0 + (size_t)s_path[w][t] * H;
            const float a = cur.a, vc = cur.vc;
            // this wave's copies of k, beta k and q (one wave: in-order LDS)
            s_k[w][l] = cur.k0;
            s_k[w][64 + l] = cur.k1;
            s_bk[w][l] = cur.be * cur.k0;
            s_bk[w][64 + l] = cur.be * cur.k1;
            s_q[w][l] = cur.q0;
            s_q[w][64 + l] = cur.q1;
            // w = S^T k: this lane's 64 rows (four independent partial sums),
            // then the other half of the column
            float wp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 k4 = *reinterpret_cast<const float4 *>(&s_k[w][32 * qq + 8 * g + 4 * h]);
                    wp[0] = fmaf(st[qq][4 * g + 0], k4.x, wp[0]);
                    wp[1] = fmaf(st[qq][4 * g + 1], k4.y, wp[1]);
                    wp[2] = fmaf(st[qq][4 * g + 2], k4.z, wp[2]);
                    wp[3] = fmaf(st[qq][4 * g + 3], k4.w, wp[3]);
                }
            const float wl = (wp[0] + wp[1]) + (wp[2] + wp[3]);
            const float wc = wl + __shfl_xor(wl, 32);
            // S <- alpha (S - beta k w^T) + beta k v^T = alpha S + (beta k)(v - alpha w)
            const float cf = vc - a * wc;
            float opp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 k4 = *reinterpret_cast<const float4 *>(&s_bk[w][32 * qq + 8 * g + 4 * h]);
                    const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[w][32 * qq + 8 * g + 4 * h]);
                    const float kk[4] = {k4.x, k4.y, k4.z, k4.w}, qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = fmaf(kk[e], cf, a * st[qq][4 * g + e]);
                        st[qq][4 * g + e] = x;
                        opp[e] = fmaf(x, qv[e], opp[e]);
                    }
                }
            const float op = (opp[0] + opp[1]) + (opp[2] + opp[3]);
            const float o = op + __shfl_xor(op, 32);
            if (h == 0) out[row * kD + col] = o;
        }
    }
}

}  // namespace

hipError_t launch_branch_verify(const VerifyArgs &a, hipStream_t s) {
    if (a.dk == kD && a.dv == kD) {
        // eight workgroups per (sequence, head), each looping over leaf ranks
        dim3 grid((unsigned)(a.batch * a.H), 8u);
        if (a.dtype == GDN_DTYPE_BF16)
            hipLaunchKernelGGL(branch_verify_d128_kernel<uint16_t>, grid, dim3(kThreads), 0, s,
                               (const uint16_t *)a.q, (const uint16_t *)a.k,
                               (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.S0, a.out,
                               a.n, a.H, a.status);
        else
            hipLaunchKernelGGL(branch_verify_d128_kernel<float>, grid, dim3(kThreads), 0, s,
                               (const float *)a.q, (const float *)a.k, (const float *)a.v,
                               a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, a.status);
        return hipGetLastError();
    }
    // other head sizes: one workgroup per (sequence, head, leaf, 64 columns);
    // grid.y covers the largest possible leaf count (n) and workgroups past
    // a tree's own leaf count exit after the leaf scan
    dim3 grid((unsigned)(a.batch * a.H), (unsigned)a.n, (unsigned)((a.dv + kTileV - 1) / kTileV));
    if (a.dtype == GDN_DTYPE_BF16) {
        hipLaunchKernelGGL(branch_verify_kernel<uint16_t>, grid, dim3(kThreads), 0, s,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, a.dk, a.dv,
                           a.status);
    } else {
        hipLaunchKernelGGL(branch_verify_kernel<float>, grid, dim3(kThreads), 0, s,
                           (const float *)a.q, (const float *)a.k, (const float *)a.v, a.alpha,
                           a.beta, a.parent, a.S0, a.out, a.n, a.H, a.dk, a.dv, a.status);
    }
    return hipGetLastError();
}

}  // namespace gdn
