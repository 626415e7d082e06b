// Generic tree-verify kernel: any supported shape, fp32 or bf16 q/k/v, all
// arithmetic in fp32 on the vector ALUs.  It serves the all-fp32 dtype and
// every shape the MFMA kernel does not specialise.
//
// Method (DFlash-TfM page, section on rollback-free tree verification for
// GDN): the tree is treated as one chunk of the linear recurrence.  Writing
// the update as S_t = alpha_t S_{t-1} + k_t u_t^T with pseudo-values
// u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t), and g_i = sum of log alpha over
// the root..i path, one gets
//     (I + X) U = beta (V - e^g (K S0)),   X_is = beta_i e^{g_i-g_s} k_i.k_s
//     o_i = e^{g_i} S0^T q_i + sum_{s in anc*(i)} Y_is u_s,
//     Y_is = e^{g_i-g_s} q_i.k_s,
// with X over strict ancestors s of i and Y over ancestors-or-self.  The
// page's right-hand side beta V is the S0 = 0 case; the S0 term is carried
// in the right-hand side here.  u_s is shared by every branch through s,
// which is why one solve serves the whole tree and S0 is never written.
//
// Work split: one workgroup per (sequence, head, 64-column tile of d_v).
// Decays are kept in log space (g), so deep chains never form a product of
// alphas that underflows fp32: every weight used is e^{g_i - g_s} <= 1.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTileV = 64;
constexpr int kMaxN = GDN_MAX_NODES;
constexpr int kMaxEntries = kMaxN * (kMaxN + 1) / 2;  // sum of (depth+1) <= n(n+1)/2

template <typename T>
__device__ float dot_rows(const T *a, const T *b, int d) {
    float acc = 0.f;
    for (int r = 0; r < d; ++r) acc = fmaf(to_f32(a[r]), to_f32(b[r]), acc);
    return acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void verify_generic_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0,
    float *__restrict__ out, int n, int H, int dk, int dv,
    int32_t *__restrict__ status, bool status_or) {
    __shared__ int s_par[kMaxN], s_depth[kMaxN], s_off[kMaxN + 1];
    __shared__ float s_g[kMaxN], s_eg[kMaxN], s_beta[kMaxN];
    __shared__ float s_X[kMaxEntries], s_Y[kMaxEntries];
    __shared__ uint8_t s_idx[kMaxEntries], s_row[kMaxEntries];
    __shared__ float s_U[kMaxN * kTileV];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int c0 = blockIdx.y * kTileV;
    const bool writer = (h == 0 && blockIdx.y == 0 && tid == 0);

    // topology: validate, depth, entry offsets and the log-decay prefix g
    if (tid == 0) {
        int bad = 0, off = 0;
        for (int i = 0; i < n; ++i) {
            const int p = parent[(size_t)b * n + i];
            if (!parent_ok(p, i)) { bad = 1; break; }
            const size_t row = ((size_t)b * n + i) * H + h;
            s_par[i] = p;
            s_depth[i] = p < 0 ? 0 : s_depth[p] + 1;
            s_off[i] = off;
            off += s_depth[i] + 1;
            s_g[i] = (p < 0 ? 0.f : s_g[p]) + logf(alpha[row]);
            s_eg[i] = expf(s_g[i]);
            s_beta[i] = beta[row];
        }
        s_off[n] = off;
        s_bad = bad;
        if (writer && status) status[b] = (status_or ? status[b] : 0) | (bad ? kFaultBadParent : 0);
    }
    __syncthreads();
    if (s_bad) {
        for (int it = tid; it < n * kTileV; it += kThreads) {
            const int i = it / kTileV, c = c0 + it % kTileV;
            if (c < dv) out[(((size_t)b * n + i) * H + h) * dv + c] = __builtin_nanf("");
        }
        return;
    }

    // ancestor-or-self lists, root first: entry off[i] + depth(s) holds s
    for (int i = tid; i < n; i += kThreads) {
        for (int t = i; t >= 0; t = s_par[t]) {
            s_idx[s_off[i] + s_depth[t]] = (uint8_t)t;
            s_row[s_off[i] + s_depth[t]] = (uint8_t)i;
        }
    }
    __syncthreads();

    // interaction matrices X (strict ancestors) and Y (ancestors-or-self)
    const size_t hstride = (size_t)H;
    const int total = s_off[n];
    for (int e = tid; e < total; e += kThreads) {
        const int i = s_row[e], s = s_idx[e];
        const T *ki = k + (((size_t)b * n + i) * hstride + h) * dk;
        const T *qi = q + (((size_t)b * n + i) * hstride + h) * dk;
        const T *ks = k + (((size_t)b * n + s) * hstride + h) * dk;
        const float w = expf(s_g[i] - s_g[s]);
        s_Y[e] = w * dot_rows(qi, ks, dk);
        s_X[e] = (s == i) ? 0.f : s_beta[i] * w * dot_rows(ki, ks, dk);
    }

    // right-hand side beta_i (v_i - e^{g_i} S0^T k_i) for this column tile
    const float *s0 = S0 + (size_t)bh * dk * dv;
    for (int it = tid; it < n * kTileV; it += kThreads) {
        const int i = it / kTileV, cl = it % kTileV, c = c0 + cl;
        if (c >= dv) continue;
        const size_t row = ((size_t)b * n + i) * hstride + h;
        const T *ki = k + row * dk;
        float r = 0.f;
        for (int d = 0; d < dk; ++d) r = fmaf(to_f32(ki[d]), s0[(size_t)d * dv + c], r);
        s_U[i * kTileV + cl] = s_beta[i] * (to_f32(v[row * dv + c]) - s_eg[i] * r);
    }
    __syncthreads();

    // forward substitution in topological order, one column per thread
    if (tid < kTileV && c0 + tid < dv) {
        for (int i = 0; i < n; ++i) {
            const int o = s_off[i];
            float u = s_U[i * kTileV + tid];
            for (int t = 0; t < s_depth[i]; ++t) u = fmaf(-s_X[o + t], s_U[s_idx[o + t] * kTileV + tid], u);
            s_U[i * kTileV + tid] = u;
        }
    }
    __syncthreads();

    // output stage: e^{g_i} S0^T q_i + sum_s Y_is u_s
    for (int it = tid; it < n * kTileV; it += kThreads) {
        const int i = it / kTileV, cl = it % kTileV, c = c0 + cl;
        if (c >= dv) continue;
        const size_t row = ((size_t)b * n + i) * hstride + h;
        const T *qi = q + row * dk;
        float p = 0.f;
        for (int d = 0; d < dk; ++d) p = fmaf(to_f32(qi[d]), s0[(size_t)d * dv + c], p);
        float o = s_eg[i] * p;
        const int off = s_off[i];
        for (int t = 0; t <= s_depth[i]; ++t) o = fmaf(s_Y[off + t], s_U[s_idx[off + t] * kTileV + cl], o);
        out[row * dv + c] = o;
    }
}

}  // namespace

hipError_t launch_verify_generic(const VerifyArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.batch * a.H), (unsigned)((a.dv + kTileV - 1) / kTileV));
    if (a.dtype == GDN_DTYPE_BF16) {
        hipLaunchKernelGGL(verify_generic_kernel<uint16_t>, grid, dim3(kThreads), 0, s,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, a.dk, a.dv, a.status,
                           a.status_or);
    } else {
        hipLaunchKernelGGL(verify_generic_kernel<float>, grid, dim3(kThreads), 0, s,
                           (const float *)a.q, (const float *)a.k, (const float *)a.v,
                           a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, a.dk, a.dv, a.status,
                           a.status_or);
    }
    return hipGetLastError();
}

}  // namespace gdn
