// State commit along the accepted branch for fp32 k/v, d_k = d_v = 128
// (gfx950), on the fp32 matrix instruction v_mfma_f32_32x32x2_f32.
//
// The accepted branch is a chain, so up to 32 of its nodes at a time form
// one chunk of the delta rule (DFlash-TfM page, section on rollback-free
// tree verification for GDN: commitment is deferred until the branch is
// known).  With S the state before the chunk, g_j the log-decay prefix
// along the chunk and g_l its last value,
//     X_js = beta_j e^{g_j - g_s} k_j . k_s  (s < j),   T = (I + X)^{-1},
//     U = T (beta (V - e^{g} (K_p S))),
//     S <- e^{g_l} S + K_p^T W,   W_j = e^{g_l - g_j} u_j,
// which is the per-node recurrence S <- alpha (S - beta k k^T S) + beta k v^T
// applied node by node.  One workgroup per (sequence, head), wave w owning
// d_v columns [32 w, 32 w + 32); the state stays in registers across chunks
// and is read and written once.  Operand layout as in verify_f32.hip: an
// A-operand row keeps its 32-block contraction index c at position pos32(c),
// so that a result tile (register t = row crow(t, h)) feeds in as B.
//   per chunk: every thread loads the chunk's key rows (as A rows of K_p and
//   transposed, as A rows of K_p^T) and its column's v values, wave 0 the
//   gates and their prefix; wave 1 forms the path Gram and X while waves 0,
//   2 and 3 contract R = K_p S, then wave 0 forms T by forward substitution
//   while wave 1 contracts its R; then every wave forms U, W and the update
//   of its columns.
#include "internal.hpp"
#include "path_commit.hpp"
#include "tree_verify.hpp"

namespace gdn {
namespace {

using namespace tile;
using tv::kD;

constexpr int kThreads = 256;    // four waves
constexpr int kC = 32;           // path nodes per chunk
constexpr int kRS = kD + 4;      // LDS row stride of the 128-wide key rows (floats)
constexpr int kBS = 32 + 4;      // LDS row stride of the 32-wide operand blocks

struct Smem {
    float kp[kC][kRS];      // key rows of the chunk, column c at position pos128(c)
    float kt[kD][kBS];      // the same keys transposed: row c, node j at pos32(j)
    float xd[kC][kBS];      // X as [j][s] (strictly lower part read)
    float t[kC][kBS];       // T, row i, column j at pos32(j)
    float g[kC], eg[kC], bt[kC];
    float gl;               // the chunk's last decay prefix
    pc::PathIds pi;
};

static_assert(sizeof(Smem) <= 64 * 1024, "three workgroups per CU");

__device__ __forceinline__ int pos32(int c) {
    return 16 * ((c >> 2) & 1) + 4 * (c >> 3) + (c & 3);
}
__device__ __forceinline__ int pos128(int c) { return 32 * (c >> 5) + pos32(c & 31); }

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 lds4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}

// acc + A B for a 32-wide A-operand block (rows m, positions 16 h + t) and a
// result tile B
__device__ __forceinline__ f32x16 mm_blk(const float (*a)[kBS], int m, int h, const f32x16 &bt,
                                         f32x16 acc) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
        const float4 a4 = lds4(&a[m][16 * h + 4 * t4]);
        acc = mfma32(a4.x, bt[4 * t4], acc);
        acc = mfma32(a4.y, bt[4 * t4 + 1], acc);
        acc = mfma32(a4.z, bt[4 * t4 + 2], acc);
        acc = mfma32(a4.w, bt[4 * t4 + 3], acc);
    }
    return acc;
}

__global__ __launch_bounds__(kThreads, 2) void commit_f32_kernel(
    float *__restrict__ S, const int32_t *__restrict__ path, const int32_t *__restrict__ path_len,
    int max_path, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, int n, int H, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int m = l & 31, h = l >> 5;
    const int bh = blockIdx.x, b = bh / H, hd = bh % H;
    const int col = 32 * w + m;
    const int mlen = path_len[b];

    if (w == 0) {
        const bool ok = pc::validate_and_keep(sm.pi, parent + (size_t)b * n,
                                              path + (size_t)b * max_path, mlen, max_path, n, l);
        if (l == 0) {
            sm.pi.ok = ok;
            if (hd == 0 && status) status[b] = ok ? 0 : kFaultBadPath;
        }
    }
    lds_barrier();
    if (!sm.pi.ok || mlen == 0) return;

    float *slab = S + (size_t)bh * kD * kD;
    f32x16 st[4];
    load_state(st, slab, col, h);

    // rows of this (sequence, head): node i's row at i * rstride; ids of a
    // valid path are below n, inside the resources
    const size_t rstride = (size_t)H * kD;
    const size_t base = ((size_t)b * n * H + hd) * kD;
    const uint32_t bytes = (uint32_t)(n * rstride * 4);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base, bytes);

    for (int c0 = 0; c0 < mlen; c0 += kC) {
        const int mc = min(kC, mlen - c0);
        // ---- the chunk's key rows and this lane's v values (rows past the
        //      chunk: zero), wave 0 the gates and their prefix
        float4 kx[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = tid + kThreads * it, j = e >> 5, c4 = (e & 31) * 4;
            kx[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < mc)
                kx[it] = __builtin_bit_cast(
                    float4, load16(rk, (uint32_t)((sm.pi.pid[c0 + j] * rstride + c4) * 4)));
        }
        float vv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = crow(r, h);
            vv[r] = 0.f;
            if (j < mc)
                vv[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rv, (int)((sm.pi.pid[c0 + j] * rstride + col) * 4), 0, kNT));
        }
        if (w == 0) {
            // lane j < 32: node c0 + j; past the chunk alpha = 1, beta = 0
            float lg = 0.f, be = 0.f;
            if (l < mc) {
                const size_t row = ((size_t)b * n + sm.pi.pid[c0 + l]) * H + hd;
                lg = log2f(alpha[row]);
                be = beta[row];
            }
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                const float up = __shfl_up(lg, off);
                if ((l & 31) >= off) lg += up;
            }
            if (l < kC) {
                sm.g[l] = lg;
                sm.eg[l] = exp2f(lg);
                sm.bt[l] = be;
            }
            if (l == mc - 1) sm.gl = lg;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = tid + kThreads * it, j = e >> 5, c4 = (e & 31) * 4;
            *reinterpret_cast<float4 *>(&sm.kp[j][pos128(c4)]) = kx[it];
            const int pj = pos32(j);
            sm.kt[c4][pj] = kx[it].x;
            sm.kt[c4 + 1][pj] = kx[it].y;
            sm.kt[c4 + 2][pj] = kx[it].z;
            sm.kt[c4 + 3][pj] = kx[it].w;
        }
        lds_barrier();

        // ---- wave 1: the path Gram and X while waves 0, 2 and 3 contract
        //      R = K_p S; then wave 0: T while wave 1 contracts its R
        f32x16 R = {};
        auto contract_r = [&]() {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    const float4 a4 = lds4(&sm.kp[m][32 * q + 16 * h + 4 * t4]);
                    R = mfma32(a4.x, st[q][4 * t4], R);
                    R = mfma32(a4.y, st[q][4 * t4 + 1], R);
                    R = mfma32(a4.z, st[q][4 * t4 + 2], R);
                    R = mfma32(a4.w, st[q][4 * t4 + 3], R);
                }
        };
        if (w == 1) {
            // transposed: lane (node j = m, h), register r: s = crow(r, h)
            f32x16 ga = {};
            const float *ka = &sm.kp[m][64 * h];
#pragma unroll 4
            for (int j4 = 0; j4 < 16; ++j4) {
                const float4 a4 = lds4(&ka[4 * j4]);
                // both operands are key rows: A row s = m, B row j = m
                ga = mfma32(a4.x, a4.x, ga);
                ga = mfma32(a4.y, a4.y, ga);
                ga = mfma32(a4.z, a4.z, ga);
                ga = mfma32(a4.w, a4.w, ga);
            }
            const float gj = sm.g[m], bj = sm.bt[m];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 g4 = lds4(&sm.g[8 * q4 + 4 * h]);
                const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 8 * q4 + 4 * h + e;
                    x[e] = s < m ? bj * __builtin_amdgcn_exp2f(gj - gs[e]) * ga[4 * q4 + e] : 0.f;
                }
                *reinterpret_cast<float4 *>(&sm.xd[m][8 * q4 + 4 * h]) =
                    make_float4(x[0], x[1], x[2], x[3]);
            }
        } else {
            contract_r();
        }
        lds_barrier();   // X in
        if (w == 0) {
            if (h == 0) {
                // lane m: column j = m of T, (I + X) T = I row by row
                float t[32];
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    float acc = (i == m) ? 1.f : 0.f;
#pragma unroll
                    for (int s = 0; s < i; ++s) acc = fmaf(-sm.xd[i][s], t[s], acc);
                    t[i] = acc;
                }
                const int pj = pos32(m);
#pragma unroll
                for (int i = 0; i < 32; ++i) sm.t[i][pj] = t[i];
            }
        } else if (w == 1) {
            contract_r();
        }
        lds_barrier();   // T in

        // ---- U = T beta (V - e^g R), W = e^{g_l - g} U, S <- e^{g_l} S + K_p^T W
        f32x16 rhs;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 b4 = lds4(&sm.bt[8 * q4 + 4 * h]);
            const float4 e4 = lds4(&sm.eg[8 * q4 + 4 * h]);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                rhs[r] = bb[e] * (vv[r] - ee[e] * R[r]);
            }
        }
        const f32x16 U = mm_blk(sm.t, m, h, rhs, f32x16{});
        const float gl = sm.gl, egl = exp2f(gl);
        f32x16 W;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 g4 = lds4(&sm.g[8 * q4 + 4 * h]);
            const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                W[4 * q4 + e] = __builtin_amdgcn_exp2f(gl - gs[e]) * U[4 * q4 + e];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) st[q] = mm_blk(&sm.kt[32 * q], m, h, W, st[q] * egl);
        lds_barrier();   // the chunk's LDS is free for the next one
    }
    store_state(st, slab, col, h);
}

}  // namespace

bool commit_f32_supports(const CommitArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_F32 && a.dk == kD && a.dv == kD && a.H <= 4096 &&
           a.n <= pc::kMaxPath;
}

hipError_t launch_commit_f32(const CommitArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(commit_f32_kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0, s,
                       a.S, a.path, a.path_len, a.max_path, (const float *)a.k,
                       (const float *)a.v, a.alpha, a.beta, a.parent, a.n, a.H, a.status);
    return hipGetLastError();
}

}  // namespace gdn
