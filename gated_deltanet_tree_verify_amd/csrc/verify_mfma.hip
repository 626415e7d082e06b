// MFMA tree-verify kernel for bf16 q/k/v, d_k = d_v = 128, n <= 64 (gfx950).
//
// Method (DFlash-TfM page, section on rollback-free tree verification for
// GDN): the whole tree is one chunk of the delta-rule recurrence.  With
// g_i the log-decay summed over the root..i path and pseudo-values u,
//     (I + X) U = beta (V - e^g (K S0)),  X_is = beta_i e^{g_i-g_s} k_i.k_s  (s strict ancestor of i)
//     O = e^g (Q S0) + Y U,               Y_is = e^{g_i-g_s} q_i.k_s         (s ancestor-or-self)
// X and Y are the ancestor-masked, decay-weighted Gram matrices; S0 is only
// read.  (The page's right-hand side beta V is the S0 = 0 case; the S0 term
// rides in the right-hand side here.)  The solve is a tiled forward
// substitution over two 32-row blocks:
//     U_0 = T_0 RHS_0,  U_1 = T_1 (RHS_1 - X_10 U_0),  T_b = (I + X_bb)^{-1}.
//
// One workgroup per (sequence, head); four waves, wave w owning d_v columns
// [32w, 32w + 32).  Dense contractions run on v_mfma_f32_32x32x16_bf16:
//   * Gram Q K^T and K K^T (bf16 inputs are exact, fp32 accumulation),
//   * Q S0 and K S0 with the fp32 state split into bf16 hi + lo
//     (relative error of the split below 2^-16),
//   * the solve and output products with fp32 operands split three ways
//     (hi*hi + hi*lo + lo*hi).
// Every intermediate n x 32 tile stays in registers: an accumulator tile in
// the 32x32 MFMA result layout is fed straight back as the B operand of the
// next product, with the A operand's columns stored in the matching permuted
// order.  Only the 64x128 Q and K tiles, the 32x32 interaction blocks and
// the block inverses live in LDS (~75 KB, two workgroups per CU).
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kN = 64;          // tree size handled (padded)
constexpr int kD = 128;         // d_k = d_v
constexpr int kThreads = 256;   // four waves
constexpr int kQK = kD + 8;     // LDS row stride of the Q/K tiles (bf16)
constexpr int kBL = 40;         // LDS row stride of 32x32 operand blocks (bf16)

struct Smem {
    uint16_t q[kN][kQK];
    uint16_t k[kN][kQK];
    float d[2][32][32];                 // strictly-lower X of the two diagonal blocks
    uint16_t th[2][32][kBL], tl[2][32][kBL];   // T_b = (I + X_bb)^{-1}, hi / lo
    uint16_t xh[32][kBL], xl[32][kBL];         // -X_10, hi / lo
    uint16_t yh[3][32][kBL], yl[3][32][kBL];   // Y_00, Y_10, Y_11, hi / lo
    unsigned long long anc[kN];                // ancestor-or-self bitmask per node
    float g[kN], eg[kN], beta[kN];
    int bad;
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// row of a 32x32 MFMA result held by lane half h in register r
__device__ __forceinline__ int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// storage position of column c of an A operand whose B operand comes from a
// result tile: bits 2 and 3 of the column index swap places
__device__ __forceinline__ int perm(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// x = hi + lo + O(2^-17 |x|), hi and lo bf16 (round to nearest even)
__device__ __forceinline__ void split_bits(float x, uint16_t &hi, uint16_t &lo) {
    const __bf16 h = static_cast<__bf16>(x);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = bf16_bits(x - static_cast<float>(h));
}

__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = static_cast<__bf16>(x[j]);
        hi[j] = h;
        lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
    }
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// C += A * B for fp32 A (hi/lo blocks in LDS, permuted columns) and an fp32
// B held as a 32x32 result tile (three bf16 products)
__device__ __forceinline__ f32x16 mm3(const uint16_t (*ah)[kBL], const uint16_t (*al)[kBL],
                                      const f32x16 &b, f32x16 c, int m, int h) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        float bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = b[8 * kk + j];
        bf16x8 bh, bl;
        split8(bv, bh, bl);
        const bf16x8 a_h = lds8(&ah[m][16 * kk + 8 * h]);
        const bf16x8 a_l = lds8(&al[m][16 * kk + 8 * h]);
        c = mfma(a_h, bh, c);
        c = mfma(a_h, bl, c);
        c = mfma(a_l, bh, c);
    }
    return c;
}

__global__ __launch_bounds__(kThreads, 2) void verify_mfma_n64_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int m = l & 31, h = l >> 5;        // row / column within a 32x32 tile, lane half
    const int bh = blockIdx.x, b = bh / H, hd = bh % H;
    const int col = 32 * w + m;              // this lane's d_v column

    // ---- 1. issue loads: Q/K tiles (to LDS), gates and parents, the S0 slab
    uint4 qk[8];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        const size_t off = (((size_t)b * n + row) * H + hd) * kD + c8;
        qk[it] = row < n ? *reinterpret_cast<const uint4 *>(q + off) : make_uint4(0, 0, 0, 0);
        qk[4 + it] = row < n ? *reinterpret_cast<const uint4 *>(k + off) : make_uint4(0, 0, 0, 0);
    }
    int p = -1;
    float la = 0.f, bt = 0.f;
    const bool node_ok = (w == 3) && (l < n);
    if (node_ok) {
        const size_t row = ((size_t)b * n + l) * H + hd;
        p = parent[(size_t)b * n + l];
        la = logf(alpha[row]);
        bt = beta[row];
    }
    const float *s0p = S0 + (size_t)bh * kD * kD + col;
    float s0[8][8];     // [k-step][j]: S0 row 16 kk + 8 h + j, this lane's column
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) s0[kk][j] = s0p[(size_t)(16 * kk + 8 * h + j) * kD];

#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<uint4 *>(&sm.q[row][c8]) = qk[it];
        *reinterpret_cast<uint4 *>(&sm.k[row][c8]) = qk[4 + it];
    }
    __syncthreads();

    // ---- 2. Gram tiles (waves 0-2) and tree topology (wave 3)
    const int mt = (w == 2) ? 1 : (w == 1 ? 1 : 0);   // tiles (0,0) (1,0) (1,1)
    const int nt = (w == 2) ? 1 : 0;
    f32x16 gc = {}, ga = {};
    if (w < 3) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 aq = lds8(&sm.q[32 * mt + m][16 * kk + 8 * h]);
            const bf16x8 ak = lds8(&sm.k[32 * mt + m][16 * kk + 8 * h]);
            const bf16x8 bk = lds8(&sm.k[32 * nt + m][16 * kk + 8 * h]);
            gc = mfma(aq, bk, gc);
            ga = mfma(ak, bk, ga);
        }
    } else {
        // pointer jumping, one lane per node: after round r every node has
        // folded in its nearest 2^(r+1) path nodes (mask bits and log decays)
        const bool badi = node_ok && !parent_ok(p, l);
        const unsigned long long badm = __ballot(badi);
        unsigned long long anc = node_ok ? (1ull << l) : 0ull;
        int jmp = (node_ok && !badi) ? p : -1;
        float gs = la;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int src = jmp >= 0 ? jmp : l;
            const unsigned lo = __shfl((unsigned)anc, src), hi = __shfl((unsigned)(anc >> 32), src);
            const float g2 = __shfl(gs, src);
            const int j2 = __shfl(jmp, src);
            if (jmp >= 0) {
                anc |= ((unsigned long long)hi << 32) | lo;
                gs += g2;
                jmp = j2;
            }
        }
        sm.anc[l] = anc;
        sm.g[l] = gs;
        sm.eg[l] = node_ok ? expf(gs) : 0.f;
        sm.beta[l] = bt;
        if (l == 0) {
            sm.bad = badm != 0ull;
            if (hd == 0 && status) status[b] = badm ? kFaultBadParent : 0;
        }
    }
    __syncthreads();

    float *orow = out + ((size_t)b * n * H + hd) * kD + col;   // + i * H * kD
    if (sm.bad) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * t + crow(r, h);
                if (i < n) orow[(size_t)i * H * kD] = __builtin_nanf("");
            }
        return;
    }

    // ---- 3. mask + decay the Gram tiles into X and Y blocks
    if (w < 3) {
        const int s = 32 * nt + m;
        const float gsv = sm.g[s];
        const int yb = (w == 0) ? 0 : (w == 1 ? 1 : 2);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int il = crow(r, h), i = 32 * mt + il;
            const bool star = (sm.anc[i] >> s) & 1ull;
            const float wt = star ? expf(sm.g[i] - gsv) : 0.f;
            const float y = wt * gc[r];
            const float x = (star && s != i) ? sm.beta[i] * wt * ga[r] : 0.f;
            uint16_t yh, yl;
            split_bits(y, yh, yl);
            sm.yh[yb][il][perm(m)] = yh;
            sm.yl[yb][il][perm(m)] = yl;
            if (w == 1) {
                uint16_t xh, xl;
                split_bits(-x, xh, xl);
                sm.xh[il][perm(m)] = xh;
                sm.xl[il][perm(m)] = xl;
            } else {
                sm.d[mt][il][m] = x;
            }
        }
    }
    // values of V in the result layout of this lane's tiles
    const uint16_t *vp = v + ((size_t)b * n * H + hd) * kD + col;
    float vv[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * t + crow(r, h);
            vv[t][r] = i < n ? to_f32(vp[(size_t)i * H * kD]) : 0.f;
        }
    __syncthreads();

    // ---- 4. block inverses T_b = (I + X_bb)^{-1} (wave 3: lane = block, column)
    if (w == 3) {
        const int blk = h, c = m;
        float t[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int s4 = 0; s4 < r; s4 += 4) {
                const float4 xr = *reinterpret_cast<const float4 *>(&sm.d[blk][r][s4]);
                acc = fmaf(-xr.x, t[s4], acc);
                if (s4 + 1 < r) acc = fmaf(-xr.y, t[s4 + 1], acc);
                if (s4 + 2 < r) acc = fmaf(-xr.z, t[s4 + 2], acc);
                if (s4 + 3 < r) acc = fmaf(-xr.w, t[s4 + 3], acc);
            }
            t[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            uint16_t th, tl;
            split_bits(t[r], th, tl);
            sm.th[blk][r][perm(c)] = th;
            sm.tl[blk][r][perm(c)] = tl;
        }
    }

    // ---- 5. P = Q S0 and R = K S0 for this wave's 32 columns
    f32x16 P[2] = {}, R[2] = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        bf16x8 sh, sl;
        split8(s0[kk], sh, sl);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 aq = lds8(&sm.q[32 * t + m][16 * kk + 8 * h]);
            const bf16x8 ak = lds8(&sm.k[32 * t + m][16 * kk + 8 * h]);
            P[t] = mfma(aq, sh, P[t]);
            P[t] = mfma(aq, sl, P[t]);
            R[t] = mfma(ak, sh, R[t]);
            R[t] = mfma(ak, sl, R[t]);
        }
    }
    __syncthreads();

    // ---- 6. right-hand side, tiled forward substitution, output
    f32x16 rhs[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * t + crow(r, h);
            rhs[t][r] = sm.beta[i] * (vv[t][r] - sm.eg[i] * R[t][r]);
            P[t][r] *= sm.eg[i];
        }
    const f32x16 zero = {};
    const f32x16 u0 = mm3(sm.th[0], sm.tl[0], rhs[0], zero, m, h);
    const f32x16 z1 = mm3(sm.xh, sm.xl, u0, rhs[1], m, h);
    const f32x16 u1 = mm3(sm.th[1], sm.tl[1], z1, zero, m, h);
    f32x16 o0 = mm3(sm.yh[0], sm.yl[0], u0, P[0], m, h);
    f32x16 o1 = mm3(sm.yh[1], sm.yl[1], u0, P[1], m, h);
    o1 = mm3(sm.yh[2], sm.yl[2], u1, o1, m, h);

#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i0 = crow(r, h), i1 = 32 + i0;
        if (i0 < n) orow[(size_t)i0 * H * kD] = o0[r];
        if (i1 < n) orow[(size_t)i1 * H * kD] = o1[r];
    }
}

}  // namespace

bool verify_mfma_supports(const VerifyArgs &a) {
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n <= kN;
}

hipError_t launch_verify_mfma(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_mfma_n64_kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0,
                       s, (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, a.status);
    return hipGetLastError();
}

}  // namespace gdn
