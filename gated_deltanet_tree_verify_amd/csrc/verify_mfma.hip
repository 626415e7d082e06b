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
// order.  Gram tiles are computed transposed so that each lane already holds
// the operand fragment that the solve reads back, and leaves it with one
// 16-byte LDS write.  V and the output rows move through LDS so that global
// traffic is whole-row 16-byte accesses.
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

// LDS layout (79 KB, two workgroups per CU).  The V tile is staged once and
// moved into registers before the solve blocks are built in the same bytes;
// the Q/K tiles are reused to stage the output rows.
struct SolveBlocks {
    float d[2][32][32];                        // strictly-lower X_bb (fp32); later also Z
    float tinv[4][16][16];                     // inverses of the 16x16 diagonal sub-blocks
    uint16_t th[2][32][kBL], tl[2][32][kBL];   // T_b = (I + X_bb)^{-1}, hi / lo
    uint16_t xh[32][kBL], xl[32][kBL];         // -X_10, hi / lo
    uint16_t yh[3][32][kBL], yl[3][32][kBL];   // Y_00, Y_10, Y_11, hi / lo
};
struct QKTiles {
    uint16_t q[kN][kQK];
    uint16_t k[kN][kQK];
};
struct Smem {
    union {
        QKTiles t;
        float o[kN][kD + 4];                   // output rows, staged for 16-byte stores
    } a;
    union {
        uint16_t v[kN][kQK];
        SolveBlocks s;
    } b;
    unsigned long long anc[kN];                // ancestor-or-self bitmask per node
    float g[kN];                               // log2 of the path decay product
    float eg[kN];                              // path decay product e^{g}
    float beta[kN];
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
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
    // hi = bf16(x) (round to nearest even); the residual x - hi is exact in
    // fp32 and comes out of one dot2 per element: (-1, 0).(hi0, hi1) + x0.
    // The (-1, 0) and (0, -1) pairs are kept in scalar registers: written as
    // constants, the compiler encodes one of them as the inline float
    // constant -1.0, which the dot2 instruction reads as a different bf16
    // pair (checked on gfx950: every lane wrong).
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t n0b, n1b;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(n0b));
    asm("s_mov_b32 %0, 0xbf800000" : "=s"(n1b));
    const bf16x2 n0 = __builtin_bit_cast(bf16x2, n0b);
    const bf16x2 n1 = __builtin_bit_cast(bf16x2, n1b);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x2 h2 = {static_cast<__bf16>(x[2 * j]), static_cast<__bf16>(x[2 * j + 1])};
        const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h2, n0, x[2 * j], false);
        const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h2, n1, x[2 * j + 1], false);
        const bf16x2 l2 = {static_cast<__bf16>(r0), static_cast<__bf16>(r1)};
        hw[j] = __builtin_bit_cast(uint32_t, h2);
        lw[j] = __builtin_bit_cast(uint32_t, l2);
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void st8(uint16_t *p, const bf16x8 &x) {
    *reinterpret_cast<bf16x8 *>(p) = x;
}

// a 32x32 fp32 result tile as B operands: two k-steps, bf16 hi and lo
struct SplitTile {
    bf16x8 hi[2], lo[2];
};

__device__ __forceinline__ SplitTile split_tile(const f32x16 &b) {
    SplitTile t;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        float bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = b[8 * kk + j];
        split8(bv, t.hi[kk], t.lo[kk]);
    }
    return t;
}

// C += A * B for fp32 A (hi/lo blocks in LDS, permuted columns) and an fp32
// B given as a split result tile (three bf16 products per k-step)
__device__ __forceinline__ f32x16 mm3(const uint16_t (*ah)[kBL], const uint16_t (*al)[kBL],
                                      const SplitTile &b, f32x16 c, int m, int h) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a_h = lds8(&ah[m][16 * kk + 8 * h]);
        const bf16x8 a_l = lds8(&al[m][16 * kk + 8 * h]);
        c = mfma(a_h, b.hi[kk], c);
        c = mfma(a_h, b.lo[kk], c);
        c = mfma(a_l, b.hi[kk], c);
    }
    return c;
}

__global__ __launch_bounds__(kThreads, 2) void verify_mfma_n64_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int ncu, int32_t *__restrict__ status) {
    __shared__ Smem sm;
    // the wave index is uniform: keep it scalar so role branches stay scalar
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int m = l & 31, h = l >> 5;        // row / column within a 32x32 tile, lane half
    const int bh = blockIdx.x, b = bh / H, hd = bh % H;
    const int col = 32 * w + m;              // this lane's d_v column
    const size_t rstride = (size_t)H * kD;   // elements between consecutive nodes
    const size_t base = ((size_t)b * n * H + hd) * kD;   // node 0 of this (sequence, head)

    // ---- 1. loads: Q, K, V tiles (16-byte row chunks, to LDS), gates and
    //         parents (wave 3, one lane per node); then this wave's S0 slab
    int p = -1;
    float la = 0.f, bt = 0.f;
    const bool node_ok = (w == 3) && (l < n);
    if (node_ok) {
        const size_t row = ((size_t)b * n + l) * H + hd;
        p = parent[(size_t)b * n + l];
        la = alpha[row];
        bt = beta[row];
    }
    uint4 st[12];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        const size_t off = base + row * rstride + c8;
        const bool in = row < n;
        st[it] = in ? *reinterpret_cast<const uint4 *>(q + off) : make_uint4(0, 0, 0, 0);
        st[4 + it] = in ? *reinterpret_cast<const uint4 *>(k + off) : make_uint4(0, 0, 0, 0);
        st[8 + it] = in ? *reinterpret_cast<const uint4 *>(v + off) : make_uint4(0, 0, 0, 0);
    }
    if (w == 3) {
        // tree topology while the tiles are in flight (the gates were
        // requested first): pointer jumping, one lane per node; after round
        // r every node has folded in its nearest 2^(r+1) path nodes
        const bool badi = node_ok && !parent_ok(p, l);
        const unsigned long long badm = __ballot(badi);
        unsigned long long anc = node_ok ? (1ull << l) : 0ull;
        int jmp = (node_ok && !badi) ? p : -1;
        float gs = node_ok ? log2f(la) : 0.f;
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
        sm.eg[l] = node_ok ? exp2f(gs) : 0.f;
        sm.beta[l] = bt;
        if (l == 0) {
            sm.bad = badm != 0ull;
            if (hd == 0 && status) status[b] = badm ? kFaultBadParent : 0;
        }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<uint4 *>(&sm.a.t.q[row][c8]) = st[it];
        *reinterpret_cast<uint4 *>(&sm.a.t.k[row][c8]) = st[4 + it];
        *reinterpret_cast<uint4 *>(&sm.b.v[row][c8]) = st[8 + it];
    }
    __syncthreads();

    // The S0 slab is requested only after the Q/K/V tiles have landed, and
    // a wave that issues it stalls until the memory system has accepted the
    // whole slab.  The two workgroups resident on a CU (dispatch rounds r
    // and r + 1) therefore take opposite orders: one streams its state
    // first and builds the tree matrices afterwards, the other builds them
    // while its neighbour streams, then streams its own.
    const bool state_first = ((blockIdx.x / ncu) & 1) == 0;
    const float *s0p = S0 + (size_t)bh * kD * kD + col;
    float s0[8][8];     // [k-step][j]: S0 row 16 kk + 8 h + j, this lane's column
    if (state_first) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const float *rowp = s0p + (size_t)(16 * kk + 8 * h) * kD;
#pragma unroll
            for (int j = 0; j < 8; ++j) s0[kk][j] = rowp[j * kD];
        }
    }

    // ---- 2. transposed Gram tiles (waves 0-2), V -> registers
    // Wave w owns block (mt, nt) = (0,0), (1,0), (1,1) of the node x node
    // matrices and computes it transposed: lane (node i = 32 mt + m, half h)
    // holds k_s.q_i and k_s.k_i for s = 32 nt + crow(r, h), exactly the
    // operand order the solve and output products read back.
    const int mt = (w == 0) ? 0 : 1;
    const int nt = (w == 2) ? 1 : 0;
    f32x16 gc = {}, ga = {};
    if (w < 3) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 ks = lds8(&sm.a.t.k[32 * nt + m][16 * kk + 8 * h]);
            const bf16x8 qi = lds8(&sm.a.t.q[32 * mt + m][16 * kk + 8 * h]);
            const bf16x8 ki = lds8(&sm.a.t.k[32 * mt + m][16 * kk + 8 * h]);
            gc = mfma(ks, qi, gc);
            ga = mfma(ks, ki, ga);
        }
    }
    uint32_t vpk[2][8];   // V in this lane's result-tile layout, bf16 pairs
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
            vpk[t][r / 2] = (uint32_t)sm.b.v[32 * t + crow(r, h)][col] |
                            ((uint32_t)sm.b.v[32 * t + crow(r + 1, h)][col] << 16);
    __syncthreads();

    if (sm.bad) {
        float *orow = out + base + col;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * t + crow(r, h);
                if (i < n) orow[(size_t)i * rstride] = __builtin_nanf("");
            }
        return;
    }

    // ---- 3. mask + decay the Gram tiles into the X and Y blocks
    SolveBlocks &sb = sm.b.s;
    if (w < 3) {
        const int il = m, i = 32 * mt + m;
        // ancestor bits of node i inside key block nt, pre-shifted by this
        // lane half's row offset so that register r tests a constant bit
        const unsigned long long anc = sm.anc[i];
        const uint32_t mb = (uint32_t)(anc >> (32 * nt)) >> (4 * h);
        const float gi = sm.g[i], bi = sm.beta[i];
        float y[16], x[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 g4 = *reinterpret_cast<const float4 *>(&sm.g[32 * nt + 8 * q4 + 4 * h]);
            const float gs4[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                const bool star = (mb >> (8 * q4 + e)) & 1u;
                const float wt = star ? __builtin_amdgcn_exp2f(gi - gs4[e]) : 0.f;
                y[r] = wt * gc[r];
                // the diagonal of X is never read (strictly lower use only)
                x[r] = (bi * wt) * ga[r];
            }
        }
        const int yb = w;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 hi, lo;
            split8(&y[8 * kk], hi, lo);
            st8(&sb.yh[yb][il][16 * kk + 8 * h], hi);
            st8(&sb.yl[yb][il][16 * kk + 8 * h], lo);
        }
        if (w == 1) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = -x[r];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 hi, lo;
                split8(&x[8 * kk], hi, lo);
                st8(&sb.xh[il][16 * kk + 8 * h], hi);
                st8(&sb.xl[il][16 * kk + 8 * h], lo);
            }
        } else {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4 *>(&sb.d[mt][il][8 * q4 + 4 * h]) =
                    make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
        }
    }
    __syncthreads();

    // ---- 4. block inverses T_b = (I + X_bb)^{-1}, tiled: the four 16x16
    //         diagonal sub-blocks by forward substitution (wave 3, lane =
    //         sub-block, column), then T21 = -C^{-1} (B A^{-1}) by all threads
    if (w == 3) {
        const int sbk = l >> 4, c = l & 15, blk = sbk >> 1, o16 = 16 * (sbk & 1);
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int s4 = 0; s4 < r; s4 += 4) {
                const float4 xr = *reinterpret_cast<const float4 *>(&sb.d[blk][o16 + r][o16 + s4]);
                acc = fmaf(-xr.x, t[s4], acc);
                if (s4 + 1 < r) acc = fmaf(-xr.y, t[s4 + 1], acc);
                if (s4 + 2 < r) acc = fmaf(-xr.z, t[s4 + 2], acc);
                if (s4 + 3 < r) acc = fmaf(-xr.w, t[s4 + 3], acc);
            }
            t[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sb.tinv[sbk][r][c] = t[r];
    }
    __syncthreads();
    // Z_b = B_b A_b^{-1} into the upper-left sub-block of d[b] (read only by
    // the forward substitution above), two entries per thread
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int idx = tid + kThreads * u, blk = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) acc = fmaf(sb.d[blk][16 + r][s], sb.tinv[2 * blk][s][c], acc);
        sb.d[blk][r][c] = acc;
    }
    __syncthreads();
    // L_b = -C_b^{-1} Z_b into the lower-left sub-block (B_b is no longer read)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int idx = tid + kThreads * u, blk = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) acc = fmaf(sb.tinv[2 * blk + 1][r][s], sb.d[blk][s][c], acc);
        sb.d[blk][16 + r][c] = -acc;
    }
    __syncthreads();
    // T_b = [[A^-1, 0], [L, C^-1]] as bf16 hi/lo operand rows: each thread
    // fills one 8-entry chunk (permuted positions 8 seg .. 8 seg + 7, i.e.
    // columns 16 kb + 4 hb + {0..3} and 16 kb + 8 + 4 hb + {0..3})
    {
        const int blk = tid >> 7, r = (tid >> 2) & 31, seg = tid & 3, kb = seg >> 1, hb = seg & 1;
        const int c0 = 16 * kb + 4 * hb;
        float4 lo4, hi4;
        if (r < 16) {
            if (kb == 0) {
                lo4 = *reinterpret_cast<const float4 *>(&sb.tinv[2 * blk][r][c0]);
                hi4 = *reinterpret_cast<const float4 *>(&sb.tinv[2 * blk][r][c0 + 8]);
            } else {
                lo4 = hi4 = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        } else if (kb == 1) {
            lo4 = *reinterpret_cast<const float4 *>(&sb.tinv[2 * blk + 1][r - 16][c0 - 16]);
            hi4 = *reinterpret_cast<const float4 *>(&sb.tinv[2 * blk + 1][r - 16][c0 - 8]);
        } else {
            lo4 = *reinterpret_cast<const float4 *>(&sb.d[blk][r][c0]);
            hi4 = *reinterpret_cast<const float4 *>(&sb.d[blk][r][c0 + 8]);
        }
        const float vals[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
        bf16x8 th8, tl8;
        split8(vals, th8, tl8);
        st8(&sb.th[blk][r][8 * seg], th8);
        st8(&sb.tl[blk][r][8 * seg], tl8);
    }

    // ---- 5. P = Q S0 and R = K S0 for this wave's 32 columns
    if (!state_first) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const float *rowp = s0p + (size_t)(16 * kk + 8 * h) * kD;
#pragma unroll
            for (int j = 0; j < 8; ++j) s0[kk][j] = rowp[j * kD];
        }
    }
    f32x16 P[2] = {}, R[2] = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        bf16x8 sh, sl;
        split8(s0[kk], sh, sl);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 aq = lds8(&sm.a.t.q[32 * t + m][16 * kk + 8 * h]);
            const bf16x8 ak = lds8(&sm.a.t.k[32 * t + m][16 * kk + 8 * h]);
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
        for (int q4 = 0; q4 < 4; ++q4) {
            const int i0 = 32 * t + 8 * q4 + 4 * h;
            const float4 b4 = *reinterpret_cast<const float4 *>(&sm.beta[i0]);
            const float4 e4 = *reinterpret_cast<const float4 *>(&sm.eg[i0]);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                const uint32_t pr = vpk[t][r >> 1];
                const float vval = __uint_as_float((r & 1) ? (pr & 0xffff0000u) : (pr << 16));
                rhs[t][r] = bb[e] * (vval - ee[e] * R[t][r]);
                P[t][r] *= ee[e];
            }
        }
    const f32x16 zero = {};
    const f32x16 u0 = mm3(sb.th[0], sb.tl[0], split_tile(rhs[0]), zero, m, h);
    const SplitTile u0s = split_tile(u0);
    const f32x16 z1 = mm3(sb.xh, sb.xl, u0s, rhs[1], m, h);
    const f32x16 u1 = mm3(sb.th[1], sb.tl[1], split_tile(z1), zero, m, h);
    f32x16 o0 = mm3(sb.yh[0], sb.yl[0], u0s, P[0], m, h);
    f32x16 o1 = mm3(sb.yh[1], sb.yl[1], u0s, P[1], m, h);
    o1 = mm3(sb.yh[2], sb.yl[2], split_tile(u1), o1, m, h);

    // ---- 7. stage the output rows in LDS, then store whole rows
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        sm.a.o[crow(r, h)][col] = o0[r];
        sm.a.o[32 + crow(r, h)][col] = o1[r];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = tid + kThreads * it, row = e >> 5, c4 = (e & 31) * 4;
        if (row < n)
            *reinterpret_cast<float4 *>(out + base + row * rstride + c4) =
                *reinterpret_cast<const float4 *>(&sm.a.o[row][c4]);
    }
}

}  // namespace

bool verify_mfma_supports(const VerifyArgs &a) {
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n <= kN;
}

hipError_t launch_verify_mfma(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_mfma_n64_kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0,
                       s, (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H, device_cu_count(),
                       a.status);
    return hipGetLastError();
}

}  // namespace gdn
