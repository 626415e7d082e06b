// Stages of the MFMA tree verify for one (sequence, head), bf16 q/k/v,
// d_k = d_v = 128, n <= 64; shared by the verify kernel and the fused
// commit-verify kernel.
//
// Method (DFlash-TfM page, section on rollback-free tree verification for
// GDN): the whole tree is one chunk of the delta-rule recurrence.  With g_i
// the log-decay summed over the root..i path and pseudo-values u,
//     (I + X) U = beta (V - e^g (K S0)),  X_is = beta_i e^{g_i-g_s} k_i.k_s  (s strict ancestor of i)
//     O = e^g (Q S0) + Y U,               Y_is = e^{g_i-g_s} q_i.k_s         (s ancestor-or-self)
// X and Y are the ancestor-masked, decay-weighted Gram matrices; S0 is only
// read.  (The page's right-hand side beta V is the S0 = 0 case; the S0 term
// rides in the right-hand side here.)  The solve is a tiled forward
// substitution over two 32-row blocks, U_0 = T_0 RHS_0, U_1 = T_1 (RHS_1 -
// X_10 U_0), with T_b = (I + X_bb)^{-1} built from 16x16 pieces.
//
// Work split: four waves, wave w owning d_v columns [32w, 32w + 32).  The
// state slab of a wave is four 32x32 result tiles (rows of S0), so Q and K
// are stored with their d_k index permuted (see mfma_tile.hpp) and the slab
// feeds Q S0 and K S0 directly.  Gram tiles are computed transposed, so each
// lane ends up holding the operand fragment that the solve reads back.
#pragma once

#include "device_common.hpp"
#include "mfma_tile.hpp"

namespace gdn {
namespace tv {

using namespace tile;

constexpr int kN = 64;          // tree size handled (padded)
constexpr int kD = 128;         // d_k = d_v
constexpr int kThreads = 256;   // four waves
constexpr int kQK = kD + 8;     // LDS row stride of the Q/K/V tiles (bf16)
constexpr int kBL = 40;         // LDS row stride of 32x32 operand blocks (bf16)

struct QKTiles {
    uint16_t q[kN][kQK];        // d_k index permuted within 16-blocks
    uint16_t k[kN][kQK];
};

struct SolveBlocks {
    float d[2][32][32];                        // X_bb (strictly lower used); later Z, L
    float tinv[4][16][16];                     // inverses of the 16x16 diagonal sub-blocks
    uint16_t th[2][32][kBL], tl[2][32][kBL];   // T_b = (I + X_bb)^{-1}, hi / lo
    uint16_t xh[32][kBL], xl[32][kBL];         // -X_10, hi / lo
    uint16_t yh[3][32][kBL], yl[3][32][kBL];   // Y_00, Y_10, Y_11, hi / lo
};

struct Topo {
    unsigned long long anc[kN];                // ancestor-or-self bitmask per node
    float g[kN];                               // log2 of the path decay product
    float eg[kN];                              // path decay product e^{g}
    float beta[kN];
    int bad;
};

struct Lane {
    int tid, w, l, m, h, col;
};

__device__ __forceinline__ Lane lane_coords() {
    Lane c;
    c.tid = threadIdx.x;
    // the wave index is uniform: keep it scalar so role branches stay scalar
    c.w = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    c.l = c.tid & 63;
    c.m = c.l & 31;
    c.h = c.l >> 5;
    c.col = 32 * c.w + c.m;
    return c;
}

// (sequence, head) coordinates of a [batch][n][H][128] tensor
struct Seq {
    int b, hd, n, H;
    size_t base;      // element offset of node 0
    size_t rstride;   // elements between consecutive nodes
};

__device__ __forceinline__ Seq seq_coords(int bh, int n, int H) {
    Seq s;
    s.b = bh / H;
    s.hd = bh % H;
    s.n = n;
    s.H = H;
    s.rstride = (size_t)H * kD;
    s.base = ((size_t)s.b * n * H + s.hd) * kD;
    return s;
}

// gates and parent of node l (wave 3 lanes; other lanes return neutral values)
struct Gates {
    int p;
    float a, bt;
    bool ok;
};

__device__ __forceinline__ Gates load_gates(const Lane &c, const Seq &s, const int32_t *parent,
                                            const float *alpha, const float *beta) {
    Gates g{-1, 1.f, 0.f, (c.w == 3) && (c.l < s.n)};
    if (g.ok) {
        const size_t row = ((size_t)s.b * s.n + c.l) * s.H + s.hd;
        g.p = parent[(size_t)s.b * s.n + c.l];
        g.a = alpha[row];
        g.bt = beta[row];
    }
    return g;
}

// wave 3: parent validation, ancestor bitmasks and log2 decay prefix by
// pointer jumping (one lane per node; after round r every node has folded
// in its nearest 2^(r+1) path nodes).  Writes status[b] when write_status.
__device__ __forceinline__ void topology(const Lane &c, const Seq &s, const Gates &g, Topo &tp,
                                         int32_t *status, bool write_status) {
    const bool badi = g.ok && !parent_ok(g.p, c.l);
    const unsigned long long badm = __ballot(badi);
    unsigned long long anc = g.ok ? (1ull << c.l) : 0ull;
    int jmp = (g.ok && !badi) ? g.p : -1;
    float gs = g.ok ? log2f(g.a) : 0.f;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        const int src = jmp >= 0 ? jmp : c.l;
        const unsigned lo = __shfl((unsigned)anc, src), hi = __shfl((unsigned)(anc >> 32), src);
        const float g2 = __shfl(gs, src);
        const int j2 = __shfl(jmp, src);
        if (jmp >= 0) {
            anc |= ((unsigned long long)hi << 32) | lo;
            gs += g2;
            jmp = j2;
        }
    }
    tp.anc[c.l] = anc;
    tp.g[c.l] = gs;
    tp.eg[c.l] = g.ok ? exp2f(gs) : 0.f;
    tp.beta[c.l] = g.bt;
    if (c.l == 0) {
        tp.bad = badm != 0ull;
        if (write_status && status) status[s.b] = badm ? kFaultBadParent : 0;
    }
}

// 64 node rows of one (sequence, head) of a bf16 [batch][n][H][128] tensor:
// four 16-byte chunks per thread; rows past n lie past the end of the buffer
// resource and read as zero
// (kAux: the cache policy, non-temporal unless a caller reads the rows again)
template <int kAux = kNT>
__device__ __forceinline__ void load_rows(const Lane &c, const Seq &s, const uint16_t *src,
                                          uint4 (&x)[4]) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + s.base, (uint32_t)(s.n * s.rstride * 2));
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        x[it] = load16<kAux>(rs, (uint32_t)((row * s.rstride + c8) * 2));
    }
}

__device__ __forceinline__ void store_rows_permuted(const Lane &c, const uint4 (&x)[4],
                                                    uint16_t (*dst)[kQK]) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        store_row8_permuted(dst[row], c8, x[it]);
    }
}

__device__ __forceinline__ void store_rows(const Lane &c, const uint4 (&x)[4],
                                           uint16_t (*dst)[kQK]) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<uint4 *>(&dst[row][c8]) = x[it];
    }
}

// waves 0-2: block (mt, nt) = (0,0), (1,0), (1,1) of K Q^T and K K^T, i.e.
// transposed: lane (node i = 32 mt + m, h) holds k_s.q_i and k_s.k_i for
// s = 32 nt + crow(r, h)
__device__ __forceinline__ int gram_mt(int w) { return w == 0 ? 0 : 1; }
__device__ __forceinline__ int gram_nt(int w) { return w == 2 ? 1 : 0; }

__device__ __forceinline__ void gram(const Lane &c, const QKTiles &t, f32x16 &gc, f32x16 &ga) {
    const int mt = gram_mt(c.w), nt = gram_nt(c.w);
    gc = f32x16{};
    ga = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ks = lds8(&t.k[32 * nt + c.m][16 * kk + 8 * c.h]);
        const bf16x8 qi = lds8(&t.q[32 * mt + c.m][16 * kk + 8 * c.h]);
        const bf16x8 ki = lds8(&t.k[32 * mt + c.m][16 * kk + 8 * c.h]);
        gc = mfma(ks, qi, gc);
        ga = mfma(ks, ki, ga);
    }
}

// V values of this lane's two result tiles, as bf16 pairs
__device__ __forceinline__ void v_to_regs(const Lane &c, const uint16_t (*v)[kQK],
                                          uint32_t (&vpk)[2][8]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
            vpk[t][r / 2] = (uint32_t)v[32 * t + crow(r, c.h)][c.col] |
                            ((uint32_t)v[32 * t + crow(r + 1, c.h)][c.col] << 16);
}

// waves 0-2: ancestor mask and decay weights on the Gram tiles -> Y blocks
// (bf16 hi/lo operand rows), -X_10 (hi/lo) and the diagonal X blocks (fp32)
__device__ __forceinline__ void mask(const Lane &c, const Topo &tp, const f32x16 &gc,
                                     const f32x16 &ga, SolveBlocks &sb) {
    const int mt = gram_mt(c.w), nt = gram_nt(c.w);
    const int il = c.m, i = 32 * mt + c.m, h = c.h;
    // ancestor bits of node i inside key block nt, pre-shifted by this lane
    // half's row offset so that register r tests a constant bit
    const unsigned long long anc = tp.anc[i];
    const uint32_t mb = (uint32_t)(anc >> (32 * nt)) >> (4 * h);
    const float gi = tp.g[i], bi = tp.beta[i];
    float y[16], x[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = *reinterpret_cast<const float4 *>(&tp.g[32 * nt + 8 * q4 + 4 * h]);
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
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8 hi, lo;
        split8(&y[8 * kk], hi, lo);
        st8(&sb.yh[c.w][il][16 * kk + 8 * h], hi);
        st8(&sb.yl[c.w][il][16 * kk + 8 * h], lo);
    }
    if (c.w == 1) {
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

// All threads.  T_b = (I + X_bb)^{-1}, tiled: the four 16x16 diagonal
// sub-blocks by forward substitution (wave 3, lane = sub-block, column),
// Z_b = B_b A_b^{-1}, L_b = -C_b^{-1} Z_b, then T_b = [[A^-1, 0], [L, C^-1]]
// as bf16 hi/lo operand rows.  Starts and ends with the caller's barriers
// around it; contains three of its own.
// The parts of inverse(): the substitution is wave 3's alone, so the other
// waves may do other work in between; after inverse_zl the T rows area
// (th / tl) has not been written yet, so a caller may keep other data there
// until inverse_split, which starts with a barrier.
__device__ __forceinline__ void inverse_subst(const Lane &c, SolveBlocks &sb);
__device__ __forceinline__ void inverse_zl(const Lane &c, SolveBlocks &sb);
__device__ __forceinline__ void inverse_split(const Lane &c, SolveBlocks &sb);

__device__ __forceinline__ void inverse_finish(const Lane &c, SolveBlocks &sb) {
    inverse_zl(c, sb);
    inverse_split(c, sb);
}

__device__ __forceinline__ void inverse(const Lane &c, SolveBlocks &sb) {
    inverse_subst(c, sb);
    inverse_finish(c, sb);
}

__device__ __forceinline__ void inverse_subst(const Lane &c, SolveBlocks &sb) {
    if (c.w == 3) {
        const int sbk = c.l >> 4, col = c.l & 15, blk = sbk >> 1, o16 = 16 * (sbk & 1);
        float t[16];
        // row r's entries are requested two rows ahead of their use, so the
        // chain of rows waits on arithmetic rather than on LDS latency
        float4 xr[16][4];
#pragma unroll
        for (int r = 0; r < 16 + 2; ++r) {
            if (r < 16) {
#pragma unroll
                for (int s4 = 0; s4 < r; s4 += 4)
                    xr[r][s4 / 4] = *reinterpret_cast<const float4 *>(&sb.d[blk][o16 + r][o16 + s4]);
            }
            const int rr = r - 2;
            if (rr >= 0) {
                float acc = (rr == col) ? 1.f : 0.f;
#pragma unroll
                for (int s4 = 0; s4 < rr; s4 += 4) {
                    const float4 x4 = xr[rr][s4 / 4];
                    acc = fmaf(-x4.x, t[s4], acc);
                    if (s4 + 1 < rr) acc = fmaf(-x4.y, t[s4 + 1], acc);
                    if (s4 + 2 < rr) acc = fmaf(-x4.z, t[s4 + 2], acc);
                    if (s4 + 3 < rr) acc = fmaf(-x4.w, t[s4 + 3], acc);
                }
                t[rr] = acc;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sb.tinv[sbk][r][col] = t[r];
    }
}
__device__ __forceinline__ void inverse_zl(const Lane &c, SolveBlocks &sb) {
    // one thread per (block, row, four columns): rows of the left factor and
    // of the right one are read four entries at a time
    const int blk = (c.tid >> 6) & 1, r = (c.tid >> 2) & 15, c4 = 4 * (c.tid & 3);
    const bool zl = c.tid < 128;
    // a: 16 entries of one row; b: 16 rows, ldb floats apart, columns c4..c4+3
    auto row_times = [&](const float *a, const float *b, int ldb) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 16; s4 += 4) {
            const float4 a4 = *reinterpret_cast<const float4 *>(&a[s4]);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&b[(s4 + e) * ldb + c4]);
                acc[0] = fmaf(av[e], b4.x, acc[0]);
                acc[1] = fmaf(av[e], b4.y, acc[1]);
                acc[2] = fmaf(av[e], b4.z, acc[2]);
                acc[3] = fmaf(av[e], b4.w, acc[3]);
            }
        }
        return make_float4(acc[0], acc[1], acc[2], acc[3]);
    };
    lds_barrier();
    // Z_b = B_b A_b^-1 into the upper-left sub-block of d[b] (read only by
    // the substitution); B_b is the lower-left sub-block
    if (zl) {
        const float4 z = row_times(&sb.d[blk][16 + r][0], &sb.tinv[2 * blk][0][0], 16);
        *reinterpret_cast<float4 *>(&sb.d[blk][r][c4]) = z;
    }
    lds_barrier();
    // L_b = -C_b^-1 Z_b into the lower-left sub-block (B_b is no longer read)
    if (zl) {
        const float4 x = row_times(&sb.tinv[2 * blk + 1][r][0], &sb.d[blk][0][0], 32);
        *reinterpret_cast<float4 *>(&sb.d[blk][16 + r][c4]) = make_float4(-x.x, -x.y, -x.z, -x.w);
    }
}

__device__ __forceinline__ void inverse_split(const Lane &c, SolveBlocks &sb) {
    lds_barrier();
    {
        // one 8-entry chunk per thread: permuted positions 8 seg .. 8 seg + 7,
        // i.e. columns 16 kb + 4 hb + {0..3} and 16 kb + 8 + 4 hb + {0..3}
        const int blk = c.tid >> 7, r = (c.tid >> 2) & 31, seg = c.tid & 3, kb = seg >> 1,
                  hb = seg & 1;
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
}

// One state tile's share of P = Q S0 and R = K S0 for this wave's 32
// columns: tile q holds rows 32 q .. 32 q + 31 of S0, i.e. contraction
// indices 32 q .. 32 q + 31; it enters as the B operand, split hi/lo.  P and
// R accumulate, so the tiles may be taken one at a time as they arrive;
// taken in order 0..3 the sums are the same as contract()'s.  NT: the
// number of 32-row node blocks formed (1 when the tree has at most 32 nodes:
// the second block's rows are all zero).
template <int NT = 2>
__device__ __forceinline__ void contract_tile(const Lane &c, const QKTiles &t, const f32x16 &stq,
                                              int q, f32x16 (&P)[2], f32x16 (&R)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        float sv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = stq[8 * kk + j];
        bf16x8 sh, sl;
        split8(sv, sh, sl);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const bf16x8 aq = lds8(&t.q[32 * tt + c.m][32 * q + 16 * kk + 8 * c.h]);
            const bf16x8 ak = lds8(&t.k[32 * tt + c.m][32 * q + 16 * kk + 8 * c.h]);
            P[tt] = mfma(aq, sh, P[tt]);
            P[tt] = mfma(aq, sl, P[tt]);
            R[tt] = mfma(ak, sh, R[tt]);
            R[tt] = mfma(ak, sl, R[tt]);
        }
    }
}

// P = Q S0 and R = K S0 for this wave's 32 columns from the whole slab
// (four result tiles of S0 rows); NT as for contract_tile
template <int NT = 2>
__device__ __forceinline__ void contract(const Lane &c, const QKTiles &t, const f32x16 (&st)[4],
                                         f32x16 (&P)[2], f32x16 (&R)[2],
                                         float *store_slab = nullptr) {
    P[0] = P[1] = R[0] = R[1] = f32x16{};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        contract_tile<NT>(c, t, st[q], q, P, R);
        // optionally write the state tile back as soon as it has been read,
        // spreading the slab's stores over the contraction
        if (store_slab) store_state_tile(st[q], q, store_slab, c.col, c.h);
    }
}

// The solve in two halves, one per 32-row block, so that the first block's
// rows can be stored while the second block is still being solved.
// solve_block0: right-hand sides of both blocks (block 1's kept in the
// carry), U_0 = T_0 RHS_0 and O_0 = e^g P_0 + Y_00 U_0; P is scaled by e^g
// in place.  solve_block1: U_1 = T_1 (RHS_1 - X_10 U_0) and
// O_1 = e^g P_1 + Y_10 U_0 + Y_11 U_1.
struct SolveCarry {
    f32x16 rhs1;
    SplitTile u0s;
};

__device__ __forceinline__ void solve_block0(const Lane &c, const Topo &tp, const SolveBlocks &sb,
                                             f32x16 (&P)[2], const f32x16 (&R)[2],
                                             const uint32_t (&vpk)[2][8], f32x16 &u0,
                                             f32x16 &o0, SolveCarry &cy) {
    f32x16 rhs[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int i0 = 32 * t + 8 * q4 + 4 * c.h;
            const float4 b4 = *reinterpret_cast<const float4 *>(&tp.beta[i0]);
            const float4 e4 = *reinterpret_cast<const float4 *>(&tp.eg[i0]);
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
    u0 = mm3<kBL>(sb.th[0], sb.tl[0], split_tile(rhs[0]), zero, c.m, c.h);
    cy.u0s = split_tile(u0);
    cy.rhs1 = rhs[1];
    o0 = mm3<kBL>(sb.yh[0], sb.yl[0], cy.u0s, P[0], c.m, c.h);
}

__device__ __forceinline__ void solve_block1(const Lane &c, const SolveBlocks &sb,
                                             const f32x16 (&P)[2], const SolveCarry &cy,
                                             f32x16 &u1, f32x16 &o1) {
    const f32x16 zero = {};
    const f32x16 z1 = mm3<kBL>(sb.xh, sb.xl, cy.u0s, cy.rhs1, c.m, c.h);
    u1 = mm3<kBL>(sb.th[1], sb.tl[1], split_tile(z1), zero, c.m, c.h);
    o1 = mm3<kBL>(sb.yh[1], sb.yl[1], cy.u0s, P[1], c.m, c.h);
    o1 = mm3<kBL>(sb.yh[2], sb.yl[2], split_tile(u1), o1, c.m, c.h);
}

// Rows row0 .. row0 + 31 of one or two [batch][n][H][128] outputs, from a
// 32-row result tile each, through LDS as whole rows: tile a goes to the fp32
// dst_a through staging rows 0..31, tile b (when kPair) to dst_b through rows
// 32..63, as fp32 or, with kHalfB, as fp16 rounded to nearest (256-byte
// rows).  Contains one barrier; the staging area must be free.
template <bool kPair, bool kHalfB = false>
__device__ __forceinline__ void store_block(const Lane &c, const Seq &s, float (*ostage)[kD + 4],
                                            const f32x16 &a, float *dst_a, const f32x16 &b,
                                            void *dst_b, int row0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ostage[crow(r, c.h)][c.col] = a[r];
        if constexpr (kPair) ostage[32 + crow(r, c.h)][c.col] = b[r];
    }
    lds_barrier();
    constexpr int kFullRows = (kPair && !kHalfB) ? 64 : 32;   // rows stored as fp32
#pragma unroll
    for (int it = 0; it < kFullRows / 8; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 5, c4 = (e & 31) * 4;
        const int node = row0 + (row & 31);
        float *dst = (kPair && row >= 32) ? static_cast<float *>(dst_b) : dst_a;
        if (node < s.n)
            store16(dst + s.base + node * s.rstride + c4,
                    *reinterpret_cast<const float4 *>(&ostage[row][c4]));
    }
    if constexpr (kPair && kHalfB) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = c.tid + kThreads * it, row = e >> 4, c8 = (e & 15) * 8;
            const int node = row0 + row;
            const float4 x0 = *reinterpret_cast<const float4 *>(&ostage[32 + row][c8]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&ostage[32 + row][c8 + 4]);
            const uint4 h = make_uint4(
                (uint32_t)f16_bits(x0.x) | ((uint32_t)f16_bits(x0.y) << 16),
                (uint32_t)f16_bits(x0.z) | ((uint32_t)f16_bits(x0.w) << 16),
                (uint32_t)f16_bits(x1.x) | ((uint32_t)f16_bits(x1.y) << 16),
                (uint32_t)f16_bits(x1.z) | ((uint32_t)f16_bits(x1.w) << 16));
            if (node < s.n)
                store16h(static_cast<uint16_t *>(dst_b) + s.base + node * s.rstride + c8, h);
        }
    }
}

// NaN rows of an fp16 [batch][n][H][128] tensor (this lane's entries)
__device__ __forceinline__ void store_nan_f16(const Lane &c, const Seq &s, uint16_t *out) {
    uint16_t *orow = out + s.base + c.col;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * t + crow(r, c.h);
            if (i < s.n) orow[(size_t)i * s.rstride] = 0x7e00;   // quiet NaN
        }
}

// NaN rows for a sequence whose tree is malformed (this lane's entries)
__device__ __forceinline__ void store_nan(const Lane &c, const Seq &s, float *out) {
    float *orow = out + s.base + c.col;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * t + crow(r, c.h);
            if (i < s.n) orow[(size_t)i * s.rstride] = __builtin_nanf("");
        }
}

}  // namespace tv
}  // namespace gdn
