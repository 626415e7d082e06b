// Stages of the MFMA tree verify for trees of 65..128 nodes, bf16 q/k/v,
// d_k = d_v = 128 (gfx950).  Same method as tree_verify.hpp (the whole tree
// is one chunk of the delta rule: (I + X) U = beta (V - e^g (K S0)),
// O = e^g (Q S0) + Y U, DFlash-TfM page, section on rollback-free tree
// verification for GDN); the node range is four 32-row blocks, solved as
// two halves of 64 nodes:
//     half 0:  U_01 = (I + X_{01,01})^{-1} RHS_01,
//              O_01 = e^g P_01 + Y_{01,01} U_01
//     half 1:  U_23 = (I + X_{23,23})^{-1} (RHS_23 - X_{23,01} U_01),
//              O_23 = e^g P_23 + Y_{23,01} U_01 + Y_{23,23} U_23
// Each half reuses the 64-node solve blocks (tv::SolveBlocks, tv::inverse).
// This file holds the pieces: the 128-node topology, the masked Gram blocks,
// a half's right-hand side and solve; the schedule (which rows are in LDS
// when, and the cross blocks X_{23,01}, Y_{23,01}) is in tree_verify128h.hpp.
#pragma once

#include "tree_verify.hpp"

namespace gdn {
namespace tv128 {

using namespace tile;
using tv::kBL;
using tv::kD;
using tv::Lane;
using tv::Seq;
using tv::SolveBlocks;

constexpr int kN = 128;

// cross blocks (row block 2 + a, key block b), a, b in {0, 1}
struct Cross {
    uint16_t xh[2][2][32][kBL], xl[2][2][32][kBL];   // -X, hi / lo
    uint16_t yh[2][2][32][kBL], yl[2][2][32][kBL];   // Y, hi / lo
};

struct Topo {
    unsigned long long anc[kN][2];   // ancestor-or-self bitmask per node (bits 0..127)
    float g[kN];                     // log2 of the path decay product
    float eg[kN];                    // path decay product e^{g}
    float beta[kN];
    int bad;
};

// parent and gates of nodes l and 64 + l (one wave; dead nodes neutral)
struct Gates2 {
    int par[2];
    float a[2], bt[2];
    bool live[2];
};

__device__ __forceinline__ Gates2 load_gates2(const Lane &c, const Seq &s, const int32_t *parent,
                                              const float *alpha, const float *beta) {
    Gates2 g;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + c.l;
        g.live[u] = i < s.n;
        g.par[u] = -1;
        g.a[u] = 1.f;
        g.bt[u] = 0.f;
        if (g.live[u]) {
            const size_t row = ((size_t)s.b * s.n + i) * s.H + s.hd;
            g.par[u] = parent[(size_t)s.b * s.n + i];
            g.a[u] = alpha[row];
            g.bt[u] = beta[row];
        }
    }
    return g;
}

// one wave, two nodes per lane (l and 64 + l): parent validation, ancestor
// bitmasks and log2 decay prefix by pointer jumping (7 rounds cover 128).
// status[b] gets the fault flag (ORed into what is there when status_or).
__device__ __forceinline__ void topology(const Lane &c, const Seq &s, const Gates2 &gt, Topo &tp,
                                         int32_t *status, bool write_status, bool status_or) {
    int jmp[2];
    float gs[2], bt[2];
    bool live[2], badi[2];
    unsigned long long a0[2], a1[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + c.l;
        live[u] = gt.live[u];
        bt[u] = gt.bt[u];
        badi[u] = live[u] && !parent_ok(gt.par[u], i);
        jmp[u] = (live[u] && !badi[u]) ? gt.par[u] : -1;
        gs[u] = live[u] ? log2f(gt.a[u]) : 0.f;
        a0[u] = (live[u] && u == 0) ? (1ull << c.l) : 0ull;
        a1[u] = (live[u] && u == 1) ? (1ull << c.l) : 0ull;
    }
    const bool bad = (__ballot(badi[0]) | __ballot(badi[1])) != 0ull;
#pragma unroll
    for (int r = 0; r < 7; ++r) {
        // every lane publishes both of its nodes; a node fetches its jump
        // target from the lane and half that hold it
        const unsigned lo0[2] = {(unsigned)a0[0], (unsigned)a0[1]};
        const unsigned hi0[2] = {(unsigned)(a0[0] >> 32), (unsigned)(a0[1] >> 32)};
        const unsigned lo1[2] = {(unsigned)a1[0], (unsigned)a1[1]};
        const unsigned hi1[2] = {(unsigned)(a1[0] >> 32), (unsigned)(a1[1] >> 32)};
        int nj[2];
        float ng[2];
        unsigned long long na0[2], na1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int src = jmp[u] >= 0 ? jmp[u] : 64 * u + c.l;
            const int sl = src & 63;
            const bool up = src >= 64;
            const unsigned l0a = __shfl(lo0[0], sl), l0b = __shfl(lo0[1], sl);
            const unsigned h0a = __shfl(hi0[0], sl), h0b = __shfl(hi0[1], sl);
            const unsigned l1a = __shfl(lo1[0], sl), l1b = __shfl(lo1[1], sl);
            const unsigned h1a = __shfl(hi1[0], sl), h1b = __shfl(hi1[1], sl);
            const float ga = __shfl(gs[0], sl), gb = __shfl(gs[1], sl);
            const int ja = __shfl(jmp[0], sl), jb = __shfl(jmp[1], sl);
            na0[u] = ((unsigned long long)(up ? h0b : h0a) << 32) | (up ? l0b : l0a);
            na1[u] = ((unsigned long long)(up ? h1b : h1a) << 32) | (up ? l1b : l1a);
            ng[u] = up ? gb : ga;
            nj[u] = up ? jb : ja;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (jmp[u] >= 0) {
                a0[u] |= na0[u];
                a1[u] |= na1[u];
                gs[u] += ng[u];
                jmp[u] = nj[u];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + c.l;
        tp.anc[i][0] = a0[u];
        tp.anc[i][1] = a1[u];
        tp.g[i] = gs[u];
        tp.eg[i] = live[u] ? exp2f(gs[u]) : 0.f;
        tp.beta[i] = bt[u];
    }
    if (c.l == 0) {
        tp.bad = bad;
        if (write_status && status)
            status[s.b] = (status_or ? status[s.b] : 0) | (bad ? kFaultBadParent : 0);
    }
}


// ancestor mask and decay weights on a Gram block: y = Y entries, x = X
// entries (not yet negated; the diagonal of X is never read)
__device__ __forceinline__ void mask(const Lane &c, const Topo &tp, int a, int b, const f32x16 &gc,
                                     const f32x16 &ga, float (&y)[16], float (&x)[16]) {
    const int i = 32 * a + c.m, h = c.h;
    const uint32_t mb = (uint32_t)(tp.anc[i][b >> 1] >> (32 * (b & 1))) >> (4 * h);
    const float gi = tp.g[i], bi = tp.beta[i];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = *reinterpret_cast<const float4 *>(&tp.g[32 * b + 8 * q4 + 4 * h]);
        const float gs4[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            const bool star = (mb >> (8 * q4 + e)) & 1u;
            const float wt = star ? __builtin_amdgcn_exp2f(gi - gs4[e]) : 0.f;
            y[r] = wt * gc[r];
            x[r] = (bi * wt) * ga[r];
        }
    }
}

__device__ __forceinline__ void store_split(const Lane &c, const float (&v)[16],
                                            uint16_t (*hi)[kBL], uint16_t (*lo)[kBL]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8 h8, l8;
        split8(&v[8 * kk], h8, l8);
        st8(&hi[c.m][16 * kk + 8 * c.h], h8);
        st8(&lo[c.m][16 * kk + 8 * c.h], l8);
    }
}

// wave w < 3's masked block of a half ((0,0), (1,0) or (1,1)) into the
// 64-node solve blocks: Y into yh / yl [w]; X as -X_10 (hi / lo, wave 1) or
// as the fp32 diagonal block that the inverse reads (waves 0 and 2)
__device__ __forceinline__ void half_store(const Lane &c, float (&y)[16], float (&x)[16],
                                           SolveBlocks &sb) {
    const int la = c.w == 0 ? 0 : 1;
    store_split(c, y, sb.yh[c.w], sb.yl[c.w]);
    if (c.w == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = -x[r];
        store_split(c, x, sb.xh, sb.xl);
    } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(&sb.d[la][c.m][8 * q4 + 4 * c.h]) =
                make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
    }
}

// right-hand side beta (v - e^g R) and e^g P for rows 64 hf + 32 t + crow;
// vh[t] holds the v values of rows 64 hf + 32 t + crow as bf16 pairs
__device__ __forceinline__ void rhs_and_decay(const Lane &c, const Topo &tp, int hf,
                                              f32x16 (&P)[2], const f32x16 (&R)[2],
                                              const uint32_t (*vh)[8], f32x16 (&rhs)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int i0 = 64 * hf + 32 * t + 8 * q4 + 4 * c.h;
            const float4 b4 = *reinterpret_cast<const float4 *>(&tp.beta[i0]);
            const float4 e4 = *reinterpret_cast<const float4 *>(&tp.eg[i0]);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                const uint32_t pr = vh[t][r >> 1];
                const float vval = __uint_as_float((r & 1) ? (pr & 0xffff0000u) : (pr << 16));
                rhs[t][r] = bb[e] * (vval - ee[e] * R[t][r]);
                P[t][r] *= ee[e];
            }
        }
}

// the 64-node solve on prepared right-hand sides and decayed P:
// u0 = T_0 rhs0, u1 = T_1 (rhs1 - X_10 u0), o = P + Y u
__device__ __forceinline__ void solve_half(const Lane &c, const SolveBlocks &sb,
                                           const f32x16 (&rhs)[2], const f32x16 (&P)[2],
                                           f32x16 (&u)[2], f32x16 (&o)[2]) {
    const f32x16 zero = {};
    u[0] = mm3<kBL>(sb.th[0], sb.tl[0], split_tile(rhs[0]), zero, c.m, c.h);
    const SplitTile u0s = split_tile(u[0]);
    const f32x16 z1 = mm3<kBL>(sb.xh, sb.xl, u0s, rhs[1], c.m, c.h);
    u[1] = mm3<kBL>(sb.th[1], sb.tl[1], split_tile(z1), zero, c.m, c.h);
    o[0] = mm3<kBL>(sb.yh[0], sb.yl[0], u0s, P[0], c.m, c.h);
    o[1] = mm3<kBL>(sb.yh[1], sb.yl[1], u0s, P[1], c.m, c.h);
    o[1] = mm3<kBL>(sb.yh[2], sb.yl[2], split_tile(u[1]), o[1], c.m, c.h);
}

__device__ __forceinline__ void store_nan(const Lane &c, const Seq &s, float *out) {
    float *orow = out + s.base + c.col;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * t + crow(r, c.h);
            if (i < s.n) orow[(size_t)i * s.rstride] = __builtin_nanf("");
        }
}

}  // namespace tv128
}  // namespace gdn
