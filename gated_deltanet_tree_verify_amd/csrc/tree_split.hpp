// Stages of the d_v-split tree verify (bf16 q/k/v, d_k = d_v = 128, trees of
// at most 32 nodes) for small launches: several workgroups per (sequence,
// head), each owning a quarter of the d_v columns (gfx950).  Shared by the
// split verify kernel and the split fused commit-verify kernel.
//
// Same system as tree_verify.hpp (DFlash-TfM page, section on rollback-free
// tree verification for GDN):
//     (I + X) U = beta (V - e^g (K S0)),   O = e^g (Q S0) + Y U,
// with X and Y the ancestor-masked, decay-weighted Grams.  Every d_v column
// of U and O depends only on the same column of V and S0, so the columns
// split across workgroups with no exchange; the tree matrices (Gram, masks,
// the inverse of I + X) depend on q, k and the gates alone and each
// quarter's workgroup forms them again.
//
// Why: with one workgroup per (sequence, head), a launch of batch x H
// workgroups well below the CU count (batch 1, 32 heads) has each CU pull a
// whole 64 KiB state slab through its own memory pipeline, and the waves
// stall on issuing those loads for ~2 us before the Gram can start.  A
// quarter's workgroup pulls 16 KiB, and inside it one wave builds the tree
// matrices while another streams the state and contracts it.
//
// Lane (m = l & 31, h = l >> 5) of a wave owns d_v column 32 j + m of
// quarter j; the tree is one 32-row block: T = (I + X)^{-1} from its two
// 16x16 diagonal sub-blocks (substitution), Z = B A^{-1}, L = -C^{-1} Z.
#pragma once

#include "tree_verify.hpp"

namespace gdn {
namespace ts {

using namespace tile;
using tv::kBL;
using tv::kD;
using tv::kQK;

constexpr int kQuarters = 4;   // workgroups per (sequence, head)
constexpr int kN1 = 32;        // tree size handled: one 32-row block
constexpr int kLanes = 64;     // lanes of a wave

struct Tree {
    uint16_t q[kN1][kQK], k[kN1][kQK];   // d_k index permuted within 16-blocks
    float d[32][32];                     // X (strictly lower used); later Z, L
    float tinv[2][16][16];               // inverses of the diagonal sub-blocks
    uint16_t th[32][kBL], tl[32][kBL];   // T, hi / lo
    uint16_t yh[32][kBL], yl[32][kBL];   // Y, hi / lo
    uint32_t anc[kN1];                   // ancestor-or-self bits
    float g[kN1], eg[kN1], beta[kN1];    // log2 path decay, e^g, beta
    int bad;
};

// orders this wave's LDS writes before its later LDS reads by other lanes
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// rows 0..31 of a bf16 [batch][n][H][128] tensor (rows past n read as zero),
// eight 16-byte chunks per lane of one wave
__device__ __forceinline__ void load_rows32(const tv::Seq &s, const uint16_t *src, int l,
                                            uint4 (&x)[8]) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + s.base, (uint32_t)(s.n * s.rstride * 2));
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = l + kLanes * it, row = e >> 4, c8 = (e & 15) * 8;
        x[it] = load16(rs, (uint32_t)((row * s.rstride + c8) * 2));
    }
}

__device__ __forceinline__ void store_rows32(uint16_t (*dst)[kQK], int l, const uint4 (&x)[8]) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = l + kLanes * it;
        store_row8_permuted(dst[e >> 4], (e & 15) * 8, x[it]);
    }
}

// v of rows crow(r, h) in column col, bf16 pairs (rows past n read as zero)
__device__ __forceinline__ void load_v_col(const tv::Seq &s, const uint16_t *v, int col, int h,
                                           uint32_t (&vpk)[8]) {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + s.base, (uint32_t)(s.n * s.rstride * 2));
    const int rb = (int)(2 * s.rstride);
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        const int r0 = crow(r, h);
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rv, 2 * col + r0 * rb, 0, kNT);
        const uint32_t hi =
            __builtin_amdgcn_raw_buffer_load_b16(rv, 2 * col + (r0 + 1) * rb, 0, kNT);
        vpk[r / 2] = lo | (hi << 16);
    }
}

// One wave, lane = node: gates, then the ancestor-or-self bits and log2 decay
// prefix by pointer jumping (5 rounds cover 32 nodes) into LDS; returns
// whether some parent lies outside [-1, node) (also left in t.bad)
__device__ __forceinline__ bool topology(Tree &t, const tv::Seq &s, const int32_t *parent,
                                         const float *alpha, const float *beta, int l) {
    int par = -1;
    float a_l = 1.f, b_l = 0.f;
    const bool live = l < s.n;
    if (live) {
        const size_t row = ((size_t)s.b * s.n + l) * s.H + s.hd;
        par = parent[(size_t)s.b * s.n + l];
        a_l = alpha[row];
        b_l = beta[row];
    }
    const bool badi = live && !parent_ok(par, l);
    const bool bad = __ballot(badi) != 0ull;
    uint32_t anc = live ? (1u << (l & 31)) : 0u;
    int jmp = (live && !badi) ? par : -1;
    float gs = live ? log2f(a_l) : 0.f;
#pragma unroll
    for (int r = 0; r < 5; ++r) {
        const int src = jmp >= 0 ? jmp : l;
        const uint32_t a2 = __shfl(anc, src);
        const float g2 = __shfl(gs, src);
        const int j2 = __shfl(jmp, src);
        if (jmp >= 0) {
            anc |= a2;
            gs += g2;
            jmp = j2;
        }
    }
    if (l < kN1) {
        t.anc[l] = anc;
        t.g[l] = gs;
        t.eg[l] = live ? exp2f(gs) : 0.f;
        t.beta[l] = b_l;
    }
    if (l == 0) t.bad = bad;
    return bad;
}

// One wave: the transposed Gram tile (lane (node i = m, h) holds k_s.q_i and
// k_s.k_i for s = crow(r, h)), then the ancestor mask and decay: Y as hi /
// lo operand rows, X as fp32 rows (the Q / K tiles and topology in LDS)
__device__ __forceinline__ void gram_mask(Tree &t, int m, int h) {
    f32x16 gc = {}, ga = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 kr = lds8(&t.k[m][16 * kk + 8 * h]);
        const bf16x8 qr = lds8(&t.q[m][16 * kk + 8 * h]);
        gc = mfma(kr, qr, gc);
        ga = mfma(kr, kr, ga);
    }
    const uint32_t mb = t.anc[m] >> (4 * h);
    const float gi = t.g[m], bi = t.beta[m];
    float y[16], x[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = *reinterpret_cast<const float4 *>(&t.g[8 * q4 + 4 * h]);
        const float gs4[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            const bool star = (mb >> (8 * q4 + e)) & 1u;
            const float wt = star ? __builtin_amdgcn_exp2f(gi - gs4[e]) : 0.f;
            y[r] = wt * gc[r];
            x[r] = (bi * wt) * ga[r];   // the diagonal is never read
        }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8 hi, lo;
        split8(&y[8 * kk], hi, lo);
        st8(&t.yh[m][16 * kk + 8 * h], hi);
        st8(&t.yl[m][16 * kk + 8 * h], lo);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4 *>(&t.d[m][8 * q4 + 4 * h]) =
            make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
}

// One wave (X written and visible to it): T = (I + X)^{-1} as bf16 hi / lo
// operand rows, in two parts.  inverse_subst: the diagonal sub-blocks by
// forward substitution (lane = sub-block (l >> 4) & 1, column l & 15, lanes
// 32.. repeating 0..31; row r's entries requested two rows ahead of their
// use).  inverse_finish (the sub-block inverses visible): Z = B A^{-1} over A
// and L = -C^{-1} Z over B (lane = row, four columns), then the split.
__device__ __forceinline__ void inverse_subst(Tree &t, int l) {
    {
        const int sbk = (l >> 4) & 1, cl = l & 15, o16 = 16 * sbk;
        float tv[16];
        float4 xr[16][4];
#pragma unroll
        for (int r = 0; r < 16 + 2; ++r) {
            if (r < 16) {
#pragma unroll
                for (int s4 = 0; s4 < r; s4 += 4)
                    xr[r][s4 / 4] = *reinterpret_cast<const float4 *>(&t.d[o16 + r][o16 + s4]);
            }
            const int rr = r - 2;
            if (rr >= 0) {
                float acc = (rr == cl) ? 1.f : 0.f;
#pragma unroll
                for (int s4 = 0; s4 < rr; s4 += 4) {
                    const float4 x4 = xr[rr][s4 / 4];
                    acc = fmaf(-x4.x, tv[s4], acc);
                    if (s4 + 1 < rr) acc = fmaf(-x4.y, tv[s4 + 1], acc);
                    if (s4 + 2 < rr) acc = fmaf(-x4.z, tv[s4 + 2], acc);
                    if (s4 + 3 < rr) acc = fmaf(-x4.w, tv[s4 + 3], acc);
                }
                tv[rr] = acc;
            }
        }
        if (l < 32) {
#pragma unroll
            for (int r = 0; r < 16; ++r) t.tinv[sbk][r][cl] = tv[r];
        }
    }
}

__device__ __forceinline__ void inverse_finish(Tree &t, int l) {
    {
        const int r = l >> 2, c4 = 4 * (l & 3);
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
        const float4 z = row_times(&t.d[16 + r][0], &t.tinv[0][0][0], 16);
        *reinterpret_cast<float4 *>(&t.d[r][c4]) = z;
        wave_lds_sync();
        const float4 lz = row_times(&t.tinv[1][r][0], &t.d[0][0], 32);
        *reinterpret_cast<float4 *>(&t.d[16 + r][c4]) = make_float4(-lz.x, -lz.y, -lz.z, -lz.w);
    }
    wave_lds_sync();
    // one 8-entry chunk (permuted positions 8 seg .. 8 seg + 7) per lane and pass
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int r = 16 * pass + (l >> 2), seg = l & 3, kb = seg >> 1, hb = seg & 1;
        const int c0 = 16 * kb + 4 * hb;
        float4 lo4, hi4;
        if (r < 16) {
            if (kb == 0) {
                lo4 = *reinterpret_cast<const float4 *>(&t.tinv[0][r][c0]);
                hi4 = *reinterpret_cast<const float4 *>(&t.tinv[0][r][c0 + 8]);
            } else {
                lo4 = hi4 = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        } else if (kb == 1) {
            lo4 = *reinterpret_cast<const float4 *>(&t.tinv[1][r - 16][c0 - 16]);
            hi4 = *reinterpret_cast<const float4 *>(&t.tinv[1][r - 16][c0 - 8]);
        } else {
            lo4 = *reinterpret_cast<const float4 *>(&t.d[r][c0]);
            hi4 = *reinterpret_cast<const float4 *>(&t.d[r][c0 + 8]);
        }
        const float vals[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
        bf16x8 th8, tl8;
        split8(vals, th8, tl8);
        st8(&t.th[r][8 * seg], th8);
        st8(&t.tl[r][8 * seg], tl8);
    }
}

__device__ __forceinline__ void inverse(Tree &t, int l) {
    inverse_subst(t, l);
    wave_lds_sync();
    inverse_finish(t, l);
}

// P = Q S and R = K S for this lane's column, the slab split hi / lo (the
// same products in the same order as tv::contract_tile)
__device__ __forceinline__ void contract(const Tree &t, const f32x16 (&st)[4], int m, int h,
                                         f32x16 &P, f32x16 &R) {
    P = R = f32x16{};
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float sv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[j] = st[t4][8 * kk + j];
            bf16x8 sh, sl;
            split8(sv, sh, sl);
            const bf16x8 aq = lds8(&t.q[m][32 * t4 + 16 * kk + 8 * h]);
            const bf16x8 ak = lds8(&t.k[m][32 * t4 + 16 * kk + 8 * h]);
            P = mfma(aq, sh, P);
            P = mfma(aq, sl, P);
            R = mfma(ak, sh, R);
            R = mfma(ak, sl, R);
        }
}

// U = T beta (v - e^g R), O = e^g P + Y U (T and Y in LDS)
__device__ __forceinline__ void solve(const Tree &t, const uint32_t (&vpk)[8], f32x16 P,
                                      const f32x16 &R, int m, int h, f32x16 &u, f32x16 &o) {
    f32x16 rhs;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const int i0 = 8 * q4 + 4 * h;
        const float4 b4 = *reinterpret_cast<const float4 *>(&t.beta[i0]);
        const float4 e4 = *reinterpret_cast<const float4 *>(&t.eg[i0]);
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            const uint32_t pr = vpk[r >> 1];
            const float vval = __uint_as_float((r & 1) ? (pr & 0xffff0000u) : (pr << 16));
            rhs[r] = bb[e] * (vval - ee[e] * R[r]);
            P[r] *= ee[e];
        }
    }
    const f32x16 zero = {};
    u = mm3<kBL>(t.th, t.tl, split_tile(rhs), zero, m, h);
    o = mm3<kBL>(t.yh, t.yl, split_tile(u), P, m, h);
}

// rows i = crow(r, h) < n of column col of an fp32 [batch][n][H][128] tensor
// (each store instruction writes two 128-byte row segments)
__device__ __forceinline__ void store_col(const tv::Seq &s, float *dst, int col, int h,
                                          const f32x16 &x) {
    float *p = dst + s.base + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = crow(r, h);
        if (i < s.n) __builtin_nontemporal_store(x[r], p + (size_t)i * s.rstride);
    }
}

// the same for an fp16 tensor, rounded to nearest
__device__ __forceinline__ void store_col_f16(const tv::Seq &s, uint16_t *dst, int col, int h,
                                              const f32x16 &x) {
    uint16_t *p = dst + s.base + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = crow(r, h);
        if (i < s.n) p[(size_t)i * s.rstride] = f16_bits(x[r]);
    }
}

}  // namespace ts
}  // namespace gdn
