// MFMA tree verify for small launches: bf16 q/k/v, d_k = d_v = 128, trees of
// at most 32 nodes, one two-wave workgroup per (sequence, head, quarter of
// d_v) (gfx950).
//
// Same system as tree_verify.hpp (DFlash-TfM page, section on rollback-free
// tree verification for GDN):
//     (I + X) U = beta (V - e^g (K S0)),   O = e^g (Q S0) + Y U,
// with X and Y the ancestor-masked, decay-weighted Grams.  Every d_v column
// of U and O depends only on the same column of V and S0, so the columns
// split across workgroups with no exchange; the tree matrices (Gram, masks,
// the inverse of I + X) depend on q, k and the gates alone and are formed
// again by each quarter's workgroup.
//
// Why: with one workgroup per (sequence, head), a launch of batch x H
// workgroups well below the CU count (batch 1, 32 heads) has each CU pull a
// whole 64 KiB state slab through its own memory pipeline, and the waves
// stall on issuing those loads for ~2 us before the Gram can start.  Four
// workgroups per (sequence, head) each pull a quarter of the slab (16 KiB)
// on four CUs.  In a workgroup one wave builds the tree matrices and the
// other streams the state and contracts it, so neither waits for the other
// until the solve.
//
// Lane (m = l & 31, h = l >> 5) owns d_v column 32 j + m of quarter j; the
// 32-node tree is one 32-row block: T = (I + X)^{-1} from its two 16x16
// diagonal sub-blocks (substitution), Z = B A^{-1}, L = -C^{-1} Z.
#include "internal.hpp"
#include "tree_verify.hpp"

namespace gdn {
namespace {

using namespace tile;
using tv::kBL;
using tv::kD;
using tv::kQK;

constexpr int kQuarters = 4;   // workgroups per (sequence, head)
constexpr int kN1 = 32;        // tree size handled: one 32-row block
constexpr int kLanes = 64;     // lanes of a wave
constexpr int kThreads = 128;  // two waves

struct Smem {
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

// the 16x16 diagonal sub-blocks' inverses of I + X by forward substitution
// (lane = sub-block (l >> 4) & 1, column l & 15; lanes 32.. repeat 0..31);
// row r's entries are requested two rows ahead of their use
__device__ __forceinline__ void subst16(Smem &sm, int l) {
    const int sbk = (l >> 4) & 1, cl = l & 15, o16 = 16 * sbk;
    float t[16];
    float4 xr[16][4];
#pragma unroll
    for (int r = 0; r < 16 + 2; ++r) {
        if (r < 16) {
#pragma unroll
            for (int s4 = 0; s4 < r; s4 += 4)
                xr[r][s4 / 4] = *reinterpret_cast<const float4 *>(&sm.d[o16 + r][o16 + s4]);
        }
        const int rr = r - 2;
        if (rr >= 0) {
            float acc = (rr == cl) ? 1.f : 0.f;
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
    if (l < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.tinv[sbk][r][cl] = t[r];
    }
}

// Two waves.  Wave 0: gates and Q rows, topology, the Gram tile, masks and
// T = (I + X)^{-1}.  Wave 1: K rows, then the quarter's state columns and v
// values (its stall on issuing them is off wave 0's path), P and R while
// wave 0 builds T, then the solve and the output rows.
__global__ __launch_bounds__(kThreads) void verify_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status, bool status_or) {
    __shared__ Smem sm;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = threadIdx.x & 63, m = l & 31, h = l >> 5;
    const int bh = blockIdx.x / kQuarters, quarter = blockIdx.x % kQuarters;
    const int col = 32 * quarter + m;
    const tv::Seq s = tv::seq_coords(bh, n, H);
    const uint32_t rbytes = (uint32_t)(n * s.rstride * 2);

    // ---- loads: Q (wave 0) or K (wave 1) rows 0..31 (rows past n read as
    //      zero), 16-byte chunks into LDS with d_k permuted
    uint4 x[8];
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((w == 0 ? q : k) + s.base, rbytes);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int e = l + kLanes * it, row = e >> 4, c8 = (e & 15) * 8;
            x[it] = load16(rs, (uint32_t)((row * s.rstride + c8) * 2));
        }
    }
    f32x16 st[4];
    uint32_t vpk[8];   // v of rows crow(r, h), bf16 pairs
    if (w == 0) {
        // ---- gates (lane = node), then the topology: ancestor-or-self bits
        //      and log2 decay prefix by pointer jumping (5 rounds cover 32)
        int par = -1;
        float a_l = 1.f, b_l = 0.f;
        const bool live = l < n;
        if (live) {
            const size_t row = ((size_t)s.b * n + l) * H + s.hd;
            par = parent[(size_t)s.b * n + l];
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
            sm.anc[l] = anc;
            sm.g[l] = gs;
            sm.eg[l] = live ? exp2f(gs) : 0.f;
            sm.beta[l] = b_l;
        }
        if (l == 0) sm.bad = bad;
        if (l == 0 && quarter == 0 && s.hd == 0 && status) {
            const int f = bad ? kFaultBadParent : 0;
            status[s.b] = status_or ? (status[s.b] | f) : f;
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int e = l + kLanes * it;
            store_row8_permuted(sm.q[e >> 4], (e & 15) * 8, x[it]);
        }
    } else {
        load_state(st, S0 + (size_t)bh * kD * kD, col, h);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + s.base, rbytes);
        const int rb = (int)(2 * s.rstride);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int r0 = crow(r, h);
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rv, 2 * col + r0 * rb, 0, kNT);
            const uint32_t hi =
                __builtin_amdgcn_raw_buffer_load_b16(rv, 2 * col + (r0 + 1) * rb, 0, kNT);
            vpk[r / 2] = lo | (hi << 16);
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int e = l + kLanes * it;
            store_row8_permuted(sm.k[e >> 4], (e & 15) * 8, x[it]);
        }
    }
    lds_barrier();   // Q and K rows, the topology
    if (sm.bad) {
        if (w == 1) {
            float *orow = out + s.base + col;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = crow(r, h);
                if (i < n) orow[(size_t)i * s.rstride] = __builtin_nanf("");
            }
        }
        return;
    }

    if (w == 0) {
        // ---- transposed Gram tile: lane (node i = m, h) holds k_s.q_i and
        //      k_s.k_i for s = crow(r, h)
        f32x16 gc = {}, ga = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 kr = lds8(&sm.k[m][16 * kk + 8 * h]);
            const bf16x8 qr = lds8(&sm.q[m][16 * kk + 8 * h]);
            gc = mfma(kr, qr, gc);
            ga = mfma(kr, kr, ga);
        }
        // ---- ancestor mask and decay: Y (hi / lo operand rows), X (fp32)
        {
            const uint32_t mb = sm.anc[m] >> (4 * h);
            const float gi = sm.g[m], bi = sm.beta[m];
            float y[16], xx[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 g4 = *reinterpret_cast<const float4 *>(&sm.g[8 * q4 + 4 * h]);
                const float gs4[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q4 + e;
                    const bool star = (mb >> (8 * q4 + e)) & 1u;
                    const float wt = star ? __builtin_amdgcn_exp2f(gi - gs4[e]) : 0.f;
                    y[r] = wt * gc[r];
                    xx[r] = (bi * wt) * ga[r];   // the diagonal is never read
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 hi, lo;
                split8(&y[8 * kk], hi, lo);
                st8(&sm.yh[m][16 * kk + 8 * h], hi);
                st8(&sm.yl[m][16 * kk + 8 * h], lo);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4 *>(&sm.d[m][8 * q4 + 4 * h]) =
                    make_float4(xx[4 * q4], xx[4 * q4 + 1], xx[4 * q4 + 2], xx[4 * q4 + 3]);
        }
        wave_lds_sync();
        subst16(sm, l);
        wave_lds_sync();
        // ---- Z = B A^{-1} over A (upper left), then L = -C^{-1} Z over B
        //      (lower left); lane = (row r, columns c4 .. c4 + 3)
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
                        const float4 b4 =
                            *reinterpret_cast<const float4 *>(&b[(s4 + e) * ldb + c4]);
                        acc[0] = fmaf(av[e], b4.x, acc[0]);
                        acc[1] = fmaf(av[e], b4.y, acc[1]);
                        acc[2] = fmaf(av[e], b4.z, acc[2]);
                        acc[3] = fmaf(av[e], b4.w, acc[3]);
                    }
                }
                return make_float4(acc[0], acc[1], acc[2], acc[3]);
            };
            const float4 z = row_times(&sm.d[16 + r][0], &sm.tinv[0][0][0], 16);
            *reinterpret_cast<float4 *>(&sm.d[r][c4]) = z;
            wave_lds_sync();
            const float4 lz = row_times(&sm.tinv[1][r][0], &sm.d[0][0], 32);
            *reinterpret_cast<float4 *>(&sm.d[16 + r][c4]) =
                make_float4(-lz.x, -lz.y, -lz.z, -lz.w);
        }
        wave_lds_sync();
        // ---- T = [[A^{-1}, 0], [L, C^{-1}]] as bf16 hi / lo operand rows:
        //      one 8-entry chunk (permuted positions 8 seg .. 8 seg + 7) per
        //      lane and pass
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int r = 16 * pass + (l >> 2), seg = l & 3, kb = seg >> 1, hb = seg & 1;
            const int c0 = 16 * kb + 4 * hb;
            float4 lo4, hi4;
            if (r < 16) {
                if (kb == 0) {
                    lo4 = *reinterpret_cast<const float4 *>(&sm.tinv[0][r][c0]);
                    hi4 = *reinterpret_cast<const float4 *>(&sm.tinv[0][r][c0 + 8]);
                } else {
                    lo4 = hi4 = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            } else if (kb == 1) {
                lo4 = *reinterpret_cast<const float4 *>(&sm.tinv[1][r - 16][c0 - 16]);
                hi4 = *reinterpret_cast<const float4 *>(&sm.tinv[1][r - 16][c0 - 8]);
            } else {
                lo4 = *reinterpret_cast<const float4 *>(&sm.d[r][c0]);
                hi4 = *reinterpret_cast<const float4 *>(&sm.d[r][c0 + 8]);
            }
            const float vals[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            bf16x8 th8, tl8;
            split8(vals, th8, tl8);
            st8(&sm.th[r][8 * seg], th8);
            st8(&sm.tl[r][8 * seg], tl8);
        }
        lds_barrier();   // T and Y are in; wave 1 solves
        return;
    }

    // ---- wave 1: P = Q S0 and R = K S0 for this lane's column (the state
    //      split hi / lo), while wave 0 builds T
    f32x16 P = {}, R = {};
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float sv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[j] = st[t4][8 * kk + j];
            bf16x8 sh, sl;
            split8(sv, sh, sl);
            const bf16x8 aq = lds8(&sm.q[m][32 * t4 + 16 * kk + 8 * h]);
            const bf16x8 ak = lds8(&sm.k[m][32 * t4 + 16 * kk + 8 * h]);
            P = mfma(aq, sh, P);
            P = mfma(aq, sl, P);
            R = mfma(ak, sh, R);
            R = mfma(ak, sl, R);
        }
    lds_barrier();   // T and Y are in

    // ---- U = T beta (v - e^g R), O = e^g P + Y U
    f32x16 rhs;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const int i0 = 8 * q4 + 4 * h;
        const float4 b4 = *reinterpret_cast<const float4 *>(&sm.beta[i0]);
        const float4 e4 = *reinterpret_cast<const float4 *>(&sm.eg[i0]);
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
    const f32x16 u = mm3<kBL>(sm.th, sm.tl, split_tile(rhs), zero, m, h);
    const f32x16 o = mm3<kBL>(sm.yh, sm.yl, split_tile(u), P, m, h);

    // ---- output rows of this lane's column (each store instruction writes
    //      two 128-byte row segments)
    float *orow = out + s.base + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = crow(r, h);
        if (i < n) __builtin_nontemporal_store(o[r], orow + (size_t)i * s.rstride);
    }
}

}  // namespace

bool verify_split_supports(const VerifyArgs &a) {
    // small launches only (at most two split workgroups per CU): measured at
    // 32 nodes and 32 heads against one workgroup per (sequence, head),
    // batch 1 and 2 take 7.0 us instead of 9.4, batch 4 9.2 instead of 9.9,
    // batch 8 would take 13.9 instead of 10.5
    return a.dtype == GDN_DTYPE_BF16 && a.dk == kD && a.dv == kD && a.n <= kN1 &&
           a.H <= 4096 && (long long)a.batch * a.H * kQuarters <= 2LL * device_cu_count();
}

hipError_t launch_verify_split(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_split_kernel, dim3((unsigned)(a.batch * a.H * kQuarters)),
                       dim3(kThreads), 0, s, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.alpha, a.beta, a.parent, a.S0, a.out, a.n, a.H,
                       a.status, a.status_or);
    return hipGetLastError();
}

}  // namespace gdn
