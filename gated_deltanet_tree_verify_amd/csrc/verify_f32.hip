// Tree verify for all-fp32 q/k/v, d_k = d_v = 128, n <= 64 (gfx950), on the
// fp32 matrix instruction v_mfma_f32_32x32x2_f32: every product is an fp32
// product, so the path holds the all-fp32 accuracy gate, which bf16 hi / lo
// splits of fp32 inputs do not (their dropped lo x lo term is ~2^-16).
//
// Same system and work split as the bf16 verify (tree_verify.hpp; DFlash-TfM
// page, section on rollback-free tree verification for GDN):
//     (I + X) U = beta (V - e^g (K S0)),   O = e^g (Q S0) + Y U,
// solved over two 32-row node blocks, U_0 = T_0 RHS_0, U_1 = T_1 (RHS_1 -
// X_10 U_0), T_b = (I + X_bb)^{-1}.  One workgroup per (sequence, head),
// wave w owning d_v columns [32 w, 32 w + 32); S0 is only read.
//
// Operands.  The 32x32x2 instruction takes one value per lane for A (row
// l & 31, contraction slot l >> 5) and one for B (column l & 31, the same
// slot); its result has the layout of mfma_tile.hpp (register r of lane
// (col, h) holds row crow(r, h)).  A result tile fed back as B supplies, at
// step t, its register t, i.e. row crow(t, h) of its 32-block; so every A
// operand row keeps its 32-block contraction index c at position pos32(c),
// where crow(t, h) lands at 16 h + t, and a lane reads its sixteen values
// contiguously.  The Gram tiles take both operands from LDS rows and pair
// positions 64 h .. 64 h + 63 on both sides.
//   1. Q and K rows into LDS (16-byte loads, positions pos128); wave 3: the
//      gates and the topology (tv::topology);
//   2. waves 0-2: transposed Gram tiles K_s . Q_i and K_s . K_i of node
//      blocks (0,0), (1,0), (1,1) -> masked, decay-weighted Y blocks and
//      -X_10 (A-operand rows of node i) and the diagonal X blocks (natural
//      layout); wave 3: P = Q S0 for its columns;
//   3. wave 3: T_0 and T_1 by forward substitution (one lane per column),
//      then R = K S0; waves 0-2: P and R;
//   4. all: RHS = beta (V - e^g R), the block solve, O = e^g P + Y U, the
//      output columns stored row by row.
// LDS ~105 KB: one workgroup per CU.
#include "internal.hpp"
#include "tree_verify.hpp"

namespace gdn {
namespace {

using namespace tile;
using tv::kD;
using tv::kN;
using tv::Lane;
using tv::Seq;

constexpr int kThreads = 256;   // four waves
constexpr int kRS = kD + 4;     // LDS row stride of the 128-wide Q / K rows (floats)
constexpr int kBS = 32 + 4;     // LDS row stride of the 32-wide operand blocks

struct Smem {
    float q[kN][kRS];        // row i of Q, column c at position pos128(c)
    float k[kN][kRS];
    float y[3][32][kBS];     // Y_00, Y_10, Y_11: row i, column s at pos32(s)
    float nx10[32][kBS];     // -X_10, same layout
    float t[2][32][kBS];     // T_0, T_1, same layout
    float xd[2][32][kBS];    // X_00, X_11 as [i][s] (strictly lower part read)
    tv::Topo tp;
};

static_assert(sizeof(Smem) <= 160 * 1024, "fits one CU's LDS");

// position of contraction index c (0..31) in an A-operand row: row crow(t, h)
// of a result tile lands at 16 h + t
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

// 64 fp32 rows of one (sequence, head) into an LDS tile: 16-byte chunks
// (four columns c..c+3, which stay adjacent under pos128); rows past n lie
// past the buffer resource's end and read as zero
__device__ __forceinline__ void load_rows_f32(const Lane &c, const Seq &s, const float *src,
                                              float4 (&x)[8]) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + s.base, (uint32_t)(s.n * s.rstride * 4));
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 5, c4 = (e & 31) * 4;
        x[it] = __builtin_bit_cast(float4, load16(rs, (uint32_t)((row * s.rstride + c4) * 4)));
    }
}

__device__ __forceinline__ void store_rows_f32(const Lane &c, const float4 (&x)[8],
                                               float (*dst)[kRS]) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int e = c.tid + kThreads * it, row = e >> 5, c4 = (e & 31) * 4;
        *reinterpret_cast<float4 *>(&dst[row][pos128(c4)]) = x[it];
    }
}

// waves 0-2: node block (mt, nt) = (0,0), (1,0), (1,1); lane (node i =
// 32 mt + m, h), register r: s = 32 nt + crow(r, h), gc = k_s . q_i,
// ga = k_s . k_i (the tiles transposed, so that lane i holds row i of Y
// and X)
__device__ __forceinline__ void gram(const Lane &c, const Smem &sm, int mt, int nt, f32x16 &gc,
                                     f32x16 &ga) {
    gc = f32x16{};
    ga = f32x16{};
    const float *ka = &sm.k[32 * nt + c.m][64 * c.h];
    const float *qb = &sm.q[32 * mt + c.m][64 * c.h];
    const float *kb = &sm.k[32 * mt + c.m][64 * c.h];
#pragma unroll 4
    for (int j4 = 0; j4 < 16; ++j4) {
        const float4 a4 = lds4(&ka[4 * j4]), q4 = lds4(&qb[4 * j4]), k4 = lds4(&kb[4 * j4]);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w}, qv[4] = {q4.x, q4.y, q4.z, q4.w},
                    kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gc = mfma32(av[e], qv[e], gc);
            ga = mfma32(av[e], kv[e], ga);
        }
    }
}

// ancestor mask and decay weights on a Gram tile, stored as A-operand rows:
// Y (ancestor-or-self) into y[w], X (strict ancestors) as -X_10 (wave 1) or
// into the natural-layout diagonal block (waves 0 and 2)
__device__ __forceinline__ void mask_store(const Lane &c, Smem &sm, int mt, int nt,
                                           const f32x16 &gc, const f32x16 &ga) {
    const int i = 32 * mt + c.m;
    const uint32_t mb = (uint32_t)(sm.tp.anc[i] >> (32 * nt)) >> (4 * c.h);
    const float gi = sm.tp.g[i], bi = sm.tp.beta[i];
    float y[16], x[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = lds4(&sm.tp.g[32 * nt + 8 * q4 + 4 * c.h]);
        const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            const bool star = (mb >> (8 * q4 + e)) & 1u;
            const float wt = star ? __builtin_amdgcn_exp2f(gi - gs[e]) : 0.f;
            y[r] = wt * gc[r];
            x[r] = (bi * wt) * ga[r];   // the diagonal is never read
        }
    }
    // register r is column s_local = crow(r, h), i.e. position 16 h + r
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4 *>(&sm.y[c.w][c.m][16 * c.h + 4 * q4]) =
            make_float4(y[4 * q4], y[4 * q4 + 1], y[4 * q4 + 2], y[4 * q4 + 3]);
    if (c.w == 1) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(&sm.nx10[c.m][16 * c.h + 4 * q4]) =
                make_float4(-x[4 * q4], -x[4 * q4 + 1], -x[4 * q4 + 2], -x[4 * q4 + 3]);
    } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(&sm.xd[mt][c.m][8 * q4 + 4 * c.h]) =
                make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
    }
}

// wave 3: T_b = (I + X_bb)^{-1}, lane (b = l >> 5, column j = l & 31):
// T[i][j] = [i == j] - sum_{s < i} X[i][s] T[s][j], row by row; column j
// then goes to position pos32(j) of the A-operand rows of T_b
__device__ __forceinline__ void inverse(const Lane &c, Smem &sm) {
    const int b = c.l >> 5, j = c.l & 31;
    const float(*x)[kBS] = sm.xd[b];
    float t[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < i; ++s) acc = fmaf(-x[i][s], t[s], acc);
        t[i] = acc;
    }
    const int pj = pos32(j);
#pragma unroll
    for (int i = 0; i < 32; ++i) sm.t[b][i][pj] = t[i];
}

// this wave's columns of X S0 for node blocks 0 and 1 (X = Q or K rows):
// state tile q enters as B (its register t is row 32 q + crow(t, h)), the
// rows as A from positions 32 q + 16 h + t
__device__ __forceinline__ void contract(const Lane &c, const float (*rows)[kRS],
                                         const f32x16 (&st)[4], f32x16 (&acc)[2]) {
    acc[0] = acc[1] = f32x16{};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const float4 a0 = lds4(&rows[c.m][32 * q + 16 * c.h + 4 * t4]);
            const float4 a1 = lds4(&rows[32 + c.m][32 * q + 16 * c.h + 4 * t4]);
            const float v0[4] = {a0.x, a0.y, a0.z, a0.w}, v1[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[0] = mfma32(v0[e], st[q][4 * t4 + e], acc[0]);
                acc[1] = mfma32(v1[e], st[q][4 * t4 + e], acc[1]);
            }
        }
}

// c_out = A B + c_in for a 32x32 A-operand block (rows m, positions 16 h + t)
// and a result tile B
__device__ __forceinline__ f32x16 mm_blk(const Lane &c, const float (*a)[kBS], const f32x16 &bt,
                                         f32x16 acc) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
        const float4 a4 = lds4(&a[c.m][16 * c.h + 4 * t4]);
        acc = mfma32(a4.x, bt[4 * t4], acc);
        acc = mfma32(a4.y, bt[4 * t4 + 1], acc);
        acc = mfma32(a4.z, bt[4 * t4 + 2], acc);
        acc = mfma32(a4.w, bt[4 * t4 + 3], acc);
    }
    return acc;
}

__global__ __launch_bounds__(kThreads, 1) void verify_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const int32_t *__restrict__ parent, const float *__restrict__ S0, float *__restrict__ out,
    int n, int H, int32_t *__restrict__ status, bool status_or) {
    __shared__ Smem sm;
    const Lane c = tv::lane_coords();
    const Seq s = tv::seq_coords(blockIdx.x, n, H);

    // ---- 1. rows, gates, topology, state slab
    const tv::Gates gt = tv::load_gates(c, s, parent, alpha, beta);
    float4 rq[8], rk[8];
    load_rows_f32(c, s, q, rq);
    load_rows_f32(c, s, k, rk);
    if (c.w == 3) {
        tv::topology(c, s, gt, sm.tp, status, false);
        if (c.l == 0 && s.hd == 0 && status) {
            const int f = sm.tp.bad ? kFaultBadParent : 0;
            status[s.b] = status_or ? (status[s.b] | f) : f;
        }
    }
    store_rows_f32(c, rq, sm.q);
    store_rows_f32(c, rk, sm.k);
    f32x16 st[4];
    load_state(st, S0 + (size_t)blockIdx.x * kD * kD, c.col, c.h);
    lds_barrier();

    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + s.base, (uint32_t)(s.n * s.rstride * 4));
    if (sm.tp.bad) {
        // rows past n lie past the resource's end: their stores are dropped
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(
                    0x7fc00000u, ro,
                    (int)(((32 * t + tile::crow(r, c.h)) * s.rstride + c.col) * 4), 0, kNT);
        return;
    }

    // ---- 2. Gram tiles and masks (waves 0-2); P for wave 3
    f32x16 P[2], R[2];
    if (c.w < 3) {
        const int mt = tv::gram_mt(c.w), nt = tv::gram_nt(c.w);
        f32x16 gc, ga;
        gram(c, sm, mt, nt, gc, ga);
        mask_store(c, sm, mt, nt, gc, ga);
    } else {
        contract(c, sm.q, st, P);
    }
    // v values of this lane's column, rows 32 t + crow(r, h) (rows past n
    // read as zero), needed after the contraction
    float vv[2][16];
    {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + s.base, (uint32_t)(s.n * s.rstride * 4));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                vv[t][r] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(
                               rv, (int)(((32 * t + tile::crow(r, c.h)) * s.rstride + c.col) * 4),
                               0, kNT));
    }
    lds_barrier();   // X and Y blocks in

    // ---- 3. T (wave 3), the rest of the contraction
    if (c.w < 3) {
        contract(c, sm.q, st, P);
    } else {
        inverse(c, sm);
    }
    contract(c, sm.k, st, R);
    lds_barrier();   // T in

    // ---- 4. right-hand side, solve, output
    f32x16 rhs[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int i0 = 32 * t + 8 * q4 + 4 * c.h;
            const float4 b4 = lds4(&sm.tp.beta[i0]);
            const float4 e4 = lds4(&sm.tp.eg[i0]);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                rhs[t][r] = bb[e] * (vv[t][r] - ee[e] * R[t][r]);
                P[t][r] *= ee[e];
            }
        }
    const f32x16 zero = {};
    const f32x16 u0 = mm_blk(c, sm.t[0], rhs[0], zero);
    const f32x16 z1 = mm_blk(c, sm.nx10, u0, rhs[1]);
    const f32x16 u1 = mm_blk(c, sm.t[1], z1, zero);
    f32x16 o[2];
    o[0] = mm_blk(c, sm.y[0], u0, P[0]);
    o[1] = mm_blk(c, sm.y[2], u1, mm_blk(c, sm.y[1], u0, P[1]));
    // each element through a scalar temporary: passed to the store builtin
    // straight from the vector, the compiler stored element 0 sixteen times
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = o[t][r];
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(x), ro,
                (int)(((32 * t + tile::crow(r, c.h)) * s.rstride + c.col) * 4), 0, kNT);
        }
}

}  // namespace

bool verify_f32_supports(const VerifyArgs &a) {
    // byte extents of a head's rows must fit the 32-bit buffer ranges
    return a.dtype == GDN_DTYPE_F32 && a.dk == kD && a.dv == kD && a.n <= kN && a.H <= 4096;
}

hipError_t launch_verify_f32(const VerifyArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(verify_f32_kernel, dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0, s,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, a.alpha,
                       a.beta, a.parent, a.S0, a.out, a.n, a.H, a.status, a.status_or);
    return hipGetLastError();
}

}  // namespace gdn
