// Stages of the MFMA state commit along an accepted branch for one
// (sequence, head), bf16 k/v, d_k = d_v = 128; shared by the commit kernel
// and the fused commit-verify kernel.
//
// The commitment is deferred until the accepted branch is known (DFlash-TfM
// page, rollback-free GDN verification section), and the branch is a chain,
// so the chunked form of the delta rule applies to it directly.  For a chunk
// of path nodes j = 0..mc-1 (chunk-local log2 decay prefix g_j) entering with
// state S:
//     R = K_p S,   (I + X) U = beta (V_p - e^g R),   X_jt = beta_j e^{g_j-g_t} k_j.k_t (t < j)
//     S <- e^{g_last} S + K_p^T W,   W_j = e^{g_last - g_j} u_j.
// This is the same state the explicit update would reach along the chunk.
// Chunks of 32 nodes are applied in order.
//
// Four waves of 32 d_v columns.  The state slab of a wave (128 rows x 32
// columns, fp32) is held in registers as four 32x32 result tiles for the
// whole commit: it is the B operand of R = K_p S (with the key rows stored
// in the matching permuted order) and the accumulator of the rank-mc update,
// so S never passes through bf16 except inside R (split hi + lo).
#pragma once

#include "device_common.hpp"
#include "mfma_tile.hpp"

namespace gdn {
namespace pc {

using namespace tile;

constexpr int kD = 128;
constexpr int kC = 32;          // path nodes per chunk
constexpr int kThreads = 256;
constexpr int kKP = kD + 8;     // row stride of the path-key / path-value tiles (bf16)
constexpr int kBL = 40;         // row stride of 32-wide operand blocks (bf16)
constexpr int kMaxPath = GDN_MAX_NODES;   // a valid path has at most n <= 128 nodes

struct ChunkTiles {
    uint16_t kp[kC][kKP];       // path keys, d_k index permuted within 16-blocks
    uint16_t vp[kC][kKP];       // path values
    float d[kC][kC];            // X of the chunk (strictly lower part used); then Z, L
    float tinv[2][16][16];      // inverses of the two 16x16 diagonal sub-blocks
    uint16_t th[kC][kBL], tl[kC][kBL];   // T = (I + X)^{-1}, hi / lo, permuted columns
    float g[kC], eg[kC], wdec[kC], beta[kC];
    float glast;
};

struct PathIds {
    int pid[kMaxPath];          // path node ids, kept from the validation pass
    int ok;
};

// A path is valid when 0 <= m <= max_path, every id is in [0, n), the first
// node is a root and each later node's parent is the previous node, with
// ids strictly increasing.  Checked by one wave, one path slot per lane, so
// the path and parent reads are two round trips rather than a chain.
__device__ inline bool path_valid_wave(const int32_t *par, const int32_t *path, int m, int max_path,
                                       int n, int lane) {
    if (m < 0 || m > max_path) return false;
    bool bad = false;
    for (int j0 = 0; j0 < m; j0 += 64) {
        const int j = j0 + lane;
        if (j < m) {
            const int id = path[j];
            const int prev = j == 0 ? -1 : path[j - 1];
            if (id < 0 || id >= n || (j > 0 && prev >= id)) bad = true;
            else if (par[id] != prev) bad = true;
        }
    }
    return __ballot(bad) == 0ull;
}

// one wave: validate the path of sequence b and keep its ids in LDS
__device__ __forceinline__ bool validate_and_keep(PathIds &pi, const int32_t *parent,
                                                  const int32_t *prow, int mlen, int max_path,
                                                  int n, int lane) {
    const bool ok = path_valid_wave(parent, prow, mlen, max_path, n, lane);
    if (ok)
        for (int j = lane; j < mlen; j += 64) pi.pid[j] = prow[j];
    return ok;
}

// A path as seen by the one wave that reads it: lane l holds the ids of slots l and
// 64 + l (-1 past the path) and, after the second round of loads, the
// parents that validate them.
struct PathLanes {
    int id0, id1;
    int par0, par1;
};

// node id of path slot j (j < 128)
__device__ __forceinline__ int slot_id(const PathLanes &p, int j) {
    const int a = __shfl(p.id0, j & 63), b = __shfl(p.id1, j & 63);
    return j < 64 ? a : b;
}

// parent of node id (or -2 for an id outside [0, n)) from a parent row held
// by one wave, lane l holding the parents of nodes l (pp0) and 64 + l (pp1);
// every lane of the wave must take part
__device__ __forceinline__ int parent_of(int id, int pp0, int pp1, int n) {
    const int a = __shfl(pp0, id & 63), b = __shfl(pp1, id & 63);
    if (id < 0 || id >= n) return -2;
    return id < 64 ? a : b;
}

// every parent of a tree of n <= 128 nodes held as in parent_of lies in
// [-1, node)
__device__ __forceinline__ bool tree_valid(int pp0, int pp1, int n, int l) {
    const bool bad = (l < n && !parent_ok(pp0, l)) || (64 + l < n && !parent_ok(pp1, 64 + l));
    return __ballot(bad) == 0ull;
}

// a path is valid when 0 <= m <= max_path, its ids lie in [0, n) and
// increase, the first is a root and each later id's parent is the previous id
__device__ __forceinline__ bool path_valid(const PathLanes &p, int m, int max_path, int n,
                                           int l) {
    if (m < 0 || m > max_path || m > kMaxPath) return false;
    const int last0 = __shfl(p.id0, 63);
    bool bad = false;
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd) {
        const int j = 64 * rnd + l;
        const int id = rnd == 0 ? p.id0 : p.id1;
        const int par = rnd == 0 ? p.par0 : p.par1;
        int prev = __shfl(id, (l + 63) & 63);
        if (l == 0) prev = rnd == 0 ? -1 : last0;
        if (j < m && (id < 0 || id >= n || (j > 0 && prev >= id) || par != prev)) bad = true;
    }
    return __ballot(bad) == 0ull;
}

// Gates and key / value rows of the chunk starting at path slot c0, in
// registers (one round of loads; threads < 32 also take a gate pair).
struct ChunkRows {
    uint4 kr[2], vr[2];
    float la, bt;
};

__device__ __forceinline__ ChunkRows load_chunk(const int *pid, int c0, int mlen, int b, int hd,
                                                int n, int H, const uint16_t *__restrict__ k,
                                                const uint16_t *__restrict__ v,
                                                const float *__restrict__ alpha,
                                                const float *__restrict__ beta, int tid) {
    const int mc = min(kC, mlen - c0);
    ChunkRows r;
    // every thread reads the gates of a valid path node (slots past the
    // chunk repeat its last node and are zeroed), so no load sits in a branch
    const int jg = min(tid & (kC - 1), mc - 1);
    const size_t grow = ((size_t)b * n + pid[c0 + jg]) * H + hd;
    const float a = alpha[grow], be = beta[grow];
    const bool live = tid < mc;
    r.la = live ? log2f(a) : 0.f;
    r.bt = live ? be : 0.f;
    // key / value rows through buffer resources over this head's n rows;
    // slots past the chunk get an offset past the end and read as zero
    const size_t base = ((size_t)b * n * H + hd) * kD;
    const uint32_t bytes = (uint32_t)(n * H * kD * 2);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + base, bytes), vr = make_rsrc(v + base, bytes);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int e = tid + kThreads * it, j = e >> 4, c8 = (e & 15) * 8;
        const uint32_t off =
            j < mc ? (uint32_t)(((size_t)pid[c0 + j] * H * kD + c8) * 2) : bytes;
        r.kr[it] = load16(kr, off);
        r.vr[it] = load16(vr, off);
    }
    return r;
}

// Rows into LDS, decay prefix, Gram, T = (I + X)^{-1} for the chunk.  Every
// thread of the workgroup calls this (it contains barriers).
__device__ __forceinline__ void build_chunk(ChunkTiles &sm, const ChunkRows &cr, int c0, int mlen,
                                            int tid, int w, int l) {
    const int m = l & 31, h = l >> 5;
    const int mc = min(kC, mlen - c0);
    const float la = cr.la, bt = cr.bt;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int e = tid + kThreads * it, j = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<uint4 *>(&sm.vp[j][c8]) = cr.vr[it];
        store_row8_permuted(sm.kp[j], c8, cr.kr[it]);
    }
    if (tid < kC) {
        // inclusive prefix of the log2 decays over the chunk (32 lanes)
        const int j = tid;
        float gs = la;
#pragma unroll
        for (int o = 1; o < kC; o <<= 1) {
            const float t = __shfl_up(gs, o, kC);
            if (j >= o) gs += t;
        }
        const float gl = __shfl(gs, mc - 1, kC);
        sm.g[j] = gs;
        sm.eg[j] = exp2f(gs);
        sm.wdec[j] = j < mc ? exp2f(gl - gs) : 0.f;
        sm.beta[j] = bt;
        if (j == 0) sm.glast = exp2f(gl);
    }
    lds_barrier();

    // chunk Gram (wave 0, transposed tile): lane (j, h) holds k_t.k_j for
    // t = crow(r, h); X_jt = beta_j e^{g_j - g_t} k_j.k_t for t < j into d[j][t]
    if (w == 0) {
        f32x16 ga = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 a = lds8(&sm.kp[m][16 * kk + 8 * h]);
            ga = mfma(a, a, ga);
        }
        const int j = m;
        const float gj = sm.g[j], bj = sm.beta[j];
        float x[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 g4 = *reinterpret_cast<const float4 *>(&sm.g[8 * q4 + 4 * h]);
            const float gt[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e, t = crow(r, h);
                x[r] = (t < j) ? bj * __builtin_amdgcn_exp2f(gj - gt[e]) * ga[r] : 0.f;
            }
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(&sm.d[j][8 * q4 + 4 * h]) =
                make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
    }
    lds_barrier();

    // T = (I + X)^{-1}: 16x16 diagonal inverses by forward substitution
    // (32 lanes: sub-block, column), then Z = B A^{-1} and L = -C^{-1} Z
    if (w == 0 && l < 32) {
        const int sbk = l >> 4, c = l & 15, o16 = 16 * sbk;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int s4 = 0; s4 < r; s4 += 4) {
                const float4 xr = *reinterpret_cast<const float4 *>(&sm.d[o16 + r][o16 + s4]);
                acc = fmaf(-xr.x, t[s4], acc);
                if (s4 + 1 < r) acc = fmaf(-xr.y, t[s4 + 1], acc);
                if (s4 + 2 < r) acc = fmaf(-xr.z, t[s4 + 2], acc);
                if (s4 + 3 < r) acc = fmaf(-xr.w, t[s4 + 3], acc);
            }
            t[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.tinv[sbk][r][c] = t[r];
    }
    lds_barrier();
    // rows past the chunk length are zero, so for mc <= 16 the lower block
    // of T is [0, I]: its coupling L is zero and the two passes are skipped
    const bool two_blocks = mc > 16;
    if (two_blocks) {
        {   // Z = B A^{-1} over the upper-left sub-block (read only by the substitution)
            const int r = tid >> 4, c = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) acc = fmaf(sm.d[16 + r][s2], sm.tinv[0][s2][c], acc);
            sm.d[r][c] = acc;
        }
        lds_barrier();
        {   // L = -C^{-1} Z over the lower-left sub-block (B is no longer read)
            const int r = tid >> 4, c = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) acc = fmaf(sm.tinv[1][r][s2], sm.d[s2][c], acc);
            sm.d[16 + r][c] = -acc;
        }
        lds_barrier();
    }
    if (tid < 4 * kC) {
        // T = [[A^-1, 0], [L, C^-1]] as bf16 hi/lo operand rows, one 8-entry
        // chunk per thread (permuted positions 8 seg .. 8 seg + 7)
        const int r = tid >> 2, seg = tid & 3, kb = seg >> 1, hb = seg & 1;
        const int c0c = 16 * kb + 4 * hb;
        float4 lo4, hi4;
        if (r < 16) {
            if (kb == 0) {
                lo4 = *reinterpret_cast<const float4 *>(&sm.tinv[0][r][c0c]);
                hi4 = *reinterpret_cast<const float4 *>(&sm.tinv[0][r][c0c + 8]);
            } else {
                lo4 = hi4 = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        } else if (kb == 1) {
            lo4 = *reinterpret_cast<const float4 *>(&sm.tinv[1][r - 16][c0c - 16]);
            hi4 = *reinterpret_cast<const float4 *>(&sm.tinv[1][r - 16][c0c - 8]);
        } else if (two_blocks) {
            lo4 = *reinterpret_cast<const float4 *>(&sm.d[r][c0c]);
            hi4 = *reinterpret_cast<const float4 *>(&sm.d[r][c0c + 8]);
        } else {
            lo4 = hi4 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const float vals[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
        bf16x8 th8, tl8;
        split8(vals, th8, tl8);
        *reinterpret_cast<bf16x8 *>(&sm.th[r][8 * seg]) = th8;
        *reinterpret_cast<bf16x8 *>(&sm.tl[r][8 * seg]) = tl8;
    }
    lds_barrier();
}

// load_chunk then build_chunk
__device__ __forceinline__ void prepare_chunk(ChunkTiles &sm, const int *pid, int c0, int mlen,
                                              int b, int hd, int n, int H,
                                              const uint16_t *__restrict__ k,
                                              const uint16_t *__restrict__ v,
                                              const float *__restrict__ alpha,
                                              const float *__restrict__ beta, int tid, int w,
                                              int l) {
    build_chunk(sm, load_chunk(pid, c0, mlen, b, hd, n, H, k, v, alpha, beta, tid), c0, mlen, tid,
                w, l);
}

// identity operands that move a path-key tile into the result layout:
// k-step kb, lane (n = m, h), element e is 1 where n is the d_k index that
// the permuted key storage puts in that slot
__device__ __forceinline__ void key_identity(bf16x8 (&ident)[2], int m, int h) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ident[kb][e] = static_cast<__bf16>(
                (m == 16 * kb + 8 * (e >> 2) + 4 * h + (e & 3)) ? 1.f : 0.f);
}

// What the application of a chunk reads, from the point of view of one lane
// (row m of the path-slot operands).  Rows past the chunk are zero rows.
struct ChunkView {
    const uint16_t *kp_row;           // path keys of slot m (d_k permuted)
    const uint16_t *th_row, *tl_row;  // row m of T, hi / lo (permuted columns)
    const uint16_t *vp;               // path values, [NR][vp_stride]
    int vp_stride;
    const float *eg, *wdec, *beta;    // per path slot, 32 entries, zero past the chunk
    float glast;
};

// S <- e^{g_last} S + K_p^T W with W_j = e^{g_last - g_j} u_j, for the chunk's
// pseudo-values U held as a result tile (rows = path slots crow(r, h)).  The
// key tile of rows 32q.. is put in the result layout by an exact identity
// product; that layout is the A operand of K_p^T with the path slots in the
// order W holds them.
template <int NR>
__device__ __forceinline__ void apply_update(const ChunkView &cv, const f32x16 &U,
                                             f32x16 (&st)[4], const bf16x8 (&ident)[2], int h) {
    constexpr int KS = NR / 16;
    bf16x8 wh[2], wl[2];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        float wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = cv.wdec[crow(8 * kk + j, h)] * U[8 * kk + j];
        split8(wv, wh[kk], wl[kk]);
    }
    const float gl = cv.glast;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f32x16 kt = {};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kt = mfma(lds8(cv.kp_row + 32 * q + 16 * kb + 8 * h), ident[kb], kt);
        f32x16 acc = st[q] * gl;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = static_cast<__bf16>(kt[8 * kk + e]);
            acc = mfma(a, wh[kk], acc);
            acc = mfma(a, wl[kk], acc);
        }
        st[q] = acc;
    }
}

// One state tile's share of R = K_p S: tile q holds rows 32 q .. 32 q + 31
// of this wave's slab (the B operand, split hi + lo); kp_row is row m of the
// chunk's key tile (d_k permuted).  R accumulates, so the tiles may be taken
// one at a time as they land.
__device__ __forceinline__ void rp_tile(const uint16_t *kp_row, const f32x16 &stq, int q,
                                        f32x16 &R, int h) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        float sv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = stq[8 * kk + j];
        bf16x8 sh, sl;
        split8(sv, sh, sl);
        const bf16x8 a = lds8(kp_row + 32 * q + 16 * kk + 8 * h);
        R = mfma(a, sh, R);
        R = mfma(a, sl, R);
    }
}

// The chunk's pseudo-values once R = K_p S is complete: the right-hand side
// beta (v - e^g R) and U = T RHS (rows = path slots crow(r, h)).  vv[r] = v
// of path slot crow(r, h) in this lane's column, zero past the chunk (no
// barrier inside).
template <int NR>
__device__ __forceinline__ f32x16 chunk_u(const ChunkView &cv, const f32x16 &vv, const f32x16 &R,
                                          int h) {
    constexpr int KS = NR / 16;   // k-steps over path slots that can be nonzero
    f32x16 rhs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = crow(r, h);
        rhs[r] = j < NR ? cv.beta[j] * (vv[r] - cv.eg[j] * R[r]) : 0.f;
    }
    f32x16 U = {};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        float bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = rhs[8 * kk + j];
        bf16x8 bhh, bll;
        split8(bv, bhh, bll);
        const bf16x8 ah = lds8(cv.th_row + 16 * kk + 8 * h);
        const bf16x8 al = lds8(cv.tl_row + 16 * kk + 8 * h);
        U = mfma(ah, bhh, U);
        U = mfma(ah, bll, U);
        U = mfma(al, bhh, U);
    }
    return U;
}

// The rest of a chunk's application once R = K_p S is complete: the
// right-hand side beta (v - e^g R), U = T RHS, and the update of the slab
// (vv as for chunk_u; the same steps written out in one body)
template <int NR>
__device__ __forceinline__ void finish_rows_v(const ChunkView &cv, const f32x16 &vv,
                                              const f32x16 &R, f32x16 (&st)[4],
                                              const bf16x8 (&ident)[2], int h) {
    constexpr int KS = NR / 16;   // k-steps over path slots that can be nonzero
    // ---- right-hand side and U = T RHS, scaled by the decay to the chunk end
    f32x16 rhs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = crow(r, h);
        rhs[r] = j < NR ? cv.beta[j] * (vv[r] - cv.eg[j] * R[r]) : 0.f;
    }
    f32x16 U = {};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        float bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = rhs[8 * kk + j];
        bf16x8 bhh, bll;
        split8(bv, bhh, bll);
        const bf16x8 ah = lds8(cv.th_row + 16 * kk + 8 * h);
        const bf16x8 al = lds8(cv.tl_row + 16 * kk + 8 * h);
        U = mfma(ah, bhh, U);
        U = mfma(ah, bll, U);
        U = mfma(al, bhh, U);
    }
    apply_update<NR>(cv, U, st, ident, h);
}

// Apply a prepared chunk of NR (16 or 32) path slots to this wave's state
// slab, the chunk's values given in registers (as for finish_rows_v).
template <int NR>
__device__ __forceinline__ void apply_rows_v(const ChunkView &cv, const f32x16 &vv,
                                             f32x16 (&st)[4], const bf16x8 (&ident)[2], int h) {
    f32x16 R = {};
#pragma unroll
    for (int q = 0; q < 4; ++q) rp_tile(cv.kp_row, st[q], q, R, h);
    finish_rows_v<NR>(cv, vv, R, st, ident, h);
}

// the same with the chunk's values read from the LDS value tile
template <int NR>
__device__ __forceinline__ void apply_rows(const ChunkView &cv, f32x16 (&st)[4],
                                           const bf16x8 (&ident)[2], int h, int col) {
    f32x16 vv;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = crow(r, h);
        vv[r] = j < NR ? to_f32(cv.vp[j * cv.vp_stride + col]) : 0.f;
    }
    apply_rows_v<NR>(cv, vv, st, ident, h);
}

__device__ __forceinline__ void apply_chunk(const ChunkTiles &sm, f32x16 (&st)[4],
                                            const bf16x8 (&ident)[2], int m, int h, int col) {
    const ChunkView cv{sm.kp[m], sm.th[m], sm.tl[m], &sm.vp[0][0], kKP,
                       sm.eg,    sm.wdec,  sm.beta,  sm.glast};
    apply_rows<kC>(cv, st, ident, h, col);
}

// ---- 16-slot chunks, for the fused commit-verify kernel, where the chunk
// tiles overlay scratch of the verify's block inverse and must be small.
// One wave loads and prepares a chunk on its own (no barrier inside); every
// wave then applies it.
constexpr int kC16 = 16;

struct Chunk16 {
    uint16_t kp[kC16][kKP];               // path keys, d_k permuted within 16-blocks
    uint16_t vp[kC16][kD];                // path values
    float x[kC16][kC16];                  // X of the chunk (strictly lower)
    uint16_t th[kC16][kBL], tl[kC16][kBL];   // T hi / lo; permuted columns, 16..31 zero
};

struct Chunk16Aux {
    float g[32], eg[32], wdec[32], beta[32];   // per path slot, zero past the chunk
    float glast;
    uint16_t zk[kKP];                           // zero key row (slots 16..31)
    uint16_t zt[kBL];                           // zero T row (rows 16..31)
};

// A chunk's rows in the registers of the wave that prepares it: lane l holds
// bytes [64 (l & 3), 64 (l & 3) + 64) of slot l >> 2's key and value rows,
// and lanes < 16 hold slot l's gates (la = alpha itself).
struct Rows16 {
    uint4 k[4], v[4];
    float la, bt;
};

// slot_id(j) is the node id of chunk slot j (valid for j < mc).  k, v, alpha,
// beta point at node 0 of this (sequence, head); rs = elements between nodes
// (H * 128), gs = gate entries between nodes (H); bytes = n * rs * 2.
__device__ __forceinline__ Rows16 load_rows16(int row_id, bool row_live, int gate_id,
                                              bool gate_live, const uint16_t *k,
                                              const uint16_t *v, const float *alpha,
                                              const float *beta, int rs, int gs, uint32_t bytes,
                                              int l) {
    Rows16 r;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k, bytes), vr = make_rsrc(v, bytes);
    const uint32_t base = row_live ? (uint32_t)(row_id * rs + 32 * (l & 3)) * 2 : bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.k[i] = load16(kr, row_live ? base + 16 * i : bytes);
        r.v[i] = load16(vr, row_live ? base + 16 * i : bytes);
    }
    const int gi = gate_live ? gate_id : 0;
    const float a = alpha[(size_t)gi * gs], be = beta[(size_t)gi * gs];
    // raw values: the build masks slots past the chunk and takes the log2,
    // so nothing here makes the wave wait for the loads issued before these
    // (a slot whose gate is not live belongs to a path the build never sees)
    r.la = a;
    r.bt = be;
    return r;
}

// One wave: keys into a chunk's key tile, decay prefix, Gram and X; Ch has
// the kp, x, th and tl members of Chunk16.  k holds the lane's part of the
// key rows as loaded by load_rows16 / load_keys16, la and bt its slot's raw
// gates (lanes < 16).  LDS accesses of one wave complete in order, so no
// barrier is needed inside.
template <class Ch>
__device__ __forceinline__ void build16_x(Ch &ch, Chunk16Aux &ax, const uint4 (&k)[4], float la,
                                             float bt, int mc, int l) {
    const int m = l & 31, h = l >> 5;
    {
        const int j = l >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) store_row8_permuted(ch.kp[j], 32 * (l & 3) + 8 * i, k[i]);
    }
    // inclusive prefix of the log2 decays over the chunk (slots past mc: 0)
    {
        float gs = (l < mc) ? log2f(la) : 0.f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const float t = __shfl_up(gs, o, 32);
            if ((l & 31) >= o) gs += t;
        }
        const float gl = __shfl(gs, mc - 1, 32);
        if (l < 32) {
            ax.g[l] = gs;
            ax.eg[l] = l < mc ? exp2f(gs) : 0.f;
            ax.wdec[l] = l < mc ? exp2f(gl - gs) : 0.f;
            ax.beta[l] = l < mc ? bt : 0.f;
        }
        if (l == 0) ax.glast = exp2f(gl);
    }
    // Gram of the chunk keys (transposed tile: lane (j, h) holds k_t.k_j for
    // t = crow(r, h)); rows past 16 read the zero row
    const uint16_t *kp_row = m < kC16 ? ch.kp[m] : ax.zk;
    f32x16 ga = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = lds8(kp_row + 16 * kk + 8 * h);
        ga = mfma(a, a, ga);
    }
    // X_jt = beta_j e^{g_j - g_t} k_j.k_t for t < j (registers r < 8 hold t < 16)
    if (m < kC16) {
        const int j = m;
        const float gj = ax.g[j], bj = ax.beta[j];
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
            float x4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * q4 + e, t = crow(rr, h);
                x4[e] = (t < j) ? bj * __builtin_amdgcn_exp2f(gj - ax.g[t]) * ga[rr] : 0.f;
            }
            *reinterpret_cast<float4 *>(&ch.x[j][8 * q4 + 4 * h]) =
                make_float4(x4[0], x4[1], x4[2], x4[3]);
        }
    }
}

// One wave (any; the chunk's X written and visible): T = (I + X)^{-1} by
// forward substitution, lane = column of T (lanes 0..15); lanes 16..31
// write the zero columns 16..31.  Row r's entries are requested two rows
// ahead of their use, so the chain of rows waits on arithmetic rather than
// on LDS latency.
template <class Ch>
__device__ __forceinline__ void build16_t(Ch &ch, int l) {
    if (l < 16) {
        const int col = l;
        float t[16];
        float4 xr[16][4];
#pragma unroll
        for (int r = 0; r < 16 + 2; ++r) {
            if (r < 16) {
#pragma unroll
                for (int s4 = 0; s4 < r; s4 += 4)
                    xr[r][s4 / 4] = *reinterpret_cast<const float4 *>(&ch.x[r][s4]);
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
        const int pc = perm(col);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const __bf16 hi = static_cast<__bf16>(t[rr]);
            const __bf16 lo = static_cast<__bf16>(t[rr] - static_cast<float>(hi));
            ch.th[rr][pc] = __builtin_bit_cast(uint16_t, hi);
            ch.tl[rr][pc] = __builtin_bit_cast(uint16_t, lo);
        }
    } else if (l < 32) {
        const int pc = perm(l);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            ch.th[rr][pc] = 0;
            ch.tl[rr][pc] = 0;
        }
    }
}

// One wave: rows into the chunk tiles (values too), X, then T.
__device__ __forceinline__ void build16(Chunk16 &ch, Chunk16Aux &ax, const Rows16 &r, int mc,
                                        int l) {
    {
        const int j = l >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4 *>(&ch.vp[j][32 * (l & 3) + 8 * i]) = r.v[i];
    }
    build16_x(ch, ax, r.k, r.la, r.bt, mc, l);
    build16_t(ch, l);
}

__device__ __forceinline__ void apply16(const Chunk16 &ch, const Chunk16Aux &ax, f32x16 (&st)[4],
                                        const bf16x8 (&ident)[2], int m, int h, int col) {
    const bool live = m < kC16;
    const ChunkView cv{live ? ch.kp[m] : ax.zk, live ? ch.th[m] : ax.zt, live ? ch.tl[m] : ax.zt,
                       &ch.vp[0][0],           kD,
                       ax.eg,                  ax.wdec,
                       ax.beta,                ax.glast};
    apply_rows<kC16>(cv, st, ident, h, col);
}

// ---- the first 16-slot chunk of a solving commit, prepared while the
// verify's tree matrices are built: it holds no values (every wave keeps its
// own columns of the chunk's value rows in registers), so it fits in the
// T rows of the verify's solve blocks.
struct EarlyChunk16 {
    uint16_t kp[kC16][kKP];                  // path keys, d_k permuted within 16-blocks
    float x[kC16][kC16];                     // X of the chunk (strictly lower)
    uint16_t th[kC16][kBL], tl[kC16][kBL];   // T hi / lo; permuted columns, 16..31 zero
};

// key rows and raw gates of a chunk in the preparing wave: lane l holds
// bytes [64 (l & 3), 64 (l & 3) + 64) of slot l >> 2's key row, lanes < 16
// slot l's alpha and beta (arguments as for load_rows16)
struct KeyRows16 {
    uint4 k[4];
    float la, bt;
};

__device__ __forceinline__ KeyRows16 load_keys16(int row_id, bool row_live, int gate_id,
                                                 bool gate_live, const uint16_t *k,
                                                 const float *alpha, const float *beta, int rs,
                                                 int gs, uint32_t bytes, int l) {
    KeyRows16 r;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k, bytes);
    const uint32_t base = row_live ? (uint32_t)(row_id * rs + 32 * (l & 3)) * 2 : bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.k[i] = load16(kr, row_live ? base + 16 * i : bytes);
    const int gi = gate_live ? gate_id : 0;
    r.la = alpha[(size_t)gi * gs];
    r.bt = beta[(size_t)gi * gs];
    return r;
}

// Raw words of a chunk's per-slot values in this lane's column, one per
// result-tile register r (slot crow(r, h)): fp32 bit patterns, or 16-bit
// patterns zero-extended.  They are widened where they are used, not where
// they are loaded: a conversion next to the load would make the wave wait
// for that load, and for every load issued before it, at that point.
struct ChunkWords {
    uint32_t x[16];
};

__device__ __forceinline__ f32x16 widen_bf16(const ChunkWords &w) {
    f32x16 v;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = __uint_as_float(w.x[r] << 16);
    return v;
}

__device__ __forceinline__ f32x16 widen_f16(const ChunkWords &w) {
    f32x16 v;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        v[r] = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)w.x[r]));
    return v;
}

__device__ __forceinline__ f32x16 as_f32(const ChunkWords &w) {
    f32x16 v;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = __uint_as_float(w.x[r]);
    return v;
}

// this lane's values of the first 16 slots crow(r, h), r < 8, of the chunk
// at path slot c0, as raw bf16 words (zero past the chunk and in r >= 8):
// v_head points at node 0 of this (sequence, head) of a [batch][n][H][128]
// bf16 tensor, rs = H * 128, bytes = n * rs * 2
__device__ __forceinline__ ChunkWords load_v_chunk16(const uint16_t *v_head, uint32_t bytes,
                                                     const int *pid, int c0, int mc, int rs,
                                                     int col, int h) {
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_head, bytes);
    ChunkWords w;
#pragma unroll
    for (int r = 0; r < 16; ++r) w.x[r] = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int j = crow(r, h);
        const uint32_t off =
            j < mc ? (uint32_t)(pid[min(c0 + j, kMaxPath - 1)] * rs + col) * 2 : bytes;
        w.x[r] = __builtin_amdgcn_raw_buffer_load_b16(vr, (int)off, 0, kNT);
    }
    return w;
}

// what the application of the early chunk reads (lane row m)
__device__ __forceinline__ ChunkView early_view(const EarlyChunk16 &ch, const Chunk16Aux &ax,
                                                int m) {
    const bool live = m < kC16;
    return ChunkView{live ? ch.kp[m] : ax.zk, live ? ch.th[m] : ax.zt, live ? ch.tl[m] : ax.zt,
                     nullptr,                0,
                     ax.eg,                  ax.wdec,
                     ax.beta,                ax.glast};
}

// ---- commit from known pseudo-values (u_s written by the verify that ran on
// the same state): S <- e^{g_last} S + K_p^T W per chunk of 32 path slots, no
// solve.  One wave loads a chunk's keys and gates; every wave loads its own
// columns of the chunk's u rows.
struct KeyChunk32 {
    uint16_t kp[32][kKP];   // path keys, d_k permuted within 16-blocks; zero past the chunk
};

// lane l holds bytes [128 (l & 1), 128 (l & 1) + 128) of slot l >> 1's key
// row, and lanes < 32 slot l's decay alpha
struct KeyRows32 {
    uint4 k[8];
    float la;
};

__device__ __forceinline__ KeyRows32 load_keys32(int row_id, bool row_live, int gate_id,
                                                 bool gate_live, const uint16_t *k,
                                                 const float *alpha, int rs, int gs,
                                                 uint32_t bytes, int l) {
    KeyRows32 r;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k, bytes);
    const uint32_t base = row_live ? (uint32_t)(row_id * rs + 64 * (l & 1)) * 2 : bytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.k[i] = load16(kr, row_live ? base + 16 * i : bytes);
    const int gi = gate_live ? gate_id : 0;
    const float a = alpha[(size_t)gi * gs];
    r.la = a;   // masked and log2'd at build time (see load_rows16)
    return r;
}

// one wave: keys into the chunk tile, decay-to-chunk-end weights and the
// chunk's total decay (no barrier inside: one wave's LDS accesses are ordered)
__device__ __forceinline__ void build_keys32(KeyChunk32 &kc, Chunk16Aux &ax, const KeyRows32 &r,
                                             int mc, int l) {
    const int j = l >> 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) store_row8_permuted(kc.kp[j], 64 * (l & 1) + 8 * i, r.k[i]);
    float gs = (l < mc) ? log2f(r.la) : 0.f;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const float t = __shfl_up(gs, o, 32);
        if ((l & 31) >= o) gs += t;
    }
    const float gl = __shfl(gs, mc - 1, 32);
    if (l < 32) ax.wdec[l] = l < mc ? exp2f(gl - gs) : 0.f;
    if (l == 0) ax.glast = exp2f(gl);
}

// this lane's u entries of the chunk's slots crow(r, h) (zero past the chunk),
// as raw words: u_head points at node 0 of this (sequence, head) of a
// [batch][n][H][128] tensor of fp32 (or, with kHalf, fp16) values,
// rs = H * 128, bytes = n * rs times the element size
template <bool kHalf>
__device__ __forceinline__ ChunkWords load_u_chunk(const void *u_head, uint32_t bytes,
                                                   const int *pid, int c0, int mc, int rs,
                                                   int col, int h) {
    const __amdgpu_buffer_rsrc_t ur = make_rsrc(u_head, bytes);
    constexpr uint32_t es = kHalf ? 2 : 4;
    ChunkWords w;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = crow(r, h);
        const uint32_t off =
            j < mc ? (uint32_t)(pid[min(c0 + j, kMaxPath - 1)] * rs + col) * es : bytes;
        if constexpr (kHalf)
            w.x[r] = __builtin_amdgcn_raw_buffer_load_b16(ur, (int)off, 0, kNT);
        else
            w.x[r] = __builtin_amdgcn_raw_buffer_load_b32(ur, (int)off, 0, kNT);
    }
    return w;
}

template <bool kHalf>
__device__ __forceinline__ f32x16 u_values(const ChunkWords &w) {
    if constexpr (kHalf) return widen_f16(w);
    else return as_f32(w);
}

__device__ __forceinline__ void apply_known_u(const KeyChunk32 &kc, const Chunk16Aux &ax,
                                              const f32x16 &U, f32x16 (&st)[4],
                                              const bf16x8 (&ident)[2], int m, int h) {
    const ChunkView cv{kc.kp[m], nullptr, nullptr, nullptr, 0,
                       nullptr,  ax.wdec, nullptr, ax.glast};
    apply_update<32>(cv, U, st, ident, h);
}

}  // namespace pc
}  // namespace gdn
