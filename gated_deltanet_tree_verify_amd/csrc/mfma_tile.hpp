// 32x32x16 bf16 MFMA tile helpers shared by the verify, commit and fused
// commit-verify kernels (gfx950).
//
// Conventions used throughout:
//   * A 32x32 fp32 result tile ("result layout") is held by a wave as 16
//     registers per lane: lane (col = l & 31, half h = l >> 5), register r
//     holds row crow(r, h) = 8 (r >> 2) + 4 h + (r & 3).
//   * An A operand lane (row = l & 31, h) supplies 8 bf16 for k-step kk at
//     slots 16 kk + 8 h + e; a B operand lane (col, h) supplies the same 8
//     slots.  Both sides use the same (h, e) -> slot pairing, so any
//     consistent relabelling of the contraction index is exact.
//   * A result tile fed back as a B operand supplies, for k-step kk, its
//     registers 8 kk .. 8 kk + 7, i.e. rows crow(8 kk + e, h).  The matching
//     A operand therefore stores its contraction index with bits 2 and 3
//     swapped within each 16-block: position perm(c).
//   * A result tile of Z also is, register for register, the A operand of
//     Z^T (rows = columns of Z, contraction over the rows of Z in that same
//     permuted order).
//   * fp32 values enter a bf16 product split in two: x = hi + lo + O(2^-17 x).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier that orders LDS only.  Every exchange between threads in
// these kernels goes through LDS, so the barrier need not wait for the
// wave's outstanding global loads (a full __syncthreads() waits for all of
// them, which would stall each barrier behind whatever prefetch is in
// flight).  A global load is still waited for where its value is used.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// row of a 32x32 result tile held by lane half h in register r
__device__ __forceinline__ int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// storage position of contraction index c in an A operand whose B operand
// is a result tile: bits 2 and 3 of c swap places
__device__ __forceinline__ int perm(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void st8(uint16_t *p, const bf16x8 &x) {
    *reinterpret_cast<bf16x8 *>(p) = x;
}

// x = hi + lo: hi = bf16(x) (round to nearest even); the residual x - hi is
// exact in fp32 and comes out of one dot2 per element, (-1, 0).(hi0, hi1) + x0.
// The (-1, 0) and (0, -1) pairs are kept in scalar registers: written as
// constants, the compiler encodes one of them as the inline float constant
// -1.0, which the dot2 instruction reads as a different bf16 pair (checked on
// gfx950: every lane wrong).
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
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

// registers 8 kk .. 8 kk + 7 of a result tile as split B operands
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

// C += A B for an fp32 A stored as hi/lo bf16 rows (permuted contraction
// index, row stride LD) and an fp32 B given as a split result tile:
// hi*hi + hi*lo + lo*hi
template <int LD>
__device__ __forceinline__ f32x16 mm3(const uint16_t (*ah)[LD], const uint16_t (*al)[LD],
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

// Write 8 consecutive bf16 of a global row (c8..c8+7) into an LDS row whose
// contraction index is stored permuted within 16-blocks: entries c8..c8+3
// land at perm(c8), c8+4..c8+7 at perm(c8 + 4).
__device__ __forceinline__ void store_row8_permuted(uint16_t *row, int c8, const uint4 &x) {
    *reinterpret_cast<uint2 *>(&row[perm(c8)]) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2 *>(&row[perm(c8 + 4)]) = make_uint2(x.z, x.w);
}

// Raw buffer resource over `bytes` bytes from base (wave-uniform).  A load
// whose offset lies past the end returns zero: rows beyond a tree's n, or
// path slots beyond a path's end, read as zero with no branch around the
// load, which keeps the memory-counter waits in front of each use exact.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // word 3 = 0x00020000: 32-bit data format, the gfx9 raw-buffer setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of every global access of these kernels: non-temporal (the
// nt bit of the gfx940-family cache-policy operand).  Each byte of q, k, v,
// the state and the outputs is touched once per call, so nothing is gained
// by keeping it in L2 or the Infinity Cache; marked streaming, the reads and
// the write-backs of the previous call's dirty lines stop competing for the
// same cache space (measured: a step's memory traffic finishes ~25% sooner).
constexpr int kNT = 2;

// s_waitcnt operand that waits for the vector memory counter alone to reach
// zero (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt
// 11:8 left at their maxima)
constexpr int kVmcntZero = 0x0F70;

template <int kAux = kNT>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAux));
}

// 16-byte store of 8 fp16 values (raw bits), non-temporal
__device__ __forceinline__ void store16h(uint16_t *p, const uint4 &x) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// 16-byte store of an output row segment, non-temporal
__device__ __forceinline__ void store16(float *p, const float4 &x) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

// The state slab of a wave: rows 0..127 of its 32 columns as four result
// tiles, tile q holding rows 32 q + crow(r, h).  The 128 x 128 fp32 state of
// one (sequence, head) is addressed through a buffer resource: the lane's
// column and half go into one 32-bit lane offset and every row offset is a
// scalar constant, so the loads or stores of a lane carry no per-element
// address arithmetic and nothing address-like stays live between the load
// and the store of the slab.  The resource's size bounds every access to
// the 64 KiB of that state.  slab must be wave-uniform.  The buffer
// builtins move integers: the floats pass through them as bit patterns.
// Tiles go one at a time with 4-byte accesses (load_state_tile,
// store_state_tile: the fused kernel and the long-path commit, measured
// faster there) or whole slabs with 8-byte accesses (load_state,
// store_state: the verify, short-path commit and branch kernels, half the
// memory instructions).
constexpr int kStateDim = 128;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(const float *slab) {
    return make_rsrc(slab, kStateDim * kStateDim * 4);
}

__device__ __forceinline__ int state_lane_offset(int col, int h) {
    return 4 * (col + 4 * h * kStateDim);
}

// one tile (rows 32 q .. 32 q + 31) of the slab
__device__ __forceinline__ void load_state_tile(f32x16 &t, int q, const float *slab, int col,
                                                int h) {
    const __amdgpu_buffer_rsrc_t rs = state_rsrc(slab);
    const int vo = state_lane_offset(col, h);
#pragma unroll
    for (int r = 0; r < 16; ++r)
        t[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rs, vo, 4 * kStateDim * (32 * q + crow(r, 0)), kNT));
}

__device__ __forceinline__ void store_state_tile(const f32x16 &t, int q, float *slab, int col,
                                                 int h) {
    const __amdgpu_buffer_rsrc_t rs = state_rsrc(slab);
    const int vo = state_lane_offset(col, h);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float x = t[r];   // scalar temporary: see store_state
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, vo,
                                              4 * kStateDim * (32 * q + crow(r, 0)), kNT);
    }
}

// Lane pairs (columns 2a, 2a + 1) move 2 x 2 blocks with 8-byte accesses:
// for registers 2j, 2j + 1 (rows R = crow(2j, h) and R + 1) the even lane
// accesses row R and the odd lane row R + 1, both at columns 2a, 2a + 1, and
// one swap between the pair (DPP quad_perm 1 0 3 2) gives each lane its own
// column of both rows.  Half the memory instructions of 4-byte accesses.
constexpr int kSwapPairs = 0xB1;   // quad_perm [1, 0, 3, 2]

__device__ __forceinline__ uint32_t pair_swap(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kSwapPairs, 0xf, 0xf, false);
}

__device__ __forceinline__ int state_pair_offset(int col, int h) {
    return 4 * ((col & ~1) + kStateDim * (4 * h + (col & 1)));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load_state_tile_x2(f32x16 &t, int q, const float *slab, int col,
                                                   int h) {
    const __amdgpu_buffer_rsrc_t rs = state_rsrc(slab);
    const int vo = state_pair_offset(col, h);
    const bool odd = col & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x2 x = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                       rs, vo, 4 * kStateDim * (32 * q + crow(2 * j, 0)), kNT));
        const uint32_t recv = pair_swap(odd ? x.x : x.y);
        t[2 * j] = __uint_as_float(odd ? recv : x.x);
        t[2 * j + 1] = __uint_as_float(odd ? x.y : recv);
    }
}

__device__ __forceinline__ void store_state_tile_x2(const f32x16 &t, int q, float *slab, int col,
                                                    int h) {
    const __amdgpu_buffer_rsrc_t rs = state_rsrc(slab);
    const int vo = state_pair_offset(col, h);
    const bool odd = col & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float a = t[2 * j], b = t[2 * j + 1];   // scalar temporaries
        const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
        const uint32_t recv = pair_swap(odd ? ua : ub);
        const u32x2 x = odd ? u32x2{recv, ub} : u32x2{ua, recv};
        __builtin_amdgcn_raw_buffer_store_b64(x, rs, vo,
                                              4 * kStateDim * (32 * q + crow(2 * j, 0)), kNT);
    }
}

// the whole slab, 8-byte accesses
__device__ __forceinline__ void load_state(f32x16 (&st)[4], const float *slab, int col, int h) {
#pragma unroll
    for (int q = 0; q < 4; ++q) load_state_tile_x2(st[q], q, slab, col, h);
}

__device__ __forceinline__ void store_state(const f32x16 (&st)[4], float *slab, int col, int h) {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_state_tile_x2(st[q], q, slab, col, h);
}

}  // namespace tile
}  // namespace gdn
