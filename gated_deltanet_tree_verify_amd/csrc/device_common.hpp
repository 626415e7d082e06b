// Small device helpers shared by the HIP kernels of libgdntree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bf16 is carried as its raw 16-bit pattern; widening to fp32 is exact.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fault flags, mirroring GDN_FAULT_* of the public header
constexpr int kFaultBadParent = 1;
constexpr int kFaultBadPath = 2;

// A parent row is valid when -1 <= parent[i] < i for every node (the draft
// tree is topologically sorted).
__device__ __forceinline__ bool parent_ok(int p, int i) { return p >= -1 && p < i; }

}  // namespace gdn
