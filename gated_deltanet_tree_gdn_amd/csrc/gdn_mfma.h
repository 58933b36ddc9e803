// gdn_mfma.h -- bf16 MFMA helpers shared by the gfx950 kernels.
//
// v_mfma_f32_16x16x32_bf16, D (16 x 16) += A (16 x 32) B (32 x 16), with
// lane l of the wavefront holding
//   A: row l % 16, k-slots 8 (l / 16) .. 8 (l / 16) + 7
//   B: column l % 16, the same k-slots
//   D: column l % 16, rows 4 (l / 16) .. 4 (l / 16) + 3.
// The contraction does not care which k each slot carries as long as A and
// B agree, which the kernels use to match fragments to their data layouts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: the same layout with 4 k-slots per lane,
// 4 (l / 16) .. 4 (l / 16) + 3 (bf16 bits in shorts).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// x ~= hi + lo with hi = bf16(x) (nearest) and lo = bf16(x - hi), so a
// product with an exact bf16 operand keeps about 16 significant bits.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = static_cast<__bf16>(x[j]);
        hi[j] = h;
        lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
    }
}

__device__ __forceinline__ bf16x8 load_frag(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Two 4-element bf16 pieces (8 bytes each) as one fragment.
__device__ __forceinline__ bf16x8 load_frag2(const void* p0, const void* p1) {
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
    return __builtin_bit_cast(bf16x8, v);
}

}  // namespace gdn
