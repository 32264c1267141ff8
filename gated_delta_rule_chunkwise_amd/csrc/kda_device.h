// Device-side helpers shared by the libkda kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- scalar conversions -------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (v_cvt_pk_bf16_f32 under the default rounding mode).
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

// Split x into hi + lo bf16 parts: hi = bf16(x), lo = bf16(x - hi).  hi + lo
// carries ~16 significant bits, so a product of split operands computed as
// hi*hi + hi*lo + lo*hi on bf16 matrix cores keeps ~2^-16 relative accuracy.
__device__ __forceinline__ void split_bf16(float x, bf16_t &hi, bf16_t &lo) {
    hi = (bf16_t)x;
    lo = (bf16_t)(x - (float)hi);
}

// ---- matrix core ----------------------------------------------------------------
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane layout (wave64): lane l holds A[l%16][8*(l/16) .. 8*(l/16)+7],
// B[8*(l/16) .. +7][l%16], and D[4*(l/16) + i][l%16] for i = 0..3.
// Only the pairing of the k index between A and B matters for the result.
__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t lds_ld8(const bf16_t *p) {
    return *reinterpret_cast<const bf16x8_t *>(p);
}

__device__ __forceinline__ f32x4_t zero4() {
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

}  // namespace kda
