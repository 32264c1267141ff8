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

// ---- input prologue ---------------------------------------------------------------
// The entry points on raw projections map their inputs as the kernels read them
// (reading of the KimiLinear article, section 3.2: normalised inputs,
// constrained and reparameterised gate values):
//     log alpha = max(-softplus(a), lo),   beta = sigmoid(b),
//     q, k scaled per (token, head) by 1 / max(||x||_2, eps).
// softplus(a) = max(a, 0) + log1p(e^-|a|) cannot overflow.  log1p(t) for t in
// (0, 1] uses the correction of Goldberg, "What Every Computer Scientist Should
// Know About Floating-Point Arithmetic", theorem 4: with u = 1 + t rounded,
// log1p(t) = log(u) * t / (u - 1) (or t when u == 1), which keeps the hardware
// logarithm's relative accuracy for small t.
constexpr float kPrologueEps = 1e-6f;

__device__ __forceinline__ float pro_log1p_unit(float t) {
    const float u = 1.f + t;
    return u == 1.f ? t : __logf(u) * (t * __builtin_amdgcn_rcpf(u - 1.f));
}
__device__ __forceinline__ float pro_log_alpha(float a, float lo) {
    const float sp = fmaxf(a, 0.f) + pro_log1p_unit(__expf(-fabsf(a)));
    return fmaxf(-sp, lo);
}
__device__ __forceinline__ float pro_beta(float b) {
    const float e = __expf(-fabsf(b));
    const float r = __builtin_amdgcn_rcpf(1.f + e);
    return b >= 0.f ? r : e * r;
}
// 1 / max(sqrt(s), eps) = rsqrt(max(s, eps^2)), from the hardware reciprocal
// square root (about 1 ulp).
__device__ __forceinline__ float pro_inv_norm(float sumsq) {
    return __builtin_amdgcn_rsqf(fmaxf(sumsq, kPrologueEps * kPrologueEps));
}

// Gate layouts (a compile-time parameter GM of the kernels): one log decay per
// key channel (KDA), one per (token, head) broadcast over the channels (Gated
// DeltaNet), or none, i.e. log alpha = 0 (DeltaNet).
enum GateMode : int { kGatePerChannel = 0, kGatePerHead = 1, kGateNone = 2 };

// Gate of (token-head th, key channel c) in layout GM.
template <int GM, typename GT>
__device__ __forceinline__ float gate_at(const GT *__restrict__ g, int64_t th, int DK, int c) {
    if constexpr (GM == kGatePerChannel) return to_f32(g[th * DK + c]);
    else if constexpr (GM == kGatePerHead) return to_f32(g[th]);
    else return 0.f;
}
// log alpha as the recurrence uses it: the gate value itself, or with the
// prologue its floored -softplus (no gate stays log alpha = 0).
template <bool PRO, int GM> __device__ __forceinline__ float log_decay(float x, float lo) {
    if constexpr (PRO && GM != kGateNone) return pro_log_alpha(x, lo);
    else return x;
}

// Sum of x over the 64 lanes of a wave, returned wave-uniform: data-parallel
// moves within rows of 16 lanes (quad swaps, then half-row and row mirrors, each
// pairing a lane with one in the other half), then the four row sums.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);   // row_half_mirror
    x += dpp_mov<0x140>(x);   // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return (r0 + r1) + (r2 + r3);
}

}  // namespace kda
