// Device helpers shared by the chunkwise-forward kernels (kda_chunk.hip and
// kda_chunk2.hip): constants of the chunk decomposition, matrix-core wrappers,
// barriers, the exact per-token update and the per-chunk input registers.
#pragma once
#include "kda_device.h"

namespace kda {
namespace {

constexpr int kC = 64;            // chunk length (tokens)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxRange2 = 80.f * kLog2e;   // max in-chunk decay (log2 units) on the fast path

// The 10 lower 16x16 blocks (R, I), I <= R, of a 64x64 chunk matrix:
// (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3).
__device__ __forceinline__ void lower_block(int idx, int &R, int &I) {
    R = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    I = idx - (R * (R + 1)) / 2;
}

template <bool ACCURATE>
__device__ __forceinline__ float kexp2(float x) {
    return ACCURATE ? exp2f(x) : __builtin_amdgcn_exp2f(x);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load, which would stall the next chunk's prefetched inputs
// at the first barrier; here only LDS operations are drained before s_barrier.
// Global memory is never exchanged between waves of a workgroup in this kernel.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc += A * B for one 32-wide k-step; `lo` pointers are read only when that
// operand is split (hi*hi + hi*lo + lo*hi).
template <bool SA, bool SB>
__device__ __forceinline__ f32x4_t mma(f32x4_t acc, const bf16_t *ah, const bf16_t *al,
                                       const bf16_t *bh, const bf16_t *bl) {
    const bf16x8_t a = lds_ld8(ah), b = lds_ld8(bh);
    acc = mfma16(a, b, acc);
    if (SB) acc = mfma16(a, lds_ld8(bl), acc);
    if (SA) acc = mfma16(lds_ld8(al), b, acc);
    return acc;
}

__device__ __forceinline__ void store_split4(bf16_t *hi, bf16_t *lo, const f32x4_t &x) {
    bf16x4_t hv, lv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16_t hh, ll;
        split_bf16(x[e], hh, ll);
        hv[e] = hh;
        lv[e] = ll;
    }
    *reinterpret_cast<bf16x4_t *>(hi) = hv;
    *reinterpret_cast<bf16x4_t *>(lo) = lv;
}

// Epilogue of one 16x16 Gram tile (R, I): A (beta-scaled, strictly lower, fp32)
// or P (lower including the diagonal, hi/lo bf16).
template <typename Sm>
__device__ __forceinline__ void gram_store(Sm &sm, bool isP, int R, int I, const f32x4_t &acc, int lr, int lg) {
    const int i = 16 * I + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        if (!isP) {
            sm.A[r][i] = (i < r) ? sm.beta[r] * acc[e] : 0.f;
        } else {
            bf16_t hh, ll;
            split_bf16((i <= r) ? acc[e] : 0.f, hh, ll);
            sm.P[0][r][i] = hh;
            sm.P[1][r][i] = ll;
        }
    }
}

// Orders this wave's earlier LDS stores before its later LDS loads (lanes of one
// wave exchanging data through LDS; no other wave is involved).
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ bf16x4_t lds_ld4(const bf16_t *p) {
    return *reinterpret_cast<const bf16x4_t *>(p);
}

// Four consecutive fp32 values from LDS, split into hi/lo bf16.
__device__ __forceinline__ void load_split4(const float *p, bf16x4_t &hi, bf16x4_t &lo) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16_t hh, ll;
        split_bf16(x[e], hh, ll);
        hi[e] = hh;
        lo[e] = ll;
    }
}

__device__ __forceinline__ void split4(const f32x4_t &x, bf16x4_t &hi, bf16x4_t &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16_t hh, ll;
        split_bf16(x[e], hh, ll);
        hi[e] = hh;
        lo[e] = ll;
    }
}

// D(16x16) += A(16x16) B(16x16) with hi/lo-split operands on the 16x16x16 bf16
// matrix core.  Lane l holds A[l%16][4*(l/16)+i], B[4*(l/16)+i][l%16] and
// D[4*(l/16)+i][l%16]: an accumulator tile is already laid out as a B operand.
__device__ __forceinline__ f32x4_t mma4(f32x4_t acc, const bf16x4_t &ah, const bf16x4_t &al,
                                        const bf16x4_t &bh, const bf16x4_t &bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
    return acc;
}

// Stores an accumulator tile (rows r0 + 4*lg + e, column c0 + lr) as hi/lo bf16.
__device__ __forceinline__ void store_tile_split(bf16_t *hi, bf16_t *lo, int ld, int r0, int c0, const f32x4_t &x,
                                                 int lr, int lg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16_t hh, ll;
        split_bf16(x[e], hh, ll);
        hi[(r0 + 4 * lg + e) * ld + c0 + lr] = hh;
        lo[(r0 + 4 * lg + e) * ld + c0 + lr] = ll;
    }
}

// State tiles of one workgroup: (d_k/16) x (BV/16) tiles of 16x16, four waves
// (0-3) own ST/4 each; tile st covers key rows 16*(st/NT) + 4*lg + e and value
// column col0 + 16*(st%NT) + lr (MFMA accumulator layout).
template <int DK, int BV> struct StateTiles {
    static constexpr int NT = BV / 16;
    static constexpr int ST = (DK / 16) * NT;
    static constexpr int STW = ST / 4;
};

// One exact token update of this workgroup's state block (the per-token rule of
// the KimiLinear article, section 2.3, with the read-out o = S^T q).  Waves 0-3
// hold the state; all waves take part in the two barriers.
// Token-path reduction slots per wave: a (BV), b (BV), q.k, and with the input
// prologue also |q|^2 and |k|^2.
template <int BV> struct TokenRed { static constexpr int N = 2 * BV + 3; };

// With PRO (raw projections in), the gate and beta are mapped as they are read
// and the raw q and k enter through their squared norms: a = k^T S and b = q^T S
// are taken with the raw vectors and rescaled once the norms are reduced.
// With DEC the erase and write strengths are separate (beta erases, wr writes):
// the written row is u = wr v - beta a instead of beta (v - a).
template <int DK, int BV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__device__ __forceinline__ void token_update(f32x4_t (&Sacc)[(DK / 16) * (BV / 16) / 4],
                                             float (*red)[TokenRed<BV>::N], const IO *__restrict__ q,
                                             const IO *__restrict__ k, const IO *__restrict__ v,
                                             const GT *__restrict__ log_alpha, const GT *__restrict__ beta,
                                             const GT *__restrict__ wr, IO *__restrict__ o, int64_t tk, int H,
                                             int h, int DV, int col0, int w, int lg, int lr, float lo) {
    constexpr int NT = BV / 16, STW = StateTiles<DK, BV>::STW;
    float kc[STW][4];
    if (w < 4) {
        const int64_t kb = (tk * H + h) * (int64_t)DK;
        float pa[NT], pb[NT], pqk = 0.f, pqq = 0.f, pkk = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pa[nt] = pb[nt] = 0.f;
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w * STW + i, mt = st / NT, nt = st % NT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * mt + 4 * lg + e;
                const float kv = to_f32(k[kb + c]), qv = to_f32(q[kb + c]);
                const float la = GM == kGatePerChannel ? to_f32(log_alpha[kb + c])
                                                       : gate_at<GM>(log_alpha, tk * H + h, DK, c);
                const float av = expf(log_decay<PRO, GM>(la, lo));
                kc[i][e] = kv;
                Sacc[i][e] *= av;
                pa[nt] += kv * Sacc[i][e];
                pb[nt] += qv * Sacc[i][e];
                if (nt == 0) {   // each key channel once per wave
                    pqk += qv * kv;
                    if (PRO) {
                        pqq += qv * qv;
                        pkk += kv * kv;
                    }
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            pa[nt] += __shfl_xor(pa[nt], 16);
            pa[nt] += __shfl_xor(pa[nt], 32);
            pb[nt] += __shfl_xor(pb[nt], 16);
            pb[nt] += __shfl_xor(pb[nt], 32);
        }
        pqk += __shfl_xor(pqk, 16);
        pqk += __shfl_xor(pqk, 32);
        if (PRO) {
            pqq += __shfl_xor(pqq, 16);
            pqq += __shfl_xor(pqq, 32);
            pkk += __shfl_xor(pkk, 16);
            pkk += __shfl_xor(pkk, 32);
        }
        if (lg == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                red[w][nt * 16 + lr] = pa[nt];
                red[w][BV + nt * 16 + lr] = pb[nt];
            }
            if (lr == 0) {
                red[w][2 * BV] = pqk;
                if (PRO) {
                    red[w][2 * BV + 1] = pqq;
                    red[w][2 * BV + 2] = pkk;
                }
            }
        }
    }
    lds_barrier();
    if (w < 4) {
        float qk = red[0][2 * BV] + red[1][2 * BV] + red[2][2 * BV] + red[3][2 * BV];
        float bt = to_f32(beta[tk * H + h]);
        const float wt = DEC ? to_f32(wr[tk * H + h]) : 0.f;
        float iq = 1.f, ik = 1.f;
        if (PRO) {
            iq = pro_inv_norm(red[0][2 * BV + 1] + red[1][2 * BV + 1] + red[2][2 * BV + 1] + red[3][2 * BV + 1]);
            ik = pro_inv_norm(red[0][2 * BV + 2] + red[1][2 * BV + 2] + red[2][2 * BV + 2] + red[3][2 * BV + 2]);
            qk *= iq * ik;
            bt = pro_beta(bt);
        }
        float u[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int jl = nt * 16 + lr;
            float a = red[0][jl] + red[1][jl] + red[2][jl] + red[3][jl];
            float b = red[0][BV + jl] + red[1][BV + jl] + red[2][BV + jl] + red[3][BV + jl];
            if (PRO) {
                a *= ik;
                b *= iq;
            }
            const float vj = to_f32(v[(tk * H + h) * (int64_t)DV + col0 + jl]);
            u[nt] = DEC ? wt * vj - bt * a : bt * (vj - a);
            if (w == 0 && lg == 0) o[(tk * H + h) * (int64_t)DV + col0 + jl] = from_f32<IO>(b + u[nt] * qk);
            if (PRO) u[nt] *= ik;   // the state takes k_hat = k / |k|
        }
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int nt = (w * STW + i) % NT;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[i][e] += kc[i][e] * u[nt];
        }
    }
    lds_barrier();
}

// Raw inputs of one chunk held in registers (packed as loaded): wave w holds
// rows 8w..8w+7 of log_alpha, k and q for key channels l*CPL..; waves 4-7 hold
// the value rows their output tile needs; wave 0 holds beta (lane = token).
template <typename T, int N> struct VecT;
template <typename T> struct VecT<T, 1> { typedef T type; };
template <> struct VecT<bf16_t, 2> { typedef bf16x2_t type; };
template <> struct VecT<float, 2> { typedef float2 type; };
template <typename V> __device__ __forceinline__ float vget(const V &x, int i);
template <> __device__ __forceinline__ float vget<bf16_t>(const bf16_t &x, int) { return (float)x; }
template <> __device__ __forceinline__ float vget<float>(const float &x, int) { return x; }
template <> __device__ __forceinline__ float vget<bf16x2_t>(const bf16x2_t &x, int i) { return (float)x[i]; }
template <> __device__ __forceinline__ float vget<float2>(const float2 &x, int i) { return i ? x.y : x.x; }
template <typename V, typename S> __device__ __forceinline__ V vsplat(S x);
template <> __device__ __forceinline__ bf16_t vsplat<bf16_t, bf16_t>(bf16_t x) { return x; }
template <> __device__ __forceinline__ float vsplat<float, float>(float x) { return x; }
template <> __device__ __forceinline__ bf16x2_t vsplat<bf16x2_t, bf16_t>(bf16_t x) {
    bf16x2_t r;
    r[0] = x;
    r[1] = x;
    return r;
}
template <> __device__ __forceinline__ float2 vsplat<float2, float>(float x) { return make_float2(x, x); }

// With PRO (raw projections in) the accessors return the mapped inputs: gate()
// the floored -softplus (mapped once, at load), kval()/qval() the raw value
// times the per-token inverse norm (reduced over the wave, which holds whole
// rows), and bt is sigmoid(b).
template <int DK, int BV, typename IO, typename GT, bool PRO, int GM, bool DEC>
struct ChunkRegs {
    static constexpr int CPL = DK / 64, NT = BV / 16;
    typedef typename VecT<GT, CPL>::type GV;
    typedef typename VecT<IO, CPL>::type IV;
    GV la[8];
    IV kk[8], qq[8];
    float vv[NT][4];
    float bt, wt;   // wave 0, lane = token: beta and (DEC) the write strength
    float qs[PRO ? 8 : 1], ks[PRO ? 8 : 1];
    float lf[PRO ? 8 : 1][CPL];

    __device__ __forceinline__ float gate(int i, int cc) const {
        if constexpr (PRO) return lf[i][cc];
        else return vget(la[i], cc);
    }
    __device__ __forceinline__ float kval(int i, int cc) const {
        if constexpr (PRO) return vget(kk[i], cc) * ks[i];
        else return vget(kk[i], cc);
    }
    __device__ __forceinline__ float qval(int i, int cc) const {
        if constexpr (PRO) return vget(qq[i], cc) * qs[i];
        else return vget(qq[i], cc);
    }

    __device__ __forceinline__ void load(const IO *__restrict__ q, const IO *__restrict__ k,
                                         const IO *__restrict__ v, const GT *__restrict__ log_alpha,
                                         const GT *__restrict__ beta, const GT *__restrict__ wr, int64_t tbase,
                                         int nv, int H, int h, int DV, int col0, int w, int l, int lg, int lr,
                                         bool with_v = true) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * w + i;
            const int rr = r < nv ? r : nv - 1;
            const int64_t base = ((tbase + rr) * H + h) * (int64_t)DK + l * CPL;
            if constexpr (GM == kGatePerChannel) {
                la[i] = *reinterpret_cast<const GV *>(log_alpha + base);
            } else {   // one gate per (token, head), or none: the same value on every channel
                const GT g = GM == kGatePerHead ? log_alpha[(tbase + rr) * H + h] : (GT)0.f;
                la[i] = vsplat<GV>(g);
            }
            kk[i] = *reinterpret_cast<const IV *>(k + base);
            qq[i] = *reinterpret_cast<const IV *>(q + base);
        }
        if (with_v && w >= 4) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * (w - 4) + 4 * lg + e;
                    const int rr = r < nv ? r : nv - 1;
                    vv[nt][e] = to_f32(v[((tbase + rr) * H + h) * (int64_t)DV + col0 + nt * 16 + lr]);
                }
        }
        if (w == 0) bt = to_f32(beta[(tbase + (l < nv ? l : nv - 1)) * H + h]);
        if (DEC && w == 0) wt = to_f32(wr[(tbase + (l < nv ? l : nv - 1)) * H + h]);
    }

    // Rows past the end of a partial chunk as if absent: zero keys, queries and
    // (mapped) gates, so that they add nothing to any sum or product.  Called
    // after prepare() (which maps the gates) on partial chunks only.
    __device__ __forceinline__ void zero_tail(int nv, int w) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (8 * w + i >= nv) {
                la[i] = vsplat<GV>((GT)0.f);
                kk[i] = vsplat<IV>((IO)0.f);
                qq[i] = vsplat<IV>((IO)0.f);
                if constexpr (PRO) {
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) lf[i][cc] = 0.f;
                }
            }
        }
    }

    // The prologue maps of the loaded chunk (nothing without PRO); called once
    // per load, where the inputs are first used, so that a load issued ahead is
    // not waited for early.
    __device__ __forceinline__ void prepare(int w, float lo) {
        if constexpr (PRO) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float a = vget(qq[i], cc), b = vget(kk[i], cc);
                    sq += a * a;
                    sk += b * b;
                }
                qs[i] = pro_inv_norm(wave_sum(sq));
                ks[i] = pro_inv_norm(wave_sum(sk));
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) lf[i][cc] = log_decay<PRO, GM>(vget(la[i], cc), lo);
            }
            if (w == 0) bt = pro_beta(bt);
        }
    }
};

}  // namespace
}  // namespace kda
