// kda_chunk.hip -- chunkwise KDA forward (prefill), one fused kernel.
//
// Method (KimiLinear article, section 3.1: intra-chunk part by matrix products,
// inter-chunk part carried by the recurrent state; Kimi Linear abstract on the
// CoChat record: a specialised DPLR transition that needs one decay-weighted key
// Gram block per chunk).  For a chunk of n <= 64 tokens with start state S
// (d_k x d_v, fp32), rows r, i of the chunk and G = inclusive per-channel cumsum
// of log_alpha inside the chunk (g_n its last row):
//
//   A[r,i] = beta_r sum_c K[r,c] K[i,c] e^{G[r,c]-G[i,c]}   (i < r)
//   P[r,i] =        sum_c Q[r,c] K[i,c] e^{G[r,c]-G[i,c]}   (i <= r)
//   U      = (I + A)^{-1} diag(beta) (V - (K.e^G) S)        (UT transform)
//   O      = (Q.e^G) S + P U
//   S     <- Diag(e^{g_n}) S + (K.e^{g_n - G})^T U
//
// which unrolls the per-token update within the chunk exactly.  The exponent
// differences are split around a per-channel anchor m = g_n / 2:
//   e^{G_r - G_i} = e^{G_r - m} e^{m - G_i},
// so both factors lie in [e^{-D/2}, e^{D/2}] with D = max_c(-g_n).  While
// D <= 120 every factor is a normal fp32/bf16 number and the products run on the
// matrix cores; a chunk with a larger in-chunk decay (a near-reset gate) is
// processed token by token instead (exact, slow, never taken by ordinary gates).
// (K.e^G) S is formed as (K.e^{G-m}) (Diag(e^m) S) and K.e^{g_n-G} as
// (K.e^{m-G}) Diag(e^{g_n-m}), so one set of decayed operands serves all products.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head, block of BV
// value columns).  The value columns of the state evolve independently, so the
// blocks need no communication; the d_v-independent part (G, A, P, T) is
// recomputed per block.  The state block stays in fp32 registers for the whole
// sequence.
//
// Precision: products that feed the recurrence (S, T, X, U, P) always use
// hi/lo-split bf16 operands (hi*hi + hi*lo + lo*hi on the matrix cores).  With
// bf16 I/O the decayed key/query operands are single bf16; with fp32 I/O they
// are split too (SPLIT instances).  For fp32 I/O with d_k = 128 the split
// operands do not fit in LDS, and that instance runs the exact token-by-token
// update for every chunk.
#include "kda_device.h"
#include "kda_launch.h"

#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

namespace kda {
namespace {

constexpr int kC = 64;            // chunk length (tokens)
constexpr int kThreads = 256;     // 4 waves
constexpr float kMaxRange = 120.f;

template <int DK, int BV, bool SPLIT>
struct ChunkSmem {
    static constexpr int NP = SPLIT ? 2 : 1;   // planes of the decayed operands
    static constexpr int KS = DK + 8;          // padded stride of d_k-long bf16 rows
    static constexpr int TS = kC + 8;          // padded stride of token-long bf16 rows
    static constexpr int FS = 68;              // fp32 stride of 64x64 matrices (16 B aligned)
    bf16_t KA[NP][kC][KS];                     // K . e^{G-m}
    bf16_t QA[NP][kC][KS];                     // Q . e^{G-m}
    union {
        bf16_t KI[NP][kC][KS];                 // K . e^{m-G}: Gram phase only
        float Tf[kC][FS];                      // (I + A)^{-1} in fp32 while it is formed
        bf16_t U[2][BV][TS];                   // hi/lo of U^T, from the U phase on
    };
    bf16_t KIt[NP][DK][TS];                    // transpose of K . e^{m-G}
    union {
        float A[kC][FS];                       // beta-scaled strictly lower A (upper: scratch)
        bf16_t X[2][BV][TS];                   // hi/lo of X^T, X = diag(beta)(V - (K.e^G) S)
    };
    bf16_t T[2][kC][TS];                       // hi/lo of (I + A)^{-1}
    bf16_t P[2][kC][TS];                       // hi/lo of P
    bf16_t S[2][BV][KS];                       // hi/lo of (Diag(e^m) S)^T, this column block
    float beta[kC];
    float colM[DK];                            // e^{m}
    float colGn[DK];                           // e^{g_n}
    float colGnM[DK];                          // e^{g_n - m}
    float tot[4][DK];                          // per-16-row-block sums of log_alpha
    float red[4][2 * BV + 1];                  // token path: cross-wave partial sums
};

template <int BV>
struct ExactSmem {
    float red[4][2 * BV + 1];
};

// The 10 lower 16x16 blocks (R, I), I <= R, of a 64x64 chunk matrix:
// (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3).
__device__ __forceinline__ void lower_block(int idx, int &R, int &I) {
    R = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    I = idx - (R * (R + 1)) / 2;
}

template <bool ACCURATE>
__device__ __forceinline__ float kexp(float x) {
    return ACCURATE ? expf(x) : __expf(x);
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

// One exact token update of this workgroup's state block (the per-token rule of
// the KimiLinear article, section 2.3, with the read-out o = S^T q).  The state
// is in the MFMA accumulator layout: wave w, tile mt holds key rows
// (w*MT+mt)*16 + 4*lg + e and value column col0 + nt*16 + lr.
template <int DK, int BV, typename IO, typename GT>
__device__ __forceinline__ void token_update(f32x4_t (&Sacc)[DK / 64][BV / 16], float (*red)[2 * BV + 1],
                                             const IO *__restrict__ q, const IO *__restrict__ k,
                                             const IO *__restrict__ v, const GT *__restrict__ log_alpha,
                                             const GT *__restrict__ beta, IO *__restrict__ o, int64_t tk,
                                             int H, int h, int DV, int col0, int w, int lg, int lr) {
    constexpr int MT = DK / 64, NT = BV / 16;
    const int64_t kb = (tk * H + h) * (int64_t)DK;
    float kc[MT][4], qc[MT][4], ac[MT][4];
    float pqk = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = (w * MT + mt) * 16 + 4 * lg + e;
            kc[mt][e] = to_f32(k[kb + c]);
            qc[mt][e] = to_f32(q[kb + c]);
            ac[mt][e] = expf(to_f32(log_alpha[kb + c]));
            pqk += qc[mt][e] * kc[mt][e];
        }
    float pa[NT], pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        pa[nt] = 0.f;
        pb[nt] = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Sacc[mt][nt][e] *= ac[mt][e];
                pa[nt] += kc[mt][e] * Sacc[mt][nt][e];
                pb[nt] += qc[mt][e] * Sacc[mt][nt][e];
            }
        pa[nt] += __shfl_xor(pa[nt], 16);
        pa[nt] += __shfl_xor(pa[nt], 32);
        pb[nt] += __shfl_xor(pb[nt], 16);
        pb[nt] += __shfl_xor(pb[nt], 32);
    }
    pqk += __shfl_xor(pqk, 16);
    pqk += __shfl_xor(pqk, 32);
    if (lg == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            red[w][nt * 16 + lr] = pa[nt];
            red[w][BV + nt * 16 + lr] = pb[nt];
        }
        if (lr == 0) red[w][2 * BV] = pqk;
    }
    __syncthreads();
    const float qk = red[0][2 * BV] + red[1][2 * BV] + red[2][2 * BV] + red[3][2 * BV];
    const float bt = to_f32(beta[tk * H + h]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int jl = nt * 16 + lr;
        const float a = red[0][jl] + red[1][jl] + red[2][jl] + red[3][jl];
        const float b = red[0][BV + jl] + red[1][BV + jl] + red[2][BV + jl] + red[3][BV + jl];
        const float u = bt * (to_f32(v[(tk * H + h) * (int64_t)DV + col0 + jl]) - a);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[mt][nt][e] += kc[mt][e] * u;
        if (w == 0 && lg == 0) o[(tk * H + h) * (int64_t)DV + col0 + jl] = from_f32<IO>(b + u * qk);
    }
    __syncthreads();
}

template <int DK, int BV, typename IO, typename GT, bool SPLIT, bool EXACT>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const float *__restrict__ h0,
    const int32_t *__restrict__ cu_seqlens, IO *__restrict__ o, float *__restrict__ h_T,
    int64_t seq_len, int32_t H, int32_t DV, int64_t num_chains) {
    constexpr int CPL = DK / 64;    // key channels per lane in the load phase
    constexpr int NKS = DK / 32;    // 32-wide k-steps over d_k
    constexpr int MT = DK / 64;     // 16-row state tiles per wave
    constexpr int NT = BV / 16;     // 16-column tiles per block
    typedef ChunkSmem<DK, BV, SPLIT> Sm;
    typedef typename std::conditional<EXACT, ExactSmem<BV>, Sm>::type Smem;
    __shared__ Smem smem;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lg = l >> 4;   // MFMA row/col within tile, lane group

    const int64_t wg = blockIdx.x;
    const int64_t chain = wg % num_chains;
    const int jb = (int)(wg / num_chains);
    const int64_t n = chain / H;
    const int h = (int)(chain % H);
    int64_t bos, eos;
    if (cu_seqlens) {
        bos = cu_seqlens[n];
        eos = cu_seqlens[n + 1];
    } else {
        bos = n * seq_len;
        eos = bos + seq_len;
    }
    const int col0 = jb * BV;   // first value column of this block

    // ---- state block in registers (MFMA accumulator layout) ------------------
    f32x4_t Sacc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = (w * MT + mt) * 16 + 4 * lg + e;
                const int j = col0 + nt * 16 + lr;
                Sacc[mt][nt][e] = h0 ? h0[((n * H + h) * DK + c) * (int64_t)DV + j] : 0.f;
            }

    if constexpr (EXACT) {
        for (int64_t tk = bos; tk < eos; ++tk)
            token_update<DK, BV, IO, GT>(Sacc, smem.red, q, k, v, log_alpha, beta, o, tk, H, h, DV, col0, w,
                                         lg, lr);
    } else {
        Sm &sm = smem;
        // Upper blocks of T and P are never written: zero them once.
        for (int idx = tid; idx < 2 * kC * Sm::TS; idx += kThreads) {
            (&sm.T[0][0][0])[idx] = (bf16_t)0.f;
            (&sm.P[0][0][0])[idx] = (bf16_t)0.f;
        }

        for (int64_t tbase = bos; tbase < eos; tbase += kC) {
            const int nv = (int)((eos - tbase) < kC ? (eos - tbase) : kC);
            __syncthreads();

            // ======== phase L: cumsum of log_alpha, anchors, decayed operands ========
            // All global loads of the chunk are issued here, unconditionally: rows
            // past the end of the sequence read the last valid row and are zeroed
            // afterwards, so no load sits behind a branch and they overlap.
            const int r0 = 16 * w;
            float g[16][CPL];
            IO kraw[16][CPL], qraw[16][CPL];
            float vraw[NT][4];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = r0 + i;
                const int rr = r < nv ? r : nv - 1;
                const int64_t base = ((tbase + rr) * H + h) * (int64_t)DK + l * CPL;
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    g[i][cc] = to_f32(log_alpha[base + cc]);
                    kraw[i][cc] = k[base + cc];
                    qraw[i][cc] = q[base + cc];
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * lg + e;
                    const int rr = r < nv ? r : nv - 1;
                    vraw[nt][e] = to_f32(v[((tbase + rr) * H + h) * (int64_t)DV + col0 + nt * 16 + lr]);
                }
            const float bload = to_f32(beta[(tbase + (l < nv ? l : nv - 1)) * H + h]);
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) g[i][cc] = (r0 + i < nv) ? g[i][cc] : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) g[i][cc] += g[i - 1][cc];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) sm.tot[w][l * CPL + cc] = g[15][cc];
            if (w == 0) sm.beta[l] = (l < nv) ? bload : 0.f;
            __syncthreads();
            float m[CPL], gn[CPL];
            float dmax = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int c = l * CPL + cc;
                const float t0 = sm.tot[0][c], t1 = sm.tot[1][c], t2 = sm.tot[2][c], t3 = sm.tot[3][c];
                const float pre = (w > 0 ? t0 : 0.f) + (w > 1 ? t1 : 0.f) + (w > 2 ? t2 : 0.f);
                gn[cc] = ((t0 + t1) + t2) + t3;
                m[cc] = 0.5f * gn[cc];
#pragma unroll
                for (int i = 0; i < 16; ++i) g[i][cc] += pre;
                dmax = fmaxf(dmax, -gn[cc]);
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, off));
            const bool slow = !(dmax <= kMaxRange);   // uniform over the workgroup; catches NaN

            if (w == 0) {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const int c = l * CPL + cc;
                    sm.colM[c] = kexp<SPLIT>(m[cc]);
                    sm.colGn[c] = kexp<SPLIT>(gn[cc]);
                    sm.colGnM[c] = kexp<SPLIT>(gn[cc] - m[cc]);
                }
            }

            if (!slow) {
                bf16_t kit[Sm::NP][CPL][16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = r0 + i;
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        const int c = l * CPL + cc;
                        const float kv = (r < nv) ? to_f32(kraw[i][cc]) : 0.f;
                        const float qv = (r < nv) ? to_f32(qraw[i][cc]) : 0.f;
                        const float e1 = kexp<SPLIT>(g[i][cc] - m[cc]);
                        const float e2 = kexp<SPLIT>(m[cc] - g[i][cc]);
                        const float ka = kv * e1, qa = qv * e1, ki = kv * e2;
                        if constexpr (SPLIT) {
                            bf16_t hh, ll;
                            split_bf16(ka, hh, ll); sm.KA[0][r][c] = hh; sm.KA[1][r][c] = ll;
                            split_bf16(qa, hh, ll); sm.QA[0][r][c] = hh; sm.QA[1][r][c] = ll;
                            split_bf16(ki, hh, ll); sm.KI[0][r][c] = hh; sm.KI[1][r][c] = ll;
                            kit[0][cc][i] = hh;
                            kit[1][cc][i] = ll;
                        } else {
                            sm.KA[0][r][c] = (bf16_t)ka;
                            sm.QA[0][r][c] = (bf16_t)qa;
                            const bf16_t kib = (bf16_t)ki;
                            sm.KI[0][r][c] = kib;
                            kit[0][cc][i] = kib;
                        }
                    }
                }
#pragma unroll
                for (int pl = 0; pl < Sm::NP; ++pl)
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        bf16x8_t lo8, hi8;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            lo8[i] = kit[pl][cc][i];
                            hi8[i] = kit[pl][cc][8 + i];
                        }
                        *reinterpret_cast<bf16x8_t *>(&sm.KIt[pl][l * CPL + cc][r0]) = lo8;
                        *reinterpret_cast<bf16x8_t *>(&sm.KIt[pl][l * CPL + cc][r0 + 8]) = hi8;
                    }
            }
            __syncthreads();

            if (slow) {
                // exact token-by-token path for a chunk with a huge in-chunk decay
                for (int r = 0; r < nv; ++r)
                    token_update<DK, BV, IO, GT>(Sacc, sm.red, q, k, v, log_alpha, beta, o, tbase + r, H, h,
                                                 DV, col0, w, lg, lr);
                continue;
            }

            // ======== phase AP: S' = Diag(e^m) S (hi/lo), Gram blocks A and P ========
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int c = (w * MT + mt) * 16 + 4 * lg;
                    bf16x4_t hi, lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bf16_t hh, ll;
                        split_bf16(sm.colM[c + e] * Sacc[mt][nt][e], hh, ll);
                        hi[e] = hh;
                        lo[e] = ll;
                    }
                    *reinterpret_cast<bf16x4_t *>(&sm.S[0][nt * 16 + lr][c]) = hi;
                    *reinterpret_cast<bf16x4_t *>(&sm.S[1][nt * 16 + lr][c]) = lo;
                }
            for (int tile = w; tile < 20; tile += 4) {
                const bool isP = tile >= 10;
                int R, I;
                lower_block(isP ? tile - 10 : tile, R, I);
                const bf16_t *ah = isP ? &sm.QA[0][16 * R + lr][8 * lg] : &sm.KA[0][16 * R + lr][8 * lg];
                const bf16_t *al = ah + (SPLIT ? kC * Sm::KS : 0);
                const bf16_t *bh = &sm.KI[0][16 * I + lr][8 * lg];
                const bf16_t *bl = bh + (SPLIT ? kC * Sm::KS : 0);
                f32x4_t acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = mma<SPLIT, SPLIT>(acc, ah + 32 * ks, al + 32 * ks, bh + 32 * ks, bl + 32 * ks);
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
            __syncthreads();

            // ======== phase T: (I + A)^{-1} by blocked forward substitution (fp32) ========
            {
                // T1: diagonal 16x16 blocks, one per wave; lane j < 16 solves column j.
                const int R = w;
                const int j = lr;
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                    for (int mm = 0; mm < r; ++mm) s -= sm.A[16 * R + r][16 * R + mm] * t[mm];
                    t[r] = s;
                }
                if (lg == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        sm.Tf[16 * R + r][16 * R + j] = t[r];
#pragma unroll
                        for (int I = R + 1; I < 4; ++I) sm.Tf[16 * R + r][16 * I + j] = 0.f;
                    }
                }
            }
            __syncthreads();
            // T2: T[R+1][R] = -T[R+1][R+1] A[R+1][R] T[R][R] for R = 0, 2 (waves 0, 1);
            // the product A[R+1][R] T[R][R] is staged in A's unused block (R, R+1).
            if (w < 2) {
                const int R = 2 * w;
                float (*Wsc)[Sm::FS] = reinterpret_cast<float (*)[Sm::FS]>(&sm.A[16 * R][16 * (R + 1)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * lg + e;
                    float s = 0.f;
#pragma unroll
                    for (int mm = 0; mm < 16; ++mm)
                        s += sm.A[16 * (R + 1) + r][16 * R + mm] * sm.Tf[16 * R + mm][16 * R + lr];
                    Wsc[r][lr] = s;
                }
            }
            __syncthreads();
            if (w < 2) {
                const int R = 2 * w;
                float (*Wsc)[Sm::FS] = reinterpret_cast<float (*)[Sm::FS]>(&sm.A[16 * R][16 * (R + 1)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * lg + e;
                    float s = 0.f;
#pragma unroll
                    for (int mm = 0; mm < 16; ++mm) s += sm.Tf[16 * (R + 1) + r][16 * (R + 1) + mm] * Wsc[mm][lr];
                    sm.Tf[16 * (R + 1) + r][16 * R + lr] = -s;
                }
            }
            __syncthreads();
            // T3: lower-left 32x32 = -T[23][23] A[23][01] T[01][01]; A's upper-right 32x32 is scratch.
            {
                const int r = tid >> 3;          // 0..31
                const int j4 = 4 * (tid & 7);    // 0..28
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
                for (int mm = 0; mm < 32; ++mm) {
                    const float a = sm.A[32 + r][mm];
                    const float4 tv = *reinterpret_cast<const float4 *>(&sm.Tf[mm][j4]);
                    s0 += a * tv.x; s1 += a * tv.y; s2 += a * tv.z; s3 += a * tv.w;
                }
                float4 wv = {s0, s1, s2, s3};
                *reinterpret_cast<float4 *>(&sm.A[r][32 + j4]) = wv;
            }
            __syncthreads();
            {
                const int r = tid >> 3;
                const int j4 = 4 * (tid & 7);
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
                for (int mm = 0; mm < 32; ++mm) {
                    const float a = sm.Tf[32 + r][32 + mm];
                    const float4 wv = *reinterpret_cast<const float4 *>(&sm.A[mm][32 + j4]);
                    s0 += a * wv.x; s1 += a * wv.y; s2 += a * wv.z; s3 += a * wv.w;
                }
                float4 tv = {-s0, -s1, -s2, -s3};
                *reinterpret_cast<float4 *>(&sm.Tf[32 + r][j4]) = tv;
            }
            __syncthreads();

            // ======== phase Y: Y = (K.e^G) S, Z = (Q.e^G) S; X = diag(beta)(V - Y); T -> hi/lo ========
            for (int idx = tid; idx < kC * kC; idx += kThreads) {
                const int r = idx >> 6, i = idx & 63;
                if ((i >> 4) <= (r >> 4)) {
                    bf16_t hh, ll;
                    split_bf16(sm.Tf[r][i], hh, ll);
                    sm.T[0][r][i] = hh;
                    sm.T[1][r][i] = ll;
                }
            }
            f32x4_t accZ[NT], accY[NT];
            {
                const bf16_t *kah = &sm.KA[0][16 * w + lr][8 * lg];
                const bf16_t *qah = &sm.QA[0][16 * w + lr][8 * lg];
                const bf16_t *kal = kah + (SPLIT ? kC * Sm::KS : 0);
                const bf16_t *qal = qah + (SPLIT ? kC * Sm::KS : 0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16_t *sh = &sm.S[0][nt * 16 + lr][8 * lg];
                    const bf16_t *sl = &sm.S[1][nt * 16 + lr][8 * lg];
                    accY[nt] = zero4();
                    accZ[nt] = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int o32 = 32 * ks;
                        accY[nt] = mma<SPLIT, true>(accY[nt], kah + o32, kal + o32, sh + o32, sl + o32);
                        accZ[nt] = mma<SPLIT, true>(accZ[nt], qah + o32, qal + o32, sh + o32, sl + o32);
                    }
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int jl = nt * 16 + lr;
                bf16x4_t hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * lg + e;
                    const float vv = (r < nv) ? vraw[nt][e] : 0.f;
                    bf16_t hh, ll;
                    split_bf16(sm.beta[r] * (vv - accY[nt][e]), hh, ll);
                    hi[e] = hh;
                    lo[e] = ll;
                }
                *reinterpret_cast<bf16x4_t *>(&sm.X[0][jl][16 * w + 4 * lg]) = hi;
                *reinterpret_cast<bf16x4_t *>(&sm.X[1][jl][16 * w + 4 * lg]) = lo;
            }
            __syncthreads();

            // ======== phase U: U = T X ========
            {
                const int nks = (w >> 1) + 1;
                const bf16_t *th = &sm.T[0][16 * w + lr][8 * lg];
                const bf16_t *tl = &sm.T[1][16 * w + lr][8 * lg];
                f32x4_t accU[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16_t *xh = &sm.X[0][nt * 16 + lr][8 * lg];
                    const bf16_t *xl = &sm.X[1][nt * 16 + lr][8 * lg];
                    accU[nt] = zero4();
                    for (int ks = 0; ks < nks; ++ks)
                        accU[nt] = mma<true, true>(accU[nt], th + 32 * ks, tl + 32 * ks, xh + 32 * ks, xl + 32 * ks);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int jl = nt * 16 + lr;
                    bf16x4_t hi, lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bf16_t hh, ll;
                        split_bf16(accU[nt][e], hh, ll);
                        hi[e] = hh;
                        lo[e] = ll;
                    }
                    *reinterpret_cast<bf16x4_t *>(&sm.U[0][jl][16 * w + 4 * lg]) = hi;
                    *reinterpret_cast<bf16x4_t *>(&sm.U[1][jl][16 * w + 4 * lg]) = lo;
                }
            }
            __syncthreads();

            // ======== phase O: O = Z + P U (store); phase S: state update ========
            {
                const int nks = (w >> 1) + 1;
                const bf16_t *ph = &sm.P[0][16 * w + lr][8 * lg];
                const bf16_t *pl = &sm.P[1][16 * w + lr][8 * lg];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16_t *uh = &sm.U[0][nt * 16 + lr][8 * lg];
                    const bf16_t *ul = &sm.U[1][nt * 16 + lr][8 * lg];
                    f32x4_t acc = accZ[nt];
                    for (int ks = 0; ks < nks; ++ks)
                        acc = mma<true, true>(acc, ph + 32 * ks, pl + 32 * ks, uh + 32 * ks, ul + 32 * ks);
                    const int jl = nt * 16 + lr;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * w + 4 * lg + e;
                        if (r < nv) o[((tbase + r) * H + h) * (int64_t)DV + col0 + jl] = from_f32<IO>(acc[e]);
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int c16 = (w * MT + mt) * 16;
                const bf16_t *kh = &sm.KIt[0][c16 + lr][8 * lg];
                const bf16_t *kl = kh + (SPLIT ? DK * Sm::TS : 0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16_t *uh = &sm.U[0][nt * 16 + lr][8 * lg];
                    const bf16_t *ul = &sm.U[1][nt * 16 + lr][8 * lg];
                    f32x4_t acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc = mma<SPLIT, true>(acc, kh + 32 * ks, kl + 32 * ks, uh + 32 * ks, ul + 32 * ks);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = c16 + 4 * lg + e;
                        Sacc[mt][nt][e] = sm.colGn[c] * Sacc[mt][nt][e] + sm.colGnM[c] * acc[e];
                    }
                }
            }
        }
    }

    if (h_T) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = (w * MT + mt) * 16 + 4 * lg + e;
                    const int j = col0 + nt * 16 + lr;
                    h_T[((n * H + h) * DK + c) * (int64_t)DV + j] = Sacc[mt][nt][e];
                }
    }
}

template <int DK, int BV, typename IO, typename GT, bool SPLIT, bool EXACT>
hipError_t launch_t(const ChunkArgs &a, hipStream_t st) {
    const int64_t chains = a.num_seqs * (int64_t)a.H;
    const int64_t nwg = chains * (a.d_v / BV);
    hipLaunchKernelGGL((chunk_fwd_kernel<DK, BV, IO, GT, SPLIT, EXACT>), dim3((unsigned)nwg), dim3(kThreads), 0,
                       st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v, (const GT *)a.log_alpha,
                       (const GT *)a.beta, a.h0, a.cu_seqlens, (IO *)a.o, a.h_T, a.seq_len, a.H, a.d_v, chains);
    return hipGetLastError();
}

// bf16 I/O: single-bf16 decayed operands.  fp32 I/O: split operands (d_k = 64)
// or the exact token path (d_k = 128).
template <int DK, int BV>
hipError_t launch_types(const ChunkArgs &a, hipStream_t st) {
    if (a.io_bf16)
        return a.gate_bf16 ? launch_t<DK, BV, bf16_t, bf16_t, false, false>(a, st)
                           : launch_t<DK, BV, bf16_t, float, false, false>(a, st);
    constexpr bool EX = DK == 128;
    return a.gate_bf16 ? launch_t<DK, BV, float, bf16_t, !EX, EX>(a, st)
                       : launch_t<DK, BV, float, float, !EX, EX>(a, st);
}

// Value-column block width: 32 when that still gives at least two workgroups
// per compute unit (less recomputation of the d_v-independent part), else 16.
// LIBKDA_BLOCK_V=16|32 overrides the choice (used by the tests to cover both).
int pick_block_v(const ChunkArgs &a) {
    const char *env = getenv("LIBKDA_BLOCK_V");
    const int forced = env ? atoi(env) : 0;
    if (forced == 16 || forced == 32) return forced;
    const int64_t chains = a.num_seqs * (int64_t)a.H;
    return chains * (a.d_v / 32) >= 512 ? 32 : 16;
}

}  // namespace

size_t chunk_fwd_workspace_bytes(int64_t, int32_t, int32_t, int32_t, int64_t) { return 0; }

int launch_chunk_fwd(const ChunkArgs &a, void *stream, char *err, size_t err_len) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t nwg = a.num_seqs * (int64_t)a.H * (a.d_v / 16);
    if (nwg > 0x7fffffffLL) {
        snprintf(err, err_len, "chunk_fwd grid too large");
        return -1;
    }
    const int bv = pick_block_v(a);
    hipError_t e;
    if (a.d_k == 128)
        e = bv == 32 ? launch_types<128, 32>(a, st) : launch_types<128, 16>(a, st);
    else
        e = bv == 32 ? launch_types<64, 32>(a, st) : launch_types<64, 16>(a, st);
    if (e != hipSuccess) {
        snprintf(err, err_len, "%s", hipGetErrorString(e));
        return -1;
    }
    return 0;
}

}  // namespace kda
