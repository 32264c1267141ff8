// kda_chunk.hip -- chunkwise KDA forward (prefill), one fused kernel.
// This kernel serves fp32 I/O at d_k = 64 (and a call without tokens that only
// passes h0 on to h_T); bf16 I/O runs the kernels of kda_chunk2.hip and
// kda_fused.hip, fp32 I/O at d_k = 128 those of kda_bwd.hip.
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
// D <= 80 every factor (and every single-token gate) is a normal fp32/bf16
// number and the products run on the matrix cores; a chunk with a larger
// in-chunk decay (a near-reset gate) is processed token by token instead (exact,
// slower, not taken by ordinary gates).  (K.e^G) S is formed as
// (K.e^{G-m}) (Diag(e^m) S) and K.e^{g_n-G} as (K.e^{m-G}) Diag(e^{g_n-m}), so
// one set of decayed operands serves every product.
//
// Work decomposition: one workgroup of 8 waves per (sequence, head, block of BV
// value columns).  The value columns of the state evolve independently, so the
// blocks need no communication; the d_v-independent part (G, A, P, T) is
// recomputed per block.  Waves 0-3 hold the state block in fp32 registers for
// the whole sequence; waves 4-7 form (K.e^G)S and (Q.e^G)S and the output while
// waves 0-3 invert the diagonal blocks of (I + A) and update the state.  The
// next chunk's inputs are loaded into registers while the current one is
// processed.
//
// Precision: products that feed the recurrence (T, X, U, P) use hi/lo-split
// bf16 operands (hi*hi + hi*lo + lo*hi on the matrix cores).  With bf16 I/O the
// decayed key/query operands and Diag(e^m) S are single bf16; with fp32 I/O they
// are split too (SPLIT instances).  fp32 I/O at d_k = 128 does not come here:
// the split operands would not fit in LDS, and it runs chunkwise on the fp32
// matrix cores instead (kda_bwd.hip).
#include "kda_chunk_common.h"
#include "kda_launch.h"

#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

namespace kda {
namespace {


template <int DK, int BV, bool SPLIT>
struct alignas(16) ChunkSmem {
    static constexpr int NP = SPLIT ? 2 : 1;   // planes of the decayed operands and of S'
    static constexpr int KS = DK + 8;          // padded stride of d_k-long bf16 rows
    static constexpr int TS = kC + 8;          // padded stride of token-long bf16 rows
    static constexpr int FS = 68;              // fp32 stride of 64x64 matrices (16 B aligned)
    bf16_t KA[NP][kC][KS];                     // K . e^{G-m}
    bf16_t QA[NP][kC][KS];                     // Q . e^{G-m}
    union {
        bf16_t KI[NP][kC][KS];                 // K . e^{m-G}: Gram phase only
        bf16_t Tt[2][kC][kC + 4];              // hi/lo of (I + A)^{-1}, transposed (diagonal blocks)
    };
    bf16_t KIt[NP][DK][TS];                    // transpose of K . e^{m-G}
    union {
        float A[kC][FS];                       // beta-scaled strictly lower A (upper: scratch)
        bf16_t U[2][BV][TS];                   // hi/lo of U^T, after the inversion
    };
    bf16_t X[2][BV][TS];                       // hi/lo of X^T, X = diag(beta)(V - (K.e^G) S)
    bf16_t T[2][kC][TS];                       // hi/lo of (I + A)^{-1}
    bf16_t P[2][kC][TS];                       // hi/lo of P
    bf16_t S[NP][BV][KS];                      // (Diag(e^m) S)^T of this column block
    float beta[kC];
    float wr[kC];                              // separate write strengths (DEC)
    float colM[DK];                            // e^{m}
    float colGn[DK];                           // e^{g_n}
    float colGnM[DK];                          // e^{g_n - m}
    float tot[DK][kWaves];                     // per-8-row sums of log2(alpha)
    float red[4][TokenRed<BV>::N];             // token path: cross-wave partial sums
    float T8[4][2][8][8];                      // 8x8 diagonal inverses, per wave
    float W8[4][8][8];                         // 8x8 merge scratch, per wave
};

// PRO: q, k, log_alpha and beta are raw projections, mapped as they are read
// (input prologue; lo is the floor of log alpha).
template <int DK, int BV, typename IO, typename GT, bool SPLIT, bool PRO, int GM, bool DEC>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const GT *__restrict__ wr,
    const float *__restrict__ h0,
    const int32_t *__restrict__ cu_seqlens, IO *__restrict__ o, float *__restrict__ h_T,
    int64_t seq_len, int32_t H, int32_t DV, int64_t num_chains, float lo) {
    constexpr int CPL = DK / 64;    // key channels per lane in the load phase
    constexpr int NKS = DK / 32;    // 32-wide k-steps over d_k
    constexpr int NT = BV / 16;     // 16-column tiles per block
    constexpr int STW = StateTiles<DK, BV>::STW;
    typedef ChunkSmem<DK, BV, SPLIT> Sm;
    __shared__ Sm smem;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
    const int l = tid & 63;
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

    // ---- state block in registers of waves 0-3 ---------------------------------
    f32x4_t Sacc[STW];
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w * STW + i, mt = st / NT, nt = st % NT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * mt + 4 * lg + e;
            const int j = col0 + nt * 16 + lr;
            Sacc[i][e] = (h0 && w < 4) ? h0[((n * H + h) * DK + c) * (int64_t)DV + j] : 0.f;
        }
    }

    {
        Sm &sm = smem;
        // Upper blocks of T and P are never written: zero them once.
        for (int idx = tid; idx < 2 * kC * Sm::TS; idx += kThreads) {
            (&sm.T[0][0][0])[idx] = (bf16_t)0.f;
            (&sm.P[0][0][0])[idx] = (bf16_t)0.f;
        }
        ChunkRegs<DK, BV, IO, GT, PRO, GM, DEC> in;
        if (bos < eos) {
            const int nv0 = (int)((eos - bos) < kC ? (eos - bos) : kC);
            in.load(q, k, v, log_alpha, beta, wr, bos, nv0, H, h, DV, col0, w, l, lg, lr);
        }
        f32x4_t accZ[NT];

        for (int64_t tbase = bos; tbase < eos; tbase += kC) {
            const int nv = (int)((eos - tbase) < kC ? (eos - tbase) : kC);
            // Lane indices are re-derived from an opaque copy of the thread id each
            // chunk, so the compiler recomputes LDS addresses here instead of keeping
            // dozens of them live across the whole loop (which spills).
            int tl_;
            asm volatile("v_mov_b32 %0, %1" : "=v"(tl_) : "v"(tid));
            const int l = tl_ & 63, lr = l & 15, lg = l >> 4;
            const bool has_next = tbase + kC < eos;
            const int nv_next = has_next ? (int)((eos - tbase - kC) < kC ? (eos - tbase - kC) : kC) : 0;
            lds_barrier();

            // ======== phase L: log2-decay cumsum, anchors, decayed operands ========
            in.prepare(w, lo);
            const bool partial = nv < kC;
            float csum[8][CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float x = in.gate(i, cc) * kLog2e;
                    if (partial && 8 * w + i >= nv) x = 0.f;
                    csum[i][cc] = i ? csum[i - 1][cc] + x : x;
                }
                sm.tot[l * CPL + cc][w] = csum[7][cc];
            }
            float vcur[NT][4];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) vcur[nt][e] = in.vv[nt][e];
            if (w == 0) sm.beta[l] = (l < nv) ? in.bt : 0.f;
            if (DEC && w == 0) sm.wr[l] = (l < nv) ? in.wt : 0.f;
            lds_barrier();
            float m2[CPL];
            bool big = false;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int c = l * CPL + cc;
                const float4 ta = reinterpret_cast<const float4 *>(&sm.tot[c][0])[0];
                const float4 tb = reinterpret_cast<const float4 *>(&sm.tot[c][0])[1];
                const float tw[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
                float pre = 0.f, all = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    all += tw[ww];
                    if (ww < w) pre += tw[ww];
                }
                m2[cc] = 0.5f * all;
#pragma unroll
                for (int i = 0; i < 8; ++i) csum[i][cc] += pre;
                big = big || !(-all <= kMaxRange2);   // also true for NaN
                if (w == 0) {
                    sm.colM[c] = kexp2<SPLIT>(m2[cc]);
                    sm.colGn[c] = kexp2<SPLIT>(all);
                    sm.colGnM[c] = kexp2<SPLIT>(all - m2[cc]);
                }
            }
            // Every wave sees the same totals, so this vote is uniform over the workgroup.
            const bool slow = __ballot(big) != 0;

            if (!slow) {
                // e1[i] = 2^{G[i]-m}, e2[i] = 2^{m-G[i]}: one exact exp at each end of
                // the wave's 8 rows, then products with alpha = 2^{lam} (|.| <= 2^{58}).
                float e1[8][CPL], e2[8][CPL];
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    float al[8];
#pragma unroll
                    for (int i = 1; i < 8; ++i) {
                        float x = in.gate(i, cc) * kLog2e;
                        if (partial && 8 * w + i >= nv) x = 0.f;
                        al[i] = kexp2<SPLIT>(x);
                    }
                    e1[0][cc] = kexp2<SPLIT>(csum[0][cc] - m2[cc]);
#pragma unroll
                    for (int i = 1; i < 8; ++i) e1[i][cc] = e1[i - 1][cc] * al[i];
                    e2[7][cc] = kexp2<SPLIT>(m2[cc] - csum[7][cc]);
#pragma unroll
                    for (int i = 6; i >= 0; --i) e2[i][cc] = e2[i + 1][cc] * al[i + 1];
                }
                if (partial) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (8 * w + i >= nv) {
#pragma unroll
                            for (int cc = 0; cc < CPL; ++cc) e1[i][cc] = e2[i][cc] = 0.f;
                        }
                }
                bf16x8_t kit[Sm::NP][CPL];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * w + i;
                    float ka[CPL], qa[CPL], ki[CPL];
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        const float kv = in.kval(i, cc), qv = in.qval(i, cc);
                        ka[cc] = kv * e1[i][cc];
                        qa[cc] = qv * e1[i][cc];
                        ki[cc] = kv * e2[i][cc];
                    }
                    if constexpr (SPLIT) {
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) {
                            const int c = l * CPL + cc;
                            bf16_t hh, ll;
                            split_bf16(ka[cc], hh, ll); sm.KA[0][r][c] = hh; sm.KA[1][r][c] = ll;
                            split_bf16(qa[cc], hh, ll); sm.QA[0][r][c] = hh; sm.QA[1][r][c] = ll;
                            split_bf16(ki[cc], hh, ll); sm.KI[0][r][c] = hh; sm.KI[1][r][c] = ll;
                            kit[0][cc][i] = hh;
                            kit[Sm::NP - 1][cc][i] = ll;
                        }
                    } else if constexpr (CPL == 2) {
                        bf16x2_t p;
                        p[0] = (bf16_t)ka[0]; p[1] = (bf16_t)ka[1];
                        *reinterpret_cast<bf16x2_t *>(&sm.KA[0][r][2 * l]) = p;
                        p[0] = (bf16_t)qa[0]; p[1] = (bf16_t)qa[1];
                        *reinterpret_cast<bf16x2_t *>(&sm.QA[0][r][2 * l]) = p;
                        p[0] = (bf16_t)ki[0]; p[1] = (bf16_t)ki[1];
                        *reinterpret_cast<bf16x2_t *>(&sm.KI[0][r][2 * l]) = p;
                        kit[0][0][i] = p[0];
                        kit[0][1][i] = p[1];
                    } else {
                        sm.KA[0][r][l] = (bf16_t)ka[0];
                        sm.QA[0][r][l] = (bf16_t)qa[0];
                        const bf16_t kib = (bf16_t)ki[0];
                        sm.KI[0][r][l] = kib;
                        kit[0][0][i] = kib;
                    }
                }
#pragma unroll
                for (int pl = 0; pl < Sm::NP; ++pl)
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc)
                        *reinterpret_cast<bf16x8_t *>(&sm.KIt[pl][l * CPL + cc][8 * w]) = kit[pl][cc];
            }
            // the next chunk's inputs go in flight now
            if (has_next) in.load(q, k, v, log_alpha, beta, wr, tbase + kC, nv_next, H, h, DV, col0, w, l, lg, lr);
            lds_barrier();

            if (slow) {
                // exact token-by-token path for a chunk with a huge in-chunk decay
                for (int r = 0; r < nv; ++r)
                    token_update<DK, BV, IO, GT, PRO, GM, DEC>(Sacc, sm.red, q, k, v, log_alpha, beta, wr, o,
                                                               tbase + r, H, h, DV, col0, w, lg, lr, lo);
                continue;
            }

            // ======== phase AP: S' = Diag(e^m) S, Gram blocks A and P ========
            if (w < 4) {
#pragma unroll
                for (int i = 0; i < STW; ++i) {
                    const int st = w * STW + i, mt = st / NT, nt = st % NT;
                    const int c = 16 * mt + 4 * lg;
                    bf16x4_t hi, lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bf16_t hh, ll;
                        split_bf16(sm.colM[c + e] * Sacc[i][e], hh, ll);
                        hi[e] = hh;
                        lo[e] = ll;
                    }
                    *reinterpret_cast<bf16x4_t *>(&sm.S[0][nt * 16 + lr][c]) = hi;
                    if constexpr (SPLIT) *reinterpret_cast<bf16x4_t *>(&sm.S[Sm::NP - 1][nt * 16 + lr][c]) = lo;
                }
            }
            {
                // 20 Gram tiles: wave w takes tiles w and w + 8 together (two independent
                // MFMA chains), and waves 0-3 also tile w + 16.
                int RA, IA, RB, IB;
                const int tA = w, tB = w + 8;
                lower_block(tA, RA, IA);
                lower_block(tB >= 10 ? tB - 10 : tB, RB, IB);
                const bool pB = tB >= 10;
                const bf16_t *aAh = &sm.KA[0][16 * RA + lr][8 * lg];
                const bf16_t *aBh = pB ? &sm.QA[0][16 * RB + lr][8 * lg] : &sm.KA[0][16 * RB + lr][8 * lg];
                const bf16_t *bAh = &sm.KI[0][16 * IA + lr][8 * lg];
                const bf16_t *bBh = &sm.KI[0][16 * IB + lr][8 * lg];
                constexpr int PL = SPLIT ? kC * Sm::KS : 0;
                f32x4_t accA = zero4(), accB = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int o32 = 32 * ks;
                    accA = mma<SPLIT, SPLIT>(accA, aAh + o32, aAh + PL + o32, bAh + o32, bAh + PL + o32);
                    accB = mma<SPLIT, SPLIT>(accB, aBh + o32, aBh + PL + o32, bBh + o32, bBh + PL + o32);
                }
                gram_store(sm, false, RA, IA, accA, lr, lg);
                gram_store(sm, pB, RB, IB, accB, lr, lg);
                if (w < 4) {
                    int RC, IC;
                    lower_block(w + 6, RC, IC);   // tiles 16..19 are P blocks 6..9
                    const bf16_t *aCh = &sm.QA[0][16 * RC + lr][8 * lg];
                    const bf16_t *bCh = &sm.KI[0][16 * IC + lr][8 * lg];
                    f32x4_t accC = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int o32 = 32 * ks;
                        accC = mma<SPLIT, SPLIT>(accC, aCh + o32, aCh + PL + o32, bCh + o32, bCh + PL + o32);
                    }
                    gram_store(sm, true, RC, IC, accC, lr, lg);
                }
            }
            lds_barrier();

            // ======== waves 0-3: diagonal blocks of (I + A)^{-1};  waves 4-7: Y, Z, X ========
            if (w < 4) {
                // Block R = w of the inverse, 16x16, from two 8x8 forward substitutions
                // merged in the wave: [[Ta, 0], [-Tb A_ba Ta, Tb]].  fp32 throughout.
                const int R = w;
                float (*t8)[8][8] = sm.T8[R];
                float (*w8)[8] = sm.W8[R];
                if (l < 16) {
                    const int sb = l >> 3, j = l & 7, base = 16 * R + 8 * sb;
                    float a[8][8];
#pragma unroll
                    for (int r = 1; r < 8; ++r) {
                        const float4 a0 = *reinterpret_cast<const float4 *>(&sm.A[base + r][base]);
                        const float4 a1 = *reinterpret_cast<const float4 *>(&sm.A[base + r][base + 4]);
                        a[r][0] = a0.x; a[r][1] = a0.y; a[r][2] = a0.z; a[r][3] = a0.w;
                        a[r][4] = a1.x; a[r][5] = a1.y; a[r][6] = a1.z; a[r][7] = a1.w;
                    }
                    float t[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                        for (int mm = 0; mm < r; ++mm) {
                            if (mm & 1) s1 -= a[r][mm] * t[mm];
                            else s0 -= a[r][mm] * t[mm];
                        }
                        t[r] = s0 + s1;
                        t8[sb][r][j] = t[r];
                    }
                }
                wave_lds_sync();
                const int i8 = l >> 3, j8 = l & 7;
                {
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int mm = 0; mm < 8; mm += 2) {
                        s0 += sm.A[16 * R + 8 + i8][16 * R + mm] * t8[0][mm][j8];
                        s1 += sm.A[16 * R + 8 + i8][16 * R + mm + 1] * t8[0][mm + 1][j8];
                    }
                    w8[i8][j8] = s0 + s1;
                }
                wave_lds_sync();
                float tba;
                {
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int mm = 0; mm < 8; mm += 2) {
                        s0 += t8[1][i8][mm] * w8[mm][j8];
                        s1 += t8[1][i8][mm + 1] * w8[mm + 1][j8];
                    }
                    tba = -(s0 + s1);
                }
                // lane (i8, j8) writes entries (i8, j8), (i8, 8+j8), (8+i8, j8), (8+i8, 8+j8)
                // of the 16x16 block, row-major (T) and transposed (Tt).
                const float vals[4] = {t8[0][i8][j8], 0.f, tba, t8[1][i8][j8]};
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int rr = 16 * R + 8 * (qd >> 1) + i8, cc = 16 * R + 8 * (qd & 1) + j8;
                    bf16_t hh, ll;
                    split_bf16(vals[qd], hh, ll);
                    sm.T[0][rr][cc] = hh;
                    sm.T[1][rr][cc] = ll;
                    sm.Tt[0][cc][rr] = hh;
                    sm.Tt[1][cc][rr] = ll;
                }
            } else {
                const int rb = w - 4;
                const bf16_t *kah = &sm.KA[0][16 * rb + lr][8 * lg];
                const bf16_t *qah = &sm.QA[0][16 * rb + lr][8 * lg];
                const bf16_t *kal = kah + (SPLIT ? kC * Sm::KS : 0);
                const bf16_t *qal = qah + (SPLIT ? kC * Sm::KS : 0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16_t *sh = &sm.S[0][nt * 16 + lr][8 * lg];
                    const bf16_t *sl = sh + (SPLIT ? BV * Sm::KS : 0);
                    f32x4_t accY = zero4();
                    accZ[nt] = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int o32 = 32 * ks;
                        accY = mma<SPLIT, SPLIT>(accY, kah + o32, kal + o32, sh + o32, sl + o32);
                        accZ[nt] = mma<SPLIT, SPLIT>(accZ[nt], qah + o32, qal + o32, sh + o32, sl + o32);
                    }
                    f32x4_t x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * rb + 4 * lg + e;
                        x[e] = DEC ? sm.wr[r] * vcur[nt][e] - sm.beta[r] * accY[e]
                                   : sm.beta[r] * (vcur[nt][e] - accY[e]);
                    }
                    const int jl = nt * 16 + lr;
                    store_split4(&sm.X[0][jl][16 * rb + 4 * lg], &sm.X[1][jl][16 * rb + 4 * lg], x);
                }
            }
            lds_barrier();

            // ======== off-diagonal blocks of (I + A)^{-1}: waves 0 and 1, matrix cores ========
            // T[R+1][R] = -T[R+1][R+1] (A[R+1][R] T[R][R]) for R = 0, 2 (both waves compute
            // both; the stores are identical), then wave b forms the lower-left column block
            // b of -T[23][23] (A[23][01] T[01][01]).  16x16x16 products with hi/lo-split
            // operands; an accumulator tile is directly the B operand of the next product.
            if (w < 2) {
                const int b = w;
                f32x4_t t10, t32;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int R = 2 * pr;
                    bf16x4_t ah, al;
                    load_split4(&sm.A[16 * (R + 1) + lr][16 * R + 4 * lg], ah, al);
                    f32x4_t wacc = mma4(zero4(), ah, al, lds_ld4(&sm.Tt[0][16 * R + lr][16 * R + 4 * lg]),
                                        lds_ld4(&sm.Tt[1][16 * R + lr][16 * R + 4 * lg]));
                    bf16x4_t wh, wl;
                    split4(wacc, wh, wl);
                    f32x4_t tacc = mma4(zero4(), lds_ld4(&sm.T[0][16 * (R + 1) + lr][16 * (R + 1) + 4 * lg]),
                                        lds_ld4(&sm.T[1][16 * (R + 1) + lr][16 * (R + 1) + 4 * lg]), wh, wl);
#pragma unroll
                    for (int e = 0; e < 4; ++e) tacc[e] = -tacc[e];
                    store_tile_split(&sm.T[0][0][0], &sm.T[1][0][0], Sm::TS, 16 * (R + 1), 16 * R, tacc, lr, lg);
                    if (pr == 0) t10 = tacc;
                    else t32 = tacc;
                }
                (void)t32;
                wave_lds_sync();
                // W2[a][b] = sum_m A[a][m] T[m][b], a = 2, 3 (T[0][1] = 0)
                f32x4_t w2[2];
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2) {
                    const int a = 2 + a2;
                    bf16x4_t ah, al;
                    w2[a2] = zero4();
                    if (b == 0) {
                        load_split4(&sm.A[16 * a + lr][4 * lg], ah, al);
                        w2[a2] = mma4(w2[a2], ah, al, lds_ld4(&sm.Tt[0][lr][4 * lg]), lds_ld4(&sm.Tt[1][lr][4 * lg]));
                        bf16x4_t th, tl;
                        split4(t10, th, tl);
                        load_split4(&sm.A[16 * a + lr][16 + 4 * lg], ah, al);
                        w2[a2] = mma4(w2[a2], ah, al, th, tl);
                    } else {
                        load_split4(&sm.A[16 * a + lr][16 + 4 * lg], ah, al);
                        w2[a2] = mma4(w2[a2], ah, al, lds_ld4(&sm.Tt[0][16 + lr][16 + 4 * lg]),
                                      lds_ld4(&sm.Tt[1][16 + lr][16 + 4 * lg]));
                    }
                }
                bf16x4_t w2h[2], w2l[2];
                split4(w2[0], w2h[0], w2l[0]);
                split4(w2[1], w2h[1], w2l[1]);
                // T[2][b] = -T[2][2] W2[2][b];  T[3][b] = -(T[3][2] W2[2][b] + T[3][3] W2[3][b])
                f32x4_t t2b = mma4(zero4(), lds_ld4(&sm.T[0][32 + lr][32 + 4 * lg]),
                                   lds_ld4(&sm.T[1][32 + lr][32 + 4 * lg]), w2h[0], w2l[0]);
                f32x4_t t3b = mma4(zero4(), lds_ld4(&sm.T[0][48 + lr][32 + 4 * lg]),
                                   lds_ld4(&sm.T[1][48 + lr][32 + 4 * lg]), w2h[0], w2l[0]);
                t3b = mma4(t3b, lds_ld4(&sm.T[0][48 + lr][48 + 4 * lg]), lds_ld4(&sm.T[1][48 + lr][48 + 4 * lg]),
                           w2h[1], w2l[1]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t2b[e] = -t2b[e];
                    t3b[e] = -t3b[e];
                }
                store_tile_split(&sm.T[0][0][0], &sm.T[1][0][0], Sm::TS, 32, 16 * b, t2b, lr, lg);
                store_tile_split(&sm.T[0][0][0], &sm.T[1][0][0], Sm::TS, 48, 16 * b, t3b, lr, lg);
            }
            lds_barrier();

            // ======== phase U: U = T X ========
            if (w < 4 * NT) {
                const int R = w & 3, nt = w >> 2;
                const int nks = (R >> 1) + 1;
                const bf16_t *th = &sm.T[0][16 * R + lr][8 * lg];
                const bf16_t *tl = &sm.T[1][16 * R + lr][8 * lg];
                const bf16_t *xh = &sm.X[0][nt * 16 + lr][8 * lg];
                const bf16_t *xl = &sm.X[1][nt * 16 + lr][8 * lg];
                f32x4_t acc = zero4();
                for (int ks = 0; ks < nks; ++ks)
                    acc = mma<true, true>(acc, th + 32 * ks, tl + 32 * ks, xh + 32 * ks, xl + 32 * ks);
                const int jl = nt * 16 + lr;
                store_split4(&sm.U[0][jl][16 * R + 4 * lg], &sm.U[1][jl][16 * R + 4 * lg], acc);
            }
            lds_barrier();

            // ======== waves 4-7: O = Z + P U (store);  waves 0-3: state update ========
            if (w >= 4) {
                const int rb = w - 4;
                const int nks = (rb >> 1) + 1;
                const bf16_t *ph = &sm.P[0][16 * rb + lr][8 * lg];
                const bf16_t *pl = &sm.P[1][16 * rb + lr][8 * lg];
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
                        const int r = 16 * rb + 4 * lg + e;
                        if (r < nv) o[((tbase + r) * H + h) * (int64_t)DV + col0 + jl] = from_f32<IO>(acc[e]);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < STW; ++i) {
                    const int st = w * STW + i, mt = st / NT, nt = st % NT;
                    const bf16_t *kh = &sm.KIt[0][16 * mt + lr][8 * lg];
                    const bf16_t *kl = kh + (SPLIT ? DK * Sm::TS : 0);
                    const bf16_t *uh = &sm.U[0][nt * 16 + lr][8 * lg];
                    const bf16_t *ul = &sm.U[1][nt * 16 + lr][8 * lg];
                    f32x4_t acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc = mma<SPLIT, true>(acc, kh + 32 * ks, kl + 32 * ks, uh + 32 * ks, ul + 32 * ks);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * mt + 4 * lg + e;
                        Sacc[i][e] = sm.colGn[c] * Sacc[i][e] + sm.colGnM[c] * acc[e];
                    }
                }
            }
        }
    }

    if (h_T && w < 4) {
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w * STW + i, mt = st / NT, nt = st % NT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * mt + 4 * lg + e;
                const int j = col0 + nt * 16 + lr;
                h_T[((n * H + h) * DK + c) * (int64_t)DV + j] = Sacc[i][e];
            }
        }
    }
}

template <int DK, int BV, typename IO, typename GT, bool SPLIT, bool PRO, int GM, bool DEC>
hipError_t launch_t(const ChunkArgs &a, hipStream_t st) {
    const int64_t chains = a.num_seqs * (int64_t)a.H;
    const int64_t nwg = chains * (a.d_v / BV);
    hipLaunchKernelGGL((chunk_fwd_kernel<DK, BV, IO, GT, SPLIT, PRO, GM, DEC>), dim3((unsigned)nwg),
                       dim3(kThreads), 0, st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v,
                       (const GT *)a.log_alpha, (const GT *)a.beta, (const GT *)a.w_write, a.h0, a.cu_seqlens, (IO *)a.o, a.h_T, a.seq_len, a.H, a.d_v, chains,
                       a.log_alpha_min);
    return hipGetLastError();
}

// bf16 I/O: single-bf16 decayed operands.  fp32 I/O: split operands (d_k = 64;
// at d_k = 128 the fp32 forward runs chunkwise on the fp32 matrix cores, in
// kda_bwd.hip, and never reaches this kernel).
template <int DK, int BV, bool PRO, int GM, bool DEC>
hipError_t launch_types(const ChunkArgs &a, hipStream_t st) {
    if (a.io_bf16)
        return a.gate_bf16 ? launch_t<DK, BV, bf16_t, bf16_t, false, PRO, GM, DEC>(a, st)
                           : launch_t<DK, BV, bf16_t, float, false, PRO, GM, DEC>(a, st);
    if constexpr (DK == 128) {
        return hipErrorInvalidValue;
    } else {
        return a.gate_bf16 ? launch_t<DK, BV, float, bf16_t, true, PRO, GM, DEC>(a, st)
                           : launch_t<DK, BV, float, float, true, PRO, GM, DEC>(a, st);
    }
}

// The input variants that exist: per-channel gates with or without the prologue
// or with decoupled strengths, and the scalar-gate forms.
template <int DK, int BV>
hipError_t launch_types_pro(const ChunkArgs &a, hipStream_t st) {
    if (a.gate_mode == kGatePerHead) return launch_types<DK, BV, false, kGatePerHead, false>(a, st);
    if (a.gate_mode == kGateNone) return launch_types<DK, BV, false, kGateNone, false>(a, st);
    if (a.prologue) return launch_types<DK, BV, true, kGatePerChannel, false>(a, st);
    if (a.w_write) return launch_types<DK, BV, false, kGatePerChannel, true>(a, st);
    return launch_types<DK, BV, false, kGatePerChannel, false>(a, st);
}

// Value-column block width: 32 when that still gives at least two workgroups
// per compute unit (less recomputation of the d_v-independent part), else 16.
int pick_block_v(const ChunkArgs &a) {
    const int64_t chains = a.num_seqs * (int64_t)a.H;
    return chains * (a.d_v / 32) >= 512 ? 32 : 16;
}

}  // namespace

// Two-kernel path (kda_chunk2.hip): bf16 I/O at the dimensions the fused kernel
// does not cover.
size_t two_kernel_workspace_bytes(const ChunkArgs &a);
bool two_kernel_grids_fit(const ChunkArgs &a, int bv);
hipError_t launch_chunk_fwd_two_kernel(const ChunkArgs &a, int bv, hipStream_t st);

// fp32 I/O at d_k = 128 (kda_bwd.hip): chunkwise on the fp32 matrix cores.
size_t f32_fwd_workspace_bytes(const ChunkArgs &a);
bool f32_fwd_grids_fit(const ChunkArgs &a);
hipError_t launch_f32_chunk_fwd(const ChunkArgs &a, hipStream_t st);

// Fused path (kda_fused.hip).
bool fused_fwd_supported(const ChunkArgs &a);
size_t fused_fwd_workspace_bytes(const ChunkArgs &a);
bool fused_fwd_grids_fit(const ChunkArgs &a);
hipError_t launch_fused_fwd(const ChunkArgs &a, hipStream_t st);

// The workspace query does not know which entry point will use it, so it covers
// both forward paths where the entry point decides between them.
size_t chunk_fwd_workspace_bytes(const ChunkArgs &a) {
    if (!a.io_bf16) return a.d_k == 128 ? f32_fwd_workspace_bytes(a) : 0;
    if (a.d_k == 128 && a.d_v == 128) {
        // packed batches always run the fused kernel; equal-length ones run it
        // for the input variants and the two-kernel path for plain KDA
        const size_t f = fused_fwd_workspace_bytes(a);
        if (a.varlen || a.force_fused) return f;
        const size_t t = two_kernel_workspace_bytes(a);
        return f > t ? f : t;
    }
    return two_kernel_workspace_bytes(a);
}

bool chunk_fwd_grids_fit(const ChunkArgs &a) {
    if (fused_fwd_supported(a)) return fused_fwd_grids_fit(a);
    if (!a.io_bf16 && a.d_k == 128) return f32_fwd_grids_fit(a);
    const int bv = pick_block_v(a);
    if (a.io_bf16 && a.total_tokens > 0) return two_kernel_grids_fit(a, bv);
    return grid_fits(a.num_seqs * (int64_t)a.H * (a.d_v / bv), kThreads);
}

int launch_chunk_fwd(const ChunkArgs &a, void *stream, char *err, size_t err_len) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!chunk_fwd_grids_fit(a)) {
        snprintf(err, err_len, "chunk_fwd grid too large");
        return -1;
    }
    hipError_t e;
    if (fused_fwd_supported(a)) {
        if (a.workspace_bytes < chunk_fwd_workspace_bytes(a)) {
            snprintf(err, err_len, "workspace too small");
            return -1;
        }
        e = launch_fused_fwd(a, st);
    } else if (!a.io_bf16 && a.d_k == 128) {
        if (a.workspace_bytes < chunk_fwd_workspace_bytes(a)) {
            snprintf(err, err_len, "workspace too small");
            return -1;
        }
        e = launch_f32_chunk_fwd(a, st);
    } else {
        const int bv = pick_block_v(a);
        if (a.io_bf16 && a.total_tokens > 0) {
            if (a.workspace_bytes < chunk_fwd_workspace_bytes(a)) {
                snprintf(err, err_len, "workspace too small");
                return -1;
            }
            e = launch_chunk_fwd_two_kernel(a, bv, st);
        } else if (a.d_k == 128)
            e = bv == 32 ? launch_types_pro<128, 32>(a, st) : launch_types_pro<128, 16>(a, st);
        else
            e = bv == 32 ? launch_types_pro<64, 32>(a, st) : launch_types_pro<64, 16>(a, st);
    }
    if (e != hipSuccess) {
        snprintf(err, err_len, "%s", hipGetErrorString(e));
        return -1;
    }
    return 0;
}

}  // namespace kda
