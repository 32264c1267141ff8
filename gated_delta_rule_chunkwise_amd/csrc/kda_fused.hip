// kda_fused.hip -- chunkwise KDA forward, one fused kernel per (chain, segment).
//
// Method (KimiLinear article, section 3.1: intra-chunk products on the matrix
// cores, inter-chunk recurrence on a resident state; Kimi Linear abstract on the
// CoChat record: the specialised DPLR transition of KDA, whose low-rank pair is
// tied to the key and the decayed key).  For one chunk of n <= 64 tokens with
// start state S (d_k x d_v, fp32) and the inclusive in-chunk cumsum G of
// log alpha (per token and key channel, g_n its last row):
//
//   A[r,i] = b_r sum_c K[r,c] K[i,c] e^{G[r,c]-G[i,c]}   (i < r)
//   P[r,i] =     sum_c Q[r,c] K[i,c] e^{G[r,c]-G[i,c]}   (i <= r)
//   T      = (I + A)^{-1}                                  (UT transform)
//   U      = T (w.V - b.(K.e^G) S)                        (rows written)
//   O      = (Q.e^G) S + P U
//   S     <- Diag(e^{g_n}) S + (K.e^{g_n - G})^T U
//
// with b = w = beta for KDA (b erases, w writes in the decoupled form).  This
// unrolls the per-token update of section 2.3 within the chunk exactly.
//
// Decay anchoring.  Every factor outside the Gram blocks is at most 1 (G <= 0,
// g_n <= G).  Inside them each key channel is anchored at the middle of its
// chunk decay, m = g_n / 2:
//   e^{G_r - G_i} = e^{G_r - m} . e^{m - G_i},
// so either factor is at most e^{-g_n / 2}, and the operands are Q.e^{G-m},
// K.e^{G-m} (left) and K.e^{m-G} (right), one row each.  A channel whose chunk
// decay exceeds kBig nats is left out of the Gram products (its operands are
// zero there) and its pairs are added exactly on the vector units; the state
// products still take it, through its factors e^G and e^{g_n - G} (at most 1).
//
// Work decomposition.  One workgroup of 8 waves owns one (sequence, head) chain,
// or one segment of it, with all d_v value columns: nothing is shared between
// workgroups.  Per chunk, all waves form the operands and the Gram blocks; waves
// 0-3 invert the four diagonal 16x16 blocks of I + A while waves 4-7 convert P
// and the blocks of A below the diagonal to fp16; then every wave advances its
// 16 value columns of the state (fp32, registers) while the next chunk's inputs
// are in flight.  T = (I + A)^{-1} is never formed: each wave solves
// (I + A) U = Y for its columns by substitution over the four token tiles,
// U_R = D_R (Y_R - sum_{I<R} A_RI U_I) with D_R the inverted diagonal blocks.  The state's accumulator tiles are used directly as matrix-core
// operands: the k index of each 32-wide step is permuted (slot 8g+4h+i holds
// index 16h+4g+i) so that an accumulator pair is one operand fragment; the
// shared operands are stored in LDS in that order.
//
// Segments.  A chain too long for the parallelism the GPU needs is cut into
// segments.  The state at a segment's end is an affine map of the state at its
// start, S_end = Phi S_start + S_loc.  A first kernel runs the first segment of
// every chain exactly from h0 (its o, and its end state, which is the second
// segment's start state), and beside it every segment but the first and the
// last from the pair (S_loc, Phi) = (0, I) (waves 0-3 the d_v columns of S_loc,
// waves 4-7 the d_k columns of Phi, the same chunk step with no value input for
// Phi); a short scan from the second segment's start state gives the start
// states of the rest; a last kernel runs every segment but the first from its
// start state and writes o and h_T.  The two launches then hold the same
// number of workgroups.  Each column of S and Phi evolves independently under
// the same chunk step, so this is the recurrence regrouped, not approximated.
//
// Precision.  The Gram products take K.e^{G-m} as single bf16 and Q.e^{G-m},
// K.e^{m-G} as hi/lo bf16 pairs (about 2^-16 relative).  The diagonal blocks
// of I + A are inverted in fp32.  The state products (X = K.e^G S, Q.e^G S,
// the substitution for U, P U, (K.e^{g_n-G})^T U) run on fp16 operands, each
// scaled by a power of two to the top of the fp16 range (the state per wave,
// each token tile's right-hand side and U per wave, K and Q per chunk, A, D and
// P per row), which keeps 11 significant bits whatever the magnitudes; every
// scale is undone exactly on the fp32 accumulators.
#include "kda_chunk_common.h"
#include "kda_launch.h"
#include "kda_plan.h"

#include <stdio.h>
#include <stdlib.h>

namespace kda {
namespace {

constexpr int kFW = 8;                         // waves per workgroup
constexpr int kFT = 64 * kFW;                  // threads per workgroup

// Slot of index x inside its 32-wide k-step (see the header): x = 32ks + 16h + 4g + i.
__device__ __forceinline__ int kslot(int x) {
    return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}

typedef _Float16 f16_t;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma16h(const f16x8_t &a, const f16x8_t &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int DK, int DV> struct alignas(16) FusedSmem {
    static constexpr int KS = DK + 8;   // stride of channel-long 16-bit rows
    static constexpr int TS = kC + 8;   // stride of token-long 16-bit rows
    static constexpr int FS = kC + 4;   // fp32 stride of 64 x 64 matrices
    static constexpr int XQ = 32;       // channels per pass of the exact terms
    union {
        struct {                        // Gram operands, natural channel order
            bf16_t KA[kC][KS];          // K.e^{G-m}
            bf16_t QA[2][kC][KS];       // hi/lo of Q.e^{G-m}
            bf16_t KI[2][kC][KS];       // hi/lo of K.e^{m-G}
        } g;
        struct {                        // after the Gram products
            union {
                struct {
                    float A[kC][FS];    // b-scaled strictly lower A
                    float P[kC][FS];    // lower P (upper part not written)
                } ap;
                bf16_t Vt[DV][TS];      // V^T, written once A and P are consumed
            };
            union {
                struct {                // exact terms of channels left out of the Gram products
                    float G[kC][XQ];
                    float K[kC][XQ];
                    float Q[kC][XQ];
                } x;
                struct {                // inverses of the diagonal blocks of I + A
                    float D[4][16][17];
                    float T8[4][2][8][8];
                    float W8[4][8][8];
                } t;
            };
        } r;
    };
    // state-phase operands, fp16, k index in slot order (see the header)
    f16_t KE[kC][KS];                   // K.e^G . sk
    f16_t QE[kC][KS];                   // Q.e^G . sq
    f16_t KIt[DK][TS];                  // (K.e^{g_n-G})^T . sk
    union {
        float tot[DK][kFW];             // per-wave sums of log2 alpha (cumsum phase only)
        f16_t AD16[kC][TS];             // A below the diagonal blocks (rows scaled by 1 / rsA) and
                                        // the diagonal blocks' inverses D (rows scaled by 1 / rsD)
    };
    f16_t P16[kC][TS];                  // P, rows scaled by 1 / rsP
    float rsA[kC], rsD[kC], rsP[kC];    // row scales (powers of 2)
    float egn[DK];                      // e^{g_n}
    float beta[kC];                     // erase strength b (= beta)
    float wr[kC];                       // write strength w (= beta unless decoupled)
    float wmax[2][kFW];                 // per-wave max |k|, |q|
    uint8_t big[DK];                    // channel left out of the Gram products
    int32_t anybig;
};

struct FusedArgs {
    const void *q, *k, *v, *log_alpha, *beta, *wr;
    const float *h0;
    const int32_t *cu;       // device cu_seqlens, or null (equal-length sequences of T tokens)
    const int32_t *order;    // single pass: sequences by decreasing length, or null (natural order)
    void *o;
    float *h_T;
    float *seg_in;           // [chains][nseg - 1][DK*DV]  start state of segment 1 + i
    float *seg_loc;          // [chains][nseg - 2][DK*DV]  end state of segment 1 + i run from zero
    float *seg_phi;          // [chains][nseg - 2][DK*DK]  transition of segment 1 + i
    int64_t N, T;
    int32_t H;
    int32_t nseg, seg_chunks, head_chunks;   // segment 0 has head_chunks chunks, the rest seg_chunks
    int32_t pass;            // 0: one pass; 1: first launch of a segmented call; 2: last launch
    float lo;
};

struct Task {
    int64_t n, chain, t0, t1;
    int h, seg;
    bool phi;
};

__device__ __forceinline__ Task fused_task(const FusedArgs &a) {
    const int64_t id = blockIdx.x;
    const int64_t chains = a.N * a.H;
    Task t;
    t.seg = 0;
    t.phi = false;
    if (a.pass == 0) {
        const int64_t r = id / a.H;
        t.h = (int)(id % a.H);
        t.n = a.order ? (int64_t)a.order[r] : r;
        t.chain = t.n * a.H + t.h;
    } else {
        if (a.pass == 1 && id < chains) {   // segment 0 of chain id, exactly from h0
            t.chain = id;
        } else if (a.pass == 1) {           // transitions of segments 1 .. nseg - 2
            t.chain = (id - chains) / (a.nseg - 2);
            t.seg = 1 + (int)((id - chains) % (a.nseg - 2));
            t.phi = true;
        } else {                            // outputs of segments 1 .. nseg - 1
            t.chain = id / (a.nseg - 1);
            t.seg = 1 + (int)(id % (a.nseg - 1));
        }
        t.n = t.chain / a.H;
        t.h = (int)(t.chain % a.H);
    }
    int64_t bos, eos;
    if (a.cu) {
        bos = a.cu[t.n];
        eos = a.cu[t.n + 1];
    } else {
        bos = t.n * a.T;
        eos = bos + a.T;
    }
    if (a.pass == 0) {
        t.t0 = bos;
        t.t1 = eos;
    } else {
        const int64_t span = (int64_t)a.seg_chunks * kC, head = (int64_t)a.head_chunks * kC;
        t.t0 = t.seg == 0 ? bos : bos + head + span * (t.seg - 1);
        const int64_t len = t.seg == 0 ? head : span;
        t.t1 = t.t0 + len < eos ? t.t0 + len : eos;
    }
    return t;
}

// Power of two p with |x| * p in [0.5, 1) for the largest |x| = mx (1 when mx = 0),
// its exponent clamped to [-126, 126] so that p and 1 / p are normal fp32 numbers
// (a state that has decayed into the denormal range is scaled up by 2^126 only).
__device__ __forceinline__ float pow2_scale(float mx) {
    const int e = __builtin_amdgcn_frexp_expf(mx);
    return __builtin_amdgcn_ldexpf(1.f, -(e < -126 ? -126 : e > 126 ? 126 : e));
}

// Largest x over the 64 lanes, wave-uniform: data-parallel moves within rows of
// 16 lanes, then the four row maxima.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_mov<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp_mov<0x140>(x));   // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// fp16 fragment (8 values) of an accumulator pair scaled by s: rows 4g..4g+3 of
// tile a, then of tile b, at this lane's column -- the slot order of a k-step.
__device__ __forceinline__ f16x8_t pair_h(const f32x4_t &a, const f32x4_t &b, float s) {
    f16x8_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (f16_t)(a[e] * s);
        r[4 + e] = (f16_t)(b[e] * s);
    }
    return r;
}

__device__ __forceinline__ f16x8_t lds_ld8h(const f16_t *p) { return *reinterpret_cast<const f16x8_t *>(p); }
__device__ __forceinline__ f16x4_t lds_ld4h(const f16_t *p) { return *reinterpret_cast<const f16x4_t *>(p); }

// D(16x16) += A(16x16) B(16x16) on fp16 operands: lane l holds A[l%16][4(l/16)+i],
// B[4(l/16)+i][l%16] and D[4(l/16)+i][l%16], so an accumulator tile is a B operand.
__device__ __forceinline__ f32x4_t mfma16h16(const f16x4_t &a, const f16x4_t &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// acc += A B with hi/lo bf16 A and B (hi*hi + hi*lo + lo*hi).
__device__ __forceinline__ f32x4_t mfma3(const bf16x8_t &ah, const bf16x8_t &al, const bf16x8_t &bh,
                                         const bf16x8_t &bl, f32x4_t acc) {
    acc = mfma16(ah, bh, acc);
    acc = mfma16(ah, bl, acc);
    acc = mfma16(al, bh, acc);
    return acc;
}

// One chunk of the state recurrence for NT 16-column tiles of the state held by
// this wave (columns col0.. of the value space, or of Phi when HAS_V is false).
// The state-side products run on fp16 operands scaled by powers of two: the
// state by ss (this wave's columns), each token tile of the right-hand side and
// of U by its own power of two and U again by su, the shared operands
// by sk, sq and the row scales of A, D and P; every scale is undone exactly on
// the fp32 accumulators.
//   X = K.e^G S,  O^T = S^T (Q.e^G)^T            (WITH_O)
//   Y = w.V - b.X,  (I + A) U = Y,  O^T += U^T P^T, o    (WITH_O)
//   S <- Diag(e^{g_n}) S + (K.e^{g_n-G})^T U
// issue(p), p = 0..3, is called at four points of the phase (the next chunk's
// input loads).
template <int DK, int DV, int NT, bool WITH_O, bool HAS_V, typename IO, typename LF>
__device__ __forceinline__ void state_chunk(FusedSmem<DK, DV> &sm, f32x4_t (&S)[DK / 16][NT], int col0,
                                            float isk, float isq,
                                            IO *__restrict__ o, int64_t tbase, int nv, int H, int h, int l,
                                            LF &&issue) {
    constexpr int NKS = DK / 32, MT = DK / 16;
    const int lr = l & 15, lg = l >> 4;
    float mx = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(S[mt][nt][e]));
    issue(0);
    const float ss = pow2_scale(wave_max(mx)), iss = 1.f / ss;
    f32x4_t X[4][NT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) X[tt][nt] = zero4();
    f16x8_t sf[NKS][NT];   // the state as fp16 operand fragments, kept for the output
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sf[ks][nt] = pair_h(S[2 * ks][nt], S[2 * ks + 1][nt], ss);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f16x8_t ke = lds_ld8h(&sm.KE[16 * tt + lr][32 * ks + 8 * lg]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) X[tt][nt] = mfma16h(ke, sf[ks][nt], X[tt][nt]);
        }
    }
    issue(1);
    // Y = w.V - b.X (rows 16tt + 4lg + e)
    const float xs = isk * iss;
    f32x4_t Y[4][NT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const f32x4_t bb = *reinterpret_cast<const f32x4_t *>(&sm.beta[16 * tt + 4 * lg]);
        const f32x4_t ww = *reinterpret_cast<const f32x4_t *>(&sm.wr[16 * tt + 4 * lg]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            bf16x4_t vv;
            if (HAS_V) vv = lds_ld4(&sm.r.Vt[col0 + 16 * nt + lr][16 * tt + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Y[tt][nt][e] = (HAS_V ? ww[e] * (float)vv[e] : 0.f) - bb[e] * (X[tt][nt][e] * xs);
        }
    }
    // U = (I + A)^{-1} Y by substitution over the four 16-token tiles,
    //   U_R = D_R (Y_R - sum_{I<R} A_RI U_I),   D_R = (I + A_RR)^{-1},
    // on 16x16x16 fp16 products (a U tile's accumulator layout is the B
    // operand layout); each tile's right-hand side and U take their own power
    // of two, undone on the fp32 accumulators with the row scales of A and D.
    f32x4_t U[4][NT];
    f16x4_t uh[3][NT];
    float isub[3];
    float mu = 0.f;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const f32x4_t ra = *reinterpret_cast<const f32x4_t *>(&sm.rsA[16 * R + 4 * lg]);
        const f32x4_t rd = *reinterpret_cast<const f32x4_t *>(&sm.rsD[16 * R + 4 * lg]);
        f32x4_t yp[NT];
        float m = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4_t z = zero4();
#pragma unroll
            for (int I = 0; I < R; ++I) {
                const f16x4_t a = lds_ld4h(&sm.AD16[16 * R + lr][16 * I + 4 * lg]);
                const f32x4_t pr = mfma16h16(a, uh[I][nt], zero4());
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] += pr[e] * isub[I];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yp[nt][e] = Y[R][nt][e] - z[e] * ra[e];
                m = fmaxf(m, fabsf(yp[nt][e]));
            }
        }
        const float sy = pow2_scale(wave_max(m)), isy = 1.f / sy;
        const f16x4_t dd = lds_ld4h(&sm.AD16[16 * R + lr][16 * R + 4 * lg]);
        float mR = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f16x4_t yh;
#pragma unroll
            for (int e = 0; e < 4; ++e) yh[e] = (f16_t)(yp[nt][e] * sy);
            U[R][nt] = mfma16h16(dd, yh, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                U[R][nt][e] *= rd[e] * isy;
                mR = fmaxf(mR, fabsf(U[R][nt][e]));
            }
        }
        mu = fmaxf(mu, mR);
        if (R < 3) {
            const float s = pow2_scale(wave_max(mR));
            isub[R] = 1.f / s;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) uh[R][nt][e] = (f16_t)(U[R][nt][e] * s);
        }
    }
    issue(2);
    const float su = pow2_scale(wave_max(mu)), isu = 1.f / su;
    f16x8_t uf[2][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        uf[0][nt] = pair_h(U[0][nt], U[1][nt], su);
        uf[1][nt] = pair_h(U[2][nt], U[3][nt], su);
    }
    if (WITH_O) {
        // O^T = (S^T QE^T) / (sq ss) + (U^T P^T) / (rsP su), one token tile at a time:
        // the lane holds o[16tt + lr][col0 + 16nt + 4lg + e]
        const float c1 = isq * iss;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4_t O1[NT], O2[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O1[nt] = O2[nt] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const f16x8_t qe = lds_ld8h(&sm.QE[16 * tt + lr][32 * ks + 8 * lg]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) O1[nt] = mfma16h(sf[ks][nt], qe, O1[nt]);
            }
#pragma unroll
            for (int k2 = 0; k2 <= (tt >> 1); ++k2) {
                const f16x8_t pf = lds_ld8h(&sm.P16[16 * tt + lr][32 * k2 + 8 * lg]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) O2[nt] = mfma16h(uf[k2][nt], pf, O2[nt]);
            }
            const int r = 16 * tt + lr;
            const float c2 = sm.rsP[r] * isu;
            if (r < nv) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4_t ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = O1[nt][e] * c1 + O2[nt][e] * c2;
                    IO *dst = &o[((tbase + r) * H + h) * (int64_t)DV + col0 + 16 * nt + 4 * lg];
                    if constexpr (sizeof(IO) == 2) {
                        bf16x4_t b4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) b4[e] = from_f32<bf16_t>(ov[e]);
                        *reinterpret_cast<bf16x4_t *>(dst) = b4;
                    } else {
                        *reinterpret_cast<f32x4_t *>(dst) = ov;
                    }
                }
            }
        }
    }
    issue(3);
    // S <- Diag(e^{g_n}) S + (KIn^T U) / (sk su)
    const float cs = isk * isu;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const f32x4_t eg = *reinterpret_cast<const f32x4_t *>(&sm.egn[16 * mt + 4 * lg]);
        f32x4_t acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const f16x8_t kf = lds_ld8h(&sm.KIt[16 * mt + lr][32 * k2 + 8 * lg]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16h(kf, uf[k2][nt], acc[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[mt][nt][e] = eg[e] * S[mt][nt][e] + acc[nt][e] * cs;
    }
}

// D_R = (I + A_RR)^{-1} for the four diagonal 16x16 blocks of the b-scaled
// strictly lower A in sm.r.ap.A (fp32), each by two 8x8 forward substitutions
// and a merge (waves 0-3, one block each), into sm.r.t.D.  Waves 4-7 run
// `other` meanwhile.  Every wave takes part in the closing barrier.  The blocks
// below the diagonal are not inverted: the state phase solves with A and D.
template <typename Sm, typename F>
__device__ __forceinline__ void diag_inverse(Sm &sm, int w, int l, F &&other) {
    if (w < 4) {
        const int R = w;
        float(*t8)[8][8] = sm.r.t.T8[R];
        float(*w8)[8] = sm.r.t.W8[R];
        if (l < 16) {
            const int sb = l >> 3, j = l & 7, base = 16 * R + 8 * sb;
            float av[8][8];
#pragma unroll
            for (int r = 1; r < 8; ++r) {
                const float4 x0 = *reinterpret_cast<const float4 *>(&sm.r.ap.A[base + r][base]);
                const float4 x1 = *reinterpret_cast<const float4 *>(&sm.r.ap.A[base + r][base + 4]);
                av[r][0] = x0.x; av[r][1] = x0.y; av[r][2] = x0.z; av[r][3] = x0.w;
                av[r][4] = x1.x; av[r][5] = x1.y; av[r][6] = x1.z; av[r][7] = x1.w;
            }
            float t[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                for (int mm = 0; mm < r; ++mm) {
                    if (mm & 1) s1 -= av[r][mm] * t[mm];
                    else s0 -= av[r][mm] * t[mm];
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
                s0 += sm.r.ap.A[16 * R + 8 + i8][16 * R + mm] * t8[0][mm][j8];
                s1 += sm.r.ap.A[16 * R + 8 + i8][16 * R + mm + 1] * t8[0][mm + 1][j8];
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
        const float vals[4] = {t8[0][i8][j8], 0.f, tba, t8[1][i8][j8]};
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) sm.r.t.D[R][8 * (qd >> 1) + i8][8 * (qd & 1) + j8] = vals[qd];
    } else {
        other();
    }
    lds_barrier();
}

// P (fp32, lower) to fp16 rows scaled by powers of two, k index in slot order
// (waves 4-7, t = 0..255: row t/4, columns 16(t%4)..+15).
template <typename Sm> __device__ __forceinline__ void p_convert(Sm &sm, int t) {
    const int r = t >> 2, b = t & 3, ks = b >> 1, hh = b & 1;
    float x[16], mx = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int c = 16 * b + j;
        x[j] = c <= r ? sm.r.ap.P[r][c] : 0.f;
        mx = fmaxf(mx, fabsf(x[j]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float sc = pow2_scale(mx);
    if (b == 0) sm.rsP[r] = 1.f / sc;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        f16x4_t y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = (f16_t)(x[4 * g + i] * sc);
        *reinterpret_cast<f16x4_t *>(&sm.P16[r][32 * ks + 8 * g + 4 * hh]) = y;
    }
}

// A below the diagonal blocks (fp32) to fp16 rows scaled by powers of two, in
// natural column order (waves 4-7, t = 0..255: row t/4, columns 16(t%4)..+15;
// block rows 1-3 only).
template <typename Sm> __device__ __forceinline__ void a_convert(Sm &sm, int t) {
    const int r = t >> 2, b = t & 3, R = r >> 4;
    float x[16], mx = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        x[j] = b < R ? sm.r.ap.A[r][16 * b + j] : 0.f;
        mx = fmaxf(mx, fabsf(x[j]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float sc = pow2_scale(mx);
    if (b == 0) sm.rsA[r] = 1.f / sc;
    if (b < R) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f16x4_t y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (f16_t)(x[4 * g + i] * sc);
            *reinterpret_cast<f16x4_t *>(&sm.AD16[r][16 * b + 4 * g]) = y;
        }
    }
}

// The diagonal blocks' inverses (fp32) to fp16 rows scaled by powers of two
// (t = 0..255: row t/4, columns 16(r/16) + 4(t%4)..+3).
template <typename Sm> __device__ __forceinline__ void d_convert(Sm &sm, int t) {
    const int r = t >> 2, b = t & 3, R = r >> 4;
    float x[4], mx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = sm.r.t.D[R][r & 15][4 * b + i];
        mx = fmaxf(mx, fabsf(x[i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float sc = pow2_scale(mx);
    if (b == 0) sm.rsD[r] = 1.f / sc;
    f16x4_t y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (f16_t)(x[i] * sc);
    *reinterpret_cast<f16x4_t *>(&sm.AD16[r][16 * R + 4 * b]) = y;
}

constexpr float kBig = 80.f;              // chunk decay (nats) beyond which a channel leaves the Gram products
constexpr float kBig2 = kBig * kLog2e;   // the same in log2 units

// The chunk loop of one task.  Every wave runs the operand phases; waves with
// HAS_STATE also hold NT 16-column tiles of the state (columns col0.. of the
// value space, or of Phi without HAS_V) and run the state phase.  All
// instantiations execute the same barrier sequence.
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC, int NT, bool WITH_O, bool HAS_V,
          bool HAS_STATE>
__device__ __forceinline__ void chain_loop(FusedSmem<DK, DV> &sm, const FusedArgs &a, const Task &tk, int w, int tid,
                                           int col0, const float *__restrict__ src, bool ident, float *__restrict__ dst,
                                           int ld, bool need_o) {
    constexpr int CPL = DK / 64, NKS = DK / 32, MT = DK / 16;
    static_assert(CPL == 2, "lanes hold two key channels");
    constexpr int NTX = NT > 0 ? NT : 1;
    const IO *__restrict__ q = (const IO *)a.q;
    const IO *__restrict__ k = (const IO *)a.k;
    const IO *__restrict__ v = (const IO *)a.v;
    const GT *__restrict__ la = (const GT *)a.log_alpha;
    const GT *__restrict__ be = (const GT *)a.beta;
    const GT *__restrict__ wrp = (const GT *)a.wr;
    IO *__restrict__ o = (IO *)a.o;
    const int H = a.H, h = tk.h;
    const int l0 = tid & 63, lr0 = l0 & 15, lg0 = l0 >> 4;

    // ---- state tiles (accumulator layout: rows 16mt + 4lg + e, column col0 + 16nt + lr)
    f32x4_t S[MT][NTX];
    if (HAS_STATE) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * mt + 4 * lg0 + e, c = col0 + 16 * nt + lr0;
                    S[mt][nt][e] = ident ? (r == c ? 1.f : 0.f) : (src ? src[(int64_t)r * ld + c] : 0.f);
                }
    }

    constexpr int CPV = DV / 64;
    typedef typename VecT<IO, CPV>::type VV;
    ChunkRegs<DK, 16, IO, GT, PRO, GM, DEC> in;
    VV vr[8];   // value rows 8w.., columns CPV*l..
    auto load_in = [&](int64_t tb, int nvv, int l) {
        in.load(q, k, v, la, be, wrp, tb, nvv, H, h, DV, 0, w, l, l >> 4, l & 15, false);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * w + i, rr = r < nvv ? r : nvv - 1;
            vr[i] = *reinterpret_cast<const VV *>(v + ((tb + rr) * H + h) * (int64_t)DV + l * CPV);
        }
    };
    // The next chunk's inputs, issued in four parts spread over the state phase
    // (gates and strengths, keys, queries, values), so that the waves are not
    // held at one point while the loads drain through the memory pipeline.
    typedef typename ChunkRegs<DK, 16, IO, GT, PRO, GM, DEC>::GV GVt;
    typedef typename ChunkRegs<DK, 16, IO, GT, PRO, GM, DEC>::IV IVt;
    auto load_part = [&](int part, int64_t tb, int nvv, int l) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * w + i, rr = r < nvv ? r : nvv - 1;
            const int64_t row = (tb + rr) * H + h;
            const int64_t base = row * (int64_t)DK + l * CPL;
            if (part == 0) {
                if constexpr (GM == kGatePerChannel) in.la[i] = *reinterpret_cast<const GVt *>(la + base);
                else in.la[i] = vsplat<GVt>(GM == kGatePerHead ? la[row] : (GT)0.f);
            } else if (part == 1) {
                in.kk[i] = *reinterpret_cast<const IVt *>(k + base);
            } else if (part == 2) {
                in.qq[i] = *reinterpret_cast<const IVt *>(q + base);
            } else {
                vr[i] = *reinterpret_cast<const VV *>(v + row * (int64_t)DV + l * CPV);
            }
        }
        if (part == 0 && w == 0) {
            const int64_t row = (tb + (l < nvv ? l : nvv - 1)) * H + h;
            in.bt = to_f32(be[row]);
            if (DEC) in.wt = to_f32(wrp[row]);
        }
    };
    if (tk.t0 < tk.t1) load_in(tk.t0, (int)((tk.t1 - tk.t0) < kC ? (tk.t1 - tk.t0) : kC), l0);

    for (int64_t tbase = tk.t0; tbase < tk.t1; tbase += kC) {
        const int nv = (int)((tk.t1 - tbase) < kC ? (tk.t1 - tbase) : kC);
        int tl_;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tl_) : "v"(tid));
        const int l = tl_ & 63, lr = l & 15, lg = l >> 4;
        lds_barrier();   // the previous chunk's state phase is done with the operands

        // ======== cumsum (log2 units), strengths, largest |k| and |q|
        in.prepare(w, a.lo);
        const bool partial = nv < kC;
        if (partial) in.zero_tail(nv, w);   // rows past the end: zero keys, queries, gates
        float G[8][CPL], mk = 0.f, mq = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = in.gate(i, cc) * kLog2e;
                G[i][cc] = i ? G[i - 1][cc] + x : x;
                mk = fmaxf(mk, fabsf(in.kval(i, cc)));
                mq = fmaxf(mq, fabsf(in.qval(i, cc)));
            }
            sm.tot[l * CPL + cc][w] = G[7][cc];
        }
        mk = wave_max(mk);
        mq = wave_max(mq);
        if (l == 0) {
            sm.wmax[0][w] = mk;
            sm.wmax[1][w] = mq;
        }
        if (w == 0) {
            sm.beta[l] = (l < nv) ? in.bt : 0.f;
            sm.wr[l] = (l < nv) ? (DEC ? in.wt : in.bt) : 0.f;
        }
        if (tid == 0) sm.anybig = 0;
        lds_barrier();   // B0

        // ======== anchors m = g_n / 2 per channel, scales, channels beyond the range
        float gn[CPL], m[CPL];
        bool bigc[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int c = l * CPL + cc;
            const float4 ta = reinterpret_cast<const float4 *>(&sm.tot[c][0])[0];
            const float4 tb = reinterpret_cast<const float4 *>(&sm.tot[c][0])[1];
            const float tw[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
            float run = 0.f, pre = 0.f;
#pragma unroll
            for (int ww = 0; ww < kFW; ++ww) {
                if (ww == w) pre = run;
                run += tw[ww];
            }
            gn[cc] = run;
            m[cc] = 0.5f * run;
            bigc[cc] = -run > kBig2;
#pragma unroll
            for (int i = 0; i < 8; ++i) G[i][cc] += pre;
        }
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int ww = 0; ww < kFW; ++ww) {
            sk = fmaxf(sk, sm.wmax[0][ww]);
            sq = fmaxf(sq, sm.wmax[1][ww]);
        }
        sk = pow2_scale(sk);
        sq = pow2_scale(sq);
        const bool wbig = __ballot(bigc[0] || bigc[1]) != 0;   // the same channels in every wave
        if (w == 0) {
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                sm.big[l * CPL + cc] = bigc[cc] ? 1 : 0;
                sm.egn[l * CPL + cc] = kexp2<false>(gn[cc]);
            }
            if (wbig && l == 0) sm.anybig = 1;
        }

        // ======== operands: Gram (bf16, anchored at m) and state phase (fp16, scaled)
        if (!wbig) {   // no channel beyond the range in this wave: one form for all
            float emk[CPL], emq[CPL], egk[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const float em = kexp2<false>(m[cc]);
                emk[cc] = em * sk;
                emq[cc] = em * sq;
                egk[cc] = kexp2<false>(gn[cc] - m[cc]) * sk;
            }
            // e^{G-m} and e^{m-G} along this wave's eight rows as running products
            // of the per-token decays (one exponential per token and channel)
            float ex1[8][CPL], ex2[8][CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                float al[8];
#pragma unroll
                for (int i = 1; i < 8; ++i) al[i] = kexp2<false>(in.gate(i, cc) * kLog2e);
                ex1[0][cc] = kexp2<false>(G[0][cc] - m[cc]);
                ex2[7][cc] = kexp2<false>(m[cc] - G[7][cc]);
#pragma unroll
                for (int i = 1; i < 8; ++i) ex1[i][cc] = ex1[i - 1][cc] * al[i];
#pragma unroll
                for (int i = 6; i >= 0; --i) ex2[i][cc] = ex2[i + 1][cc] * al[i + 1];
            }
            f16x4_t kit[CPL][2];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * w + i;
                bf16x2_t ka2, qh2, ql2, kh2, kl2;
                f16x2_t ke2, qe2;
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float kv = in.kval(i, cc), qv = in.qval(i, cc);
                    const float e1 = ex1[i][cc], e2 = ex2[i][cc];
                    const float ka = kv * e1, qa = qv * e1, ki = kv * e2;
                    bf16_t hh, ll;
                    ka2[cc] = (bf16_t)ka;
                    split_bf16(qa, hh, ll);
                    qh2[cc] = hh;
                    ql2[cc] = ll;
                    split_bf16(ki, hh, ll);
                    kh2[cc] = hh;
                    kl2[cc] = ll;
                    ke2[cc] = (f16_t)(ka * emk[cc]);
                    qe2[cc] = (f16_t)(qa * emq[cc]);
                    kit[cc][i >> 2][i & 3] = (f16_t)(ki * egk[cc]);
                }
                const int c0 = l * CPL, s0 = kslot(c0);
                *reinterpret_cast<bf16x2_t *>(&sm.g.KA[r][c0]) = ka2;
                *reinterpret_cast<bf16x2_t *>(&sm.g.KI[0][r][c0]) = kh2;
                *reinterpret_cast<bf16x2_t *>(&sm.g.KI[1][r][c0]) = kl2;
                *reinterpret_cast<f16x2_t *>(&sm.KE[r][s0]) = ke2;
                if (need_o) {
                    *reinterpret_cast<bf16x2_t *>(&sm.g.QA[0][r][c0]) = qh2;
                    *reinterpret_cast<bf16x2_t *>(&sm.g.QA[1][r][c0]) = ql2;
                    *reinterpret_cast<f16x2_t *>(&sm.QE[r][s0]) = qe2;
                }
            }
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    *reinterpret_cast<f16x4_t *>(&sm.KIt[l * CPL + cc][kslot(8 * w + 4 * half)]) = kit[cc][half];
        } else {
            float Em[CPL], Egm[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                Em[cc] = kexp2<false>(m[cc]);
                Egm[cc] = kexp2<false>(gn[cc] - m[cc]);
            }
            f16x4_t kit[CPL][2];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * w + i;
                const bool valid = r < nv;
                bf16x2_t ka2, qh2, ql2, kh2, kl2;
                f16_t ke2[CPL], qe2[CPL];
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float kv = valid ? in.kval(i, cc) : 0.f, qv = valid ? in.qval(i, cc) : 0.f;
                    const float e1 = kexp2<false>(G[i][cc] - m[cc]), e2 = kexp2<false>(m[cc] - G[i][cc]);
                    float eG = e1 * Em[cc], eI = e2 * Egm[cc];
                    if (wbig && bigc[cc]) {
                        eG = kexp2<false>(G[i][cc]);
                        eI = kexp2<false>(gn[cc] - G[i][cc]);
                    }
                    const float ka = bigc[cc] ? 0.f : kv * e1, qa = bigc[cc] ? 0.f : qv * e1;
                    const float ki = bigc[cc] ? 0.f : kv * e2;
                    bf16_t hh, ll;
                    ka2[cc] = (bf16_t)ka;
                    split_bf16(qa, hh, ll);
                    qh2[cc] = hh;
                    ql2[cc] = ll;
                    split_bf16(ki, hh, ll);
                    kh2[cc] = hh;
                    kl2[cc] = ll;
                    ke2[cc] = (f16_t)(kv * eG * sk);
                    qe2[cc] = (f16_t)(qv * eG * sq);
                    kit[cc][i >> 2][i & 3] = (f16_t)(kv * eI * sk);
                }
                const int c0 = l * CPL, s0 = kslot(c0);   // two adjacent channels: adjacent slots
                *reinterpret_cast<bf16x2_t *>(&sm.g.KA[r][c0]) = ka2;
                *reinterpret_cast<bf16x2_t *>(&sm.g.KI[0][r][c0]) = kh2;
                *reinterpret_cast<bf16x2_t *>(&sm.g.KI[1][r][c0]) = kl2;
                {
                    f16x2_t x2;
                    x2[0] = ke2[0];
                    x2[1] = ke2[1];
                    *reinterpret_cast<f16x2_t *>(&sm.KE[r][s0]) = x2;
                }
                if (need_o) {
                    *reinterpret_cast<bf16x2_t *>(&sm.g.QA[0][r][c0]) = qh2;
                    *reinterpret_cast<bf16x2_t *>(&sm.g.QA[1][r][c0]) = ql2;
                    f16x2_t x2;
                    x2[0] = qe2[0];
                    x2[1] = qe2[1];
                    *reinterpret_cast<f16x2_t *>(&sm.QE[r][s0]) = x2;
                }
            }
            // rows 8w..8w+3 and 8w+4..8w+7 each fill four consecutive token slots
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    *reinterpret_cast<f16x4_t *>(&sm.KIt[l * CPL + cc][kslot(8 * w + 4 * half)]) = kit[cc][half];
        }
        lds_barrier();   // B1

        // ======== Gram blocks A = b.KA KI^T and P = QA KI^T, ten 16x16 block pairs
        f32x4_t accA[2], accP[2];
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
            const int p = w + 8 * pi;
            accA[pi] = zero4();
            accP[pi] = zero4();
            if (p < 10) {
                int Rp, Ip;
                lower_block(p, Rp, Ip);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int c0 = 32 * ks + 8 * lg;
                    const bf16x8_t bh = lds_ld8(&sm.g.KI[0][16 * Ip + lr][c0]);
                    const bf16x8_t bl = lds_ld8(&sm.g.KI[1][16 * Ip + lr][c0]);
                    const bf16x8_t ka = lds_ld8(&sm.g.KA[16 * Rp + lr][c0]);
                    accA[pi] = mfma16(ka, bh, accA[pi]);
                    accA[pi] = mfma16(ka, bl, accA[pi]);
                    if (need_o) {
                        const bf16x8_t qh = lds_ld8(&sm.g.QA[0][16 * Rp + lr][c0]);
                        const bf16x8_t ql = lds_ld8(&sm.g.QA[1][16 * Rp + lr][c0]);
                        accP[pi] = mfma3(qh, ql, bh, bl, accP[pi]);
                    }
                }
            }
        }
        lds_barrier();   // B2: the Gram operands are consumed
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
            const int p = w + 8 * pi;
            if (p < 10) {
                int Rp, Ip;
                lower_block(p, Rp, Ip);
                const int i = 16 * Ip + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * Rp + 4 * lg + e;
                    sm.r.ap.A[r][i] = (i < r) ? sm.beta[r] * accA[pi][e] : 0.f;
                    if (need_o) sm.r.ap.P[r][i] = (i <= r) ? accP[pi][e] : 0.f;
                }
            }
        }
        lds_barrier();   // B3

        // ======== exact terms of the channels left out (rare): all pairs i <= r
        if (sm.anybig) {
            constexpr int NPAIR = kC * (kC + 1) / 2, PPT = (NPAIR + kFT - 1) / kFT;
            constexpr int XQ = FusedSmem<DK, DV>::XQ;
            float sa[PPT], sp[PPT];
#pragma unroll
            for (int j = 0; j < PPT; ++j) sa[j] = sp[j] = 0.f;
            for (int qi = 0; qi < DK / XQ; ++qi) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * w + i;
                    const bool valid = r < nv;
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        const int c = l * CPL + cc;
                        if (c / XQ == qi) {
                            sm.r.x.G[r][c % XQ] = G[i][cc];
                            sm.r.x.K[r][c % XQ] = valid ? in.kval(i, cc) : 0.f;
                            sm.r.x.Q[r][c % XQ] = valid ? in.qval(i, cc) : 0.f;
                        }
                    }
                }
                lds_barrier();
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    const int p = tid + kFT * j;
                    if (p < NPAIR) {
                        int r = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
                        if ((r + 1) * (r + 2) / 2 <= p) ++r;
                        if (r * (r + 1) / 2 > p) --r;
                        const int i = p - r * (r + 1) / 2;
                        for (int cq = 0; cq < XQ; ++cq) {
                            if (sm.big[XQ * qi + cq]) {
                                const float kk = sm.r.x.K[i][cq] * kexp2<false>(sm.r.x.G[r][cq] - sm.r.x.G[i][cq]);
                                sa[j] += sm.r.x.K[r][cq] * kk;
                                sp[j] += sm.r.x.Q[r][cq] * kk;
                            }
                        }
                    }
                }
                lds_barrier();
            }
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int p = tid + kFT * j;
                if (p < NPAIR) {
                    int r = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
                    if ((r + 1) * (r + 2) / 2 <= p) ++r;
                    if (r * (r + 1) / 2 > p) --r;
                    const int i = p - r * (r + 1) / 2;
                    if (i < r) sm.r.ap.A[r][i] += sm.beta[r] * sa[j];
                    if (need_o) sm.r.ap.P[r][i] += sp[j];
                }
            }
            lds_barrier();
        }

        // ======== D_R = (I + A_RR)^{-1} (waves 0-3) while waves 4-7 convert P and
        // the blocks of A below the diagonal; then D to fp16
        diag_inverse(sm, w, l, [&] {
            if (need_o) p_convert(sm, tid - 256);
            a_convert(sm, tid - 256);
        });
        if (tid < 256) d_convert(sm, tid);
        // V^T over A and P, which the transform has consumed (rows past the chunk zero)
#pragma unroll
        for (int cv = 0; cv < CPV; ++cv) {
            bf16x8_t x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (8 * w + i < nv) ? (bf16_t)vget(vr[i], cv) : (bf16_t)0.f;
            *reinterpret_cast<bf16x8_t *>(&sm.r.Vt[l * CPV + cv][8 * w]) = x;
        }
        lds_barrier();   // B5: the state-phase operands are complete

        // ======== next chunk's inputs in flight, then the state phase
        const bool more = tbase + kC < tk.t1;
        const int64_t tn = tbase + kC;
        const int nvn = more ? (int)((tk.t1 - tn) < kC ? (tk.t1 - tn) : kC) : 0;
        auto issue = [&](int part) {
            if (more) load_part(part, tn, nvn, l);
        };
        if (HAS_STATE) {
            state_chunk<DK, DV, NTX, WITH_O, HAS_V, IO>(sm, S, col0, 1.f / sk, 1.f / sq, o, tbase, nv, H, h, l, issue);
        } else {
#pragma unroll
            for (int part = 0; part < 4; ++part) issue(part);
        }
    }

    if (HAS_STATE && dst) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * mt + 4 * lg0 + e, c = col0 + 16 * nt + lr0;
                    dst[(int64_t)r * ld + c] = S[mt][nt][e];
                }
    }
}

// A chain, or a segment of one, with o: every wave holds DV / 8 value columns
// of the state (16 at d_v = 128), from src (or zero) to dst (if given).
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__device__ __forceinline__ void out_task(FusedSmem<DK, DV> &sm, const FusedArgs &a, const Task &tk, int w, int tid,
                                         const float *src, float *dst) {
    static_assert(DV == 128, "eight waves of 16 value columns");
    chain_loop<DK, DV, IO, GT, PRO, GM, DEC, DV / 128, true, true, true>(sm, a, tk, w, tid, w * (DV / 8), src, false,
                                                                         dst, DV, true);
}

// First launch of a segmented call: blocks below the chain count run segment
// 0 of their chain exactly from h0 (o, and its end state as the start state of
// segment 1); the others run segments 1 .. nseg - 2 from (S, Phi) = (0, I) and
// store the end state S_loc and the transition Phi.
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__global__ __launch_bounds__(kFT, 1) void fused_phi_kernel(const FusedArgs a) {
    typedef FusedSmem<DK, DV> Sm;
    static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
    __shared__ Sm sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Task tk = fused_task(a);
    const size_t sv = (size_t)DK * DV, sp = (size_t)DK * DK;
    if (!tk.phi) {
        out_task<DK, DV, IO, GT, PRO, GM, DEC>(sm, a, tk, w, tid, a.h0 ? a.h0 + tk.chain * sv : nullptr,
                                               a.seg_in + tk.chain * (a.nseg - 1) * sv);
        return;
    }
    const int64_t slot = tk.chain * (a.nseg - 2) + (tk.seg - 1);
    if (w < 4)   // S from zero over the segment
        chain_loop<DK, DV, IO, GT, PRO, GM, DEC, DV / 64, false, true, true>(
            sm, a, tk, w, tid, w * (DV / 4), nullptr, false, a.seg_loc + slot * sv, DV, false);
    else         // Phi from the identity: the same step with no value input
        chain_loop<DK, DV, IO, GT, PRO, GM, DEC, DK / 64, false, false, true>(
            sm, a, tk, w, tid, (w - 4) * (DK / 4), nullptr, true, a.seg_phi + slot * sp, DK, false);
}

// One pass (pass 0), or the last launch of a segmented call (segments 1 ..
// nseg - 1 from their start states): o, and h_T at the end of the chain.
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__global__ __launch_bounds__(kFT, 1) void fused_out_kernel(const FusedArgs a) {
    typedef FusedSmem<DK, DV> Sm;
    static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
    __shared__ Sm sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Task tk = fused_task(a);
    const size_t sv = (size_t)DK * DV;
    const float *src;
    float *dst;
    if (a.pass == 2) {
        src = a.seg_in + (tk.chain * (a.nseg - 1) + (tk.seg - 1)) * sv;
        dst = (tk.seg == a.nseg - 1 && a.h_T) ? a.h_T + tk.chain * sv : nullptr;
    } else {
        src = a.h0 ? a.h0 + tk.chain * sv : nullptr;
        dst = a.h_T ? a.h_T + tk.chain * sv : nullptr;
    }
    out_task<DK, DV, IO, GT, PRO, GM, DEC>(sm, a, tk, w, tid, src, dst);
}

// Start states of segments 2 .. nseg - 1 of every chain, from that of segment
// 1 (the exact end state of segment 0):
// S_in[s + 1] = Phi[s] S_in[s] + S_loc[s] for s = 1 .. nseg - 2, in fp32 on the
// fp32 matrix cores.  One workgroup per (chain, 16 value columns): the columns
// are independent.
template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_kernel(float *__restrict__ seg_in, const float *__restrict__ seg_loc,
                                                       const float *__restrict__ seg_phi, int nseg) {
    constexpr int NCB = DV / 16, MTW = DK / 64;   // row tiles per wave
    __shared__ float xin[DK][17];
    const int64_t chain = blockIdx.x / NCB;
    const int col0 = 16 * (int)(blockIdx.x % NCB);
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const size_t sv = (size_t)DK * DV, sp = (size_t)DK * DK;
    const float *in1 = seg_in + chain * (nseg - 1) * sv;
    for (int idx = tid; idx < DK * 16; idx += 256) xin[idx >> 4][idx & 15] = in1[(size_t)(idx >> 4) * DV + col0 + (idx & 15)];
    for (int s = 1; s + 1 < nseg; ++s) {
        __syncthreads();
        const float *phi = seg_phi + (chain * (nseg - 2) + (s - 1)) * sp;
        const float *loc = seg_loc + (chain * (nseg - 2) + (s - 1)) * sv;
        f32x4_t acc[MTW];
#pragma unroll
        for (int j = 0; j < MTW; ++j) {
            const int mt = wv + 4 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] = loc[(size_t)(16 * mt + 4 * lg + e) * DV + col0 + lr];
#pragma unroll 8
            for (int kk = 0; kk < DK / 4; ++kk)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(phi[(size_t)(16 * mt + lr) * DK + 4 * kk + lg],
                                                              xin[4 * kk + lg][lr], acc[j], 0, 0, 0);
        }
        __syncthreads();
        float *out = seg_in + (chain * (nseg - 1) + s) * sv;
#pragma unroll
        for (int j = 0; j < MTW; ++j) {
            const int mt = wv + 4 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mt + 4 * lg + e;
                xin[r][lr] = acc[j][e];
                out[(size_t)r * DV + col0 + lr] = acc[j][e];
            }
        }
    }
}

// Sequences of a packed batch in order of decreasing length (ties by index):
// rank by counting, one thread per sequence.
__global__ __launch_bounds__(256) void seq_order_kernel(const int32_t *__restrict__ cu, int64_t N,
                                                        int32_t *__restrict__ order) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int32_t len = cu[n + 1] - cu[n];
    int64_t rank = 0;
    for (int64_t m = 0; m < N; ++m) {
        const int32_t lm = cu[m + 1] - cu[m];
        rank += (lm > len) || (lm == len && m < n);
    }
    order[rank] = (int32_t)n;
}

constexpr int64_t kFusedTargetBlocks = 256;   // one workgroup per compute unit
constexpr int64_t kMinSegChunks = 4;          // shortest segment worth its transition pass
constexpr int64_t kOrderMaxSeqs = 16384;      // longest-first order up to this many sequences

struct FusedPlan {
    int64_t chains;
    int nseg, seg_chunks, head_chunks;
    bool order;
    size_t order_off, in_off, loc_off, phi_off, bytes;
};

FusedPlan fused_plan(const ChunkArgs &a) {
    FusedPlan p = {};
    p.chains = a.num_seqs * (int64_t)a.H;
    p.nseg = 1;
    p.seg_chunks = 0;
    if (!a.varlen && p.chains > 0) {
        // both launches of a segmented call run chains * (nseg - 1) <= target
        // workgroups, one round on the chip
        const int64_t nch = (a.seq_len + kC - 1) / kC;
        int64_t ns = kFusedTargetBlocks / p.chains + 1;
        if (ns > nch / kMinSegChunks) ns = nch / kMinSegChunks;
        if (ns >= 3) {
            const int64_t sc = (nch + ns - 1) / ns;
            ns = (nch + sc - 1) / sc;   // no empty segment
            if (ns >= 3) {
                p.nseg = (int)ns;
                p.seg_chunks = (int)sc;
                p.head_chunks = (int)sc;
                // The first launch's exact first segment runs slower per chunk
                // than the transitions beside it (about 8 : 7): give it about
                // 7/8 of the others' length (measured best between 0.85 and
                // 0.9) where that shortens the two launches together, whose
                // time goes as max(head, 7/8 segment) + segment.
                const int64_t s2 = (8 * nch + 8 * ns - 2) / (8 * ns - 1);   // ceil(nch / (ns - 1/8))
                int64_t h2 = 7 * s2 / 8;
                if (h2 < 1) h2 = 1;
                const int64_t n2 = 1 + (nch - h2 + s2 - 1) / s2;
                const int64_t t_even = 16 * sc, t_head = (8 * h2 > 7 * s2 ? 8 * h2 : 7 * s2) + 8 * s2;
                if (n2 >= 3 && n2 <= ns && h2 <= s2 && t_head < t_even) {
                    p.nseg = (int)n2;
                    p.seg_chunks = (int)s2;
                    p.head_chunks = (int)h2;
                }
            }
        }
    }
    p.order = a.varlen && a.num_seqs > 1 && a.num_seqs <= kOrderMaxSeqs;
    size_t off = 0;
    p.order_off = off;
    if (p.order) off += plan_bytes(a.num_seqs);
    const size_t sv = (size_t)a.d_k * a.d_v * 4, sp = (size_t)a.d_k * a.d_k * 4;
    const size_t in_slots = p.nseg >= 3 ? (size_t)p.chains * (p.nseg - 1) : 0;
    const size_t mid_slots = p.nseg >= 3 ? (size_t)p.chains * (p.nseg - 2) : 0;
    p.in_off = off;
    off += in_slots * sv;
    p.loc_off = off;
    off += mid_slots * sv;
    p.phi_off = off;
    off += mid_slots * sp;
    p.bytes = off;
    return p;
}

template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
hipError_t launch_fused_t(const ChunkArgs &a, hipStream_t st) {
    const FusedPlan p = fused_plan(a);
    uint8_t *ws = reinterpret_cast<uint8_t *>(a.workspace);
    FusedArgs f = {};
    f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.beta = a.beta; f.wr = a.w_write;
    f.h0 = a.h0; f.cu = a.varlen ? a.cu_seqlens : nullptr; f.o = a.o; f.h_T = a.h_T;
    f.N = a.num_seqs; f.T = a.seq_len; f.H = a.H; f.lo = a.log_alpha_min;
    f.nseg = p.nseg; f.seg_chunks = p.seg_chunks; f.head_chunks = p.head_chunks;
    if (p.chains == 0) return hipSuccess;
    if (p.nseg < 3) {
        if (p.order) {
            int32_t *order = reinterpret_cast<int32_t *>(ws + p.order_off);
            hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((a.num_seqs + 255) / 256)), dim3(256), 0, st,
                               a.cu_seqlens, a.num_seqs, order);
            f.order = order;
        }
        f.pass = 0;
        hipLaunchKernelGGL((fused_out_kernel<DK, DV, IO, GT, PRO, GM, DEC>), dim3((unsigned)p.chains), dim3(kFT), 0, st,
                           f);
        return hipGetLastError();
    }
    f.seg_in = reinterpret_cast<float *>(ws + p.in_off);
    f.seg_loc = reinterpret_cast<float *>(ws + p.loc_off);
    f.seg_phi = reinterpret_cast<float *>(ws + p.phi_off);
    f.pass = 1;
    hipLaunchKernelGGL((fused_phi_kernel<DK, DV, IO, GT, PRO, GM, DEC>), dim3((unsigned)(p.chains * (p.nseg - 1))),
                       dim3(kFT), 0, st, f);
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV>), dim3((unsigned)(p.chains * (DV / 16))), dim3(256), 0, st, f.seg_in,
                       (const float *)f.seg_loc, (const float *)f.seg_phi, p.nseg);
    f.pass = 2;
    hipLaunchKernelGGL((fused_out_kernel<DK, DV, IO, GT, PRO, GM, DEC>), dim3((unsigned)(p.chains * (p.nseg - 1))),
                       dim3(kFT), 0, st, f);
    return hipGetLastError();
}

template <int DK, int DV, bool PRO, int GM, bool DEC>
hipError_t launch_fused_types(const ChunkArgs &a, hipStream_t st) {
    return a.gate_bf16 ? launch_fused_t<DK, DV, bf16_t, bf16_t, PRO, GM, DEC>(a, st)
                       : launch_fused_t<DK, DV, bf16_t, float, PRO, GM, DEC>(a, st);
}

template <int DK, int DV>
hipError_t launch_fused_variants(const ChunkArgs &a, hipStream_t st) {
    if (a.gate_mode == kGatePerHead) return launch_fused_types<DK, DV, false, kGatePerHead, false>(a, st);
    if (a.gate_mode == kGateNone) return launch_fused_types<DK, DV, false, kGateNone, false>(a, st);
    if (a.prologue) return launch_fused_types<DK, DV, true, kGatePerChannel, false>(a, st);
    if (a.w_write) return launch_fused_types<DK, DV, false, kGatePerChannel, true>(a, st);
    return launch_fused_types<DK, DV, false, kGatePerChannel, false>(a, st);
}

}  // namespace

// bf16 I/O at d_k = d_v = 128 runs the fused kernel.
// Which forward runs a call: the fused kernel takes bf16 I/O at d_k = d_v = 128
// for packed batches, raw projections and separate write strengths (whose
// long-context outputs need its hi/lo and scaled fp16 operands to stay within
// the bf16 bound); plain KDA and the scalar gates over an equal-length batch run
// the two-kernel path (prep + state kernels), which is faster there.  A packed
// batch gives bitwise the results of each of its sequences packed alone.  The
// forward that allocates nothing takes the fused kernel for every batch shape,
// since its workspace (segment states of at most about 380 chains) is bounded.
bool fused_fwd_supported(const ChunkArgs &a) {
    if (!a.io_bf16 || a.d_k != 128 || a.d_v != 128) return false;
    return a.force_fused || a.varlen || a.prologue || a.w_write != nullptr;
}

// Chains are split only when nseg = floor(target / chains) + 1 >= 3, i.e. chains
// <= target / 2, and then chains * (nseg - 1) <= target.  The segment states
// take chains * (3 nseg - 5) = 3 chains (nseg - 1) - 2 chains < 3 target
// matrices of d_k x d_v (or d_k x d_k) fp32: those of any call fit the scratch
// of the forward that allocates nothing.
static_assert((size_t)3 * kFusedTargetBlocks * 128 * 128 * 4 <= kNoAllocScratchBytes,
              "fused segment states exceed the no-allocation scratch");

size_t fused_fwd_workspace_bytes(const ChunkArgs &a) { return fused_plan(a).bytes; }

// Every launch of the call within the HIP limits: the chain kernels (one
// workgroup per chain or segment), the sequence order and the segment scan.
bool fused_fwd_grids_fit(const ChunkArgs &a) {
    const FusedPlan p = fused_plan(a);
    if (!grid_fits(p.nseg >= 3 ? p.chains * (p.nseg - 1) : p.chains, kFT)) return false;
    if (p.order && !grid_fits((a.num_seqs + 255) / 256, 256)) return false;
    return p.nseg < 3 || grid_fits(p.chains * (a.d_v / 16), 256);
}

hipError_t launch_fused_fwd(const ChunkArgs &a, hipStream_t st) {
    return launch_fused_variants<128, 128>(a, st);
}

}  // namespace kda
