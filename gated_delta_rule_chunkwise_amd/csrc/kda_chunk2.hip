// kda_chunk2.hip -- chunkwise KDA forward for bf16 I/O in two kernels.
//
// The chunkwise form (KimiLinear article, section 3.1) splits each chunk's work
// into a part that does not depend on the state -- the in-chunk log-decay
// cumsum, the decayed key/query operands, the decay-weighted Gram blocks A and
// P and the UT transform T = (I + A)^{-1} -- and a part that carries the state
// from chunk to chunk.  Only the second part is sequential.  Here:
//
//   chunk_prep_kernel   one workgroup per (chunk, head), all chunks in parallel:
//                       computes the state-independent part once and writes a
//                       compact record per chunk-head to the workspace;
//   chunk_state_kernel  one workgroup per (sequence, head, block of BV value
//                       columns): walks the chunks of its sequence, keeping the
//                       fp32 state block in registers, and reads the records.
//
// Per chunk with start state S, with the operands of the record
// (m = g_n / 2 per channel, see kda_chunk.hip for the derivation):
//   Y = KA (e^m . S),  Z = QA (e^m . S)            KA = K.e^{G-m}, QA = Q.e^{G-m}
//   X = diag(beta) (V - Y),  U = T X
//   O = Z + P U
//   S <- Diag(e^{g_n}) S + Diag(e^{g_n-m}) (KI^T U)    KI = K.e^{m-G}
// Chunks whose in-chunk decay exceeds the matrix-core range are flagged by the
// prep kernel and run token by token in the state kernel.
//
// Record layout: matrix operands are stored in the order the state kernel's
// lanes hold them, so that every wave-wide load reads one contiguous 1 KiB (or
// 512 B) run.  A "fragment" is one 16x32 bf16 operand of the 16x16x32 matrix
// instruction, lane l holding row l%16, columns 8*(l/16)..+7 (16 bytes at l*16).
//   KA, QA   fragments (row block rb, k-step ks), rb*NKS + ks, NKS = DK/32
//   KIt      fragments (key block mt, token k-step ks) of KI^T, mt*2 + ks
//   T        the six fragments (R, ks <= R/2) of T that a 32-wide k-step reads,
//            each as hi then lo; blocks above the diagonal inside them are zero
//   PT       the ten lower tiles (R, I <= R) of P, transposed and in the 16x16x16
//            operand layout (lane l: P[16R + l%16][16I + 4*(l/16)..+3], 8 bytes),
//            each as hi then lo
//   e^m, e^{g_n}, e^{g_n-m} fp32[3][DK], beta fp32[64], flags int32[4];
// padded to a multiple of 256 bytes.
#include "kda_chunk_common.h"
#include "kda_launch.h"

#include <stdio.h>
#include <stdlib.h>

namespace kda {
namespace {

template <int DK> struct Rec {
    static constexpr int NKS = DK / 32;
    static constexpr size_t FRAG = 1024;                          // 64 lanes x 16 bytes
    static constexpr size_t TILE = 512;                           // 64 lanes x 8 bytes
    static constexpr size_t KA = 0;
    static constexpr size_t QA = KA + 4 * NKS * FRAG;
    static constexpr size_t KIT = QA + 4 * NKS * FRAG;
    static constexpr size_t T = KIT + (DK / 16) * 2 * FRAG;
    static constexpr size_t PT = T + 6 * 2 * FRAG;
    static constexpr size_t COL = PT + 10 * 2 * TILE;
    static constexpr size_t BETA = COL + 3 * (size_t)DK * 4;
    static constexpr size_t FLAG = BETA + (size_t)kC * 4;
    static constexpr size_t BYTES = ((FLAG + 16) + 255) / 256 * 256;
};

// Index of the stored T fragment (row block R, k-step ks); k-steps right of the
// diagonal block are never read and map to ks = 0 (a harmless duplicate load).
__device__ __forceinline__ int t_frag(int R, int ks) {
    ks = ks <= (R >> 1) ? ks : 0;
    return R < 2 ? R : 2 + 2 * (R - 2) + ks;
}
// Slot of the lower tile (R, I), I <= R; I > R maps to I = R.
__device__ __forceinline__ int p_tile(int R, int I) { return (R * (R + 1)) / 2 + (I <= R ? I : R); }

constexpr size_t kHeaderBytes = 256;

size_t plan_bytes(int64_t num_seqs) { return ((size_t)(num_seqs + 1) * 4 + 255) / 256 * 256; }

int64_t max_chunks(const ChunkArgs &a) {
    if (a.varlen) return (a.total_tokens + kC - 1) / kC + a.num_seqs;
    return a.num_seqs * ((a.seq_len + kC - 1) / kC);
}

// chunk_off[n] = number of chunks of sequences 0..n-1 (exclusive prefix sum of
// ceil(L_n / 64)); chunk_off[N] = total.  One workgroup.
__global__ __launch_bounds__(256) void chunk_plan_kernel(const int32_t *__restrict__ cu, int64_t N,
                                                         int32_t *__restrict__ chunk_off) {
    __shared__ int32_t part[256];
    __shared__ int32_t carry;
    const int t = threadIdx.x;
    if (t == 0) carry = 0;
    __syncthreads();
    for (int64_t base = 0; base <= N; base += 256) {
        const int64_t n = base + t;
        int32_t cnt = 0;
        if (n < N) cnt = (cu[n + 1] - cu[n] + kC - 1) / kC;
        part[t] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {   // inclusive Hillis-Steele scan
            const int32_t x = t >= off ? part[t - off] : 0;
            __syncthreads();
            part[t] += x;
            __syncthreads();
        }
        if (n <= N) chunk_off[n] = carry + part[t] - cnt;
        __syncthreads();
        if (t == 255) carry += part[255];
        __syncthreads();
    }
}

// Finds the sequence and token range of chunk `chunk`; false if past the end.
__device__ __forceinline__ bool locate_chunk(int64_t chunk, const int32_t *__restrict__ cu,
                                             const int32_t *__restrict__ chunk_off, int64_t N, int64_t T,
                                             int64_t &n, int64_t &t0, int &nv) {
    if (cu) {
        if (chunk >= chunk_off[N]) return false;
        int64_t lo = 0, hi = N - 1;   // largest n with chunk_off[n] <= chunk (and a non-empty sequence)
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (chunk_off[mid] <= chunk) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        t0 = cu[n] + (int64_t)kC * (chunk - chunk_off[n]);
        const int64_t rem = cu[n + 1] - t0;
        nv = (int)(rem < kC ? rem : kC);
        return true;
    }
    const int64_t cps = (T + kC - 1) / kC;
    n = chunk / cps;
    const int64_t c = chunk % cps;
    t0 = n * T + (int64_t)kC * c;
    const int64_t rem = T - (int64_t)kC * c;
    nv = (int)(rem < kC ? rem : kC);
    return true;
}

template <int DK>
struct alignas(16) PrepSmem {
    static constexpr int KS = DK + 8;
    static constexpr int TS = kC + 8;
    static constexpr int FS = 68;
    union {
        struct {
            bf16_t KA[kC][KS];
            bf16_t QA[kC][KS];
        } g;                                   // Gram phase
        struct {
            bf16_t T[2][kC][TS];               // hi/lo of (I + A)^{-1}
            float T8[4][2][8][8];
            float W8[4][8][8];
        } t;                                   // inversion phase
    };
    union {
        bf16_t KI[kC][KS];                     // K . e^{m-G}
        bf16_t Tt[2][kC][kC + 4];              // transposed diagonal blocks of T
    };
    float A[kC][FS];
    float tot[DK][kWaves];
    float beta[kC];
};

// ---------------------------------------------------------------------------------
// Prep: one workgroup (8 waves) per (chunk, head).
template <int DK, typename IO, typename GT>
__global__ __launch_bounds__(kThreads, 4) void chunk_prep_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const GT *__restrict__ log_alpha,
    const GT *__restrict__ beta, const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
    uint8_t *__restrict__ recs, int64_t N, int64_t T, int32_t H) {
    constexpr int CPL = DK / 64;
    constexpr int NKS = DK / 32;
    typedef PrepSmem<DK> Sm;
    typedef Rec<DK> RL;
    __shared__ Sm sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    const int64_t chunk = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int64_t n, t0;
    int nv;
    if (!locate_chunk(chunk, cu, chunk_off, N, T, n, t0, nv)) return;
    uint8_t *rec = recs + (size_t)blockIdx.x * RL::BYTES;
    float *gCol = reinterpret_cast<float *>(rec + RL::COL);
    float *gBeta = reinterpret_cast<float *>(rec + RL::BETA);
    int32_t *gFlag = reinterpret_cast<int32_t *>(rec + RL::FLAG);

    // ---- load this chunk (rows past the end read the last row and are zeroed)
    ChunkRegs<DK, 16, IO, GT> in;
    in.load(q, k, q, log_alpha, beta, t0, nv, H, h, 0, 0, w, l, lg, lr, false);
    const bool partial = nv < kC;
    float csum[8][CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x = vget(in.la[i], cc) * kLog2e;
            if (partial && 8 * w + i >= nv) x = 0.f;
            csum[i][cc] = i ? csum[i - 1][cc] + x : x;
        }
        sm.tot[l * CPL + cc][w] = csum[7][cc];
    }
    if (w == 0) {
        const float b = (l < nv) ? in.bt : 0.f;
        sm.beta[l] = b;
        gBeta[l] = b;
    }
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
        big = big || !(-all <= kMaxRange2);
        if (w == 0) {
            gCol[c] = kexp2<false>(m2[cc]);
            gCol[DK + c] = kexp2<false>(all);
            gCol[2 * DK + c] = kexp2<false>(all - m2[cc]);
        }
    }
    const bool slow = __ballot(big) != 0;   // same totals in every wave: uniform
    if (tid == 0) gFlag[0] = slow ? 1 : 0;
    if (slow) return;                        // the state kernel runs this chunk token by token

    // ---- decayed operands: LDS for the Gram products, record for the state kernel
    {
        float e1[8][CPL], e2[8][CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float al[8];
            al[0] = 1.f;
#pragma unroll
            for (int i = 1; i < 8; ++i) {
                float x = vget(in.la[i], cc) * kLog2e;
                if (partial && 8 * w + i >= nv) x = 0.f;
                al[i] = kexp2<false>(x);
            }
            e1[0][cc] = kexp2<false>(csum[0][cc] - m2[cc]);
#pragma unroll
            for (int i = 1; i < 8; ++i) e1[i][cc] = e1[i - 1][cc] * al[i];
            e2[7][cc] = kexp2<false>(m2[cc] - csum[7][cc]);
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
        bf16x8_t kit[CPL];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * w + i;
            bf16_t ka[CPL], qa[CPL], ki[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const float kv = vget(in.kk[i], cc), qv = vget(in.qq[i], cc);
                ka[cc] = (bf16_t)(kv * e1[i][cc]);
                qa[cc] = (bf16_t)(qv * e1[i][cc]);
                ki[cc] = (bf16_t)(kv * e2[i][cc]);
                kit[cc][i] = ki[cc];
            }
            if constexpr (CPL == 2) {
                bf16x2_t p;
                p[0] = ka[0]; p[1] = ka[1];
                *reinterpret_cast<bf16x2_t *>(&sm.g.KA[r][2 * l]) = p;
                p[0] = qa[0]; p[1] = qa[1];
                *reinterpret_cast<bf16x2_t *>(&sm.g.QA[r][2 * l]) = p;
                p[0] = ki[0]; p[1] = ki[1];
                *reinterpret_cast<bf16x2_t *>(&sm.KI[r][2 * l]) = p;
            } else {
                sm.g.KA[r][l] = ka[0];
                sm.g.QA[r][l] = qa[0];
                sm.KI[r][l] = ki[0];
            }
        }
        // KI^T: this lane holds 8 consecutive tokens 8w.. of key channel c, i.e. the
        // 16-byte piece of lane (c%16 + 16*(w%4)) of fragment (c/16, w/4)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int c = l * CPL + cc;
            const int f = (c >> 4) * 2 + (w >> 2), ln = (c & 15) + 16 * (w & 3);
            *reinterpret_cast<bf16x8_t *>(rec + RL::KIT + f * RL::FRAG + ln * 16) = kit[cc];
        }
    }
    lds_barrier();

    // ---- KA and QA to the record, fragment by fragment (1 KiB per wave-wide store)
#pragma unroll
    for (int it = 0; it < (2 * 4 * NKS * 64) / kThreads; ++it) {
        const int pc = tid + kThreads * it;
        const int mat = pc / (4 * NKS * 64);
        const int f = (pc >> 6) % (4 * NKS), ln = pc & 63;
        const int rb = f / NKS, ks = f % NKS;
        const int r = 16 * rb + (ln & 15), c = 32 * ks + 8 * (ln >> 4);
        const bf16x8_t x = lds_ld8(mat ? &sm.g.QA[r][c] : &sm.g.KA[r][c]);
        *reinterpret_cast<bf16x8_t *>(rec + (mat ? RL::QA : RL::KA) + f * RL::FRAG + ln * 16) = x;
    }

    // ---- Gram blocks: A (fp32, LDS) and P (hi/lo, record)
    {
        // A tiles as A[r][i] (rows of KA, columns of KI); P tiles transposed,
        // P^T[i][r] (rows of KI, columns of QA), so that the accumulator is the
        // 16x16x16 operand layout the record stores
        auto gram = [&](int tile, f32x4_t &acc, bool &isP, int &R, int &I) {
            isP = tile >= 10;
            lower_block(isP ? tile - 10 : tile, R, I);
            const bf16_t *xh = isP ? &sm.g.QA[16 * R + lr][8 * lg] : &sm.g.KA[16 * R + lr][8 * lg];
            const bf16_t *kh = &sm.KI[16 * I + lr][8 * lg];
            acc = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8_t xa = lds_ld8(xh + 32 * ks), kb = lds_ld8(kh + 32 * ks);
                acc = isP ? mfma16(kb, xa, acc) : mfma16(xa, kb, acc);
            }
        };
        auto finish = [&](bool isP, int R, int I, const f32x4_t &acc) {
            if (!isP) {
                const int i = 16 * I + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * R + 4 * lg + e;
                    sm.A[r][i] = (i < r) ? sm.beta[r] * acc[e] : 0.f;
                }
            } else {
                // lane holds P^T[16I + 4lg + e][16R + lr] = P[r][i], kept for i <= r
                const int r = 16 * R + lr;
                f32x4_t x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (16 * I + 4 * lg + e <= r) ? acc[e] : 0.f;
                uint8_t *dst = rec + RL::PT + (size_t)p_tile(R, I) * 2 * RL::TILE + l * 8;
                store_split4(reinterpret_cast<bf16_t *>(dst), reinterpret_cast<bf16_t *>(dst + RL::TILE), x);
            }
        };
        f32x4_t a0, a1;
        bool p0, p1;
        int R0, I0, R1, I1;
        gram(w, a0, p0, R0, I0);
        gram(w + 8, a1, p1, R1, I1);
        finish(p0, R0, I0, a0);
        finish(p1, R1, I1, a1);
        if (w < 4) {
            gram(w + 16, a0, p0, R0, I0);
            finish(p0, R0, I0, a0);
        }
    }
    lds_barrier();

    // ---- diagonal 16x16 blocks of T (waves 0-3)
    if (w < 4) {
        const int R = w;
        float (*t8)[8][8] = sm.t.T8[R];
        float (*w8)[8] = sm.t.W8[R];
        if (l < 16) {
            const int sb = l >> 3, j = l & 7, base = 16 * R + 8 * sb;
            float a[8][8];
#pragma unroll
            for (int r = 1; r < 8; ++r) {
                const float4 x0 = *reinterpret_cast<const float4 *>(&sm.A[base + r][base]);
                const float4 x1 = *reinterpret_cast<const float4 *>(&sm.A[base + r][base + 4]);
                a[r][0] = x0.x; a[r][1] = x0.y; a[r][2] = x0.z; a[r][3] = x0.w;
                a[r][4] = x1.x; a[r][5] = x1.y; a[r][6] = x1.z; a[r][7] = x1.w;
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
        const float vals[4] = {t8[0][i8][j8], 0.f, tba, t8[1][i8][j8]};
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int rr = 16 * R + 8 * (qd >> 1) + i8, cc = 16 * R + 8 * (qd & 1) + j8;
            bf16_t hh, ll;
            split_bf16(vals[qd], hh, ll);
            sm.t.T[0][rr][cc] = hh;
            sm.t.T[1][rr][cc] = ll;
            sm.Tt[0][cc][rr] = hh;
            sm.Tt[1][cc][rr] = ll;
        }
    }
    lds_barrier();

    // ---- off-diagonal blocks of T (waves 0 and 1, matrix cores)
    if (w < 2) {
        const int b = w;
        f32x4_t t10 = zero4();
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const int R = 2 * pr;
            bf16x4_t ah, al;
            load_split4(&sm.A[16 * (R + 1) + lr][16 * R + 4 * lg], ah, al);
            f32x4_t wacc = mma4(zero4(), ah, al, lds_ld4(&sm.Tt[0][16 * R + lr][16 * R + 4 * lg]),
                                lds_ld4(&sm.Tt[1][16 * R + lr][16 * R + 4 * lg]));
            bf16x4_t wh, wl;
            split4(wacc, wh, wl);
            f32x4_t tacc = mma4(zero4(), lds_ld4(&sm.t.T[0][16 * (R + 1) + lr][16 * (R + 1) + 4 * lg]),
                                lds_ld4(&sm.t.T[1][16 * (R + 1) + lr][16 * (R + 1) + 4 * lg]), wh, wl);
#pragma unroll
            for (int e = 0; e < 4; ++e) tacc[e] = -tacc[e];
            store_tile_split(&sm.t.T[0][0][0], &sm.t.T[1][0][0], Sm::TS, 16 * (R + 1), 16 * R, tacc, lr, lg);
            if (pr == 0) t10 = tacc;
        }
        wave_lds_sync();
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
        f32x4_t t2b = mma4(zero4(), lds_ld4(&sm.t.T[0][32 + lr][32 + 4 * lg]), lds_ld4(&sm.t.T[1][32 + lr][32 + 4 * lg]),
                           w2h[0], w2l[0]);
        f32x4_t t3b = mma4(zero4(), lds_ld4(&sm.t.T[0][48 + lr][32 + 4 * lg]), lds_ld4(&sm.t.T[1][48 + lr][32 + 4 * lg]),
                           w2h[0], w2l[0]);
        t3b = mma4(t3b, lds_ld4(&sm.t.T[0][48 + lr][48 + 4 * lg]), lds_ld4(&sm.t.T[1][48 + lr][48 + 4 * lg]), w2h[1],
                   w2l[1]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            t2b[e] = -t2b[e];
            t3b[e] = -t3b[e];
        }
        store_tile_split(&sm.t.T[0][0][0], &sm.t.T[1][0][0], Sm::TS, 32, 16 * b, t2b, lr, lg);
        store_tile_split(&sm.t.T[0][0][0], &sm.t.T[1][0][0], Sm::TS, 48, 16 * b, t3b, lr, lg);
    }
    lds_barrier();

    // ---- the six stored fragments of T, both planes, zeros above the block diagonal
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int pc = tid + kThreads * it;          // 0..767: (fragment, plane, lane)
        if (pc < 6 * 2 * 64) {
            const int fp = pc >> 6, f = fp >> 1, pl = fp & 1, ln = pc & 63;
            const int R = f < 2 ? f : 2 + ((f - 2) >> 1), ks = f < 2 ? 0 : ((f - 2) & 1);
            const int r = 16 * R + (ln & 15), c = 32 * ks + 8 * (ln >> 4);
            bf16x8_t v = lds_ld8(&sm.t.T[pl][r][c]);
            if ((c >> 4) > R) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (bf16_t)0.f;
            }
            *reinterpret_cast<bf16x8_t *>(rec + RL::T + (size_t)fp * RL::FRAG + ln * 16) = v;
        }
    }
}

// ---------------------------------------------------------------------------------
// State: one workgroup (8 waves) per (sequence, head, BV value columns).  The
// waves split into two roles with the same barrier sequence per chunk:
//   state role  (waves 0-3): own the fp32 state tiles; write e^m.S to LDS, form
//                            U = T X, update the state with KI^T U;
//   output role (waves 4-7): row block w-4 of the chunk: Y, Z, X and O = Z + P U.
// Each role runs its own loop, so each keeps only its own record operands in
// registers and its loads retire in a fixed order: every operand is reloaded for
// the next chunk right after its last use, about one chunk ahead of its next use.
template <int DK, int BV>
struct alignas(16) StateSmem {
    static constexpr int KS = DK + 8;
    static constexpr int TS = kC + 8;
    bf16_t S[BV][KS];          // (Diag(e^m) S)^T, single bf16
    bf16_t X[2][BV][TS];       // hi/lo of X^T
    bf16_t U[2][BV][TS];       // hi/lo of U^T
    float red[4][2 * BV + 1];  // token path
};

// The flag is read through a lane-dependent address (always element 0) so that
// it arrives by a vector load, counted in order with the other record loads,
// and not by a scalar load that every LDS barrier would wait for.
__device__ __forceinline__ int load_flag(const uint8_t *rec, size_t off, int tl) {
    return reinterpret_cast<const int32_t *>(rec + off)[tl >> 10];
}

template <int DK, int BV> struct StateRole {
    static constexpr int NT = BV / 16, STW = StateTiles<DK, BV>::STW;
    bf16x8_t th[2], tl[2];    // rows 16w.. of T (hi, lo)
    bf16x8_t kit[STW][2];     // KI^T rows of the wave's state tiles
    f32x4_t cm[STW], cg[STW], cgm[STW];
    int flag;

    __device__ __forceinline__ void load_cm(const uint8_t *rec, int w, int lg, int tid) {
        const float *col = reinterpret_cast<const float *>(rec + Rec<DK>::COL);
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int mt = (w * STW + i) / NT;
            cm[i] = *reinterpret_cast<const f32x4_t *>(col + 16 * mt + 4 * lg);
        }
        flag = load_flag(rec, Rec<DK>::FLAG, tid);
    }
    __device__ __forceinline__ void load_t(const uint8_t *rec, int w, int ln) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint8_t *t = rec + Rec<DK>::T + (size_t)t_frag(w, ks) * 2 * Rec<DK>::FRAG + ln * 16;
            th[ks] = *reinterpret_cast<const bf16x8_t *>(t);
            tl[ks] = *reinterpret_cast<const bf16x8_t *>(t + Rec<DK>::FRAG);
        }
    }
    __device__ __forceinline__ void load_kit(const uint8_t *rec, int w, int ln, int lg) {
        const float *col = reinterpret_cast<const float *>(rec + Rec<DK>::COL);
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int mt = (w * STW + i) / NT;
            const uint8_t *kt = rec + Rec<DK>::KIT + (size_t)(2 * mt) * Rec<DK>::FRAG + ln * 16;
            kit[i][0] = *reinterpret_cast<const bf16x8_t *>(kt);
            kit[i][1] = *reinterpret_cast<const bf16x8_t *>(kt + Rec<DK>::FRAG);
            cg[i] = *reinterpret_cast<const f32x4_t *>(col + DK + 16 * mt + 4 * lg);
            cgm[i] = *reinterpret_cast<const f32x4_t *>(col + 2 * DK + 16 * mt + 4 * lg);
        }
    }
};

template <int DK, int BV, typename IO> struct OutRole {
    static constexpr int NKS = DK / 32, NT = BV / 16;
    bf16x8_t ka[NKS], qa[NKS];  // fragments (rb, ks) of KA, QA
    bf16x4_t ph[4], pl[4];      // tiles (rb, I) of P^T, I <= rb (hi, lo)
    IO vv[NT][4];               // values of the rows this lane produces, as loaded
    f32x4_t bt;                 // beta of those rows
    int flag;

    __device__ __forceinline__ void load_kqvb(const uint8_t *rec, const IO *__restrict__ v, int64_t tbase, int nv,
                                              int H, int h, int DV, int col0, int rb, int lr, int lg, int tid) {
        const uint8_t *a = rec + Rec<DK>::KA + (size_t)(rb * NKS) * Rec<DK>::FRAG + (tid & 63) * 16;
        const uint8_t *b = rec + Rec<DK>::QA + (size_t)(rb * NKS) * Rec<DK>::FRAG + (tid & 63) * 16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            ka[ks] = *reinterpret_cast<const bf16x8_t *>(a + ks * Rec<DK>::FRAG);
            qa[ks] = *reinterpret_cast<const bf16x8_t *>(b + ks * Rec<DK>::FRAG);
        }
        bt = *reinterpret_cast<const f32x4_t *>(reinterpret_cast<const float *>(rec + Rec<DK>::BETA) + 16 * rb + 4 * lg);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const int rr = r < nv ? r : nv - 1;
                vv[nt][e] = v[((tbase + rr) * H + h) * (int64_t)DV + col0 + nt * 16 + lr];
            }
        flag = load_flag(rec, Rec<DK>::FLAG, tid);
    }
    __device__ __forceinline__ void load_p(const uint8_t *rec, int rb, int ln) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const uint8_t *p = rec + Rec<DK>::PT + (size_t)p_tile(rb, I) * 2 * Rec<DK>::TILE + ln * 8;
            ph[I] = *reinterpret_cast<const bf16x4_t *>(p);
            pl[I] = *reinterpret_cast<const bf16x4_t *>(p + Rec<DK>::TILE);
        }
    }
};

// Chunk geometry of one state workgroup.
struct ChainRange {
    int64_t bos, eos, c0;  // token range, index of the first chunk record
    int64_t n;             // sequence
    int h, col0;
};

template <int DK, int BV, typename IO, typename GT>
__device__ __forceinline__ void state_role_loop(StateSmem<DK, BV> &sm, const ChainRange &cr,
                                                const IO *__restrict__ q, const IO *__restrict__ k,
                                                const IO *__restrict__ v, const GT *__restrict__ log_alpha,
                                                const GT *__restrict__ beta, const float *__restrict__ h0,
                                                const uint8_t *__restrict__ recs, IO *__restrict__ o,
                                                float *__restrict__ h_T, int H, int DV, int w, int tid) {
    constexpr int NT = BV / 16, STW = StateTiles<DK, BV>::STW;
    typedef Rec<DK> RL;
    const int h = cr.h, col0 = cr.col0;
    const int lr0 = tid & 15, lg0 = (tid & 63) >> 4;
    f32x4_t Sacc[STW];
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w * STW + i, mt = st / NT, nt = st % NT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * mt + 4 * lg0 + e;
            Sacc[i][e] = h0 ? h0[((cr.n * H + h) * DK + c) * (int64_t)DV + col0 + nt * 16 + lr0] : 0.f;
        }
    }
    StateRole<DK, BV> R;
    if (cr.bos < cr.eos) {
        const uint8_t *rec = recs + (size_t)(cr.c0 * H + h) * RL::BYTES;
        R.load_cm(rec, w, lg0, tid);
        R.load_t(rec, w, tid & 63);
        R.load_kit(rec, w, tid & 63, lg0);
    }
    // Each operand group has a single load site per chunk, right after its last
    // use; the token path of a flagged chunk runs right after the first barrier
    // and the matrix-core steps are skipped, so both paths share the loads.
    int64_t ci = cr.c0;
    for (int64_t tbase = cr.bos; tbase < cr.eos; tbase += kC, ++ci) {
        int tl_;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tl_) : "v"(tid));
        const int lr = tl_ & 15, lg = (tl_ & 63) >> 4;
        const int nv = (int)((cr.eos - tbase) < kC ? (cr.eos - tbase) : kC);
        // next chunk's record (the current one again on the last chunk, so that
        // every load is issued on every path and the wait counts stay exact)
        const int64_t cn = tbase + kC < cr.eos ? ci + 1 : ci;
        const uint8_t *recn = recs + (size_t)(cn * H + h) * RL::BYTES;
        lds_barrier();  // B0
        const bool slow = __builtin_amdgcn_readfirstlane(R.flag) != 0;
        if (slow) {
            for (int r = 0; r < nv; ++r)
                token_update<DK, BV, IO, GT>(Sacc, sm.red, q, k, v, log_alpha, beta, o, tbase + r, H, h, DV, col0,
                                             w, lg, lr);
        } else {
            // S' = Diag(e^m) S, transposed, to LDS
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w * STW + i, mt = st / NT, nt = st % NT;
                bf16x4_t sv;
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[e] = (bf16_t)(R.cm[i][e] * Sacc[i][e]);
                *reinterpret_cast<bf16x4_t *>(&sm.S[nt * 16 + lr][16 * mt + 4 * lg]) = sv;
            }
        }
        R.load_cm(recn, w, lg, tl_);
        lds_barrier();  // B1: S' visible
        lds_barrier();  // B2: X visible
        if (!slow) {
            // U = T X for row block w (T is lower triangular: blocks right of w are zero)
            const int nks = (w >> 1) + 1;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *xh = &sm.X[0][nt * 16 + lr][8 * lg];
                const bf16_t *xl = &sm.X[1][nt * 16 + lr][8 * lg];
                f32x4_t acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks < nks) {
                        const bf16x8_t bh = lds_ld8(xh + 32 * ks), bl = lds_ld8(xl + 32 * ks);
                        acc = mfma16(R.th[ks], bh, acc);
                        acc = mfma16(R.th[ks], bl, acc);
                        acc = mfma16(R.tl[ks], bh, acc);
                    }
                }
                const int jl = nt * 16 + lr;
                store_split4(&sm.U[0][jl][16 * w + 4 * lg], &sm.U[1][jl][16 * w + 4 * lg], acc);
            }
        }
        R.load_t(recn, w, tl_ & 63);
        lds_barrier();  // B3: U visible
        if (!slow) {
            // S <- Diag(e^{g_n}) S + Diag(e^{g_n - m}) KI^T U
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int nt = (w * STW + i) % NT;
                const bf16_t *uh = &sm.U[0][nt * 16 + lr][8 * lg];
                const bf16_t *ul = &sm.U[1][nt * 16 + lr][8 * lg];
                f32x4_t acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    acc = mfma16(R.kit[i][ks], lds_ld8(uh + 32 * ks), acc);
                    acc = mfma16(R.kit[i][ks], lds_ld8(ul + 32 * ks), acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) Sacc[i][e] = R.cg[i][e] * Sacc[i][e] + R.cgm[i][e] * acc[e];
            }
        }
        R.load_kit(recn, w, tl_ & 63, lg);
    }
    if (h_T) {
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w * STW + i, mt = st / NT, nt = st % NT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * mt + 4 * lg0 + e;
                h_T[((cr.n * H + h) * DK + c) * (int64_t)DV + col0 + nt * 16 + lr0] = Sacc[i][e];
            }
        }
    }
}

template <int DK, int BV, typename IO>
__device__ __forceinline__ void output_role_loop(StateSmem<DK, BV> &sm, const ChainRange &cr,
                                                 const IO *__restrict__ v, const uint8_t *__restrict__ recs,
                                                 IO *__restrict__ o, int H, int DV, int rb, int tid) {
    static_assert(sizeof(IO) == 2, "the two-kernel path stores bf16 outputs");
    constexpr int NKS = DK / 32, NT = BV / 16;
    typedef Rec<DK> RL;
    const int h = cr.h, col0 = cr.col0;
    OutRole<DK, BV, IO> R;
    if (cr.bos < cr.eos) {
        const uint8_t *rec = recs + (size_t)(cr.c0 * H + h) * RL::BYTES;
        const int nv0 = (int)((cr.eos - cr.bos) < kC ? (cr.eos - cr.bos) : kC);
        const int lr0 = tid & 15, lg0 = (tid & 63) >> 4;
        R.load_kqvb(rec, v, cr.bos, nv0, H, h, DV, col0, rb, lr0, lg0, tid);
        R.load_p(rec, rb, tid & 63);
    }
    f32x4_t accZ[NT];
    int64_t ci = cr.c0;
    for (int64_t tbase = cr.bos; tbase < cr.eos; tbase += kC, ++ci) {
        int tl_;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tl_) : "v"(tid));
        const int lr = tl_ & 15, lg = (tl_ & 63) >> 4;
        const int nv = (int)((cr.eos - tbase) < kC ? (cr.eos - tbase) : kC);
        // next chunk (the current one again on the last chunk: loads on every path)
        const bool has_next = tbase + kC < cr.eos;
        const int64_t cn = has_next ? ci + 1 : ci;
        const int64_t tn = has_next ? tbase + kC : tbase;
        const int nvn = (int)((cr.eos - tn) < kC ? (cr.eos - tn) : kC);
        const uint8_t *recn = recs + (size_t)(cn * H + h) * RL::BYTES;
        lds_barrier();  // B0
        const bool slow = __builtin_amdgcn_readfirstlane(R.flag) != 0;
        if (slow) {
            // the state role runs the chunk token by token: two barriers per token
            for (int r = 0; r < nv; ++r) {
                lds_barrier();
                lds_barrier();
            }
        }
        lds_barrier();  // B1: S' visible
        if (!slow) {
            // Y = KA S', Z = QA S', X = diag(beta) (V - Y) for rows 16rb..16rb+15
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *sh = &sm.S[nt * 16 + lr][8 * lg];
                f32x4_t accY = zero4();
                accZ[nt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8_t sb = lds_ld8(sh + 32 * ks);
                    accY = mfma16(R.ka[ks], sb, accY);
                    accZ[nt] = mfma16(sb, R.qa[ks], accZ[nt]);   // Z^T[j][r]
                }
                f32x4_t x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    x[e] = (r < nv) ? R.bt[e] * (to_f32(R.vv[nt][e]) - accY[e]) : 0.f;
                }
                const int jl = nt * 16 + lr;
                store_split4(&sm.X[0][jl][16 * rb + 4 * lg], &sm.X[1][jl][16 * rb + 4 * lg], x);
            }
        }
        R.load_kqvb(recn, v, tn, nvn, H, h, DV, col0, rb, lr, lg, tl_);
        lds_barrier();  // B2: X visible
        lds_barrier();  // B3: U visible
        if (!slow) {
            // O^T = Z^T + U^T P^T: lane holds O[16rb + lr][16nt + 4lg + e]
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *uh = &sm.U[0][nt * 16 + lr][4 * lg];
                const bf16_t *ul = &sm.U[1][nt * 16 + lr][4 * lg];
                f32x4_t acc = accZ[nt];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if (I <= rb) acc = mma4(acc, lds_ld4(uh + 16 * I), lds_ld4(ul + 16 * I), R.ph[I], R.pl[I]);
                }
                const int r = 16 * rb + lr;
                if (r < nv) {
                    bf16x4_t ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = from_f32<bf16_t>(acc[e]);
                    *reinterpret_cast<bf16x4_t *>(&o[((tbase + r) * H + h) * (int64_t)DV + col0 + nt * 16 + 4 * lg]) = ov;
                }
            }
        }
        R.load_p(recn, rb, tl_ & 63);
    }
}

template <int DK, int BV, typename IO, typename GT>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const float *__restrict__ h0,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ chunk_off,
    const uint8_t *__restrict__ recs, IO *__restrict__ o, float *__restrict__ h_T, int64_t seq_len,
    int32_t H, int32_t DV, int64_t num_chains) {
    __shared__ StateSmem<DK, BV> sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t wg = blockIdx.x;
    const int64_t chain = wg % num_chains;
    ChainRange cr;
    cr.n = chain / H;
    cr.h = (int)(chain % H);
    cr.col0 = (int)(wg / num_chains) * BV;
    if (cu_seqlens) {
        cr.bos = cu_seqlens[cr.n];
        cr.eos = cu_seqlens[cr.n + 1];
        cr.c0 = chunk_off[cr.n];
    } else {
        cr.bos = cr.n * seq_len;
        cr.eos = cr.bos + seq_len;
        cr.c0 = cr.n * ((seq_len + kC - 1) / kC);
    }
    if (w < 4)
        state_role_loop<DK, BV, IO, GT>(sm, cr, q, k, v, log_alpha, beta, h0, recs, o, h_T, H, DV, w, tid);
    else
        output_role_loop<DK, BV, IO>(sm, cr, v, recs, o, H, DV, w - 4, tid);
}

template <int DK, typename IO, typename GT>
hipError_t launch_two_kernel(const ChunkArgs &a, int bv, hipStream_t st) {
    uint8_t *ws = reinterpret_cast<uint8_t *>(a.workspace);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws + kHeaderBytes);
    uint8_t *recs = ws + kHeaderBytes + plan_bytes(a.num_seqs);
    if (a.varlen)
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.num_seqs, chunk_off);
    const int64_t nprep = max_chunks(a) * a.H;
    if (nprep > 0)
        hipLaunchKernelGGL((chunk_prep_kernel<DK, IO, GT>), dim3((unsigned)nprep), dim3(kThreads), 0, st,
                           (const IO *)a.q, (const IO *)a.k, (const GT *)a.log_alpha, (const GT *)a.beta,
                           a.cu_seqlens, (const int32_t *)chunk_off, recs, a.num_seqs, a.seq_len, a.H);
    const int64_t chains = a.num_seqs * (int64_t)a.H;
    if (bv == 32)
        hipLaunchKernelGGL((chunk_state_kernel<DK, 32, IO, GT>), dim3((unsigned)(chains * (a.d_v / 32))),
                           dim3(kThreads), 0, st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v,
                           (const GT *)a.log_alpha, (const GT *)a.beta, a.h0, a.cu_seqlens,
                           (const int32_t *)chunk_off, recs, (IO *)a.o, a.h_T, a.seq_len, a.H, a.d_v, chains);
    else
        hipLaunchKernelGGL((chunk_state_kernel<DK, 16, IO, GT>), dim3((unsigned)(chains * (a.d_v / 16))),
                           dim3(kThreads), 0, st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v,
                           (const GT *)a.log_alpha, (const GT *)a.beta, a.h0, a.cu_seqlens,
                           (const int32_t *)chunk_off, recs, (IO *)a.o, a.h_T, a.seq_len, a.H, a.d_v, chains);
    return hipGetLastError();
}

}  // namespace

size_t two_kernel_workspace_bytes(const ChunkArgs &a) {
    if (a.total_tokens <= 0) return 0;
    const size_t rec = a.d_k == 128 ? Rec<128>::BYTES : Rec<64>::BYTES;
    return kHeaderBytes + plan_bytes(a.num_seqs) + (size_t)max_chunks(a) * a.H * rec;
}

hipError_t launch_chunk_fwd_two_kernel(const ChunkArgs &a, int bv, hipStream_t st) {
    if (a.d_k == 128)
        return a.gate_bf16 ? launch_two_kernel<128, bf16_t, bf16_t>(a, bv, st)
                           : launch_two_kernel<128, bf16_t, float>(a, bv, st);
    return a.gate_bf16 ? launch_two_kernel<64, bf16_t, bf16_t>(a, bv, st)
                       : launch_two_kernel<64, bf16_t, float>(a, bv, st);
}

}  // namespace kda
