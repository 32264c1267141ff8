// kda_chunk2.hip -- chunkwise KDA forward for bf16 I/O in two kernels.
//
// The chunkwise form (KimiLinear article, section 3.1) splits each chunk's work
// into a part that does not depend on the state and a part that carries the
// state from chunk to chunk; only the second part is sequential.  With the
// in-chunk log-decay cumsum G (per token and key channel), its chunk total g_n
// and the per-channel anchor m = g_n / 2, the decayed operands
//     KA = K.e^{G-m},  QA = Q.e^{G-m},  KI = K.e^{m-G}
// give the intra-chunk blocks A = strictly-lower(diag(beta) KA KI^T),
// P = lower(QA KI^T) and the UT transform T = (I + A)^{-1} (WY form of the
// delta rule, section 3.1 and the DPLR discussion of the same article).  The
// state-independent factors of the chunk update are folded here into
//     Tb = T diag(beta),   W = Tb KA,   U0 = Tb V,
// so that, with S' = Diag(e^m) S, one chunk of the recurrence is
//     U = U0 - W S'                       (rows written into the state)
//     O = QA S' + P U
//     S <- Diag(e^{g_n}) S + Diag(e^{g_n - m}) KI^T U.
// This is the same U = T diag(beta) (V - K.e^G S) as the WY/UT form; only the
// rounding points differ.
//
//   chunk_prep_kernel   one workgroup per (chunk, head), all chunks in parallel:
//                       computes the state-independent operands once and writes
//                       a compact record per chunk-head to the workspace;
//   chunk_state_kernel  one workgroup per (sequence, head, block of BV value
//                       columns): walks the chunks of its sequence, keeping the
//                       fp32 state block in registers, and streams the records.
// A key channel whose in-chunk decay exceeds the anchored range (80 nats) leaves
// the Gram products; the prep kernel adds its pairs exactly (e^{G_r - G_i} <= 1)
// and gives its state-side operands no anchor (K.e^G, Q.e^G, K.e^{g_n - G}), so
// every chunk takes the same path through the state kernel.
//
// Compile-time input variants of both kernels: PRO (raw projections mapped as
// they are read), GM (gate per key channel, per token and head, or none) and
// DEC (separate erase and write strengths); the chunk algebra is shared.  A
// single long sequence runs as segments whose records stay in the last-level
// cache between the two kernels (segment_chunks below).
//
// Record layout: matrix operands are stored in the order the state kernel's
// lanes hold them, so that each wave-wide load reads one contiguous 1 KiB (or
// 512 B) run.  A "fragment" is one 16x32 bf16 operand of the 16x16x32 matrix
// instruction, lane l holding row l%16, columns 8*(l/16)..+7 (16 bytes at l*16).
//   WN    fragments (row block rb, k-step ks) of -W, rb*NKS + ks, NKS = DK/32
//   QA    fragments (rb, ks) of QA
//   KIt   fragments (key block mt, token k-step ks) of KI^T, mt*2 + ks
//   PT    the ten lower tiles (R, I <= R) of P in the 16x16x16 operand layout
//         (lane l: P[16R + l%16][16I + 4*(l/16)..+3], 8 bytes), hi then lo
//   U0    accumulator tiles (rb, value block nt) of U0, fp32: lane l holds
//         U0[16rb + 4*(l/16) + e][16nt + l%16], e = 0..3 (16 bytes)
//   e^m, e^{g_n}, e^{g_n-m} fp32[3][DK]; flags int32[4]
// padded to a multiple of 256 bytes.
#include "kda_chunk_common.h"
#include "kda_launch.h"
#include "kda_plan.h"

#include <stdio.h>
#include <stdlib.h>

namespace kda {
namespace {

static_assert(kPlanChunk == kC, "the varlen plan and the kernels use one chunk length");

template <int DK, int DV> struct Rec {
    static constexpr int NKS = DK / 32;
    static constexpr size_t FRAG = 1024;                          // 64 lanes x 16 bytes
    static constexpr size_t TILE = 512;                           // 64 lanes x 8 bytes
    static constexpr size_t WN = 0;
    static constexpr size_t QA = WN + 4 * NKS * FRAG;
    static constexpr size_t KIT = QA + 4 * NKS * FRAG;
    static constexpr size_t PT = KIT + (DK / 16) * 2 * FRAG;
    static constexpr size_t U0 = PT + 10 * 2 * TILE;
    static constexpr size_t COL = U0 + 4 * (DV / 16) * FRAG;
    static constexpr size_t FLAG = COL + 3 * (size_t)DK * 4;
    static constexpr size_t BYTES = ((FLAG + 16) + 255) / 256 * 256;
};

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Slot of the lower tile (R, I), I <= R; I > R maps to I = R (a harmless
// duplicate load: those tiles are never used).
__device__ __forceinline__ int p_tile(int R, int I) { return (R * (R + 1)) / 2 + (I <= R ? I : R); }

constexpr size_t kHeaderBytes = 256;

int64_t max_chunks(const ChunkArgs &a) {
    if (a.varlen) return (a.total_tokens + kC - 1) / kC + a.num_seqs;
    return a.num_seqs * ((a.seq_len + kC - 1) / kC);
}

// A single long sequence (B = 1, no cu_seqlens) runs as consecutive segments of
// whole chunks, each a prep pass then a state pass.  A segment holds at most
// kSegRecords chunk-heads of records (about 190 MB), so the records the prep
// kernel writes are still in the 256 MB last-level cache when the state kernel
// reads them back; the state crosses each boundary in fp32 through the
// workspace, so the result is bitwise that of a single pass.
constexpr int64_t kSegRecords = 2048;

// Chunks per segment, or 0 when the call runs as one pass.
int64_t pipe_chunks(const ChunkArgs &a);
int64_t segment_chunks(const ChunkArgs &a) {
    if (a.varlen || a.num_seqs != 1 || pipe_chunks(a) > 0) return 0;
    const int64_t per = kSegRecords / a.H;
    const int64_t nch = (a.seq_len + kC - 1) / kC;
    return (per >= 1 && nch > per) ? per : 0;
}

// Pipelined segments (chunk_pipe_kernel) for one sequence whose state pass
// has at most half as many workgroups as the chip has compute units (256):
// d_k = 128, per-channel or per-head gates, input as given.  Each segment holds
// half the sequence, at most kPipeRecords chunk-heads, so that the two record
// buffers together stay within the last-level cache; sequences shorter than
// kPipeMinChunks chunks run as one pass.  (Measured at H = 16: two segments
// beat four or eight, each launch boundary costing a few microseconds.)
constexpr int64_t kPipeStateBlocks = 128;
constexpr int64_t kPipeRecords = 1024;
constexpr int64_t kPipeMinChunks = 16;
int64_t state_grid(int64_t chains, int nvb);

// Chunks per pipelined segment, or 0 when the call does not pipeline.
int64_t pipe_chunks(const ChunkArgs &a) {
    if (a.varlen || a.num_seqs != 1 || a.d_k != 128 || a.prologue || a.w_write) return 0;
    if (state_grid(a.H, a.d_v / 16) > kPipeStateBlocks) return 0;
    const int64_t nch = (a.seq_len + kC - 1) / kC;
    if (nch < kPipeMinChunks) return 0;
    int64_t per = (nch + 1) / 2;
    if (per * a.H > kPipeRecords) per = kPipeRecords / a.H;
    return per >= 1 ? per : 0;
}

size_t carry_bytes(const ChunkArgs &a) { return ((size_t)a.H * a.d_k * a.d_v * 4 + 255) / 256 * 256; }

template <int DK, int DV>
struct alignas(16) PrepSmem {
    static constexpr int KS = DK + 8;
    static constexpr int TS = kC + 8;
    static constexpr int FS = 68;
    bf16_t KA[kC][KS];                         // KA; after the UT transform, -W
    union {
        bf16_t QA[kC][KS];                     // Gram phase
        struct {
            bf16_t T[2][kC][TS];               // hi/lo of (I + A)^{-1}, then of T diag(beta)
            float T8[4][2][8][8];
            float W8[4][8][8];
        } t;                                   // inversion phase
    };
    union {
        bf16_t KI[kC][KS];                     // K . e^{m-G}
        bf16_t Tt[2][kC][kC + 4];              // transposed diagonal blocks of T
        bf16_t KAt[DK][TS];                    // KA^T
    };
    union {
        float A[kC][FS];
        bf16_t Vt[DV][TS];                     // V^T
    };
    float tot[DK][kWaves];
    float gs[kC];                              // scalar gates: the in-chunk cumsum per row (log2 units)
    float beta[kC];
    float wr[kC];                              // separate write strengths (DEC)
    float nrm[2][kC];                          // PRO: inverse norms of q and k per row (big channels only)
    int32_t chan[16];                          // exact pairs: the channels of the current group
    int32_t xbig[2];                           // paired prep: any big channel, their count
};

// Numbering of the key channels left out of the Gram products ("big": chunk
// decay beyond the anchored range) in channel order, the same in every wave.
template <int DK> struct BigNumbering {
    int slot[DK / 64];   // number of each of this lane's channels among the big ones
    int nb;              // number of big channels (uniform)
    __device__ __forceinline__ void init(const bool (&bigc)[DK / 64], int l) {
        constexpr int CPL = DK / 64;
        // channel l*CPL + cc comes after the big channels of lanes < l
        const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
        int s0 = 0;
        nb = 0;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const uint64_t msk = __ballot(bigc[cc]);
            s0 += __popcll(msk & below);
            nb += __popcll(msk);
        }
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            slot[cc] = s0;
            s0 += bigc[cc] ? 1 : 0;
        }
    }
};

// Exact pairs of the big channels,
//   A[r,i] += beta_r sum_c k_rc k_ic e^{G_rc - G_ic}  (i < r)
//   P[r,i] +=        sum_c q_rc k_ic e^{G_rc - G_ic}  (i <= r)
// every factor at most 1, taken 16 channels at a time from fp32 [64][16] rows of
// G (log2 units), K and Q (row pitch kXS = 17 floats, so that the lanes of a
// wave, which take consecutive columns i of one row r, read distinct banks),
// so one fast-forgetting channel costs one channel's pairs.  With at most 16 big channels the rows were staged in the area of A
// during operand formation, from the registers that held them; otherwise each
// group is staged here over the area of QA from the inputs (G by one wave-wide
// inclusive scan of the chunk's gates).  The sums are left in the area of QA as
// a 64x64 fp32 matrix of row pitch kSS = 65: the A part (without beta) below
// the diagonal, the P part on and above it (transposed), for the Gram epilogue.  Called by every wave
// after the Gram operands are consumed; returns after a barrier.
// PAIRED: two chunk-heads share the workgroup (and its barriers), so every
// barrier here is taken for nbU channels, the larger count of the two; a half
// with fewer (or none) does empty work between them.
constexpr int kXS = 17;       // row pitch (floats) of the staged G, K, Q rows of the big channels
constexpr int kSS = kC + 1;   // row pitch (floats) of the exact pair sums

template <int DK, bool PRO, int GM, bool PAIRED, typename Sm, typename IO, typename GT>
__device__ __forceinline__ void exact_pairs(Sm &sm, const bool (&bigc)[DK / 64], const BigNumbering<DK> &bn, int nbU,
                                            const IO *__restrict__ q, const IO *__restrict__ k,
                                            const GT *__restrict__ log_alpha, int64_t t0, int nv, int H, int h,
                                            float lo, int w, int l, int tid) {
    constexpr int CPL = DK / 64;
    const int nb = bn.nb;
    const bool staged = nb <= 16;
    const bool bars = PAIRED || !staged;   // the staging barriers are taken
    float *xG = staged ? reinterpret_cast<float *>(&sm.A[0][0]) : reinterpret_cast<float *>(&sm.t);
    float *xK = xG + kC * kXS, *xQ = xK + kC * kXS;
    float *xS = reinterpret_cast<float *>(&sm.t);
    static_assert(kC * kSS * 4 <= sizeof(sm.t) && 3 * kC * kXS * 4 <= sizeof(sm.t),
                  "staging and sums fit in the area of QA");
    static_assert(3 * kC * kXS * 4 <= sizeof(sm.A), "staging fits in the area of A");
    const int64_t rp = (int64_t)H * DK;   // row pitch of q, k and per-channel gates
    constexpr int NPAIR = kC * (kC + 1) / 2, PPT = (NPAIR + kThreads - 1) / kThreads;
    float sA[PPT], sP[PPT];
    int pr[PPT], pc[PPT];   // the pairs (r, i) of this thread, p = tid + kThreads j
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        sA[j] = sP[j] = 0.f;
        const int p = tid + kThreads * j;
        // r = floor((sqrt(8p + 1) - 1) / 2), from the hardware square root and
        // corrected by one either way
        int r = (int)((__builtin_amdgcn_sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
        if ((r + 1) * (r + 2) / 2 <= p) ++r;
        if (r * (r + 1) / 2 > p) --r;
        pr[j] = r;
        pc[j] = p - r * (r + 1) / 2;
    }
    int32_t *chan = sm.chan;   // the channel of number g0 + j
#pragma unroll 1
    for (int g0 = 0; g0 < nbU; g0 += 16) {
        const int cnt = nb - g0 < 0 ? 0 : nb - g0 < 16 ? nb - g0 : 16;
        if (bars) {
            if (!staged) {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const int j = bn.slot[cc] - g0;
                    if (w == 0 && bigc[cc] && j >= 0 && j < 16) chan[j] = l * CPL + cc;
                }
            }
            lds_barrier();
            if (!staged) {
            // G of numbers g0 + 2w and g0 + 2w + 1: lane r holds token r
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * w + jj;
                if (j < cnt) {   // uniform per wave
                    const int c = chan[j];
                    float x = 0.f;
                    if (l < nv) {
                        if constexpr (GM == kGatePerChannel)
                            x = log_decay<PRO, GM>(to_f32(log_alpha[(t0 + l) * rp + (int64_t)h * DK + c]), lo);
                        else if constexpr (GM == kGatePerHead)
                            x = log_decay<PRO, GM>(to_f32(log_alpha[(t0 + l) * H + h]), lo);
                    }
                    x *= kLog2e;
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const float y = __shfl_up(x, d);
                        if (l >= d) x += y;
                    }
                    xG[l * kXS + j] = x;
                }
            }
            // K and Q (with the input prologue: times the rows' inverse norms)
            for (int e = tid; e < kC * 16; e += kThreads) {
                const int r = e >> 4, j = e & 15, x = r * kXS + j;
                float kv = 0.f, qv = 0.f;
                if (r < nv && j < cnt) {
                    const int64_t o = (t0 + r) * rp + (int64_t)h * DK + chan[j];
                    kv = to_f32(k[o]);
                    qv = to_f32(q[o]);
                    if constexpr (PRO) {
                        qv *= sm.nrm[0][r];
                        kv *= sm.nrm[1][r];
                    }
                }
                xK[x] = kv;
                xQ[x] = qv;
            }
            }
            lds_barrier();
        }
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int p = tid + kThreads * j;
            const int r = pr[j], i = pc[j];
            if (p < NPAIR && r < nv) {
                float a = 0.f, b = 0.f;
                for (int c = 0; c < cnt; ++c) {
                    const float kk = xK[i * kXS + c] * kexp2<false>(xG[r * kXS + c] - xG[i * kXS + c]);
                    a += xK[r * kXS + c] * kk;
                    b += xQ[r * kXS + c] * kk;
                }
                sA[j] += a;
                sP[j] += b;
            }
        }
        if (bars) lds_barrier();   // staging read before it is overwritten
    }
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int p = tid + kThreads * j;
        if (p < NPAIR) {
            const int r = pr[j], i = pc[j];
            if (i < r) {
                xS[r * kSS + i] = sA[j];
                xS[i * kSS + r] = sP[j];
            } else {
                xS[r * kSS + r] = sP[j];
            }
        }
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------------
// Prep: one workgroup (8 waves) per (chunk, head).
// PRO: q, k, log_alpha and beta are raw projections, mapped as they are read
// (input prologue; lo is the floor of log alpha).  GM: gate layout; with one
// decay per (token, head) (or none) the decay of a pair is a scalar, so A and P
// are plain products of the raw keys and queries with the mask e^{G_r - G_i}
// applied to the fp32 results, and the state-side operands take no anchor.
// DEC: beta erases and wr writes (decoupled strengths): A and W take beta, U0
// takes wr.
// The body of one prep workgroup (threads tid = 0..kThreads-1) for chunk-head
// bid.  PAIRED: two chunk-heads share a workgroup of 2 kThreads threads, each
// half with its own LDS; every barrier is the whole workgroup's, so both halves
// take the same barriers: the choice of Gram path and the number of exact-pair
// groups follow the larger need of the two (partner: the other half's LDS, or
// null when the other half has no chunk-head).
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC, bool PAIRED = false>
__device__ __forceinline__ void prep_body(
    PrepSmem<DK, DV> &sm, const PrepSmem<DK, DV> *partner, const int tid, const unsigned bid,
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const GT *__restrict__ wr,
    const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, uint8_t *__restrict__ recs, int64_t N, int64_t T, int32_t H,
    float lo) {
    constexpr int CPL = DK / 64;
    constexpr int CPV = DV / 64;
    constexpr int NKS = DK / 32;
    constexpr bool SG = GM != kGatePerChannel;   // one decay per (token, head), or none
    typedef PrepSmem<DK, DV> Sm;
    typedef Rec<DK, DV> RL;

    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    const int64_t chunk = bid / H;
    const int h = (int)(bid % H);
    int64_t n, t0;
    int nv;
    if (!locate_chunk(chunk, cu, chunk_off, N, T, n, t0, nv)) return;
    uint8_t *rec = recs + (size_t)bid * RL::BYTES;
    float *gCol = reinterpret_cast<float *>(rec + RL::COL);
    int32_t *gFlag = reinterpret_cast<int32_t *>(rec + RL::FLAG);

    // ---- load this chunk (rows past the end read the last row; their gates,
    // keys and beta are zeroed below, so they contribute nothing)
    ChunkRegs<DK, 16, IO, GT, PRO, GM, DEC> in;
    in.load(q, k, q, log_alpha, beta, wr, t0, nv, H, h, 0, 0, w, l, lg, lr, false);
    in.prepare(w, lo);
    typedef typename VecT<IO, CPV>::type VV;
    VV vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 8 * w + i;
        const int rr = r < nv ? r : nv - 1;
        vr[i] = *reinterpret_cast<const VV *>(v + ((t0 + rr) * H + h) * (int64_t)DV + l * CPV);
    }
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
    if (w == 0) sm.beta[l] = (l < nv) ? in.bt : 0.f;
    if (DEC && w == 0) sm.wr[l] = (l < nv) ? in.wt : 0.f;
    lds_barrier();
    // Anchors: m = g_n / 2 for both factors of the Gram products.  A channel
    // whose chunk decay exceeds kMaxRange2 ("big") leaves the Gram products (its
    // KI columns are zero there) and its pairs are added exactly below; its
    // state-side operands take no anchor: K e^G and Q e^G (mA = 0) and
    // K e^{g_n - G} (mI = g_n), every factor at most 1.
    float mA2[CPL], mI2[CPL];
    bool bigc[CPL];
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
#pragma unroll
        for (int i = 0; i < 8; ++i) csum[i][cc] += pre;
        if constexpr (SG) {
            // one decay per row: the Gram products run on the raw keys and
            // queries with the pairwise decay applied to the fp32 products, so
            // no channel leaves them; the state side takes no anchor
            bigc[cc] = false;
            mA2[cc] = 0.f;
            mI2[cc] = all;
        } else {
            bigc[cc] = !(-all <= kMaxRange2);    // also true for NaN
            mA2[cc] = bigc[cc] ? 0.f : 0.5f * all;
            mI2[cc] = bigc[cc] ? all : 0.5f * all;
        }
        if (w == 0) {
            gCol[c] = kexp2<false>(mA2[cc]);
            gCol[DK + c] = kexp2<false>(all);
            gCol[2 * DK + c] = kexp2<false>(all - mI2[cc]);
        }
    }
    if constexpr (SG) {
        if (l == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) sm.gs[8 * w + i] = csum[i][0];
        }
    }
    bool lbig = false;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) lbig = lbig || bigc[cc];
    const bool anybig = __ballot(lbig) != 0;   // same channels in every wave: uniform
    BigNumbering<DK> bn;
    bn.nb = 0;
    if (anybig || PAIRED) bn.init(bigc, l);
    if (anybig) {
        if (bn.nb <= 16) {   // stage the big channels' G, K, Q rows for the exact pairs
            float *xG = reinterpret_cast<float *>(&sm.A[0][0]);
            float *xK = xG + kC * kXS, *xQ = xK + kC * kXS;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                if (bigc[cc]) {
                    const int j = bn.slot[cc];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = 8 * w + i;
                        const bool valid = r < nv;
                        xG[r * kXS + j] = csum[i][cc];
                        xK[r * kXS + j] = valid ? in.kval(i, cc) : 0.f;
                        xQ[r * kXS + j] = valid ? in.qval(i, cc) : 0.f;
                    }
                }
            }
        }
    }
    if (tid == 0) gFlag[0] = 0;
    if (PAIRED && tid == 0) {   // read by the other half after the next barrier
        sm.xbig[0] = anybig ? 1 : 0;
        sm.xbig[1] = bn.nb;
    }
    if constexpr (PRO) {
        if (anybig && l < 8) {   // for the exact pairs of the big channels
            sm.nrm[0][8 * w + l] = in.qs[l];
            sm.nrm[1][8 * w + l] = in.ks[l];
        }
    }
    // ---- decayed operands: LDS for the Gram products, KI^T to the record
    bf16_t kak[8][CPL];                      // this lane's KA values, for KA^T later
    {
        float e1[8][CPL], e2[8][CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float al[8];
            al[0] = 1.f;
#pragma unroll
            for (int i = 1; i < 8; ++i) {
                float x = in.gate(i, cc) * kLog2e;
                if (partial && 8 * w + i >= nv) x = 0.f;
                al[i] = kexp2<false>(x);
            }
            e1[0][cc] = kexp2<false>(csum[0][cc] - mA2[cc]);
#pragma unroll
            for (int i = 1; i < 8; ++i) e1[i][cc] = e1[i - 1][cc] * al[i];
            e2[7][cc] = kexp2<false>(mI2[cc] - csum[7][cc]);
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
                const float kv = in.kval(i, cc), qv = in.qval(i, cc);
                kit[cc][i] = (bf16_t)(kv * e2[i][cc]);
                if constexpr (SG) {   // Gram operands K and Q; Q e^G staged in KI's area for the record
                    const bool valid = 8 * w + i < nv;
                    ka[cc] = valid ? (bf16_t)kv : (bf16_t)0.f;
                    qa[cc] = valid ? (bf16_t)qv : (bf16_t)0.f;
                    ki[cc] = (bf16_t)(qv * e1[i][cc]);
                    kak[i][cc] = (bf16_t)(kv * e1[i][cc]);
                } else {
                    ka[cc] = (bf16_t)(kv * e1[i][cc]);
                    qa[cc] = (bf16_t)(qv * e1[i][cc]);
                    ki[cc] = bigc[cc] ? (bf16_t)0.f : kit[cc][i];   // big channels: out of the Gram
                    kak[i][cc] = ka[cc];
                }
            }
            if constexpr (CPL == 2) {
                bf16x2_t p;
                p[0] = ka[0]; p[1] = ka[1];
                *reinterpret_cast<bf16x2_t *>(&sm.KA[r][2 * l]) = p;
                p[0] = qa[0]; p[1] = qa[1];
                *reinterpret_cast<bf16x2_t *>(&sm.QA[r][2 * l]) = p;
                p[0] = ki[0]; p[1] = ki[1];
                *reinterpret_cast<bf16x2_t *>(&sm.KI[r][2 * l]) = p;
            } else {
                sm.KA[r][l] = ka[0];
                sm.QA[r][l] = qa[0];
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

    // ---- QA to the record, fragment by fragment (1 KiB per wave-wide store)
#pragma unroll
    for (int it = 0; it < (4 * NKS * 64) / kThreads; ++it) {
        const int pc = tid + kThreads * it;
        const int f = pc >> 6, ln = pc & 63;
        const int rb = f / NKS, ks = f % NKS;
        const bf16x8_t x = SG ? lds_ld8(&sm.KI[16 * rb + (ln & 15)][32 * ks + 8 * (ln >> 4)])
                              : lds_ld8(&sm.QA[16 * rb + (ln & 15)][32 * ks + 8 * (ln >> 4)]);
        *reinterpret_cast<bf16x8_t *>(rec + RL::QA + f * RL::FRAG + ln * 16) = x;
    }

    // ---- Gram blocks: A (fp32, LDS) and P (hi/lo, record)
    {
        // A tiles as A[r][i] (rows of KA, columns of KI); P tiles transposed,
        // P^T[i][r] (rows of KI, columns of QA), so that the accumulator is the
        // 16x16x16 operand layout the record stores
        auto gram = [&](int tile, f32x4_t &acc) {
            const bool isP = tile >= 10;
            int R, I;
            lower_block(isP ? tile - 10 : tile, R, I);
            const bf16_t *xh = isP ? &sm.QA[16 * R + lr][8 * lg] : &sm.KA[16 * R + lr][8 * lg];
            const bf16_t *kh = SG ? &sm.KA[16 * I + lr][8 * lg] : &sm.KI[16 * I + lr][8 * lg];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8_t xa = lds_ld8(xh + 32 * ks), kb = lds_ld8(kh + 32 * ks);
                acc = isP ? mfma16(kb, xa, acc) : mfma16(xa, kb, acc);
            }
        };
        // With big channels (anybig), xS below holds their exact pair sums: the A
        // part below the diagonal, the P part on and above it (transposed).
        const float *xS = reinterpret_cast<const float *>(&sm.t);
        auto finish = [&](bool isP, int R, int I, const f32x4_t &acc) {
            if (!isP) {
                const int i = 16 * I + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * R + 4 * lg + e;
                    float x = anybig ? acc[e] + xS[r * kSS + i] : acc[e];
                    if constexpr (SG) x *= kexp2<false>(sm.gs[r] - sm.gs[i]);   // at most 1 for i < r
                    sm.A[r][i] = (i < r) ? sm.beta[r] * x : 0.f;
                }
            } else {
                // lane holds P^T[16I + 4lg + e][16R + lr] = P[r][i], kept for i <= r
                const int r = 16 * R + lr;
                f32x4_t x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * I + 4 * lg + e;
                    float y = anybig ? acc[e] + xS[i * kSS + r] : acc[e];
                    if constexpr (SG) y *= kexp2<false>(sm.gs[r] - sm.gs[i]);   // at most 1 for i <= r
                    x[e] = (i <= r) ? y : 0.f;
                }
                uint8_t *dst = rec + RL::PT + (size_t)p_tile(R, I) * 2 * RL::TILE + l * 8;
                store_split4(reinterpret_cast<bf16_t *>(dst), reinterpret_cast<bf16_t *>(dst + RL::TILE), x);
            }
        };
        // tiles w, w + 8 and (waves 0-3) w + 16: 0-9 are the lower 16x16 blocks of
        // A, 10-19 those of P (accumulated transposed)
        constexpr int NTL = 3;
        bool anyU = anybig;
        int nbU = bn.nb;
        if (PAIRED && partner != nullptr) {   // the same in every lane and wave of both halves
            const int pbig = __builtin_amdgcn_readfirstlane(partner->xbig[0]);
            const int pnb = __builtin_amdgcn_readfirstlane(partner->xbig[1]);
            anyU = anyU || pbig != 0;
            nbU = nbU > pnb ? nbU : pnb;
        }
        if (!anyU) {
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                if (t == 2 && w >= 4) break;
                const int tile = w + 8 * t;
                const bool isP = tile >= 10;
                int R, I;
                lower_block(isP ? tile - 10 : tile, R, I);
                f32x4_t acc = zero4();
                gram(tile, acc);
                finish(isP, R, I, acc);
            }
        } else {
            f32x4_t accs[NTL];
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                accs[t] = zero4();
                if (t < 2 || w < 4) gram(w + 8 * t, accs[t]);
            }
            lds_barrier();   // the Gram operands are consumed
            exact_pairs<DK, PRO, GM, PAIRED>(sm, bigc, bn, nbU, q, k, log_alpha, t0, nv, H, h, lo, w, l, tid);
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                if (t < 2 || w < 4) {
                    const int tile = w + 8 * t;
                    const bool isP = tile >= 10;
                    int R, I;
                    lower_block(isP ? tile - 10 : tile, R, I);
                    finish(isP, R, I, accs[t]);
                }
            }
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

    // ---- Tb = T diag(beta) in place (hi/lo); KA^T and V^T to LDS.  With DEC, T
    // stays unscaled here: W and U0 scale their rows of T by beta or wr below.
    {
        const int r = tid >> 3, i0 = 8 * (tid & 7);
        const bf16x8_t hv = lds_ld8(&sm.t.T[0][r][i0]), lv = lds_ld8(&sm.t.T[1][r][i0]);
        bf16x8_t h2, l2;
        // blocks above the diagonal were never written (stale LDS): zero
        const bool upper = (i0 >> 4) > (r >> 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = upper ? 0.f : ((float)hv[e] + (float)lv[e]) * (DEC ? 1.f : sm.beta[i0 + e]);
            bf16_t hh, ll;
            split_bf16(x, hh, ll);
            h2[e] = hh;
            l2[e] = ll;
        }
        *reinterpret_cast<bf16x8_t *>(&sm.t.T[0][r][i0]) = h2;
        *reinterpret_cast<bf16x8_t *>(&sm.t.T[1][r][i0]) = l2;
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        bf16x8_t x;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = kak[i][cc];
        *reinterpret_cast<bf16x8_t *>(&sm.KAt[l * CPL + cc][8 * w]) = x;
    }
#pragma unroll
    for (int cv = 0; cv < CPV; ++cv) {
        bf16x8_t x;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (bf16_t)vget(vr[i], cv);
        *reinterpret_cast<bf16x8_t *>(&sm.Vt[l * CPV + cv][8 * w]) = x;
    }
    lds_barrier();

    // ---- W = Tb KA (stored negated, bf16, to LDS) and U0 = Tb V (fp32, record):
    // waves 0-3 the W tiles, waves 4-7 the U0 tiles, of row block w % 4
    {
        const int rb = w & 3;
        const bool isW = w < 4;
        bf16x8_t th[2], tlo[2];   // this row block of Tb, hi and lo, read once
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks <= (rb >> 1)) {   // Tb is lower triangular
                th[ks] = lds_ld8(&sm.t.T[0][16 * rb + lr][32 * ks + 8 * lg]);
                tlo[ks] = lds_ld8(&sm.t.T[1][16 * rb + lr][32 * ks + 8 * lg]);
                if constexpr (DEC) {   // T diag(beta) for W, T diag(wr) for U0
                    const float *sc = isW ? sm.beta : sm.wr;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = ((float)th[ks][e] + (float)tlo[ks][e]) * sc[32 * ks + 8 * lg + e];
                        bf16_t hh, ll;
                        split_bf16(x, hh, ll);
                        th[ks][e] = hh;
                        tlo[ks][e] = ll;
                    }
                }
            }
        }
        // one 16-column tile of Tb times the operand rows at src
        auto tb_tile = [&](const bf16_t *bsrc) {
            f32x4_t acc = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks <= (rb >> 1)) {
                    const bf16x8_t b = lds_ld8(bsrc + 32 * ks);
                    acc = mfma16(th[ks], b, acc);
                    acc = mfma16(tlo[ks], b, acc);
                }
            }
            return acc;
        };
        if (isW) {
#pragma unroll
            for (int ct = 0; ct < DK / 16; ++ct) {
                const f32x4_t acc = tb_tile(&sm.KAt[16 * ct + lr][8 * lg]);
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.KA[16 * rb + 4 * lg + e][16 * ct + lr] = (bf16_t)(-acc[e]);
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct) {
                const f32x4_t acc = tb_tile(&sm.Vt[16 * ct + lr][8 * lg]);
                *reinterpret_cast<f32x4_t *>(rec + RL::U0 + (size_t)(rb * (DV / 16) + ct) * RL::FRAG + l * 16) = acc;
            }
        }
    }
    lds_barrier();

    // ---- -W to the record, fragment by fragment
#pragma unroll
    for (int it = 0; it < (4 * NKS * 64) / kThreads; ++it) {
        const int pc = tid + kThreads * it;
        const int f = pc >> 6, ln = pc & 63;
        const int rb = f / NKS, ks = f % NKS;
        const bf16x8_t x = lds_ld8(&sm.KA[16 * rb + (ln & 15)][32 * ks + 8 * (ln >> 4)]);
        *reinterpret_cast<bf16x8_t *>(rec + RL::WN + f * RL::FRAG + ln * 16) = x;
    }
}

template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__global__ __launch_bounds__(kThreads, 4) void chunk_prep_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const GT *__restrict__ wr,
    const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, uint8_t *__restrict__ recs, int64_t N, int64_t T, int32_t H,
    float lo) {
    __shared__ PrepSmem<DK, DV> sm;
    prep_body<DK, DV, IO, GT, PRO, GM, DEC>(sm, nullptr, threadIdx.x, blockIdx.x, q, k, v, log_alpha, beta, wr, cu,
                                            chunk_off, recs, N, T, H, lo);
}

// ---------------------------------------------------------------------------------
// State: one workgroup of 16 waves per (sequence, head, BV value columns).  The
// waves split into three roles with the same barrier sequence per chunk:
//   state role  (waves 0-3):  own the fp32 state tiles; write e^m.S to LDS and
//                             update the state with KI^T U;
//   output role (waves 4-7):  row block w-4 of the chunk: U = U0 - W S' (to LDS),
//                             Z = QA S' and O = Z + P U;
//   loader role (waves 8-15): stream this workgroup's part of each chunk record
//                             from global memory into a two-slot LDS ring, two
//                             records ahead.
// Two barriers per chunk: B1 (S' written) and B2 (U written); everything else
// is ordered by them.  The state waves write S'(j+1) after B2(j), when the reads
// of S'(j) are complete; U(j+1) is written after B1(j+1), after every read of
// U(j).  So the output waves' O(j) overlaps the state waves' update of chunk j
// and their S'(j+1).
// The loaders absorb the stalls of the global-load pipe, spreading the fetch of
// each record over the phases of a chunk so that the pipe stays busy.  Record j
// goes to ring slot j%2 right after B2 of chunk j-2 (i.e. at the start of chunk
// j-1; the slot held record j-2, whose last reads were before B1 of chunk j-2)
// and is complete at B2 of chunk j-1, after which the other roles read it into
// registers, ahead of compute that hides the LDS latency.
constexpr int kStateWaves = 16;
constexpr int kStateThreads = 64 * kStateWaves;
constexpr int kLoaderLanes = 512;

// This workgroup's part of a record, in LDS: -W and QA as in the record, the U0
// tiles of its value columns, the column scales and flags, then KI^T and P.
template <int DK, int DV, int BV> struct Slot {
    typedef Rec<DK, DV> RL;
    static constexpr int NT = BV / 16;
    static constexpr int P_WQ = (int)(RL::KIT / 16);                   // -W, QA: as in the record
    static constexpr int P_U = P_WQ + 4 * NT * 64;                       // + U0 tiles of this block
    static constexpr int P_C = P_U + (int)((3 * DK * 4 + 16) / 16);      // + scales, flags
    static constexpr int NP = P_C + (int)((RL::U0 - RL::KIT) / 16);      // + KI^T, P
    static constexpr size_t U0 = (size_t)P_WQ * 16;
    static constexpr size_t COL = (size_t)P_U * 16;
    static constexpr size_t FLAG = COL + 3 * (size_t)DK * 4;
    static constexpr size_t KIT = (size_t)P_C * 16;
    static constexpr size_t PT = KIT + (RL::PT - RL::KIT);
    static constexpr size_t BYTES = (size_t)NP * 16;
    static constexpr int ITERS = (NP + kLoaderLanes - 1) / kLoaderLanes;
    // loader schedule per chunk, in units of ITERS: the ring write and the fetch
    // of the record two chunks ahead are split at B1
    static constexpr int F1 = (ITERS + 1) / 2;
    // 16-byte piece p: its offset in the global record and in the slot
    __device__ __forceinline__ static void piece(int p, int nt0, size_t &g, size_t &s) {
        if (p < P_WQ) {
            g = s = (size_t)p * 16;
        } else if (p < P_U) {
            const int q = p - P_WQ, rb = q / (NT * 64), rem = q % (NT * 64);
            g = RL::U0 + (size_t)(rb * (DV / 16) + nt0) * RL::FRAG + (size_t)rem * 16;
            s = U0 + (size_t)q * 16;
        } else if (p < P_C) {
            const int q = p - P_U;
            g = RL::COL + (size_t)q * 16;
            s = COL + (size_t)q * 16;
        } else {
            const int q = p - P_C;
            g = RL::KIT + (size_t)q * 16;
            s = KIT + (size_t)q * 16;
        }
    }
};

template <int DK, int DV, int BV>
struct alignas(16) StateSmem {
    static constexpr int KS = DK + 8;
    static constexpr int TS = kC + 8;
    uint8_t ring[2][Slot<DK, DV, BV>::BYTES];
    bf16_t S[BV][KS];          // (Diag(e^m) S)^T, single bf16
    bf16_t U[2][BV][TS];       // hi/lo of U^T
};

// Barrier for a wave whose outstanding LDS operations (ring writes) need not be
// complete yet; a later lds_barrier() orders them.
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int DK, int DV, int BV> struct StateRole {
    typedef Slot<DK, DV, BV> SL;
    static constexpr int NT = BV / 16, STW = StateTiles<DK, BV>::STW;
    bf16x8_t kit[STW][2];     // KI^T fragments of the wave's state tiles
    f32x4_t cm[STW], cg[STW], cgm[STW];

    __device__ __forceinline__ void load_cm(const uint8_t *slot, int w, int lg) {
        const float *col = reinterpret_cast<const float *>(slot + SL::COL);
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int mt = (w * STW + i) / NT;
            cm[i] = *reinterpret_cast<const f32x4_t *>(col + 16 * mt + 4 * lg);
        }
    }
    __device__ __forceinline__ void load_kit(const uint8_t *slot, int w, int ln, int lg) {
        const float *col = reinterpret_cast<const float *>(slot + SL::COL);
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int mt = (w * STW + i) / NT;
            const uint8_t *kt = slot + SL::KIT + (size_t)(2 * mt) * SL::RL::FRAG + ln * 16;
            kit[i][0] = *reinterpret_cast<const bf16x8_t *>(kt);
            kit[i][1] = *reinterpret_cast<const bf16x8_t *>(kt + SL::RL::FRAG);
            cg[i] = *reinterpret_cast<const f32x4_t *>(col + DK + 16 * mt + 4 * lg);
            cgm[i] = *reinterpret_cast<const f32x4_t *>(col + 2 * DK + 16 * mt + 4 * lg);
        }
    }
};

template <int DK, int DV, int BV> struct OutRole {
    typedef Slot<DK, DV, BV> SL;
    typedef Rec<DK, DV> RL;
    static constexpr int NKS = DK / 32, NT = BV / 16;
    bf16x8_t wn[NKS], qa[NKS];  // fragments (rb, ks) of -W and QA
    bf16x4_t ph[4], pl[4];      // tiles (rb, I) of P^T, I <= rb (hi, lo)
    f32x4_t u0[NT];             // accumulator tiles (rb, nt) of U0

    __device__ __forceinline__ void load_wq(const uint8_t *slot, int rb, int ln) {
        const uint8_t *a = slot + RL::WN + (size_t)(rb * NKS) * RL::FRAG + ln * 16;
        const uint8_t *b = slot + RL::QA + (size_t)(rb * NKS) * RL::FRAG + ln * 16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            wn[ks] = *reinterpret_cast<const bf16x8_t *>(a + ks * RL::FRAG);
            qa[ks] = *reinterpret_cast<const bf16x8_t *>(b + ks * RL::FRAG);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            u0[nt] = *reinterpret_cast<const f32x4_t *>(slot + SL::U0 + (size_t)(rb * NT + nt) * RL::FRAG + ln * 16);
    }
    __device__ __forceinline__ void load_p(const uint8_t *slot, int rb, int ln) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const uint8_t *p = slot + SL::PT + (size_t)p_tile(rb, I) * 2 * RL::TILE + ln * 8;
            ph[I] = *reinterpret_cast<const bf16x4_t *>(p);
            pl[I] = *reinterpret_cast<const bf16x4_t *>(p + RL::TILE);
        }
    }
};

// Chunk geometry of one state workgroup.
struct ChainRange {
    int64_t bos, eos, c0;  // token range, index of the first chunk record
    int64_t n;             // sequence
    int h, col0;
};

__device__ __forceinline__ int chunk_count(const ChainRange &cr) { return (int)((cr.eos - cr.bos + kC - 1) / kC); }

template <int DK, int DV, int BV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__device__ __forceinline__ void state_role_loop(StateSmem<DK, DV, BV> &sm, const ChainRange &cr,
                                                const IO *__restrict__ q, const IO *__restrict__ k,
                                                const IO *__restrict__ v, const GT *__restrict__ log_alpha,
                                                const GT *__restrict__ beta, const GT *__restrict__ wr,
                                                const float *__restrict__ h0,
                                                IO *__restrict__ o, float *__restrict__ h_T, int H, int w, int tid,
                                                float lo) {
    constexpr int NT = BV / 16, STW = StateTiles<DK, BV>::STW;
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
    const int nch = chunk_count(cr);
    lds_barrier();  // ring slot 0 holds record 0
    StateRole<DK, DV, BV> R;
    if (nch > 0) {
        R.load_cm(sm.ring[0], w, lg0);
        R.load_kit(sm.ring[0], w, tid & 63, lg0);
    }
    for (int j = 0; j < nch; ++j) {
        int tl_;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tl_) : "v"(tid));
        const int lr = tl_ & 15, lg = (tl_ & 63) >> 4;
        // S' = Diag(e^m) S, transposed, to LDS
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w * STW + i, mt = st / NT, nt = st % NT;
            bf16x4_t sv;
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e] = (bf16_t)(R.cm[i][e] * Sacc[i][e]);
            *reinterpret_cast<bf16x4_t *>(&sm.S[nt * 16 + lr][16 * mt + 4 * lg]) = sv;
        }
        lds_barrier();  // B1: S' visible
        lds_barrier();  // B2: U visible; slot (j+1)%2 holds record j+1
        R.load_cm(sm.ring[(j + 1) & 1], w, lg);   // e^m of chunk j+1, read during the update
        {
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
        R.load_kit(sm.ring[(j + 1) & 1], w, tl_ & 63, lg);
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

template <int DK, int DV, int BV, typename IO>
__device__ __forceinline__ void output_role_loop(StateSmem<DK, DV, BV> &sm, const ChainRange &cr,
                                                 IO *__restrict__ o, int H, int rb, int tid) {
    static_assert(sizeof(IO) == 2, "the two-kernel path stores bf16 outputs");
    constexpr int NKS = DK / 32, NT = BV / 16;
    const int h = cr.h, col0 = cr.col0;
    const int nch = chunk_count(cr);
    lds_barrier();  // ring slot 0 holds record 0
    OutRole<DK, DV, BV> R;
    if (nch > 0) {
        R.load_wq(sm.ring[0], rb, tid & 63);
        R.load_p(sm.ring[0], rb, tid & 63);
    }
    f32x4_t accZ[NT];
    for (int j = 0; j < nch; ++j) {
        int tl_;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tl_) : "v"(tid));
        const int lr = tl_ & 15, lg = (tl_ & 63) >> 4;
        const int64_t tbase = cr.bos + (int64_t)j * kC;
        const int nv = (int)((cr.eos - tbase) < kC ? (cr.eos - tbase) : kC);
        lds_barrier();  // B1: S' visible
        {
            // U = U0 - W S' (rows 16rb..16rb+15, to LDS) and Z^T = S'^T QA^T
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *sh = &sm.S[nt * 16 + lr][8 * lg];
                f32x4_t accU = R.u0[nt];
                accZ[nt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8_t sb = lds_ld8(sh + 32 * ks);
                    accU = mfma16(R.wn[ks], sb, accU);
                    accZ[nt] = mfma16(sb, R.qa[ks], accZ[nt]);   // Z^T[j][r]
                }
                const int jl = nt * 16 + lr;
                bf16x4_t uh, ul;
                split4(accU, uh, ul);
                *reinterpret_cast<bf16x4_t *>(&sm.U[0][jl][16 * rb + 4 * lg]) = uh;
                *reinterpret_cast<bf16x4_t *>(&sm.U[1][jl][16 * rb + 4 * lg]) = ul;
                // the diagonal block of P U needs only this wave's own U tile, whose
                // accumulator layout is the 16x16x16 A-operand layout of U^T: add it now
#pragma unroll
                for (int I = 0; I < 4; ++I)   // I == rb, with a compile-time register index
                    if (I == rb) accZ[nt] = mma4(accZ[nt], uh, ul, R.ph[I], R.pl[I]);
            }
        }
        lds_barrier();  // B2: U visible; slot (j+1)%2 holds record j+1
        R.load_wq(sm.ring[(j + 1) & 1], rb, tl_ & 63);
        {
            // O^T = Z^T + U^T P^T (blocks left of the diagonal): lane holds O[16rb + lr][16nt + 4lg + e]
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_t *uh = &sm.U[0][nt * 16 + lr][4 * lg];
                const bf16_t *ul = &sm.U[1][nt * 16 + lr][4 * lg];
                // two accumulators (even and odd column blocks) halve the dependent chain
                f32x4_t acc = accZ[nt], acc1 = zero4();
#pragma unroll
                for (int I = 0; I < 3; ++I) {
                    if (I < rb) {   // the diagonal block I = rb is already in Z
                        if (I & 1) acc1 = mma4(acc1, lds_ld4(uh + 16 * I), lds_ld4(ul + 16 * I), R.ph[I], R.pl[I]);
                        else acc = mma4(acc, lds_ld4(uh + 16 * I), lds_ld4(ul + 16 * I), R.ph[I], R.pl[I]);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += acc1[e];
                const int r = 16 * rb + lr;
                if (r < nv) {
                    bf16x4_t ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = from_f32<bf16_t>(acc[e]);
                    *reinterpret_cast<bf16x4_t *>(&o[((tbase + r) * H + h) * (int64_t)DV + col0 + nt * 16 + 4 * lg]) = ov;
                }
            }
        }
        R.load_p(sm.ring[(j + 1) & 1], rb, tl_ & 63);
    }
}

// Loader: register buffers A and B alternate between two records in flight.
// Entering chunk j, the buffer for j+1 holds (or is receiving) record j+1 and
// the other record j+2; during chunk j the first is written to slot (j+1)%2 and
// refilled with record j+3.  Records past the last chunk re-read the last one.
template <int DK, int DV, int BV, int I0, int I1, int N>
__device__ __forceinline__ void loader_fetch(u32x4_t (&buf)[N], const uint8_t *rec, int nt0, int lid) {
    typedef Slot<DK, DV, BV> SL;
    static_assert(N == SL::ITERS, "loader buffer size");
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const int p = lid + kLoaderLanes * i;
        if (i + 1 < SL::ITERS || p < SL::NP) {
            size_t g, s;
            SL::piece(p, nt0, g, s);
            buf[i] = *reinterpret_cast<const u32x4_t *>(rec + g);
        }
    }
}

template <int DK, int DV, int BV, int I0, int I1, int N>
__device__ __forceinline__ void loader_store(const u32x4_t (&buf)[N], uint8_t *slot, int nt0, int lid) {
    typedef Slot<DK, DV, BV> SL;
    static_assert(N == SL::ITERS, "loader buffer size");
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const int p = lid + kLoaderLanes * i;
        if (i + 1 < SL::ITERS || p < SL::NP) {
            size_t g, s;
            SL::piece(p, nt0, g, s);
            *reinterpret_cast<u32x4_t *>(slot + s) = buf[i];
        }
    }
}

// One chunk of the loader: the barrier sequence of the other roles, with the
// ring write of record j+1 and the fetch of record j+3 spread over it.
template <int DK, int DV, int BV, int N>
__device__ __forceinline__ void loader_chunk(StateSmem<DK, DV, BV> &sm, u32x4_t (&buf)[N], const uint8_t *rec3,
                                             int jj, int nt0, int lid) {
    typedef Slot<DK, DV, BV> SL;
    uint8_t *dst = sm.ring[(jj + 1) & 1];
    // record jj+1 to its slot in two halves, at the start of the chunk and after
    // B1 (complete at B2), each followed by the fetch of the same half of record
    // jj+3 into the registers it frees
    loader_store<DK, DV, BV, 0, SL::F1>(buf, dst, nt0, lid);
    loader_fetch<DK, DV, BV, 0, SL::F1>(buf, rec3, nt0, lid);
    plain_barrier();  // B1
    loader_store<DK, DV, BV, SL::F1, SL::ITERS>(buf, dst, nt0, lid);
    loader_fetch<DK, DV, BV, SL::F1, SL::ITERS>(buf, rec3, nt0, lid);
    lds_barrier();    // B2: the ring writes are complete
}

template <int DK, int DV, int BV>
__device__ __forceinline__ void loader_role_loop(StateSmem<DK, DV, BV> &sm, const ChainRange &cr,
                                                 const uint8_t *__restrict__ recs, int H, int lid) {
    typedef Rec<DK, DV> RL;
    typedef Slot<DK, DV, BV> SL;
    const int nch = chunk_count(cr);
    const int nt0 = cr.col0 / 16;
    auto rec_of = [&](int j) -> const uint8_t * {
        const int jj = j < nch ? j : nch - 1;
        return recs + (size_t)((cr.c0 + jj) * H + cr.h) * RL::BYTES;
    };
    u32x4_t a[SL::ITERS], b[SL::ITERS];
    if (nch > 0) {
        loader_fetch<DK, DV, BV, 0, SL::ITERS>(a, rec_of(0), nt0, lid);
        loader_store<DK, DV, BV, 0, SL::ITERS>(a, sm.ring[0], nt0, lid);
        loader_fetch<DK, DV, BV, 0, SL::ITERS>(a, rec_of(1), nt0, lid);
        loader_fetch<DK, DV, BV, 0, SL::ITERS>(b, rec_of(2), nt0, lid);
    }
    lds_barrier();  // ring slot 0 holds record 0
    // two chunks per iteration so that the buffers keep fixed registers
    for (int j = 0; j < nch; j += 2) {
        loader_chunk<DK, DV, BV>(sm, a, rec_of(j + 3), j, nt0, lid);
        if (j + 1 < nch) loader_chunk<DK, DV, BV>(sm, b, rec_of(j + 4), j + 1, nt0, lid);
    }
}

// Block id -> (chain = sequence * H + head, value-column block).  Workgroups go
// to the 8 XCDs round-robin by block id; the nvb column blocks of one chain get
// ids that are equal modulo 8 and within 8 * nvb of each other, so they run on
// one XCD at about the same time and read each chunk record from that XCD's L2
// once, however many chains there are.  Ids past the last chain return.
constexpr int kXcds = 8;
__device__ __forceinline__ bool state_block(int64_t id, int64_t chains, int nvb, int64_t &chain, int &vb) {
    const int64_t q = id / kXcds;
    vb = (int)(q % nvb);
    chain = id % kXcds + kXcds * (q / nvb);
    return chain < chains;
}
int64_t state_grid(int64_t chains, int nvb) { return (chains + kXcds - 1) / kXcds * kXcds * nvb; }

// The body of one state workgroup (all kStateThreads threads) for block id bid.
template <int DK, int DV, int BV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__device__ __forceinline__ void state_body(
    StateSmem<DK, DV, BV> &sm, const unsigned bid,
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const GT *__restrict__ wr,
    const float *__restrict__ h0,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ chunk_off,
    const uint8_t *__restrict__ recs, IO *__restrict__ o, float *__restrict__ h_T, int64_t seq_len,
    int32_t H, int64_t num_chains, float lo) {
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int64_t chain;
    int vb;
    if (!state_block(bid, num_chains, DV / BV, chain, vb)) return;
    ChainRange cr;
    cr.n = chain / H;
    cr.h = (int)(chain % H);
    cr.col0 = vb * BV;
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
        state_role_loop<DK, DV, BV, IO, GT, PRO, GM, DEC>(sm, cr, q, k, v, log_alpha, beta, wr, h0, o, h_T, H, w, tid,
                                                          lo);
    else if (w < 8)
        output_role_loop<DK, DV, BV, IO>(sm, cr, o, H, w - 4, tid);
    else
        loader_role_loop<DK, DV, BV>(sm, cr, recs, H, tid - 512);
}

template <int DK, int DV, int BV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const GT *__restrict__ wr,
    const float *__restrict__ h0,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ chunk_off,
    const uint8_t *__restrict__ recs, IO *__restrict__ o, float *__restrict__ h_T, int64_t seq_len,
    int32_t H, int64_t num_chains, float lo) {
    __shared__ StateSmem<DK, DV, BV> sm;
    state_body<DK, DV, BV, IO, GT, PRO, GM, DEC>(sm, blockIdx.x, q, k, v, log_alpha, beta, wr, h0, cu_seqlens,
                                                 chunk_off, recs, o, h_T, seq_len, H, num_chains, lo);
}

// Pipelined segments: one launch runs the state pass of segment j on its own
// blocks and the prep pass of segment j+1 on the rest, so the compute units the
// state pass leaves free (it has one workgroup per compute unit and fewer
// workgroups than half the chip) prepare the next records meanwhile.  The two
// parts share nothing: the state blocks read segment j's records and the prep
// blocks write segment j+1's into the other buffer.  A prep block takes two
// chunk-heads, one per half of its 16 waves, each half with its own LDS, so a
// compute unit prepares two at a time as with the prep kernel.  A half without
// a chunk-head (an odd count) ends at once, on a wave-uniform branch, so it
// reaches no barrier; a barrier counts only the waves still running.
template <typename IO, typename GT> struct StatePart {
    const IO *q, *k, *v;
    const GT *log_alpha, *beta;
    const float *h0;
    const uint8_t *recs;
    IO *o;
    float *h_T;
    int64_t seq_len;
    int64_t blocks;   // workgroups of the state pass
};
template <typename IO, typename GT> struct PrepPart {
    const IO *q, *k, *v;
    const GT *log_alpha, *beta;
    uint8_t *recs;
    int64_t seq_len;
    unsigned count;   // chunk-heads of the segment
};
template <int DK, int DV> union PipeSmem {
    StateSmem<DK, DV, 16> st;
    PrepSmem<DK, DV> pr[2];
};

template <int DK, int DV, typename IO, typename GT, int GM>
__global__ __launch_bounds__(kStateThreads) void chunk_pipe_kernel(const StatePart<IO, GT> sp,
                                                                   const PrepPart<IO, GT> pp, int32_t H, float lo) {
    __shared__ PipeSmem<DK, DV> sm;
    if (blockIdx.x < sp.blocks) {
        state_body<DK, DV, 16, IO, GT, false, GM, false>(sm.st, blockIdx.x, sp.q, sp.k, sp.v, sp.log_alpha, sp.beta,
                                                          nullptr, sp.h0, nullptr, nullptr, sp.recs, sp.o, sp.h_T,
                                                          sp.seq_len, H, H, lo);
    } else {
        // waves 0-7 take chunk-head 2b, waves 8-15 chunk-head 2b + 1
        const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kWaves ? 1 : 0;
        const unsigned bid = 2 * (blockIdx.x - (unsigned)sp.blocks) + half;
        if (bid >= pp.count) return;   // uniform per wave
        const PrepSmem<DK, DV> *partner = (bid ^ 1u) < pp.count ? &sm.pr[half ^ 1] : nullptr;
        prep_body<DK, DV, IO, GT, false, GM, false, true>(sm.pr[half], partner, threadIdx.x & (kThreads - 1), bid,
                                                           pp.q, pp.k, pp.v, pp.log_alpha, pp.beta, nullptr, nullptr,
                                                           nullptr, pp.recs, 1, pp.seq_len, H, lo);
    }
}

// One prep pass and one state pass over the tokens described by a, with the
// records at recs.
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
hipError_t launch_pass(const ChunkArgs &a, int bv, int32_t *chunk_off, uint8_t *recs, hipStream_t st) {
    if (a.varlen)
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.num_seqs, chunk_off);
    const int64_t nprep = max_chunks(a) * a.H;
    if (nprep > 0)
        hipLaunchKernelGGL((chunk_prep_kernel<DK, DV, IO, GT, PRO, GM, DEC>), dim3((unsigned)nprep), dim3(kThreads), 0,
                           st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v, (const GT *)a.log_alpha,
                           (const GT *)a.beta, (const GT *)a.w_write, a.cu_seqlens, (const int32_t *)chunk_off, recs,
                           a.num_seqs, a.seq_len, a.H, a.log_alpha_min);
    const int64_t chains = a.num_seqs * (int64_t)a.H;
    // 32 value columns per workgroup only at d_k = 64.  At d_k = 128 the
    // 32-column instance compiles within the 16-wave budget (100 VGPRs, 153 KiB
    // of LDS) and gives the same bits, but its chunk step is about 1.3x longer
    // while the state pass runs on half as many compute units: the long-context
    // call took 2.53 ms against 2.13-2.18 ms with 16 columns.
    if constexpr (DK == 64) {
        if (bv == 32) {
            hipLaunchKernelGGL((chunk_state_kernel<DK, DV, 32, IO, GT, PRO, GM, DEC>),
                               dim3((unsigned)state_grid(chains, DV / 32)), dim3(kStateThreads), 0, st, (const IO *)a.q,
                               (const IO *)a.k, (const IO *)a.v, (const GT *)a.log_alpha, (const GT *)a.beta,
                               (const GT *)a.w_write, a.h0, a.cu_seqlens,
                               (const int32_t *)chunk_off, recs, (IO *)a.o, a.h_T, a.seq_len, a.H, chains,
                               a.log_alpha_min);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((chunk_state_kernel<DK, DV, 16, IO, GT, PRO, GM, DEC>), dim3((unsigned)state_grid(chains, DV / 16)),
                           dim3(kStateThreads), 0, st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v,
                           (const GT *)a.log_alpha, (const GT *)a.beta, (const GT *)a.w_write, a.h0, a.cu_seqlens,
                           (const int32_t *)chunk_off, recs, (IO *)a.o, a.h_T, a.seq_len, a.H, chains,
                           a.log_alpha_min);
    return hipGetLastError();
}

// The arguments of segment [t0, t0 + len) of a single sequence.
template <int DK, int DV, typename IO, typename GT, int GM>
ChunkArgs segment_args(const ChunkArgs &a, int64_t t0, int64_t len, float *carry) {
    const int64_t H = a.H;
    ChunkArgs s = a;
    s.seq_len = len;
    s.total_tokens = len;
    s.q = (const IO *)a.q + t0 * H * DK;
    s.k = (const IO *)a.k + t0 * H * DK;
    s.v = (const IO *)a.v + t0 * H * DV;
    s.o = (IO *)a.o + t0 * H * DV;
    if (GM == kGatePerChannel) s.log_alpha = (const GT *)a.log_alpha + t0 * H * DK;
    else if (GM == kGatePerHead) s.log_alpha = (const GT *)a.log_alpha + t0 * H;
    s.beta = (const GT *)a.beta + t0 * H;
    if (a.w_write) s.w_write = (const GT *)a.w_write + t0 * H;
    s.h0 = t0 == 0 ? a.h0 : carry;
    s.h_T = t0 + len >= a.seq_len ? a.h_T : carry;
    return s;
}

// Pipelined segments of segc chunks: the prep pass of segment 0, then per
// segment j one launch with the state pass of j and the prep pass of j + 1
// (records alternating between two buffers), the last segment's state pass on
// its own.  The state crosses segments in fp32 through carry, as with plain
// segments.
template <int DK, int DV, typename IO, typename GT, int GM>
hipError_t launch_pipelined(const ChunkArgs &a, int64_t segc, float *carry, uint8_t *recs0, hipStream_t st) {
    const int64_t seg = segc * kC;
    uint8_t *recs[2] = {recs0, recs0 + (size_t)segc * a.H * Rec<DK, DV>::BYTES};
    const int64_t nseg = (a.seq_len + seg - 1) / seg;
    const int64_t blocks = state_grid(a.H, DV / 16);
    auto seg_len = [&](int64_t j) { return a.seq_len - j * seg < seg ? a.seq_len - j * seg : seg; };
    {
        const ChunkArgs p = segment_args<DK, DV, IO, GT, GM>(a, 0, seg_len(0), carry);
        const int64_t nprep = (p.seq_len + kC - 1) / kC * a.H;
        hipLaunchKernelGGL((chunk_prep_kernel<DK, DV, IO, GT, false, GM, false>), dim3((unsigned)nprep), dim3(kThreads),
                           0, st, (const IO *)p.q, (const IO *)p.k, (const IO *)p.v, (const GT *)p.log_alpha,
                           (const GT *)p.beta, (const GT *)nullptr, (const int32_t *)nullptr,
                           (const int32_t *)nullptr, recs[0], (int64_t)1, p.seq_len, a.H, a.log_alpha_min);
    }
    for (int64_t j = 0; j < nseg; ++j) {
        const ChunkArgs s = segment_args<DK, DV, IO, GT, GM>(a, j * seg, seg_len(j), carry);
        if (j + 1 == nseg) {
            hipLaunchKernelGGL((chunk_state_kernel<DK, DV, 16, IO, GT, false, GM, false>), dim3((unsigned)blocks),
                               dim3(kStateThreads), 0, st, (const IO *)s.q, (const IO *)s.k, (const IO *)s.v,
                               (const GT *)s.log_alpha, (const GT *)s.beta, (const GT *)nullptr, s.h0,
                               (const int32_t *)nullptr, (const int32_t *)nullptr, (const uint8_t *)recs[j & 1],
                               (IO *)s.o, s.h_T, s.seq_len, a.H, (int64_t)a.H, a.log_alpha_min);
            break;
        }
        const ChunkArgs p = segment_args<DK, DV, IO, GT, GM>(a, (j + 1) * seg, seg_len(j + 1), carry);
        const StatePart<IO, GT> sp{(const IO *)s.q, (const IO *)s.k, (const IO *)s.v, (const GT *)s.log_alpha,
                                   (const GT *)s.beta, s.h0, recs[j & 1], (IO *)s.o, s.h_T, s.seq_len, blocks};
        const int64_t nprep = (p.seq_len + kC - 1) / kC * a.H;
        const PrepPart<IO, GT> pp{(const IO *)p.q, (const IO *)p.k, (const IO *)p.v, (const GT *)p.log_alpha,
                                  (const GT *)p.beta, recs[(j + 1) & 1], p.seq_len, (unsigned)nprep};
        hipLaunchKernelGGL((chunk_pipe_kernel<DK, DV, IO, GT, GM>), dim3((unsigned)(blocks + (nprep + 1) / 2)),
                           dim3(kStateThreads), 0, st, sp, pp, a.H, a.log_alpha_min);
    }
    return hipGetLastError();
}

template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
hipError_t launch_two_kernel(const ChunkArgs &a, int bv, hipStream_t st) {
    uint8_t *ws = reinterpret_cast<uint8_t *>(a.workspace);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws + kHeaderBytes);
    uint8_t *after_plan = ws + kHeaderBytes + plan_bytes(a.num_seqs);
    if constexpr (DK == 128 && !PRO && !DEC) {
        const int64_t pc = pipe_chunks(a);
        if (pc > 0)
            return launch_pipelined<DK, DV, IO, GT, GM>(a, pc, reinterpret_cast<float *>(after_plan),
                                                        after_plan + carry_bytes(a), st);
    }
    const int64_t segc = segment_chunks(a);
    if (segc == 0) return launch_pass<DK, DV, IO, GT, PRO, GM, DEC>(a, bv, chunk_off, after_plan, st);
    // segments of one sequence: the state is carried in the workspace
    float *carry = reinterpret_cast<float *>(after_plan);
    uint8_t *recs = after_plan + carry_bytes(a);
    const int64_t seg = segc * kC;
    for (int64_t t0 = 0; t0 < a.seq_len; t0 += seg) {
        const int64_t len = a.seq_len - t0 < seg ? a.seq_len - t0 : seg;
        const ChunkArgs s = segment_args<DK, DV, IO, GT, GM>(a, t0, len, carry);
        const hipError_t e = launch_pass<DK, DV, IO, GT, PRO, GM, DEC>(s, bv, chunk_off, recs, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename GT, bool PRO, int GM, bool DEC>
hipError_t launch_two_kernel_dims(const ChunkArgs &a, int bv, hipStream_t st) {
    if (a.d_k == 128)
        return a.d_v == 128 ? launch_two_kernel<128, 128, bf16_t, GT, PRO, GM, DEC>(a, bv, st)
                            : launch_two_kernel<128, 64, bf16_t, GT, PRO, GM, DEC>(a, bv, st);
    return a.d_v == 128 ? launch_two_kernel<64, 128, bf16_t, GT, PRO, GM, DEC>(a, bv, st)
                        : launch_two_kernel<64, 64, bf16_t, GT, PRO, GM, DEC>(a, bv, st);
}

// The input variants that exist: per-channel gates with or without the prologue
// or with decoupled strengths, and the scalar-gate forms.
template <typename GT>
hipError_t launch_two_kernel_variant(const ChunkArgs &a, int bv, hipStream_t st) {
    if (a.gate_mode == kGatePerHead) return launch_two_kernel_dims<GT, false, kGatePerHead, false>(a, bv, st);
    if (a.gate_mode == kGateNone) return launch_two_kernel_dims<GT, false, kGateNone, false>(a, bv, st);
    if (a.prologue) return launch_two_kernel_dims<GT, true, kGatePerChannel, false>(a, bv, st);
    if (a.w_write) return launch_two_kernel_dims<GT, false, kGatePerChannel, true>(a, bv, st);
    return launch_two_kernel_dims<GT, false, kGatePerChannel, false>(a, bv, st);
}

size_t record_bytes(int d_k, int d_v) {
    if (d_k == 128) return d_v == 128 ? Rec<128, 128>::BYTES : Rec<128, 64>::BYTES;
    return d_v == 128 ? Rec<64, 128>::BYTES : Rec<64, 64>::BYTES;
}

}  // namespace

// The prep kernel runs one workgroup per chunk-head of a pass (a segment's when
// the sequence runs in segments), the state kernel the padded chains times the
// value-column blocks.
bool two_kernel_grids_fit(const ChunkArgs &a, int bv) {
    const int64_t pc = pipe_chunks(a);
    if (pc > 0) return grid_fits(state_grid(a.H, a.d_v / 16) + (pc * a.H + 1) / 2, kStateThreads);
    const int64_t segc = segment_chunks(a);
    const int64_t nprep = (segc > 0 ? segc : max_chunks(a)) * a.H;
    const int width = (a.d_k == 64 && bv == 32) ? 32 : 16;
    return grid_fits(nprep, kThreads) && grid_fits(state_grid(a.num_seqs * (int64_t)a.H, a.d_v / width), kStateThreads);
}

size_t two_kernel_workspace_bytes(const ChunkArgs &a) {
    if (a.total_tokens <= 0) return 0;
    const int64_t pc = pipe_chunks(a);
    if (pc > 0)
        return kHeaderBytes + plan_bytes(a.num_seqs) + carry_bytes(a) +
               2 * (size_t)pc * a.H * record_bytes(a.d_k, a.d_v);
    const int64_t segc = segment_chunks(a);
    if (segc > 0)
        return kHeaderBytes + plan_bytes(a.num_seqs) + carry_bytes(a) +
               (size_t)segc * a.H * record_bytes(a.d_k, a.d_v);
    return kHeaderBytes + plan_bytes(a.num_seqs) + (size_t)max_chunks(a) * a.H * record_bytes(a.d_k, a.d_v);
}

hipError_t launch_chunk_fwd_two_kernel(const ChunkArgs &a, int bv, hipStream_t st) {
    return a.gate_bf16 ? launch_two_kernel_variant<bf16_t>(a, bv, st) : launch_two_kernel_variant<float>(a, bv, st);
}

}  // namespace kda
