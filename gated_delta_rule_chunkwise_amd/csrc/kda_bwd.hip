// kda_bwd.hip -- chunkwise KDA backward: gradients with respect to q, k, v,
// log_alpha, beta and h0, given those of o and h_T.
//
// The KimiLinear article motivates the chunkwise form by training throughput
// (sections 3 and 4.1) and notes that only a chunk-sized score block has to be
// kept per chunk for the backward pass (section 3.2).  The gradient is that of
// the forward recurrence (section 2.3); here it is taken through the chunk form
// of the forward.  Per chunk, with the in-chunk cumsum G of log alpha, its
// total g_n, the anchor m = g_n / 2 and the decayed operands
//     QA = Q.e^{G-m},  KA = K.e^{G-m},  KI = K.e^{m-G},
//     M = strictly-lower(KA KI^T),  A = diag(beta) M,  T = (I + A)^{-1},
//     P = lower(QA KI^T),  W = T diag(beta) KA,
// and S' = Diag(e^m) S for the chunk's start state S, the forward is
//     X = V - KA S',  U = T diag(beta) X,  O = QA S' + P U,
//     S_next = Diag(e^{g_n}) S + Diag(e^{g_n-m}) KI^T U.
// Given dO and dS_next, reverse-mode differentiation of these lines gives
//     dU  = P^T dO + KI Diag(e^{g_n-m}) dS_next
//     dS  = Diag(e^m) (QA^T dO - W^T dU) + Diag(e^{g_n}) dS_next
//     dY  = T^T dU,  dV = diag(beta) dY,  dA = -strictly-lower(dY U^T)
//     dP  = lower(dO U^T),  dM = diag(beta) dA
//     dQA = dO S'^T + dP KI
//     dKA = -diag(beta) dY S'^T + dM KI
//     dKI = dP^T QA + dM^T KA + Diag-cols(e^{g_n-m}) (U dS_next^T)
//     dbeta_r = sum_j dY[r,j] X[r,j] + sum_i dA[r,i] M[r,i]
//             (sum_j dY X taken as sum_j dY V - sum_c KA (dY S'^T), so X is never formed)
//     dQ = dQA.e^{G-m},  dK = dKA.e^{G-m} + dKI.e^{m-G}
//     dG = dQA.QA + dKA.KA - dKI.KI
//     dg_n[c] = e^{g_n-m}[c] (sum_j dS_next[c,j] S'[c,j] + sum_r (U dS_next^T)[r,c] KI[r,c])
//     dlog_alpha[t,c] = sum_{r >= t} dG[r,c] + dg_n[c]
// (the anchor m cancels from every result, so it is held fixed; g_n enters
// through e^{g_n} and e^{g_n-m}).
// With separate erase and write strengths (b, w) beta above is b, except in
// U's V term: U = T (diag(w) V - diag(b) KA S').  Then dV = diag(w) dY, and
// dbeta splits into dw_r = sum_j dY[r,j] V[r,j] and db_r = the other two terms.
//
// Three kernels, all in fp32 on the fp32 matrix cores:
//   bwd_prep_kernel    per (chunk, head), all in parallel: QA, KI, W, T, P, M
//                      and the anchor factors into a record per chunk-head;
//   bwd_state_kernel   two independent passes side by side in one launch, each
//                      per (sequence, head, 32 value columns):
//                        replay: the state recurrence, storing each chunk's
//                        start state and U;
//                        reverse: chunks in reverse order, the state gradient
//                        at each chunk's end and dU; dh0 after the first chunk;
//   bwd_grad_kernel    per (chunk, head), all in parallel: everything else,
//                      with the d_v contractions accumulated over 16-column
//                      blocks in registers.
// The value columns of the state evolve independently, so the two sequential
// passes split d_v across workgroups; the gradients of q, k, log alpha and
// beta sum over all columns and are formed per chunk-head in one workgroup,
// so no cross-workgroup reduction (and no atomic) is needed: results are
// bitwise deterministic.
//
// Range: the anchored factors e^{+-(G-m)} reach e^{D/2}, D = max_c(-g_n[c]).
// A chunk with D above about 159 nats (kBwdMaxRange2 in log2 units) would
// overflow fp32, so the prep kernel runs it exact and marks its record: no
// anchor (m = 0 for Q e^G and K e^G, m = g_n for K e^{g_n - G}, every factor at
// most 1), M and P formed pair by pair with e^{G_r - G_i} <= 1, and in the
// gradient kernel the intra-chunk parts of dq, dk and dG formed the same way:
//     dq_r  += sum_{i<=r} dP[r,i] k_i E(r,i)
//     dk_r  += sum_{i<r} dM[r,i] k_i E(r,i) + sum_{j>=r} (dP[j,r] q_j + dM[j,r] k_j) E(j,r)
//     dG_r  += q_r (first sum) + k_r (second) - k_r (third)
// per key channel, with E(r,i) = e^{G_r - G_i}.  The state passes need no
// change: they read the factors e^m, e^{g_n}, e^{g_n-m} from the record.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_plan.h"

#include <stdio.h>

namespace kda {
namespace {

constexpr int kB = kPlanChunk;                    // chunk length, 64
constexpr float kBL2E = 1.4426950408889634f;
constexpr float kBwdMaxRange2 = 230.f;            // max in-chunk decay, log2 units
constexpr int kBV = 16;                           // value columns per block of the gradient kernel
// Column scans over a chunk (the in-chunk cumsum of log alpha and the reverse
// cumsum of its gradient) run as kSeg segments of kSegRows rows per key
// channel, in parallel: G_r = (sum of the earlier segments' totals) + (running
// sum within r's segment).  The chunk total, summed from the same segment
// totals in the same order, then equals G at the last row bitwise, and every
// kernel that forms G forms it identically.
constexpr int kSeg = 4, kSegRows = kB / kSeg;

// D(16x16) += A(16x4) B(4x16), fp32.  Lane l holds A[l%16][l/16],
// B[l/16][l%16] and D[4*(l/16) + e][l%16], e = 0..3.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive-k values of an operand for one lane: one 16-byte LDS read
// when the operand is contiguous along k (stride 1), else four reads.
template <int STRIDE>
__device__ __forceinline__ f32x4_t k4(const float *p) {
    if constexpr (STRIDE == 1) {
        return *reinterpret_cast<const f32x4_t *>(p);
    } else {
        f32x4_t v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = p[u * STRIDE];
        return v;
    }
}

// acc += A B over one 16x16 tile, K a multiple of 16, with
// A(i, k) = a[i*AI + k*AK] and B(k, j) = b[k*BK + j*BJ].  Within each group of
// 16 k values, lane group kq = lane/16 takes k = 16g + 4kq + u at step u, so an
// operand with unit stride along k is read 4 values at a time.  (The matrix
// instruction only requires A and B to agree on which k each lane supplies.)
template <int K, int AI, int AK, int BK, int BJ>
__device__ __forceinline__ f32x4_t mm(f32x4_t acc, const float *a, const float *b, int lane) {
    static_assert(K % 16 == 0, "K must be a multiple of 16");
    constexpr int NG = K / 16;
    const float *pa = a + (lane & 15) * AI + 4 * (lane >> 4) * AK;
    const float *pb = b + 4 * (lane >> 4) * BK + (lane & 15) * BJ;
    f32x4_t av[NG], bv[NG];                  // every operand read is issued first
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        av[g] = k4<AK>(pa + 16 * g * AK);
        bv[g] = k4<BK>(pb + 16 * g * BK);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma4(av[g][u], bv[g][u], acc);
    return acc;
}

__device__ __forceinline__ int acc_row(int lane, int e) { return 4 * (lane >> 4) + e; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

// Lower 16x16 blocks (R, I), I <= R, of a 64x64 chunk matrix, in order
// (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3).
__device__ __forceinline__ void low_tile(int idx, int &R, int &I) {
    R = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    I = idx - (R * (R + 1)) / 2;
}

// Per chunk-head record (fp32, row-major, offsets in floats).  The forward
// replay reads [T, QA) and the reverse pass [KI, M), each one contiguous span.
// Records, like every per-chunk array of the workspace, are indexed
// [head][chunk slot], so that a chain walks through contiguous memory.
template <int DK> struct BRec {
    static constexpr size_t T = 0;
    static constexpr size_t KI = T + kB * kB;
    static constexpr size_t W = KI + (size_t)kB * DK;
    static constexpr size_t QA = W + (size_t)kB * DK;
    static constexpr size_t P = QA + (size_t)kB * DK;
    static constexpr size_t M = P + kB * kB;
    static constexpr size_t EM = M + kB * kB;     // e^m
    static constexpr size_t EG = EM + DK;         // e^{g_n}
    static constexpr size_t EGM = EG + DK;        // e^{g_n - m}
    static constexpr size_t FLAG = EGM + DK;      // nonzero: decay out of range
    static constexpr size_t FLOATS = (FLAG + 4 + 63) / 64 * 64;
};

struct BwdLayout {
    int64_t nch;                 // chunk slots (upper bound over sequences)
    size_t plan, rec, sc, uc, dsc, duc, total;
};

int64_t bwd_max_chunks(const BwdArgs &a) {
    if (a.varlen) return (a.total_tokens + kB - 1) / kB + a.num_seqs;
    return a.num_seqs * ((a.seq_len + kB - 1) / kB);
}

template <int DK> size_t rec_floats() { return BRec<DK>::FLOATS; }

BwdLayout bwd_layout(const BwdArgs &a) {
    BwdLayout L;
    L.nch = bwd_max_chunks(a);
    const size_t ch = (size_t)L.nch * a.H;
    const size_t recf = a.d_k == 128 ? rec_floats<128>() : rec_floats<64>();
    L.plan = 0;
    L.rec = plan_bytes(a.num_seqs);
    L.sc = L.rec + ch * recf * 4;
    L.uc = L.sc + ch * a.d_k * a.d_v * 4;
    L.dsc = L.uc + ch * kB * a.d_v * 4;
    L.duc = L.dsc + ch * a.d_k * a.d_v * 4;
    L.total = L.duc + ch * kB * a.d_v * 4;
    return L;
}

// Token range [bos, eos) and first chunk slot of sequence n.
__device__ __forceinline__ void seq_range(int64_t n, const int32_t *__restrict__ cu,
                                          const int32_t *__restrict__ chunk_off, int64_t T, int64_t &bos,
                                          int64_t &eos, int64_t &slot0) {
    if (cu) {
        bos = cu[n];
        eos = cu[n + 1];
        slot0 = chunk_off[n];
    } else {
        bos = n * T;
        eos = bos + T;
        slot0 = n * ((T + kB - 1) / kB);
    }
}

// 16-byte vectors of X, converted to fp32 on the way into LDS.
template <typename X> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    typedef f32x4_t raw;
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    typedef bf16x8_t raw;
};

template <typename X>
__device__ __forceinline__ void put_f32(float *dst, const typename Vec16<X>::raw &v, float scale) {
    if constexpr (Vec16<X>::N == 4) {
        *reinterpret_cast<f32x4_t *>(dst) = v * scale;
    } else {
        f32x4_t a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = (float)v[e] * scale;
            b[e] = (float)v[e + 4] * scale;
        }
        *reinterpret_cast<f32x4_t *>(dst) = a;
        *reinterpret_cast<f32x4_t *>(dst + 4) = b;
    }
}

// A ROWS x COLS block of X (row r at src + r * pitch, rows >= nv read as zero)
// moved into an fp32 LDS array with row stride LS by NT threads: load() issues
// the 16-byte loads into registers, store() writes them out later (optionally
// scaled per row).
template <int ROWS, int COLS, int NT, typename X> struct Stage {
    static constexpr int VE = Vec16<X>::N, PER = COLS / VE, TOT = ROWS * PER, IT = (TOT + NT - 1) / NT;
    static_assert(COLS % VE == 0, "row length must be a whole number of 16-byte vectors");
    typename Vec16<X>::raw buf[IT];
    __device__ __forceinline__ void load(const X *__restrict__ src, size_t pitch, int nv, int tid) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + NT * it, r = i / PER;
            typename Vec16<X>::raw z = {};
            buf[it] = z;
            if (i < TOT && r < nv)
                buf[it] = *reinterpret_cast<const typename Vec16<X>::raw *>(src + (size_t)r * pitch + (i % PER) * VE);
        }
    }
    // Transposed: element (r, c) goes to dst[c * LS + r].
    template <int LS>
    __device__ __forceinline__ void store_t(float *dst, int tid) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + NT * it, r = i / PER, c = (i % PER) * VE;
            if (i < TOT) {
#pragma unroll
                for (int e = 0; e < VE; ++e) dst[(c + e) * LS + r] = (float)buf[it][e];
            }
        }
    }
    template <int LS>
    __device__ __forceinline__ void store(float *dst, int tid, const float *rscale = nullptr) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + NT * it, r = i / PER;
            if (i < TOT) put_f32<X>(dst + r * LS + (i % PER) * VE, buf[it], rscale ? rscale[r] : 1.f);
        }
    }
};

// For the layouts without a per-channel gate: the chunk's log alpha per row,
// one value per (token, head) (Gated DeltaNet) or 0 (DeltaNet), into gv[kB] by
// the first kB threads; rows >= nv are 0.  The column scans read gv[r] in place
// of a staged [row][channel] block.
template <int GM, typename GT>
__device__ __forceinline__ void load_gate_rows(float *gv, const GT *__restrict__ la, int64_t t0, int H, int h,
                                               int nv, int tid) {
    if (tid < kB) gv[tid] = (GM == kGatePerHead && tid < nv) ? to_f32(la[(t0 + tid) * H + h]) : 0.f;
}

// ----------------------------------------------------------------------------
// Prep: one workgroup of 4 waves per (chunk, head).  The key channels are taken
// 64 at a time (the column scan is per channel and the Gram products are sums
// over channels, accumulated in registers across the passes in the order of a
// single pass); only KA is kept for all channels, for W.  This keeps the
// workgroup within half of the LDS, so that two share a CU.
template <int DK> struct alignas(16) PrepBS {
    static constexpr int CH = DK < 64 ? DK : 64;   // channels per pass
    static constexpr int KS = DK + 4, HS = CH + 4, CS = kB + 4;
    float KA[kB][KS];                        // k, then K e^{G-m}, then diag(beta) KA
    union {
        struct {
            float QA[kB][HS];                // this pass's channels: q, then QA
            float KI[kB][HS];                // log alpha, then K e^{m-G}
        } g;
        struct {
            float A[kB][CS];                 // beta M
            float T[kB][CS];                 // (I + A)^{-1}
        } t;
    };
    float X[4][16][20];                      // per-wave product tile
    float beta[kB];
    float gv[kB];                            // log alpha per row (scalar-gate layouts)
    float part[kSeg][CH];                    // segment totals of the column scan
    float pre[256];                          // partial channel totals of the mode scan
    int flag;                                // the chunk runs exact (see the header)
};

// GM: gate layout (per key channel, per (token, head), or none).
template <int DK, typename IO, typename GT, int GM>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                                                       const GT *__restrict__ log_alpha, const GT *__restrict__ beta,
                                                       const int32_t *__restrict__ cu,
                                                       const int32_t *__restrict__ chunk_off, int64_t N, int64_t T,
                                                       int H, int64_t nch, float *__restrict__ recs) {
    using R = BRec<DK>;
    using S = PrepBS<DK>;
    __shared__ S sm;
    const int64_t chunk = blockIdx.x;
    const int h = blockIdx.y;
    int64_t n, t0;
    int nv;
    if (!locate_chunk(chunk, cu, chunk_off, N, T, n, t0, nv)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float *rec = recs + ((size_t)h * nch + chunk) * R::FLOATS;

    if (tid == 0) sm.flag = 0;
    if (tid < kB) sm.beta[tid] = tid < nv ? to_f32(beta[(t0 + tid) * H + h]) : 0.f;
    {   // the chunk's mode: exact once any key channel decays by more than kBwdMaxRange2
        constexpr int NP = 256 / DK;         // threads per channel
        const int c = tid % DK, p = tid / DK;
        float l = 0.f;
        if constexpr (GM == kGatePerChannel) {
            for (int r = p; r < nv; r += NP) l += to_f32(log_alpha[((t0 + r) * H + h) * DK + c]);
        } else if constexpr (GM == kGatePerHead) {
            for (int r = p; r < nv; r += NP) l += to_f32(log_alpha[(t0 + r) * H + h]);
        }
        sm.pre[tid] = l;
        __syncthreads();
        if (tid < DK) {
            float tot = 0.f;
#pragma unroll
            for (int i = 0; i < NP; ++i) tot += sm.pre[tid + DK * i];
            if (-tot * kBL2E > kBwdMaxRange2) sm.flag = 1;
        }
        __syncthreads();
    }
    const bool exact = sm.flag != 0;
    // Wave w accumulates tile (s, w) of P = lower(QA KI^T) and of
    // M = strictly-lower(KA KI^T) for block rows s >= w.
    constexpr int CH = S::CH, NH = DK / CH;
    f32x4_t accP[4], accM[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) accP[s4] = accM[s4] = zero4();
    // exact mode: thread t owns the pairs (r, i <= r) numbered t + 256 j
    constexpr int NPAIR = kB * (kB + 1) / 2, PPT = (NPAIR + 255) / 256;
    float xP[PPT], xM[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) xP[j] = xM[j] = 0.f;
    const size_t base = ((size_t)t0 * H + h) * DK, pitch = (size_t)H * DK;
    for (int hf = 0; hf < NH; ++hf) {
        const int c0 = hf * CH;
        {   // q -> QA, k -> KA, log alpha -> KI, as fp32 (rows >= nv zero)
            Stage<kB, CH, 256, IO> sq, sk;
            Stage<kB, CH, 256, GT> sl;
            sq.load(q + base + c0, pitch, nv, tid);
            sk.load(k + base + c0, pitch, nv, tid);
            if constexpr (GM == kGatePerChannel) sl.load(log_alpha + base + c0, pitch, nv, tid);
            if (hf > 0) __syncthreads();     // the previous pass's reads of QA and KI are done
            sq.template store<S::HS>(&sm.g.QA[0][0], tid);
            sk.template store<S::KS>(&sm.KA[0][c0], tid);
            if constexpr (GM == kGatePerChannel) sl.template store<S::HS>(&sm.g.KI[0][0], tid);
            else if (hf == 0) load_gate_rows<GM>(sm.gv, log_alpha, t0, H, h, nv, tid);
        }
        __syncthreads();
        {   // G (log2 units) per key channel, segment totals first
            constexpr int PT = 256 / CH;
            const int c = tid % CH, p = tid / CH;
            for (int sg = p; sg < kSeg; sg += PT) {
                const int r0 = sg * kSegRows, r1 = min(r0 + kSegRows, nv);
                float l = 0.f;
                for (int r = r0; r < r1; ++r) l += (GM == kGatePerChannel ? sm.g.KI[r][c] : sm.gv[r]) * kBL2E;
                sm.part[sg][c] = l;
            }
        }
        __syncthreads();
        if (exact) {   // G in place of log alpha; then the pairs; then the operands without anchor
            constexpr int PT = 256 / CH;
            const int c = tid % CH, p = tid / CH;
            float g2 = 0.f;
#pragma unroll
            for (int i = 0; i < kSeg; ++i) g2 += sm.part[i][c];
            for (int sg = p; sg < kSeg; sg += PT) {
                float pre = 0.f;
                for (int i = 0; i < sg; ++i) pre += sm.part[i][c];
                const int r0 = sg * kSegRows, r1 = min(r0 + kSegRows, nv);
                float l = 0.f;
                for (int r = r0; r < r1; ++r) {
                    l += (GM == kGatePerChannel ? sm.g.KI[r][c] : sm.gv[r]) * kBL2E;
                    sm.g.KI[r][c] = pre + l;
                }
            }
            __syncthreads();
            // M[r,i] += sum_c k_rc k_ic e^{G_rc - G_ic} (i < r), P[r,i] += sum_c q_rc k_ic e^{...}
            // (i <= r), over this pass's channels: every factor at most 1
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int pi = tid + 256 * j;
                int r = (int)((sqrtf(8.f * pi + 1.f) - 1.f) * 0.5f);
                if ((r + 1) * (r + 2) / 2 <= pi) ++r;
                if (r * (r + 1) / 2 > pi) --r;
                const int i = pi - r * (r + 1) / 2;
                if (pi < NPAIR && r < nv) {
                    float sp = 0.f, sq = 0.f;
                    for (int cc = 0; cc < CH; cc += 4) {
                        const f32x4_t gr = *reinterpret_cast<const f32x4_t *>(&sm.g.KI[r][cc]);
                        const f32x4_t gi = *reinterpret_cast<const f32x4_t *>(&sm.g.KI[i][cc]);
                        const f32x4_t kr = *reinterpret_cast<const f32x4_t *>(&sm.KA[r][c0 + cc]);
                        const f32x4_t ki = *reinterpret_cast<const f32x4_t *>(&sm.KA[i][c0 + cc]);
                        const f32x4_t qr = *reinterpret_cast<const f32x4_t *>(&sm.g.QA[r][cc]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float kk = ki[e] * __builtin_amdgcn_exp2f(gr[e] - gi[e]);
                            sp += kr[e] * kk;
                            sq += qr[e] * kk;
                        }
                    }
                    xM[j] += i < r ? sp : 0.f;
                    xP[j] += sq;
                }
            }
            __syncthreads();
            for (int sg = p; sg < kSeg; sg += PT) {
                const int r0 = sg * kSegRows;
                for (int r = r0; r < r0 + kSegRows; ++r) {
                    float ea = 0.f, ei = 0.f;
                    if (r < nv) {
                        const float G = sm.g.KI[r][c];
                        ea = __builtin_amdgcn_exp2f(G);
                        ei = __builtin_amdgcn_exp2f(g2 - G);
                    }
                    const float kv = sm.KA[r][c0 + c];
                    sm.g.QA[r][c] *= ea;
                    sm.KA[r][c0 + c] = kv * ea;
                    sm.g.KI[r][c] = kv * ei;
                }
            }
            if (p == 0) {
                rec[R::EM + c0 + c] = 1.f;
                rec[R::EG + c0 + c] = __builtin_amdgcn_exp2f(g2);
                rec[R::EGM + c0 + c] = 1.f;
            }
        } else {   // then the decayed operands in place
            constexpr int PT = 256 / CH;
            const int c = tid % CH, p = tid / CH;
            float g2 = 0.f;
#pragma unroll
            for (int i = 0; i < kSeg; ++i) g2 += sm.part[i][c];
            const float m2 = 0.5f * g2;
            for (int sg = p; sg < kSeg; sg += PT) {
                float pre = 0.f;
                for (int i = 0; i < sg; ++i) pre += sm.part[i][c];
                const int r0 = sg * kSegRows, r1 = min(r0 + kSegRows, nv);
                float l = 0.f;
                for (int r = r0; r < r1; ++r) {
                    l += (GM == kGatePerChannel ? sm.g.KI[r][c] : sm.gv[r]) * kBL2E;
                    const float G = pre + l;
                    const float ea = __builtin_amdgcn_exp2f(G - m2), ei = __builtin_amdgcn_exp2f(m2 - G);
                    const float kv = sm.KA[r][c0 + c];
                    sm.g.QA[r][c] *= ea;
                    sm.KA[r][c0 + c] = kv * ea;
                    sm.g.KI[r][c] = kv * ei;
                }
            }
            if (p == 0) {
                rec[R::EM + c0 + c] = __builtin_amdgcn_exp2f(m2);
                rec[R::EG + c0 + c] = __builtin_amdgcn_exp2f(g2);
                rec[R::EGM + c0 + c] = __builtin_amdgcn_exp2f(g2 - m2);
            }
        }
        __syncthreads();
        // QA and KI of these channels go to the record as they are.
        for (int i = tid; i < kB * CH / 4; i += 256) {
            const int r = i / (CH / 4), c = (i % (CH / 4)) * 4;
            *reinterpret_cast<f32x4_t *>(rec + R::QA + r * DK + c0 + c) =
                *reinterpret_cast<const f32x4_t *>(&sm.g.QA[r][c]);
            *reinterpret_cast<f32x4_t *>(rec + R::KI + r * DK + c0 + c) =
                *reinterpret_cast<const f32x4_t *>(&sm.g.KI[r][c]);
        }
        // the Gram products over these channels
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            if (!exact && w <= s4) {
                accP[s4] = mm<CH, S::HS, 1, 1, S::HS>(accP[s4], &sm.g.QA[16 * s4][0], &sm.g.KI[16 * w][0], lane);
                accM[s4] = mm<CH, S::KS, 1, 1, S::HS>(accM[s4], &sm.KA[16 * s4][c0], &sm.g.KI[16 * w][0], lane);
            }
        }
    }
    if (tid == 0) rec[R::FLAG] = exact ? 1.f : 0.f;
    if (exact) {   // P and M from the pairs, zero above the diagonal; A = diag(beta) M
        for (int i = tid; i < kB * kB; i += 256) {
            if (i % kB > i / kB) {
                rec[R::P + i] = 0.f;
                rec[R::M + i] = 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int pi = tid + 256 * j;
            int r = (int)((sqrtf(8.f * pi + 1.f) - 1.f) * 0.5f);
            if ((r + 1) * (r + 2) / 2 <= pi) ++r;
            if (r * (r + 1) / 2 > pi) --r;
            const int i = pi - r * (r + 1) / 2;
            if (pi < NPAIR) {
                rec[R::P + r * kB + i] = xP[j];
                rec[R::M + r * kB + i] = xM[j];
            }
        }
        __syncthreads();   // QA and KI no longer read
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int pi = tid + 256 * j;
            int r = (int)((sqrtf(8.f * pi + 1.f) - 1.f) * 0.5f);
            if ((r + 1) * (r + 2) / 2 <= pi) ++r;
            if (r * (r + 1) / 2 > pi) --r;
            const int i = pi - r * (r + 1) / 2;
            if (pi < NPAIR) sm.t.A[r][i] = sm.beta[r] * xM[j];
        }
        for (int i = tid; i < kB * kB; i += 256)
            if (i % kB > i / kB) sm.t.A[i / kB][i % kB] = 0.f;
    }
    if (!exact) {   // P and M to the record (tiles above the diagonal are zero); A = diag(beta) M
        f32x4_t mt[4];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bool isM = s >= 4;
            const int Rt = s & 3, It = w;
            f32x4_t acc = isM ? accM[Rt] : accP[Rt];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * Rt + acc_row(lane, e), c = 16 * It + acc_col(lane);
                const bool keep = isM ? r > c : r >= c;
                acc[e] = keep ? acc[e] : 0.f;
                rec[(isM ? R::M : R::P) + r * kB + c] = acc[e];
            }
            if (isM) mt[s & 3] = acc;
        }
        __syncthreads();   // QA and KI no longer read
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * s + acc_row(lane, e), c = 16 * w + acc_col(lane);
                sm.t.A[r][c] = sm.beta[r] * mt[s][e];
            }
        }
    }
    // KA <- diag(beta) KA for W
    for (int i = tid; i < kB * DK; i += 256) {
        const int r = i / DK, c = i % DK;
        sm.KA[r][c] *= sm.beta[r];
    }
    __syncthreads();
    // T = (I + A)^{-1}, unit lower triangular.  Diagonal 16x16 blocks by forward
    // substitution (wave 0, lane 16b + j holds column j of block b); the other
    // waves clear the blocks above the diagonal.
    if (w == 0) {
        const int b = lane >> 4, j = lane & 15;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s += sm.t.A[16 * b + i][16 * b + m] * t[m];
            t[i] = i < j ? 0.f : (i == j ? 1.f : -s);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.t.T[16 * b + i][16 * b + j] = t[i];
    } else {
        for (int i = tid - 64; i < kB * kB; i += 192) {
            const int r = i / kB, c = i % kB;
            if ((c >> 4) > (r >> 4)) sm.t.T[r][c] = 0.f;
        }
    }
    __syncthreads();
    // Off-diagonal blocks, block row by block row:
    //     T_RI = -T_RR sum_{m=I}^{R-1} A_Rm T_mI.
    for (int Rb = 1; Rb < 4; ++Rb) {
        if (w < Rb) {
            const int Ib = w;
            f32x4_t acc = zero4();
            for (int m = Ib; m < Rb; ++m)
                acc = mm<16, S::CS, 1, S::CS, 1>(acc, &sm.t.A[16 * Rb][16 * m], &sm.t.T[16 * m][16 * Ib], lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.X[w][acc_row(lane, e)][acc_col(lane)] = acc[e];
        }
        __syncthreads();
        if (w < Rb) {
            const int Ib = w;
            f32x4_t acc = zero4();
            acc = mm<16, S::CS, 1, 20, 1>(acc, &sm.t.T[16 * Rb][16 * Rb], &sm.X[w][0][0], lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.t.T[16 * Rb + acc_row(lane, e)][16 * Ib + acc_col(lane)] = -acc[e];
        }
        __syncthreads();
    }
    for (int i = tid; i < kB * kB; i += 256) {
        const int r = i / kB, c = i % kB;
        rec[R::T + i] = sm.t.T[r][c];
    }
    // W = T diag(beta) KA: 4 x DK/16 tiles.
    constexpr int NWT = 4 * (DK / 16);
    for (int idx = w; idx < NWT; idx += 4) {
        const int Rt = idx / (DK / 16), Ct = idx % (DK / 16);
        f32x4_t acc = zero4();
        acc = mm<kB, S::CS, 1, S::KS, 1>(acc, &sm.t.T[16 * Rt][0], &sm.KA[0][16 * Ct], lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) rec[R::W + (16 * Rt + acc_row(lane, e)) * DK + 16 * Ct + acc_col(lane)] = acc[e];
    }
}

// ----------------------------------------------------------------------------
// The two sequential passes: one workgroup of 8 waves per (sequence, head,
// block of value columns), walking the sequence's chunks.  Waves 0-3 compute;
// waves 4-7 only move data: they hold the next chunk's record span in registers
// (slot s of loader thread t: float4 number t + 256 s of the span), write it
// into LDS at the chunk boundary, issue the following chunk's loads while the
// compute waves work, and store the per-chunk results, so that the compute
// waves issue no global memory instruction.
constexpr int kSP = 512;                     // threads per workgroup
constexpr int kLT = 256;                     // loader threads (waves 4-7)
constexpr int kXCD = 8;

// Block id -> (chain = sequence * H + head, column block).  Workgroups go to the
// 8 XCDs round-robin by block id, so the NVB column blocks of one chain get ids
// that are equal modulo 8: they run on one XCD, where the chunk records they
// all read can be served from that XCD's L2.  Ids past the last chain return.
template <int NVB>
__device__ __forceinline__ bool chain_of(int64_t id, int64_t chains, int64_t &chain, int &vb) {
    const int64_t q = id / kXCD;
    vb = (int)(q % NVB);
    chain = id % kXCD + kXCD * (q / NVB);
    return chain < chains;
}

int64_t chain_grid(int64_t chains, int nvb) { return (chains + kXCD - 1) / kXCD * kXCD * nvb; }

template <int NS> struct SpanRegs {
    f32x4_t r[NS];
    __device__ __forceinline__ void load(const float *__restrict__ span, int lt) {
#pragma unroll
        for (int s = 0; s < NS; ++s) r[s] = *reinterpret_cast<const f32x4_t *>(span + 4 * (lt + kLT * s));
    }
};

// Writes float4 number fl of a [rows][COLS] block into an LDS array of row stride LS.
template <int COLS, int LS>
__device__ __forceinline__ void put4(float *dst, int fl, const f32x4_t &x) {
    *reinterpret_cast<f32x4_t *>(dst + (fl / (COLS / 4)) * LS + (fl % (COLS / 4)) * 4) = x;
}

// The per-channel factors and the flag: floats [EM, EM + 3 DK + 4) of a record.
template <int DK> struct ColRegs {
    f32x4_t r;
    __device__ __forceinline__ void load(const float *__restrict__ rec, int lt) {
        if (lt < 3 * DK / 4 + 1) r = *reinterpret_cast<const f32x4_t *>(rec + BRec<DK>::EM + 4 * lt);
    }
    __device__ __forceinline__ void store(float *cv, int lt) const {
        if (lt < 3 * DK / 4 + 1) *reinterpret_cast<f32x4_t *>(cv + 4 * lt) = r;
    }
};

// acc += A diag(bs) B over one 16x16 tile (B's rows scaled by bs), k mapped as in mm.
template <int K, int AI, int AK, int BK, int BJ>
__device__ __forceinline__ f32x4_t mm_bs(f32x4_t acc, const float *a, const float *b, const float *bs, int lane) {
    static_assert(K % 16 == 0, "K must be a multiple of 16");
    constexpr int NG = K / 16;
    const float *pa = a + (lane & 15) * AI + 4 * (lane >> 4) * AK;
    const float *pb = b + 4 * (lane >> 4) * BK + (lane & 15) * BJ;
    const float *ps = bs + 4 * (lane >> 4);
    f32x4_t av[NG], bv[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        av[g] = k4<AK>(pa + 16 * g * AK);
        bv[g] = k4<BK>(pb + 16 * g * BK) * k4<1>(ps + 16 * g);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma4(av[g][u], bv[g][u], acc);
    return acc;
}

// Stores a [ROWS][BV] block held transposed in LDS (element (r, c) at
// src[c * LS + r]) to global rows of the given pitch, with NT threads.
template <int ROWS, int BV, int LS, int NT>
__device__ __forceinline__ void block_out_t(float *__restrict__ dst, size_t pitch, const float *src, int t) {
#pragma unroll
    for (int i = t; i < ROWS * BV / 4; i += NT) {
        const int r = i / (BV / 4), c = (i % (BV / 4)) * 4;
        f32x4_t x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = src[(c + e) * LS + r];
        *reinterpret_cast<f32x4_t *>(dst + (size_t)r * pitch + c) = x;
    }
}

// Blocks with the BV value columns as rows (Vt, Ut, St) are kept transposed, so
// that they are contiguous along the contraction index as B operands.
template <int DK, int BV> struct alignas(16) FwdBS {
    static constexpr int KS = DK + 4, CS = kB + 4;
    float T[kB][CS];
    float KI[kB][KS];
    float W[kB][KS];
    float Vt[BV][CS];                        // V^T block
    float beta[kB];
    float Ut[BV][CS];
    float St[BV][KS];                        // S^T block
    float cv[3 * DK + 4];                    // e^m, e^{g_n}, e^{g_n-m}, flag
};

// Forward replay of one (sequence, head, BV value columns): S at every chunk's
// start and U, from h0, walking the chunks forwards.
template <int DK, int DV, int BV, typename IO, typename GT>
__device__ __forceinline__ void fwd_state_body(FwdBS<DK, BV> &sm, int64_t id, const IO *__restrict__ v,
                                               const GT *__restrict__ beta, const float *__restrict__ h0,
                                               const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
                                               int64_t N, int64_t T, int H, int64_t nch,
                                               const float *__restrict__ recs, float *__restrict__ Sc,
                                               float *__restrict__ Uc, float *__restrict__ hT) {
    using R = BRec<DK>;
    using S = FwdBS<DK, BV>;
    constexpr int NVB = DV / BV;
    constexpr int ST = kB * kB / 4 / kLT, SK = kB * DK / 4 / kLT;
    static_assert(ST * kLT * 4 == kB * kB && SK * kLT * 4 == kB * DK, "span slots");
    int64_t chain;
    int vb;
    if (!chain_of<NVB>(id, (int64_t)N * H, chain, vb)) return;
    const int h = (int)(chain % H);
    const int64_t n = chain / H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool loader = tid >= kSP - kLT;
    const int lt = tid - (kSP - kLT);
    const int j0 = vb * BV;
    int64_t bos, eos, slot0;
    seq_range(n, cu, chunk_off, T, bos, eos, slot0);
    const int nchunks = (int)((eos - bos + kB - 1) / kB);

    for (int i = tid; i < DK * BV; i += kSP) {
        const int c = i / BV, j = i % BV;
        sm.St[j][c] = h0 ? h0[(((size_t)n * H + h) * DK + c) * DV + j0 + j] : 0.f;
    }
    // Loader schedule per chunk: at the boundary, T, W, the factors, V and beta
    // go into LDS; during the U products KI goes in (it is first read by the
    // state update), the next chunk's T, W, V, beta and factors are requested and
    // the start state is stored; during the state update the next KI is
    // requested and U is stored.
    SpanRegs<ST> pT;
    SpanRegs<SK> pW, pK;
    ColRegs<DK> pc;
    Stage<kB, BV, kLT, IO> pv;
    float pb = 0.f;
    auto rec_of = [&](int ci) { return recs + ((size_t)h * nch + slot0 + ci) * R::FLOATS; };
    auto fetch_a = [&](int ci) {
        const int64_t t0 = bos + (int64_t)kB * ci;
        const int nv = (int)(eos - t0 < kB ? eos - t0 : kB);
        const float *rec = rec_of(ci);
        pT.load(rec + R::T, lt);
        pW.load(rec + R::W, lt);
        pc.load(rec, lt);
        pv.load(v + ((size_t)t0 * H + h) * DV + j0, (size_t)H * DV, nv, lt);
        const int r = lt - (kLT - kB);
        if (r >= 0) pb = r < nv ? to_f32(beta[(t0 + r) * H + h]) : 0.f;
    };
    if (loader && nchunks > 0) {
        fetch_a(0);
        pK.load(rec_of(0) + R::KI, lt);
    }
    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t slot = slot0 + ci;
        if (loader) {
#pragma unroll
            for (int s = 0; s < ST; ++s) put4<kB, S::CS>(&sm.T[0][0], lt + kLT * s, pT.r[s]);
#pragma unroll
            for (int s = 0; s < SK; ++s) put4<DK, S::KS>(&sm.W[0][0], lt + kLT * s, pW.r[s]);
            pc.store(sm.cv, lt);
            pv.template store_t<S::CS>(&sm.Vt[0][0], lt);
            if (lt >= kLT - kB) sm.beta[lt - (kLT - kB)] = pb;
        }
        __syncthreads();
        const float *em = sm.cv, *eg = sm.cv + DK, *egm = sm.cv + 2 * DK;
        if (loader) {
#pragma unroll
            for (int s = 0; s < SK; ++s) put4<DK, S::KS>(&sm.KI[0][0], lt + kLT * s, pK.r[s]);
            if (ci + 1 < nchunks) fetch_a(ci + 1);
            block_out_t<DK, BV, S::KS, kLT>(Sc + ((size_t)h * nch + slot) * DK * DV + j0, DV, &sm.St[0][0], lt);
        } else {   // U = T diag(beta) V - W Diag(e^m) S: one row tile per wave, each 16-column tile
#pragma unroll
            for (int jt = 0; jt < BV / 16; ++jt) {
                f32x4_t a = zero4(), b = zero4();
                a = mm_bs<kB, S::CS, 1, 1, S::CS>(a, &sm.T[16 * w][0], &sm.Vt[16 * jt][0], sm.beta, lane);
                b = mm_bs<DK, S::KS, 1, 1, S::KS>(b, &sm.W[16 * w][0], &sm.St[16 * jt][0], em, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.Ut[16 * jt + acc_col(lane)][16 * w + acc_row(lane, e)] = a[e] - b[e];
            }
        }
        __syncthreads();
        if (loader) {
            if (ci + 1 < nchunks) pK.load(rec_of(ci + 1) + R::KI, lt);
            block_out_t<kB, BV, S::CS, kLT>(Uc + ((size_t)h * nch + slot) * kB * DV + j0, DV, &sm.Ut[0][0], lt);
        } else {   // S <- Diag(e^{g_n}) S + Diag(e^{g_n-m}) KI^T U
#pragma unroll
            for (int ct = w; ct < DK / 16; ct += 4) {
#pragma unroll
                for (int jt = 0; jt < BV / 16; ++jt) {
                    f32x4_t a = zero4();
                    a = mm<kB, 1, S::KS, 1, S::CS>(a, &sm.KI[0][16 * ct], &sm.Ut[16 * jt][0], lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * ct + acc_row(lane, e), j = 16 * jt + acc_col(lane);
                        sm.St[j][c] = eg[c] * sm.St[j][c] + egm[c] * a[e];
                    }
                }
            }
        }
        __syncthreads();
    }
    if (hT) {   // the state after the last chunk (the forward's h_T)
        for (int i = tid; i < DK * BV; i += kSP) {
            const int c = i / BV, j = i % BV;
            hT[(((size_t)n * H + h) * DK + c) * DV + j0 + j] = sm.St[j][c];
        }
    }
}

// Reverse state-gradient pass: same roles, chunks in reverse order.
template <int DK, int BV> struct alignas(16) RevBS {
    static constexpr int KS = DK + 4, CS = kB + 4;
    float KI[kB][KS];
    float W[kB][KS];
    float QA[kB][KS];
    float P[kB][CS];
    float dOt[BV][CS];                       // dO^T block
    float dUt[BV][CS];
    float dSt[BV][KS];                       // (dL/dS at the chunk's end)^T
    float cv[3 * DK + 4];                    // e^m, e^{g_n}, e^{g_n-m}, flag
};

template <int DK, int DV, int BV, typename IO>
__device__ __forceinline__ void rev_state_body(RevBS<DK, BV> &sm, int64_t id, const IO *__restrict__ d_o,
                                               const float *__restrict__ d_hT, const int32_t *__restrict__ cu,
                                               const int32_t *__restrict__ chunk_off, int64_t N, int64_t T, int H,
                                               int64_t nch, const float *__restrict__ recs, float *__restrict__ dSc,
                                               float *__restrict__ dUc, float *__restrict__ dh0) {
    using R = BRec<DK>;
    using S = RevBS<DK, BV>;
    constexpr int NVB = DV / BV;
    constexpr int ST = kB * kB / 4 / kLT, SK = kB * DK / 4 / kLT;
    static_assert(ST * kLT * 4 == kB * kB && SK * kLT * 4 == kB * DK, "span slots");
    int64_t chain;
    int vb;
    if (!chain_of<NVB>(id, (int64_t)N * H, chain, vb)) return;
    const int h = (int)(chain % H);
    const int64_t n = chain / H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool loader = tid >= kSP - kLT;
    const int lt = tid - (kSP - kLT);
    const int j0 = vb * BV;
    int64_t bos, eos, slot0;
    seq_range(n, cu, chunk_off, T, bos, eos, slot0);
    const int nchunks = (int)((eos - bos + kB - 1) / kB);

    for (int i = tid; i < DK * BV; i += kSP) {
        const int c = i / BV, j = i % BV;
        sm.dSt[j][c] = d_hT ? d_hT[(((size_t)n * H + h) * DK + c) * DV + j0 + j] : 0.f;
    }
    // Loader schedule per chunk: at the boundary, KI, P, the factors and dO go
    // into LDS; during the dU products QA and W go in (first read by the
    // state-gradient update), the previous chunk's KI, P, factors and dO are
    // requested and the state gradient is stored; during the update the previous
    // QA and W are requested and dU is stored.
    SpanRegs<SK> pK;
    SpanRegs<ST> pP;
    SpanRegs<2 * SK> pWQ;                    // W and QA are adjacent in the record
    ColRegs<DK> pc;
    Stage<kB, BV, kLT, IO> po;
    auto rec_of = [&](int ci) { return recs + ((size_t)h * nch + slot0 + ci) * R::FLOATS; };
    auto fetch_a = [&](int ci) {
        const int64_t t0 = bos + (int64_t)kB * ci;
        const int nv = (int)(eos - t0 < kB ? eos - t0 : kB);
        const float *rec = rec_of(ci);
        pK.load(rec + R::KI, lt);
        pP.load(rec + R::P, lt);
        pc.load(rec, lt);
        po.load(d_o + ((size_t)t0 * H + h) * DV + j0, (size_t)H * DV, nv, lt);
    };
    if (loader && nchunks > 0) {
        fetch_a(nchunks - 1);
        pWQ.load(rec_of(nchunks - 1) + R::W, lt);
    }
    for (int ci = nchunks - 1; ci >= 0; --ci) {
        const int64_t slot = slot0 + ci;
        if (loader) {
#pragma unroll
            for (int s = 0; s < SK; ++s) put4<DK, S::KS>(&sm.KI[0][0], lt + kLT * s, pK.r[s]);
#pragma unroll
            for (int s = 0; s < ST; ++s) put4<kB, S::CS>(&sm.P[0][0], lt + kLT * s, pP.r[s]);
            pc.store(sm.cv, lt);
            po.template store_t<S::CS>(&sm.dOt[0][0], lt);
        }
        __syncthreads();
        const float *em = sm.cv, *eg = sm.cv + DK, *egm = sm.cv + 2 * DK;
        if (loader) {
#pragma unroll
            for (int s = 0; s < 2 * SK; ++s) {
                if (s < SK) put4<DK, S::KS>(&sm.W[0][0], lt + kLT * s, pWQ.r[s]);
                else put4<DK, S::KS>(&sm.QA[0][0], lt + kLT * (s - SK), pWQ.r[s]);
            }
            if (ci > 0) fetch_a(ci - 1);
            block_out_t<DK, BV, S::KS, kLT>(dSc + ((size_t)h * nch + slot) * DK * DV + j0, DV, &sm.dSt[0][0], lt);
        } else {   // dU = P^T dO + KI Diag(e^{g_n-m}) dS: one row tile per wave, each 16-column tile
#pragma unroll
            for (int jt = 0; jt < BV / 16; ++jt) {
                f32x4_t a = zero4(), b = zero4();
                a = mm<kB, 1, S::CS, 1, S::CS>(a, &sm.P[0][16 * w], &sm.dOt[16 * jt][0], lane);
                b = mm_bs<DK, S::KS, 1, 1, S::KS>(b, &sm.KI[16 * w][0], &sm.dSt[16 * jt][0], egm, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.dUt[16 * jt + acc_col(lane)][16 * w + acc_row(lane, e)] = a[e] + b[e];
            }
        }
        __syncthreads();
        if (loader) {
            if (ci > 0) pWQ.load(rec_of(ci - 1) + R::W, lt);
            block_out_t<kB, BV, S::CS, kLT>(dUc + ((size_t)h * nch + slot) * kB * DV + j0, DV, &sm.dUt[0][0], lt);
        } else {   // dS <- Diag(e^m) (QA^T dO - W^T dU) + Diag(e^{g_n}) dS
#pragma unroll
            for (int ct = w; ct < DK / 16; ct += 4) {
#pragma unroll
                for (int jt = 0; jt < BV / 16; ++jt) {
                    f32x4_t a = zero4(), b = zero4();
                    a = mm<kB, 1, S::KS, 1, S::CS>(a, &sm.QA[0][16 * ct], &sm.dOt[16 * jt][0], lane);
                    b = mm<kB, 1, S::KS, 1, S::CS>(b, &sm.W[0][16 * ct], &sm.dUt[16 * jt][0], lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * ct + acc_row(lane, e), j = 16 * jt + acc_col(lane);
                        sm.dSt[j][c] = em[c] * (a[e] - b[e]) + eg[c] * sm.dSt[j][c];
                    }
                }
            }
        }
        __syncthreads();
    }
    if (dh0) {
        for (int i = tid; i < DK * BV; i += kSP) {
            const int c = i / BV, j = i % BV;
            dh0[(((size_t)n * H + h) * DK + c) * DV + j0 + j] = sm.dSt[j][c];
        }
    }
}

// The two sequential passes read only the prep kernel's records (the reverse
// pass needs neither S nor U), so they run side by side in one launch: blocks
// [0, fwd_blocks) replay forwards, the rest walk backwards.  With kSBV value
// columns per workgroup each pass has half as many workgroups as with 16, and
// at the long-context shape both fit the chip at once.
constexpr int kSBV = 32;
template <int DK, int BV> union StateBS {
    FwdBS<DK, BV> f;
    RevBS<DK, BV> r;
};

template <int DK, int DV, int BV, typename IO, typename GT>
__global__ __launch_bounds__(kSP) void bwd_state_kernel(const IO *__restrict__ v, const GT *__restrict__ beta,
                                                        const float *__restrict__ h0, const IO *__restrict__ d_o,
                                                        const float *__restrict__ d_hT, const int32_t *__restrict__ cu,
                                                        const int32_t *__restrict__ chunk_off, int64_t N, int64_t T,
                                                        int H, int64_t nch, const float *__restrict__ recs,
                                                        float *__restrict__ Sc, float *__restrict__ Uc,
                                                        float *__restrict__ dSc,
                                                        float *__restrict__ dUc, float *__restrict__ dh0,
                                                        int64_t fwd_blocks, float *__restrict__ hT) {
    __shared__ StateBS<DK, BV> sm;
    const int64_t id = blockIdx.x;
    if (id < fwd_blocks)
        fwd_state_body<DK, DV, BV, IO, GT>(sm.f, id, v, beta, h0, cu, chunk_off, N, T, H, nch, recs, Sc, Uc, hT);
    else
        rev_state_body<DK, DV, BV, IO>(sm.r, id - fwd_blocks, d_o, d_hT, cu, chunk_off, N, T, H, nch, recs, dSc, dUc,
                                       dh0);
}

// ----------------------------------------------------------------------------
// Gradient kernel: one workgroup of 8 waves per (chunk, head).
template <int DK> struct alignas(16) GradBS {
    static constexpr int KS = DK + 4, CS = kB + 4, VS = kBV + 4;
    float KA[kB][KS];
    union {
        struct {
            float T[kB][CS];                 // loop: (I + A)^{-1}; after: dP
            float dM[kB][CS];
        } m;
        float G2[kB][DK];                    // in-chunk log2-decay cumsum, at the end
    } r2;
    union {
        struct {
            float dO[kB][VS], U[kB][VS], dU[kB][VS], V[kB][VS], dY[kB][VS];
            float Sp[DK][VS], dSn[DK][VS];
        } lp;
        struct {
            float QA[kB][KS];                // then dG
            float KI[kB][KS];                // then (U dS_next^T) . KI
        } pt;
    } r3;
    float beta[kB];                          // beta, or the erase strengths b
    float wv[kB];                            // the write strengths w (separate strengths only)
    float gv[kB];                            // log alpha per row (scalar-gate layouts)
    float dbr[kB];
    float dbA[4][kB];
    float m2[DK], em[DK], eg[DK], egm[DK];
    float part[kSeg][DK], partk[kSeg][DK];   // segment totals of the column scans
    float dgn1[DK];
    float dbK[DK / 16][kB];                  // per key tile: sum_c KA (dY S'^T) of a row
};

// KT: the type of k, dq and dk (the io type, or fp32 with bf16 v and dO when
// the input prologue's fp32 mapped q and k are the inputs).
template <int DK, int DV, typename IO, typename GT, typename KT, int GM>
__global__ __launch_bounds__(512) void bwd_grad_kernel(
    const KT *__restrict__ q, const KT *__restrict__ k, const IO *__restrict__ v, const GT *__restrict__ log_alpha,
    const GT *__restrict__ beta, const IO *__restrict__ d_o, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int64_t N, int64_t T, int H, int64_t nch, const float *__restrict__ recs,
    const float *__restrict__ Sc, const float *__restrict__ Uc, const float *__restrict__ dSc,
    const float *__restrict__ dUc, KT *__restrict__ dq, KT *__restrict__ dk,
    IO *__restrict__ dv, GT *__restrict__ dla, GT *__restrict__ dbeta, const GT *__restrict__ wr,
    GT *__restrict__ dwr) {
    using R = BRec<DK>;
    using S = GradBS<DK>;
    __shared__ S sm;
    const int64_t chunk = blockIdx.x;
    const int h = blockIdx.y;
    int64_t n, t0;
    int nv;
    if (!locate_chunk(chunk, cu, chunk_off, N, T, n, t0, nv)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float *rec = recs + ((size_t)h * nch + chunk) * R::FLOATS;
    const size_t ch = (size_t)h * nch + chunk;
    const bool exact = rec[R::FLAG] != 0.f;  // the chunk's mode, as the prep kernel chose it
    constexpr int NCT = DK / 16;             // key-column tiles
    constexpr int NOWN = 4 * NCT / 8;        // (row, key) tiles per wave

    if (tid < kB) {
        sm.beta[tid] = tid < nv ? to_f32(beta[(t0 + tid) * H + h]) : 0.f;
        sm.wv[tid] = (wr && tid < nv) ? to_f32(wr[(t0 + tid) * H + h]) : 0.f;
        sm.dbr[tid] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.dbA[i][tid] = 0.f;
    }
    float dgn1 = 0.f;                        // thread c < DK: sum_j dS_next[c,j] S'[c,j]
    {   // k and log alpha staged through the (still free) loop area; T from the record
        const size_t base = ((size_t)t0 * H + h) * DK, pitch = (size_t)H * DK;
        Stage<kB, DK, 512, KT> sk;
        Stage<kB, DK, 512, GT> sl;
        Stage<kB, kB, 512, float> st;
        sk.load(k + base, pitch, nv, tid);
        if constexpr (GM == kGatePerChannel) sl.load(log_alpha + base, pitch, nv, tid);
        st.load(rec + R::T, kB, kB, tid);
        sk.template store<S::KS>(&sm.r3.pt.QA[0][0], tid);
        if constexpr (GM == kGatePerChannel) sl.template store<S::KS>(&sm.r3.pt.KI[0][0], tid);
        else load_gate_rows<GM>(sm.gv, log_alpha, t0, H, h, nv, tid);
        st.template store<S::CS>(&sm.r2.m.T[0][0], tid);
    }
    __syncthreads();
    const int sc_c = tid % DK, sc_p = tid / DK;   // column-scan roles: channel, segment
    if (tid < DK) {
        sm.em[tid] = rec[R::EM + tid];
        sm.eg[tid] = rec[R::EG + tid];
        sm.egm[tid] = rec[R::EGM + tid];
    }
    if (sc_p < kSeg) {   // G (log2 units), as the prep kernel forms it: segment totals
        const int r0 = sc_p * kSegRows, r1 = min(r0 + kSegRows, nv);
        float l = 0.f;
        for (int r = r0; r < r1; ++r) l += (GM == kGatePerChannel ? sm.r3.pt.KI[r][sc_c] : sm.gv[r]) * kBL2E;
        sm.part[sc_p][sc_c] = l;
    }
    __syncthreads();
    if (sc_p < kSeg) {   // then KA = K e^{G - m} per segment
        const int c = sc_c;
        float g2 = 0.f, pre = 0.f;
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            g2 += sm.part[i][c];
            if (i < sc_p) pre += sm.part[i][c];
        }
        // anchors: m = g_n / 2 for both factors; in exact mode none for K e^G and
        // g_n for K e^{g_n - G} (m2 holds the latter)
        const float m2 = exact ? 0.f : 0.5f * g2;
        if (sc_p == 0) sm.m2[c] = exact ? g2 : m2;
        const int r0 = sc_p * kSegRows, r1 = min(r0 + kSegRows, nv);
        float l = 0.f;
        for (int r = r0; r < kSegRows + r0; ++r) {
            float ka = 0.f;
            if (r < r1) {
                l += (GM == kGatePerChannel ? sm.r3.pt.KI[r][c] : sm.gv[r]) * kBL2E;
                ka = sm.r3.pt.QA[r][c] * __builtin_amdgcn_exp2f((pre + l) - m2);
            }
            sm.KA[r][c] = ka;
        }
    }

    f32x4_t aQ[NOWN], aK[NOWN], aB[NOWN];    // dQA, dY S'^T, U dS_next^T
#pragma unroll
    for (int s = 0; s < NOWN; ++s) aQ[s] = aK[s] = aB[s] = zero4();
    f32x4_t aL[3];                           // lower tiles: idx < 10 dP, else dY U^T
#pragma unroll
    for (int s = 0; s < 3; ++s) aL[s] = zero4();
    f32x4_t dbp = zero4();                   // waves 4-7: the dY.V part of dbeta

    const float *sc = Sc + ch * DK * DV;
    const float *uc = Uc + ch * kB * DV;
    const float *dsc = dSc + ch * DK * DV;
    const float *duc = dUc + ch * kB * DV;

    // The next 16-column block's operands are requested (into registers) before
    // the current block's products.
    Stage<kB, kBV, 512, IO> pO, pV;
    Stage<kB, kBV, 512, float> pU, pdU;
    Stage<DK, kBV, 512, float> pS, pdS;
    auto fetch = [&](int vb) {
        const int j0 = vb * kBV;
        const size_t tb = ((size_t)t0 * H + h) * DV + j0, tp = (size_t)H * DV;
        pO.load(d_o + tb, tp, nv, tid);
        pV.load(v + tb, tp, nv, tid);
        pU.load(uc + j0, DV, kB, tid);
        pdU.load(duc + j0, DV, kB, tid);
        pS.load(sc + j0, DV, DK, tid);
        pdS.load(dsc + j0, DV, DK, tid);
    };
    fetch(0);
    for (int vb = 0; vb < DV / kBV; ++vb) {
        const int j0 = vb * kBV;
        __syncthreads();                     // previous block's reads done
        pO.template store<S::VS>(&sm.r3.lp.dO[0][0], tid);
        pV.template store<S::VS>(&sm.r3.lp.V[0][0], tid);
        pU.template store<S::VS>(&sm.r3.lp.U[0][0], tid);
        pdU.template store<S::VS>(&sm.r3.lp.dU[0][0], tid);
        pS.template store<S::VS>(&sm.r3.lp.Sp[0][0], tid, sm.em);
        pdS.template store<S::VS>(&sm.r3.lp.dSn[0][0], tid);
        __syncthreads();
        if (vb + 1 < DV / kBV) fetch(vb + 1);
        if (w >= 4) {   // dY = T^T dU; dV = diag(beta) dY; the dY.V part of dbeta
            const int rt = w - 4;
            f32x4_t a = zero4();
            a = mm<kB, 1, S::CS, S::VS, 1>(a, &sm.r2.m.T[0][16 * rt], &sm.r3.lp.dU[0][0], lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + acc_row(lane, e), j = acc_col(lane);
                sm.r3.lp.dY[r][j] = a[e];
                dbp[e] += a[e] * sm.r3.lp.V[r][j];
                if (r < nv) dv[((t0 + r) * H + h) * DV + j0 + j] = from_f32<IO>((wr ? sm.wv[r] : sm.beta[r]) * a[e]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int idx = w + 8 * s;
            if (idx < 20) {
                int Rt, It;
                low_tile(idx % 10, Rt, It);
                const float *a = idx < 10 ? &sm.r3.lp.dO[16 * Rt][0] : &sm.r3.lp.dY[16 * Rt][0];
                aL[s] = mm<kBV, S::VS, 1, 1, S::VS>(aL[s], a, &sm.r3.lp.U[16 * It][0], lane);
            }
        }
#pragma unroll
        for (int s = 0; s < NOWN; ++s) {
            const int ti = w + 8 * s, rt = ti / NCT, ct = ti % NCT;
            aQ[s] = mm<kBV, S::VS, 1, 1, S::VS>(aQ[s], &sm.r3.lp.dO[16 * rt][0], &sm.r3.lp.Sp[16 * ct][0], lane);
            aK[s] = mm<kBV, S::VS, 1, 1, S::VS>(aK[s], &sm.r3.lp.dY[16 * rt][0], &sm.r3.lp.Sp[16 * ct][0], lane);
            aB[s] = mm<kBV, S::VS, 1, 1, S::VS>(aB[s], &sm.r3.lp.U[16 * rt][0], &sm.r3.lp.dSn[16 * ct][0], lane);
        }
        if (tid < DK) {
#pragma unroll
            for (int j = 0; j < kBV; ++j) dgn1 += sm.r3.lp.dSn[tid][j] * sm.r3.lp.Sp[tid][j];
        }
    }
    __syncthreads();                         // loop buffers and T free

    // dbeta_r = sum_j dY[r,j] X[r,j] with X = V - KA S', taken as
    // sum_j dY[r,j] V[r,j] - sum_c KA[r,c] (dY S'^T)[r,c]: the first part here
    // (a sum over the 16 columns of each tile row), the second below.
    if (w >= 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = dbp[e];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            if ((lane & 15) == 0) sm.dbr[16 * (w - 4) + acc_row(lane, e)] = x;
        }
    }
    // dP (inclusive lower) and dM = diag(beta) dA, dA = -strictly-lower(dY U^T).
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int idx = w + 8 * s;
        if (idx < 20) {
            int Rt, It;
            low_tile(idx % 10, Rt, It);
            const bool isA = idx >= 10;
            float rowsum[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * Rt + acc_row(lane, e), c = 16 * It + acc_col(lane);
                if (!isA) {
                    sm.r2.m.T[r][c] = r >= c ? aL[s][e] : 0.f;     // dP
                    rowsum[e] = 0.f;
                } else {
                    const float dA = r > c ? -aL[s][e] : 0.f;
                    sm.r2.m.dM[r][c] = sm.beta[r] * dA;
                    rowsum[e] = dA * rec[R::M + r * kB + c];
                }
            }
            if (isA) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = rowsum[e];
                    x += __shfl_xor(x, 1);
                    x += __shfl_xor(x, 2);
                    x += __shfl_xor(x, 4);
                    x += __shfl_xor(x, 8);
                    if ((lane & 15) == 0) sm.dbA[It][16 * Rt + acc_row(lane, e)] = x;
                }
            }
        }
    }
    // Upper blocks of dP and dM are never written above: clear them.
    for (int i = tid; i < kB * kB; i += 512) {
        const int r = i / kB, c = i % kB;
        if ((c >> 4) > (r >> 4)) {
            sm.r2.m.T[r][c] = 0.f;
            sm.r2.m.dM[r][c] = 0.f;
        }
    }
    if (!exact) {   // the record's QA and KI
        Stage<kB, DK, 512, float> sq, si;
        sq.load(rec + R::QA, DK, kB, tid);
        si.load(rec + R::KI, DK, kB, tid);
        sq.template store<S::KS>(&sm.r3.pt.QA[0][0], tid);
        si.template store<S::KS>(&sm.r3.pt.KI[0][0], tid);
    } else {        // exact mode: k and q themselves (QA and KI areas)
        const size_t base = ((size_t)t0 * H + h) * DK, pitch = (size_t)H * DK;
        Stage<kB, DK, 512, KT> sk, sq;
        sk.load(k + base, pitch, nv, tid);
        sq.load(q + base, pitch, nv, tid);
        sk.template store<S::KS>(&sm.r3.pt.QA[0][0], tid);
        sq.template store<S::KS>(&sm.r3.pt.KI[0][0], tid);
    }
    __syncthreads();

    f32x4_t aI[NOWN];                        // dKI
#pragma unroll
    for (int s = 0; s < NOWN; ++s) {
        const int ti = w + 8 * s, rt = ti / NCT, ct = ti % NCT;
        const float *dP = &sm.r2.m.T[0][0];
        const float *dM = &sm.r2.m.dM[0][0];
        if (!exact) aQ[s] = mm<kB, S::CS, 1, S::KS, 1>(aQ[s], dP + 16 * rt * S::CS, &sm.r3.pt.KI[0][16 * ct], lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // sum_c KA[r,c] (dY S'^T)[r,c] over this tile's 16 columns
            float x = sm.KA[16 * rt + acc_row(lane, e)][16 * ct + acc_col(lane)] * aK[s][e];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            if ((lane & 15) == 0) sm.dbK[ct][16 * rt + acc_row(lane, e)] = x;
        }
        // the intra-chunk parts (dM KI, dP^T QA + dM^T KA) on the matrix cores;
        // in exact mode they are formed pair by pair below
        f32x4_t t = zero4(), u = zero4();
        if (!exact) {
            t = mm<kB, S::CS, 1, S::KS, 1>(t, dM + 16 * rt * S::CS, &sm.r3.pt.KI[0][16 * ct], lane);
            u = mm<kB, 1, S::CS, S::KS, 1>(u, dP + 16 * rt, &sm.r3.pt.QA[0][16 * ct], lane);
            u = mm<kB, 1, S::CS, S::KS, 1>(u, dM + 16 * rt, &sm.KA[0][16 * ct], lane);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) aK[s][e] = t[e] - sm.beta[16 * rt + acc_row(lane, e)] * aK[s][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] += sm.egm[16 * ct + acc_col(lane)] * aB[s][e];
        aI[s] = u;
    }
    __syncthreads();                         // dP, dM, QA, KI reads done (exact mode: KA's)

    // G (log2 units) again: into the freed area, or in exact mode (where dP and
    // dM are still needed) over KA
    float *Gp = exact ? &sm.KA[0][0] : &sm.r2.G2[0][0];
    const int gl = exact ? S::KS : DK;
    if constexpr (GM == kGatePerChannel) {
        Stage<kB, DK, 512, GT> sl;
        sl.load(log_alpha + ((size_t)t0 * H + h) * DK, (size_t)H * DK, nv, tid);
        if (exact) sl.template store<S::KS>(Gp, tid);
        else sl.template store<DK>(Gp, tid);
    }
    __syncthreads();
    if (sc_p < kSeg) {   // segment totals, then G in place (as above)
        const int r0 = sc_p * kSegRows, r1 = min(r0 + kSegRows, nv);
        float l = 0.f;
        for (int r = r0; r < r1; ++r) l += (GM == kGatePerChannel ? Gp[r * gl + sc_c] : sm.gv[r]) * kBL2E;
        sm.part[sc_p][sc_c] = l;
    }
    __syncthreads();
    if (sc_p < kSeg) {
        float pre = 0.f;
#pragma unroll
        for (int i = 0; i < kSeg; ++i)
            if (i < sc_p) pre += sm.part[i][sc_c];
        const int r0 = sc_p * kSegRows, r1 = min(r0 + kSegRows, nv);
        float l = 0.f;
        for (int r = r0; r < r1; ++r) {
            l += (GM == kGatePerChannel ? Gp[r * gl + sc_c] : sm.gv[r]) * kBL2E;
            Gp[r * gl + sc_c] = pre + l;
        }
    }
    __syncthreads();
    if (!exact) {
#pragma unroll
        for (int s = 0; s < NOWN; ++s) {
            const int ti = w + 8 * s, rt = ti / NCT, ct = ti % NCT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + acc_row(lane, e), c = 16 * ct + acc_col(lane);
                float dG = 0.f, kb = 0.f;
                if (r < nv) {
                    const float g = sm.r2.G2[r][c] - sm.m2[c];
                    const float ea = __builtin_amdgcn_exp2f(g), ei = __builtin_amdgcn_exp2f(-g);
                    const size_t o = ((t0 + r) * H + h) * DK + c;
                    const float ki = sm.r3.pt.KI[r][c];
                    dq[o] = from_f32<KT>(aQ[s][e] * ea);
                    dk[o] = from_f32<KT>(aK[s][e] * ea + aI[s][e] * ei);
                    dG = aQ[s][e] * sm.r3.pt.QA[r][c] + aK[s][e] * sm.KA[r][c] - aI[s][e] * ki;
                    kb = aB[s][e] * ki;
                }
                sm.r3.pt.QA[r][c] = dG;
                sm.r3.pt.KI[r][c] = kb;
            }
        }
    } else {
        // Exact mode.  With E(r, i) = e^{G_rc - G_ic} <= 1 (i <= r) per channel c,
        // the intra-chunk products P = sum_c q_r k_i E and M = sum_c k_r k_i E
        // (i < r) give, for this element (r, c):
        //   dq_x  = sum_{i<=r} dP[r,i] k_i E(r,i)
        //   dk_r  = sum_{i<r}  dM[r,i] k_i E(r,i)
        //   dk_i  = sum_{j>=r} (dP[j,r] q_j + dM[j,r] k_j) E(j,r)
        //   dG_x  = q_r dq_x + k_r dk_r - k_r dk_i
        // and the state-side operands are Q e^G, K e^G, K e^{g_n - G} (no anchor).
        const float *dP = &sm.r2.m.T[0][0];
        const float *dM = &sm.r2.m.dM[0][0];
        const float *kk = &sm.r3.pt.QA[0][0];
        const float *qq = &sm.r3.pt.KI[0][0];
        float xg[NOWN][4], xb[NOWN][4];
#pragma unroll
        for (int s = 0; s < NOWN; ++s) {
            const int ti = w + 8 * s, rt = ti / NCT, ct = ti % NCT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + acc_row(lane, e), c = 16 * ct + acc_col(lane);
                float dG = 0.f, kb = 0.f;
                if (r < nv) {
                    const float Gr = Gp[r * gl + c];
                    float dqx = 0.f, dkr = 0.f, dki = 0.f;
                    for (int i = 0; i <= r; ++i) {
                        const float ki = kk[i * S::KS + c] * __builtin_amdgcn_exp2f(Gr - Gp[i * gl + c]);
                        dqx += dP[r * S::CS + i] * ki;
                        dkr += dM[r * S::CS + i] * ki;
                    }
                    for (int j = r; j < nv; ++j) {
                        const float x = dP[j * S::CS + r] * qq[j * S::KS + c] + dM[j * S::CS + r] * kk[j * S::KS + c];
                        dki += x * __builtin_amdgcn_exp2f(Gp[j * gl + c] - Gr);
                    }
                    const float ea = __builtin_amdgcn_exp2f(Gr), ei = __builtin_amdgcn_exp2f(sm.m2[c] - Gr);
                    const float kr = kk[r * S::KS + c], qr = qq[r * S::KS + c];
                    const size_t o = ((t0 + r) * H + h) * DK + c;
                    dq[o] = from_f32<KT>(aQ[s][e] * ea + dqx);
                    dk[o] = from_f32<KT>(aK[s][e] * ea + aI[s][e] * ei + dkr + dki);
                    dG = aQ[s][e] * (qr * ea) + aK[s][e] * (kr * ea) - aI[s][e] * (kr * ei) + qr * dqx + kr * dkr -
                         kr * dki;
                    kb = aB[s][e] * (kr * ei);
                }
                xg[s][e] = dG;
                xb[s][e] = kb;
            }
        }
        __syncthreads();   // k and q no longer read
#pragma unroll
        for (int s = 0; s < NOWN; ++s) {
            const int ti = w + 8 * s, rt = ti / NCT, ct = ti % NCT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + acc_row(lane, e), c = 16 * ct + acc_col(lane);
                sm.r3.pt.QA[r][c] = xg[s][e];
                sm.r3.pt.KI[r][c] = xb[s][e];
            }
        }
    }
    __syncthreads();
    if (sc_p < kSeg) {   // segment totals of dG and of the KI-weighted U dS_next^T
        const int r0 = sc_p * kSegRows;
        float d = 0.f, kb = 0.f;
        for (int r = r0; r < r0 + kSegRows; ++r) {
            d += sm.r3.pt.QA[r][sc_c];
            kb += sm.r3.pt.KI[r][sc_c];
        }
        sm.part[sc_p][sc_c] = d;
        sm.partk[sc_p][sc_c] = kb;
    }
    if (tid < DK) sm.dgn1[tid] = dgn1;
    if (tid < kB && tid < nv) {
        const int r = tid;
        float kx = 0.f;
#pragma unroll
        for (int i = 0; i < DK / 16; ++i) kx += sm.dbK[i][r];
        const float ma = (sm.dbA[0][r] + sm.dbA[1][r]) + (sm.dbA[2][r] + sm.dbA[3][r]);
        if (wr) {   // separate strengths: the V term is the write strength's, the rest the erase's
            dwr[(t0 + r) * H + h] = from_f32<GT>(sm.dbr[r]);
            dbeta[(t0 + r) * H + h] = from_f32<GT>(ma - kx);
        } else {
            const float x = (sm.dbr[r] - kx) + ma;
            dbeta[(t0 + r) * H + h] = from_f32<GT>(x);
        }
    }
    __syncthreads();
    if (sc_p < kSeg) {   // dlog alpha: reverse cumsum of dG plus dg_n
        const int c = sc_c;
        float kbs = 0.f, suf = 0.f;
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            kbs += sm.partk[i][c];
            if (i > sc_p) suf += sm.part[i][c];
        }
        // dg_n = e^{g_n} sum_j dS_next S + e^{g_n - m} sum_r (U dS_next^T) KI, with
        // dgn1 = sum_j dS_next S' and S' = e^m S (m = 0 in exact mode)
        const float dgn = exact ? sm.eg[c] * sm.dgn1[c] + sm.egm[c] * kbs : sm.egm[c] * (sm.dgn1[c] + kbs);
        const int r0 = sc_p * kSegRows, r1 = min(r0 + kSegRows, nv);
        float sacc = suf;
        for (int r = r1 - 1; r >= r0; --r) {
            sacc += sm.r3.pt.QA[r][c];
            if constexpr (GM == kGatePerChannel) dla[((t0 + r) * H + h) * DK + c] = from_f32<GT>(sacc + dgn);
            else sm.r2.G2[r][c] = sacc + dgn;   // G2 is free: summed over the channels below
        }
    }
    if constexpr (GM == kGatePerHead) {
        // one gate shared by every key channel: its gradient is the channel sum,
        // 8 threads per row over DK / 8 channels each, then an xor butterfly
        // across the 8 (a fixed order: deterministic)
        __syncthreads();
        const int r = tid >> 3, sub = tid & 7;
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < DK / 8; ++i) x += sm.r2.G2[r][sub * (DK / 8) + i];
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 1);
        if (sub == 0 && r < nv) dla[(t0 + r) * H + h] = from_f32<GT>(x);
    }
}

template <int DK, int DV, typename IO, typename GT, typename KT = IO, int GM = kGatePerChannel>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
    const BwdLayout L = bwd_layout(a);
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    int32_t *chunk_off = a.varlen ? reinterpret_cast<int32_t *>(ws + L.plan) : nullptr;
    float *recs = reinterpret_cast<float *>(ws + L.rec);
    float *Sc = reinterpret_cast<float *>(ws + L.sc);
    float *Uc = reinterpret_cast<float *>(ws + L.uc);
    float *dSc = reinterpret_cast<float *>(ws + L.dsc);
    float *dUc = reinterpret_cast<float *>(ws + L.duc);
    const KT *q = static_cast<const KT *>(a.q), *k = static_cast<const KT *>(a.k);
    const IO *v = static_cast<const IO *>(a.v);
    const GT *la = static_cast<const GT *>(a.log_alpha), *be = static_cast<const GT *>(a.beta);
    const GT *wr = static_cast<const GT *>(a.w_write);     // separate write strengths, or NULL
    const IO *dO = static_cast<const IO *>(a.d_o);
    const int64_t T = a.seq_len;
    if (a.varlen)
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.num_seqs, chunk_off);
    if (L.nch > 0 && a.total_tokens > 0)
        hipLaunchKernelGGL((bwd_prep_kernel<DK, KT, GT, GM>), dim3((unsigned)L.nch, (unsigned)a.H), dim3(256), 0, st, q, k,
                           la, be, a.cu_seqlens, chunk_off, a.num_seqs, T, a.H, L.nch, recs);
    const int64_t grid = chain_grid(a.num_seqs * a.H, DV / kSBV);   // per pass (a multiple of 8)
    if (grid > 0) {
        const int64_t fb = a.total_tokens > 0 ? grid : 0;   // no replay without tokens
        // the replay's U takes the write strengths (beta when they are tied)
        hipLaunchKernelGGL((bwd_state_kernel<DK, DV, kSBV, IO, GT>), dim3((unsigned)(fb + grid)), dim3(kSP), 0, st, v,
                           wr ? wr : be, a.h0, dO, a.d_hT, a.cu_seqlens, chunk_off, a.num_seqs, T, a.H, L.nch, recs,
                           Sc, Uc, dSc, dUc, a.dh0, fb, nullptr);
    }
    if (L.nch > 0 && a.total_tokens > 0)
        hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, IO, GT, KT, GM>), dim3((unsigned)L.nch, (unsigned)a.H), dim3(512), 0, st,
                           q, k, v, la, be, dO, a.cu_seqlens, chunk_off, a.num_seqs, T, a.H, L.nch, recs, Sc, Uc,
                           dSc, dUc, static_cast<KT *>(a.dq), static_cast<KT *>(a.dk), static_cast<IO *>(a.dv),
                           static_cast<GT *>(a.dlog_alpha), static_cast<GT *>(a.dbeta), wr,
                           static_cast<GT *>(a.dw_write));
    return hipGetLastError();
}

template <int DK, int DV, int GM>
hipError_t launch_bwd_gm(const BwdArgs &a, hipStream_t st) {
    if (a.io_bf16)
        return a.gate_bf16 ? launch_bwd_t<DK, DV, bf16_t, bf16_t, bf16_t, GM>(a, st)
                           : launch_bwd_t<DK, DV, bf16_t, float, bf16_t, GM>(a, st);
    return a.gate_bf16 ? launch_bwd_t<DK, DV, float, bf16_t, float, GM>(a, st)
                       : launch_bwd_t<DK, DV, float, float, float, GM>(a, st);
}

template <int DK, int DV>
hipError_t launch_bwd_dims(const BwdArgs &a, hipStream_t st) {
    // scalar gates (Gated DeltaNet) or none (DeltaNet)
    if (a.gate_mode == kGatePerHead) return launch_bwd_gm<DK, DV, kGatePerHead>(a, st);
    if (a.gate_mode == kGateNone) return launch_bwd_gm<DK, DV, kGateNone>(a, st);
    // the input prologue's pass: fp32 mapped q, k and gates with bf16 v and dO
    if (a.qk_f32 && a.io_bf16) return launch_bwd_t<DK, DV, bf16_t, float, float>(a, st);
    if (a.io_bf16)
        return a.gate_bf16 ? launch_bwd_t<DK, DV, bf16_t, bf16_t>(a, st) : launch_bwd_t<DK, DV, bf16_t, float>(a, st);
    return a.gate_bf16 ? launch_bwd_t<DK, DV, float, bf16_t>(a, st) : launch_bwd_t<DK, DV, float, float>(a, st);
}

// ----------------------------------------------------------------------------
// Raw projections (the input prologue's entry point): the maps are applied in a
// pass of their own, into fp32 buffers; the backward runs on the mapped inputs;
// a last pass takes the chain rule back through the maps.  One wave per
// (token, head) row, DK / 64 channels per lane.
//   map:   q_hat = q / max(||q||, eps) (k likewise), log alpha =
//          max(-softplus(a), lo), beta = sigmoid(b); the row's 1 / max(||.||,
//          eps) kept, negated when ||.|| <= eps (then x_hat = x / eps);
//   chain: dq = (dq_hat - q_hat (q_hat . dq_hat)) / ||q||, or dq_hat / eps;
//          da = -sigmoid(a) dlog_alpha where the floor does not bind, else 0;
//          db = beta (1 - beta) dbeta.
template <int DK, typename IO, typename GT>
__global__ __launch_bounds__(256) void pro_map_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                                                      const GT *__restrict__ a, const GT *__restrict__ b, int64_t rows,
                                                      float lo, float *__restrict__ qh, float *__restrict__ kh,
                                                      float *__restrict__ la, float *__restrict__ be,
                                                      float *__restrict__ inq, float *__restrict__ ink) {
    constexpr int CPL = DK / 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;                 // the whole wave: one row per wave
    float qv[CPL], kv[CPL], sq = 0.f, sk = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        const int64_t o = row * DK + lane * CPL + cc;
        qv[cc] = to_f32(q[o]);
        kv[cc] = to_f32(k[o]);
        sq += qv[cc] * qv[cc];
        sk += kv[cc] * kv[cc];
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    const float iq = pro_inv_norm(sq), ik = pro_inv_norm(sk);
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        const int64_t o = row * DK + lane * CPL + cc;
        qh[o] = qv[cc] * iq;
        kh[o] = kv[cc] * ik;
        la[o] = pro_log_alpha(to_f32(a[o]), lo);
    }
    if (lane == 0) {
        const float e2 = kPrologueEps * kPrologueEps;
        be[row] = pro_beta(to_f32(b[row]));
        inq[row] = sq > e2 ? iq : -iq;
        ink[row] = sk > e2 ? ik : -ik;
    }
}

template <int DK, typename IO, typename GT>
__global__ __launch_bounds__(256) void pro_chain_kernel(
    const float *__restrict__ qh, const float *__restrict__ kh, const float *__restrict__ inq,
    const float *__restrict__ ink, const GT *__restrict__ a, const float *__restrict__ be, float lo,
    const float *__restrict__ dqh, const float *__restrict__ dkh, const float *__restrict__ dla,
    const float *__restrict__ dbe, int64_t rows, IO *__restrict__ dq, IO *__restrict__ dk, GT *__restrict__ da,
    GT *__restrict__ db) {
    constexpr int CPL = DK / 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        const int64_t o = row * DK + lane * CPL + cc;
        pq += qh[o] * dqh[o];
        pk += kh[o] * dkh[o];
    }
    pq = wave_sum(pq);
    pk = wave_sum(pk);
    const float iq = inq[row], ik = ink[row];   // negative: the eps branch
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        const int64_t o = row * DK + lane * CPL + cc;
        const float gq = iq > 0.f ? (dqh[o] - qh[o] * pq) * iq : dqh[o] * -iq;
        const float gk = ik > 0.f ? (dkh[o] - kh[o] * pk) * ik : dkh[o] * -ik;
        dq[o] = from_f32<IO>(gq);
        dk[o] = from_f32<IO>(gk);
        const float x = to_f32(a[o]);
        const float sp = fmaxf(x, 0.f) + pro_log1p_unit(__expf(-fabsf(x)));
        da[o] = from_f32<GT>(-sp > lo ? -pro_beta(x) * dla[o] : 0.f);
    }
    if (lane == 0) db[row] = from_f32<GT>(be[row] * (1.f - be[row]) * dbe[row]);
}

// Offsets of the prologue pass's fp32 buffers after the backward's own workspace.
struct ProLayout {
    size_t qh, kh, la, dqh, dkh, dla, be, inq, ink, dbe, total;
};
ProLayout pro_layout(const BwdArgs &a) {
    const size_t rows = (size_t)a.total_tokens * a.H;
    const size_t big = (rows * a.d_k * 4 + 255) / 256 * 256, small = (rows * 4 + 255) / 256 * 256;
    ProLayout P;
    P.qh = 0; P.kh = big; P.la = 2 * big; P.dqh = 3 * big; P.dkh = 4 * big; P.dla = 5 * big;
    P.be = 6 * big; P.inq = P.be + small; P.ink = P.inq + small; P.dbe = P.ink + small;
    P.total = P.dbe + small;
    return P;
}

template <int DK, typename IO, typename GT>
hipError_t launch_pro_maps(const BwdArgs &a, float lo, uint8_t *x, const ProLayout &P, int64_t rows, bool chain,
                           hipStream_t st) {
    const int64_t nblk = (rows + 3) / 4;
    auto at = [&](size_t off) { return reinterpret_cast<float *>(x + off); };
    if (!chain)
        hipLaunchKernelGGL((pro_map_kernel<DK, IO, GT>), dim3((unsigned)nblk), dim3(256), 0, st,
                           static_cast<const IO *>(a.q), static_cast<const IO *>(a.k),
                           static_cast<const GT *>(a.log_alpha), static_cast<const GT *>(a.beta), rows, lo, at(P.qh),
                           at(P.kh), at(P.la), at(P.be), at(P.inq), at(P.ink));
    else
        hipLaunchKernelGGL((pro_chain_kernel<DK, IO, GT>), dim3((unsigned)nblk), dim3(256), 0, st, at(P.qh), at(P.kh),
                           at(P.inq), at(P.ink), static_cast<const GT *>(a.log_alpha), at(P.be), lo, at(P.dqh),
                           at(P.dkh), at(P.dla), at(P.dbe), rows, static_cast<IO *>(a.dq), static_cast<IO *>(a.dk),
                           static_cast<GT *>(a.dlog_alpha), static_cast<GT *>(a.dbeta));
    return hipGetLastError();
}

template <int DK>
hipError_t launch_pro_maps_t(const BwdArgs &a, float lo, uint8_t *x, const ProLayout &P, int64_t rows, bool chain,
                             hipStream_t st) {
    if (a.io_bf16)
        return a.gate_bf16 ? launch_pro_maps<DK, bf16_t, bf16_t>(a, lo, x, P, rows, chain, st)
                           : launch_pro_maps<DK, bf16_t, float>(a, lo, x, P, rows, chain, st);
    return a.gate_bf16 ? launch_pro_maps<DK, float, bf16_t>(a, lo, x, P, rows, chain, st)
                       : launch_pro_maps<DK, float, float>(a, lo, x, P, rows, chain, st);
}


// ----------------------------------------------------------------------------
// fp32 forward at d_k = 128, chunkwise on the fp32 matrix cores.  The backward's
// prep kernel writes each chunk-head's record (QA, KI, W, T, P, the factors;
// exact mode beyond the anchored range), its forward replay walks each chain
// and stores every chunk's start state S and U (and h_T), and the output kernel
// below forms every chunk's read-out in parallel:
//     O = QA Diag(e^m) S + P U
// (the chunk form of section 3.1 of the KimiLinear article; m = 0 in exact
// mode).  Every product is fp32.
template <int DK> struct alignas(16) OutBS {
    static constexpr int KS = DK + 4, CS = kB + 4, BS = 32 + 4;
    float QA[kB][KS];                        // QA Diag(e^m)
    float P[kB][CS];
    float S[DK][BS];                         // 32 columns of the chunk's start state
    float U[kB][BS];                         // the same 32 columns of U
};

template <int DK, int DV, typename IO>
__global__ __launch_bounds__(256) void fwd_out_kernel(const int32_t *__restrict__ cu,
                                                      const int32_t *__restrict__ chunk_off, int64_t N, int64_t T,
                                                      int H, int64_t nch, const float *__restrict__ recs,
                                                      const float *__restrict__ Sc, const float *__restrict__ Uc,
                                                      IO *__restrict__ o) {
    using R = BRec<DK>;
    using S = OutBS<DK>;
    __shared__ S sm;
    const int64_t chunk = blockIdx.x;
    const int h = blockIdx.y;
    int64_t n, t0;
    int nv;
    if (!locate_chunk(chunk, cu, chunk_off, N, T, n, t0, nv)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const size_t ch = (size_t)h * nch + chunk;
    const float *rec = recs + ch * R::FLOATS;
    for (int i = tid; i < kB * DK / 4; i += 256) {
        const int r = i / (DK / 4), c = (i % (DK / 4)) * 4;
        const f32x4_t x = *reinterpret_cast<const f32x4_t *>(rec + R::QA + r * DK + c);
        const f32x4_t e = *reinterpret_cast<const f32x4_t *>(rec + R::EM + c);
        *reinterpret_cast<f32x4_t *>(&sm.QA[r][c]) = x * e;
    }
    for (int i = tid; i < kB * kB / 4; i += 256) {
        const int r = i / (kB / 4), c = (i % (kB / 4)) * 4;
        *reinterpret_cast<f32x4_t *>(&sm.P[r][c]) = *reinterpret_cast<const f32x4_t *>(rec + R::P + r * kB + c);
    }
    const float *sc = Sc + ch * DK * DV;
    const float *uc = Uc + ch * kB * DV;
    for (int j0 = 0; j0 < DV; j0 += 32) {
        __syncthreads();                     // the previous block's reads are done
        for (int i = tid; i < DK * 8; i += 256) {
            const int r = i / 8, c = (i % 8) * 4;
            *reinterpret_cast<f32x4_t *>(&sm.S[r][c]) =
                *reinterpret_cast<const f32x4_t *>(sc + (size_t)r * DV + j0 + c);
        }
        for (int i = tid; i < kB * 8; i += 256) {
            const int r = i / 8, c = (i % 8) * 4;
            *reinterpret_cast<f32x4_t *>(&sm.U[r][c]) =
                *reinterpret_cast<const f32x4_t *>(uc + (size_t)r * DV + j0 + c);
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {     // wave w: row tile w
            f32x4_t acc = zero4();
            acc = mm<DK, S::KS, 1, S::BS, 1>(acc, &sm.QA[16 * w][0], &sm.S[0][16 * ct], lane);
            acc = mm<kB, S::CS, 1, S::BS, 1>(acc, &sm.P[16 * w][0], &sm.U[0][16 * ct], lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + acc_row(lane, e), j = j0 + 16 * ct + acc_col(lane);
                if (r < nv) o[((t0 + r) * H + h) * DV + j] = from_f32<IO>(acc[e]);
            }
        }
    }
}

// Workspace of the fp32 forward: the varlen plan, the records, S and U per
// chunk-head, and the input prologue's mapped q, k, log alpha (fp32 [rows][d_k])
// and beta and inverse norms (fp32 [rows]), always reserved since the size
// query does not know the entry point.
struct F32FwdLayout {
    int64_t nch;
    size_t plan, rec, sc, uc, qh, kh, la, be, inq, ink, total;
};
F32FwdLayout f32_fwd_layout(const ChunkArgs &a) {
    F32FwdLayout L = {};
    if (a.total_tokens <= 0) return L;       // no tokens: h_T = h0, no workspace
    L.nch = a.varlen ? (a.total_tokens + kB - 1) / kB + a.num_seqs : a.num_seqs * ((a.seq_len + kB - 1) / kB);
    const size_t ch = (size_t)L.nch * a.H;
    const size_t rows = (size_t)a.total_tokens * a.H;
    const size_t big = (rows * a.d_k * 4 + 255) / 256 * 256, small = (rows * 4 + 255) / 256 * 256;
    L.plan = 0;
    L.rec = plan_bytes(a.num_seqs);
    L.sc = L.rec + ch * rec_floats<128>() * 4;
    L.uc = L.sc + ch * a.d_k * a.d_v * 4;
    L.qh = L.uc + ch * kB * a.d_v * 4;
    L.kh = L.qh + big;
    L.la = L.kh + big;
    L.be = L.la + big;
    L.inq = L.be + small;
    L.ink = L.inq + small;
    L.total = L.ink + small;
    return L;
}

// h_T = h0 (or zeros) for a call without tokens.
__global__ __launch_bounds__(256) void state_pass_kernel(const float *__restrict__ h0, float *__restrict__ h_T,
                                                         int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) h_T[i] = h0 ? h0[i] : 0.f;
}

template <int DV, typename GT, int GM>
hipError_t launch_f32_fwd_t(const ChunkArgs &a, const float *q, const float *k, const GT *la, const GT *be,
                            hipStream_t st) {
    constexpr int DK = 128;
    const F32FwdLayout L = f32_fwd_layout(a);
    if (a.total_tokens <= 0) {
        const int64_t n = a.num_seqs * a.H * (int64_t)DK * DV;
        if (a.h_T && n > 0)
            hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.h0, a.h_T, n);
        return hipGetLastError();
    }
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    int32_t *chunk_off = a.varlen ? reinterpret_cast<int32_t *>(ws + L.plan) : nullptr;
    float *recs = reinterpret_cast<float *>(ws + L.rec);
    float *Sc = reinterpret_cast<float *>(ws + L.sc);
    float *Uc = reinterpret_cast<float *>(ws + L.uc);
    const GT *wr = static_cast<const GT *>(a.w_write);
    const int64_t T = a.seq_len;
    const bool tokens = a.total_tokens > 0 && L.nch > 0;
    if (a.varlen)
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.num_seqs, chunk_off);
    if (tokens)
        hipLaunchKernelGGL((bwd_prep_kernel<DK, float, GT, GM>), dim3((unsigned)L.nch, (unsigned)a.H), dim3(256), 0, st,
                           q, k, la, be, a.cu_seqlens, chunk_off, a.num_seqs, T, a.H, L.nch, recs);
    const int64_t grid = chain_grid(a.num_seqs * a.H, DV / kSBV);
    if (grid > 0)   // the replay only (every block id below fwd_blocks)
        hipLaunchKernelGGL((bwd_state_kernel<DK, DV, kSBV, float, GT>), dim3((unsigned)grid), dim3(kSP), 0, st,
                           static_cast<const float *>(a.v), wr ? wr : be, a.h0, (const float *)nullptr,
                           (const float *)nullptr, a.cu_seqlens, chunk_off, a.num_seqs, T, a.H, L.nch, recs, Sc, Uc,
                           (float *)nullptr, (float *)nullptr, (float *)nullptr, grid, a.h_T);
    if (tokens)
        hipLaunchKernelGGL((fwd_out_kernel<DK, DV, float>), dim3((unsigned)L.nch, (unsigned)a.H), dim3(256), 0, st,
                           a.cu_seqlens, chunk_off, a.num_seqs, T, a.H, L.nch, recs, Sc, Uc, static_cast<float *>(a.o));
    return hipGetLastError();
}

template <int DV, typename GT>
hipError_t launch_f32_fwd_gate(const ChunkArgs &a, hipStream_t st) {
    const float *q = static_cast<const float *>(a.q), *k = static_cast<const float *>(a.k);
    const GT *la = static_cast<const GT *>(a.log_alpha), *be = static_cast<const GT *>(a.beta);
    if (a.gate_mode == kGatePerHead) return launch_f32_fwd_t<DV, GT, kGatePerHead>(a, q, k, la, be, st);
    if (a.gate_mode == kGateNone) return launch_f32_fwd_t<DV, GT, kGateNone>(a, q, k, la, be, st);
    return launch_f32_fwd_t<DV, GT, kGatePerChannel>(a, q, k, la, be, st);
}

// Raw projections: mapped (q/|q|, k/|k|, floored -softplus gate, sigmoid beta)
// into the workspace first, then the forward on the mapped fp32 values.
template <int DV, typename GT>
hipError_t launch_f32_fwd_prologue(const ChunkArgs &a, hipStream_t st) {
    const F32FwdLayout L = f32_fwd_layout(a);
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    auto at = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
    const int64_t rows = a.total_tokens * a.H;
    if (rows > 0)
        hipLaunchKernelGGL((pro_map_kernel<128, float, GT>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                           static_cast<const float *>(a.q), static_cast<const float *>(a.k),
                           static_cast<const GT *>(a.log_alpha), static_cast<const GT *>(a.beta), rows,
                           a.log_alpha_min, at(L.qh), at(L.kh), at(L.la), at(L.be), at(L.inq), at(L.ink));
    return launch_f32_fwd_t<DV, float, kGatePerChannel>(a, at(L.qh), at(L.kh), at(L.la), at(L.be), st);
}

template <int DV>
hipError_t launch_f32_fwd_dv(const ChunkArgs &a, hipStream_t st) {
    if (a.prologue)
        return a.gate_bf16 ? launch_f32_fwd_prologue<DV, bf16_t>(a, st) : launch_f32_fwd_prologue<DV, float>(a, st);
    return a.gate_bf16 ? launch_f32_fwd_gate<DV, bf16_t>(a, st) : launch_f32_fwd_gate<DV, float>(a, st);
}

}  // namespace

size_t chunk_bwd_workspace_bytes(const BwdArgs &a) { return bwd_layout(a).total; }

size_t f32_fwd_workspace_bytes(const ChunkArgs &a) { return f32_fwd_layout(a).total; }

// The prep and output kernels run (chunks, heads) grids of 256 threads, the
// replay the padded chains, the prologue's map four rows per workgroup.
bool f32_fwd_grids_fit(const ChunkArgs &a) {
    const F32FwdLayout L = f32_fwd_layout(a);
    return grid_fits(L.nch, 256) && a.H <= kMaxGridY && grid_fits(chain_grid(a.num_seqs * a.H, a.d_v / kSBV), kSP) &&
           grid_fits((a.total_tokens * a.H + 3) / 4, 256) &&
           grid_fits((a.num_seqs * a.H * a.d_k * (int64_t)a.d_v + 255) / 256, 256);
}

hipError_t launch_f32_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
    return a.d_v == 128 ? launch_f32_fwd_dv<128>(a, st) : launch_f32_fwd_dv<64>(a, st);
}

// Scalar gates run the same kernels with the gate layout as a compile-time
// parameter: the gate is read once per (token, head), and dlog_alpha is the
// channel sum of the per-channel gradient (the chain rule: every channel's log
// alpha is the one value), taken in the gradient kernel.
size_t gdn_chunk_bwd_workspace_bytes(const BwdArgs &a) { return bwd_layout(a).total; }

size_t pro_chunk_bwd_workspace_bytes(const BwdArgs &a) { return bwd_layout(a).total + pro_layout(a).total; }

int launch_pro_chunk_bwd(const BwdArgs &a, float lo, void *stream, char *err, size_t err_len) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t base = bwd_layout(a).total;
    const ProLayout P = pro_layout(a);
    if (a.workspace_bytes < base + P.total) {
        snprintf(err, err_len, "workspace too small");
        return -1;
    }
    const int64_t rows = a.total_tokens * a.H;
    if (!pro_chunk_bwd_grids_fit(a)) {
        snprintf(err, err_len, "chunk_bwd_prologue grid too large");
        return -1;
    }
    uint8_t *x = static_cast<uint8_t *>(a.workspace) + base;
    auto fail = [&](hipError_t e) {
        snprintf(err, err_len, "%s", hipGetErrorString(e));
        return -1;
    };
    if (rows > 0) {
        const hipError_t e = a.d_k == 128 ? launch_pro_maps_t<128>(a, lo, x, P, rows, false, st)
                                          : launch_pro_maps_t<64>(a, lo, x, P, rows, false, st);
        if (e != hipSuccess) return fail(e);
    }
    BwdArgs b = a;
    b.q = x + P.qh;
    b.k = x + P.kh;
    b.log_alpha = x + P.la;
    b.beta = x + P.be;
    b.gate_bf16 = 0;
    b.qk_f32 = 1;
    b.dq = x + P.dqh;
    b.dk = x + P.dkh;
    b.dlog_alpha = x + P.dla;
    b.dbeta = x + P.dbe;
    b.workspace_bytes = base;
    if (launch_chunk_bwd(b, stream, err, err_len) != 0) return -1;
    if (rows > 0) {
        const hipError_t e = a.d_k == 128 ? launch_pro_maps_t<128>(a, lo, x, P, rows, true, st)
                                          : launch_pro_maps_t<64>(a, lo, x, P, rows, true, st);
        if (e != hipSuccess) return fail(e);
    }
    return 0;
}

int launch_gdn_chunk_bwd(const BwdArgs &a, void *stream, char *err, size_t err_len) {
    BwdArgs b = a;
    b.gate_mode = a.log_alpha ? kGatePerHead : kGateNone;
    if (!a.log_alpha) b.dlog_alpha = nullptr;
    return launch_chunk_bwd(b, stream, err, err_len);
}

// The prep and gradient kernels run (chunks, heads) grids of 256 and 512
// threads, the state kernel up to two passes of the padded chains.
bool chunk_bwd_grids_fit(const BwdArgs &a) {
    const BwdLayout L = bwd_layout(a);
    return grid_fits(L.nch, 512) && a.H <= kMaxGridY && grid_fits(2 * chain_grid(a.num_seqs * a.H, a.d_v / kSBV), kSP);
}

// The prologue's map kernels take four rows per 256-thread workgroup.
bool pro_chunk_bwd_grids_fit(const BwdArgs &a) {
    return chunk_bwd_grids_fit(a) && grid_fits((a.total_tokens * a.H + 3) / 4, 256);
}

int launch_chunk_bwd(const BwdArgs &a, void *stream, char *err, size_t err_len) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const BwdLayout L = bwd_layout(a);
    if (!chunk_bwd_grids_fit(a)) {
        snprintf(err, err_len, "chunk_bwd grid too large");
        return -1;
    }
    if (a.workspace_bytes < L.total) {
        snprintf(err, err_len, "workspace too small");
        return -1;
    }
    hipError_t e;
    if (a.d_k == 128)
        e = a.d_v == 128 ? launch_bwd_dims<128, 128>(a, st) : launch_bwd_dims<128, 64>(a, st);
    else
        e = a.d_v == 128 ? launch_bwd_dims<64, 128>(a, st) : launch_bwd_dims<64, 64>(a, st);
    if (e != hipSuccess) {
        snprintf(err, err_len, "%s", hipGetErrorString(e));
        return -1;
    }
    return 0;
}

}  // namespace kda
