// kda_decode.hip -- one recurrent KDA step over B*H resident states (decode).
//
// Per (b, h) and every value column j (columns evolve independently):
//   s_j <- alpha (.) s_j                      (per-row decay; KimiLinear article, sec. 2.3)
//   u_j  = beta (v_j - k^T s_j)               (delta-rule correction, sec. 2.1)
//   s_j <- s_j + u_j k                        (write)
//   o_j  = q^T s_j                            (read-out, inclusive of this token)
// Both reductions are taken on the decayed column a_j = k^T (alpha.s_j),
// b_j = q^T (alpha.s_j), so o_j = b_j + u_j (q.k) and the state is read once and
// written once.  The kernel is bound by HBM bandwidth: S is 4*d_k*d_v bytes per
// (b, h) each way, everything else is O(d).
#include "kda_device.h"
#include "kda_launch.h"

#include <stdio.h>

namespace kda {
namespace {

constexpr int kDecodeThreads = 256;

// PRO: q, k, log_alpha and beta are raw projections, mapped as they are read
// (input prologue; lo is the floor of log alpha).  The reductions then run on
// the raw q and k and are rescaled by the inverse norms, reduced alongside.
// DEC: beta erases and wr writes: u = wr v - beta k^T(alpha S).
// GM: alpha per key channel, one alpha per (b, h) for every row, or none (1).
template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const GT *__restrict__ log_alpha, const GT *__restrict__ beta, const GT *__restrict__ wr, float *__restrict__ S,
    IO *__restrict__ o, float lo) {
    constexpr int NCG = DV / 4;                 // groups of 4 value columns
    constexpr int NRG = kDecodeThreads / NCG;   // row groups
    constexpr int RPT = DK / NRG;               // key rows per thread
    static_assert(RPT >= 1 && RPT * NRG == DK, "bad decode tiling");

    __shared__ float red[NRG][NCG][8];
    __shared__ float red_qk[NRG][PRO ? 3 : 1];

    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    const int cg = t % NCG, rg = t / NCG;
    const int row0 = rg * RPT;

    float *Sp = S + bh * (int64_t)(DK * DV) + 4 * cg;
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const float4 *>(Sp + (row0 + i) * DV);

    float kk[RPT], qq[RPT], al[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        kk[i] = to_f32(k[bh * DK + row0 + i]);
        qq[i] = to_f32(q[bh * DK + row0 + i]);
        al[i] = __expf(log_decay<PRO, GM>(gate_at<GM>(log_alpha, bh, DK, row0 + i), lo));
    }

    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f}, pqk = 0.f, pqq = 0.f, pkk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        s[i].x *= al[i]; s[i].y *= al[i]; s[i].z *= al[i]; s[i].w *= al[i];
        pa[0] += kk[i] * s[i].x; pa[1] += kk[i] * s[i].y; pa[2] += kk[i] * s[i].z; pa[3] += kk[i] * s[i].w;
        pb[0] += qq[i] * s[i].x; pb[1] += qq[i] * s[i].y; pb[2] += qq[i] * s[i].z; pb[3] += qq[i] * s[i].w;
        pqk += qq[i] * kk[i];
        if (PRO) {
            pqq += qq[i] * qq[i];
            pkk += kk[i] * kk[i];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        red[rg][cg][j] = pa[j];
        red[rg][cg][4 + j] = pb[j];
    }
    if (cg == 0) {
        red_qk[rg][0] = pqk;
        if (PRO) {
            red_qk[rg][1] = pqq;
            red_qk[rg][2] = pkk;
        }
    }
    __syncthreads();

    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f, nq = 0.f, nk = 0.f;
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] += red[r][cg][j];
            b[j] += red[r][cg][4 + j];
        }
        qk += red_qk[r][0];
        if (PRO) {
            nq += red_qk[r][1];
            nk += red_qk[r][2];
        }
    }
    float bt = to_f32(beta[bh]);
    float ik = 1.f;
    if (PRO) {
        const float iq = pro_inv_norm(nq);
        ik = pro_inv_norm(nk);
        qk *= iq * ik;
        bt = pro_beta(bt);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] *= ik;
            b[j] *= iq;
        }
    }
    float u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float vj = to_f32(v[bh * DV + 4 * cg + j]);
        u[j] = DEC ? to_f32(wr[bh]) * vj - bt * a[j] : bt * (vj - a[j]);
    }

    // The updated state is written with non-temporal stores: it is not read again
    // in this step, and streaming it past the caches keeps the HBM write stream
    // from competing with the state still being read (measured: 5.2 -> 6.9 TB/s).
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kh = PRO ? kk[i] * ik : kk[i];   // the state takes k / |k|
        f32x4_t r;
        r[0] = s[i].x + kh * u[0];
        r[1] = s[i].y + kh * u[1];
        r[2] = s[i].z + kh * u[2];
        r[3] = s[i].w + kh * u[3];
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4_t *>(Sp + (row0 + i) * DV));
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[bh * DV + 4 * cg + j] = from_f32<IO>(b[j] + u[j] * qk);
    }
}

template <int DK, int DV, typename IO, typename GT, bool PRO, int GM, bool DEC>
hipError_t launch_v(const DecodeArgs &a, hipStream_t st) {
    const int64_t nb = a.B * (int64_t)a.H;
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, IO, GT, PRO, GM, DEC>), dim3((unsigned)nb), dim3(kDecodeThreads),
                       0, st, (const IO *)a.q, (const IO *)a.k, (const IO *)a.v, (const GT *)a.log_alpha,
                       (const GT *)a.beta, (const GT *)a.w_write, a.S, (IO *)a.o, a.log_alpha_min);
    return hipGetLastError();
}

// The input variants that exist: per-channel gates with or without the prologue
// or with decoupled strengths, and the scalar-gate forms.
template <int DK, int DV, typename IO, typename GT>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st) {
    if (a.gate_mode == kGatePerHead) return launch_v<DK, DV, IO, GT, false, kGatePerHead, false>(a, st);
    if (a.gate_mode == kGateNone) return launch_v<DK, DV, IO, GT, false, kGateNone, false>(a, st);
    if (a.prologue) return launch_v<DK, DV, IO, GT, true, kGatePerChannel, false>(a, st);
    if (a.w_write) return launch_v<DK, DV, IO, GT, false, kGatePerChannel, true>(a, st);
    return launch_v<DK, DV, IO, GT, false, kGatePerChannel, false>(a, st);
}

template <int DK, int DV>
hipError_t launch_dims(const DecodeArgs &a, hipStream_t st) {
    if (a.io_bf16) {
        return a.gate_bf16 ? launch_t<DK, DV, bf16_t, bf16_t>(a, st) : launch_t<DK, DV, bf16_t, float>(a, st);
    }
    return a.gate_bf16 ? launch_t<DK, DV, float, bf16_t>(a, st) : launch_t<DK, DV, float, float>(a, st);
}

}  // namespace

bool decode_grids_fit(const DecodeArgs &a) { return grid_fits(a.B * (int64_t)a.H, kDecodeThreads); }

int launch_decode_step(const DecodeArgs &a, void *stream, char *err, size_t err_len) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!decode_grids_fit(a)) {
        snprintf(err, err_len, "decode grid too large");
        return -1;
    }
    hipError_t e;
    if (a.d_k == 128 && a.d_v == 128) e = launch_dims<128, 128>(a, st);
    else if (a.d_k == 128 && a.d_v == 64) e = launch_dims<128, 64>(a, st);
    else if (a.d_k == 64 && a.d_v == 128) e = launch_dims<64, 128>(a, st);
    else e = launch_dims<64, 64>(a, st);
    if (e != hipSuccess) {
        snprintf(err, err_len, "%s", hipGetErrorString(e));
        return -1;
    }
    return 0;
}

}  // namespace kda
