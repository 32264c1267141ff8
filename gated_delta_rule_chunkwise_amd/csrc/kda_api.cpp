// Host side of the libkda C ABI: argument validation, status strings and
// dispatch to the HIP launchers.  Every check here runs before any HIP call,
// so invalid arguments never reach the device.
#include "kda.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kda_launch.h"

namespace {

thread_local char g_hip_error[512] = "";

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool supported_dim(int32_t d) { return d == 64 || d == 128; }
bool valid_dtype(int32_t t) { return t == KDA_F32 || t == KDA_BF16; }
uintptr_t dsize(int32_t t) { return t == KDA_F32 ? 4 : 2; }

// Products of the sizes must stay well inside int64 for device indexing.
bool sizes_fit(int64_t a, int64_t b, int64_t c) {
    const int64_t lim = (int64_t)1 << 50;
    if (a > lim || b > lim || c > lim) return false;
    if (a != 0 && b > lim / a) return false;
    if (a * b != 0 && c > lim / (a * b)) return false;
    return true;
}

// The floor of log alpha under the input prologue: finite and <= 0.
bool valid_floor(float lo) { return isfinite(lo) && lo <= 0.f; }

kda_status_t chunk_fwd_impl(const void *q, const void *k, const void *v, const void *log_alpha,
                            const void *beta, const void *w_write, const float *h0, const int32_t *cu_seqlens,
                            int32_t num_seqs,
                            void *o, float *h_T, int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                            int32_t io_dtype, int32_t gate_dtype, void *workspace,
                            size_t workspace_bytes, void *stream, bool prologue, float lo, int gate_mode,
                            bool noalloc = false);
kda_status_t decode_step_impl(const void *q, const void *k, const void *v, const void *log_alpha,
                              const void *beta, const void *w_write, float *S, void *o, int32_t B, int32_t H, int32_t d_k,
                              int32_t d_v, int32_t io_dtype, int32_t gate_dtype, void *stream,
                              bool prologue, float lo, int gate_mode);

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return 1; }

const char *kda_status_string(int32_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_hip_error(void) { return g_hip_error; }

size_t kda_chunk_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                    int32_t num_seqs, int32_t io_dtype) {
    if (B <= 0 || T < 0 || H <= 0 || !supported_dim(d_k) || !supported_dim(d_v)) return 0;
    if (!valid_dtype(io_dtype) || num_seqs < 0 || (num_seqs > 0 && B != 1)) return 0;
    if (!sizes_fit((int64_t)B * T, H, d_k > d_v ? d_k : d_v)) return 0;
    if (!sizes_fit(num_seqs > 0 ? num_seqs : B, H, (int64_t)d_k * d_v)) return 0;
    kda::ChunkArgs a = {};
    a.varlen = num_seqs > 0;
    a.num_seqs = num_seqs > 0 ? num_seqs : B;
    a.seq_len = T;
    a.total_tokens = (int64_t)B * T;
    a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.io_bf16 = io_dtype == KDA_BF16;
    return kda::chunk_fwd_workspace_bytes(a);
}

kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *beta, const float *h0, const int32_t *cu_seqlens,
                           int32_t num_seqs, void *o, float *h_T, int32_t B, int32_t T,
                           int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                           int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                           void *stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, h0, cu_seqlens, num_seqs, o, h_T, B, T, H, d_k, d_v,
                          io_dtype, gate_dtype, workspace, workspace_bytes, stream, false, 0.f, 0);
}

kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *log_alpha,
                                   const void *beta, const float *h0, const int32_t *cu_seqlens,
                                   int32_t num_seqs, void *o, float *h_T, int32_t B, int32_t T,
                                   int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                   int32_t gate_dtype, void *stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, h0, cu_seqlens, num_seqs, o, h_T, B, T, H, d_k, d_v,
                          io_dtype, gate_dtype, nullptr, 0, stream, false, 0.f, 0, true);
}

kda_status_t kda_chunk_fwd_prologue(const void *q_raw, const void *k_raw, const void *v,
                                    const void *gate_pre, const void *beta_pre, float log_alpha_min,
                                    const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                                    void *o, float *h_T, int32_t B, int32_t T, int32_t H, int32_t d_k,
                                    int32_t d_v, int32_t io_dtype, int32_t gate_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_floor(log_alpha_min)) return KDA_ERR_INVALID_ARGUMENT;
    return chunk_fwd_impl(q_raw, k_raw, v, gate_pre, beta_pre, nullptr, h0, cu_seqlens, num_seqs, o, h_T, B, T, H, d_k,
                          d_v, io_dtype, gate_dtype, workspace, workspace_bytes, stream, true, log_alpha_min, 0);
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *log_alpha,
                             const void *beta, float *S, void *o, int32_t B, int32_t H,
                             int32_t d_k, int32_t d_v, int32_t io_dtype,
                             int32_t gate_dtype, void *stream) {
    return decode_step_impl(q, k, v, log_alpha, beta, nullptr, S, o, B, H, d_k, d_v, io_dtype, gate_dtype, stream, false,
                            0.f, 0);
}

kda_status_t kda_decode_step_prologue(const void *q_raw, const void *k_raw, const void *v,
                                      const void *gate_pre, const void *beta_pre, float log_alpha_min,
                                      float *S, void *o, int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                                      int32_t io_dtype, int32_t gate_dtype, void *stream) {
    if (!valid_floor(log_alpha_min)) return KDA_ERR_INVALID_ARGUMENT;
    return decode_step_impl(q_raw, k_raw, v, gate_pre, beta_pre, nullptr, S, o, B, H, d_k, d_v, io_dtype, gate_dtype,
                            stream, true, log_alpha_min, 0);
}

kda_status_t kda_gdn_chunk_fwd(const void *q, const void *k, const void *v, const void *log_alpha,
                               const void *beta, const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                               void *o, float *h_T, int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                               int32_t io_dtype, int32_t gate_dtype, void *workspace,
                               size_t workspace_bytes, void *stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, h0, cu_seqlens, num_seqs, o, h_T, B, T, H, d_k, d_v,
                          io_dtype, gate_dtype, workspace, workspace_bytes, stream, false, 0.f,
                          log_alpha ? 1 : 2);
}

kda_status_t kda_gdn_decode_step(const void *q, const void *k, const void *v, const void *log_alpha,
                                 const void *beta, float *S, void *o, int32_t B, int32_t H, int32_t d_k,
                                 int32_t d_v, int32_t io_dtype, int32_t gate_dtype, void *stream) {
    return decode_step_impl(q, k, v, log_alpha, beta, nullptr, S, o, B, H, d_k, d_v, io_dtype, gate_dtype, stream, false,
                            0.f, log_alpha ? 1 : 2);
}

kda_status_t kda_chunk_fwd_decoupled(const void *q, const void *k, const void *v, const void *log_alpha,
                                     const void *b_erase, const void *w_write, const float *h0,
                                     const int32_t *cu_seqlens, int32_t num_seqs, void *o, float *h_T, int32_t B,
                                     int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                     int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    if ((int64_t)B * T > 0 && (!w_write || !aligned_to(w_write, dsize(gate_dtype))))
        return valid_dtype(gate_dtype) ? KDA_ERR_INVALID_ARGUMENT : KDA_ERR_UNSUPPORTED;
    return chunk_fwd_impl(q, k, v, log_alpha, b_erase, w_write, h0, cu_seqlens, num_seqs, o, h_T, B, T, H, d_k,
                          d_v, io_dtype, gate_dtype, workspace, workspace_bytes, stream, false, 0.f, 0);
}

kda_status_t kda_decode_step_decoupled(const void *q, const void *k, const void *v, const void *log_alpha,
                                       const void *b_erase, const void *w_write, float *S, void *o, int32_t B,
                                       int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                       int32_t gate_dtype, void *stream) {
    if (!w_write || !aligned_to(w_write, dsize(gate_dtype)))
        return valid_dtype(gate_dtype) ? KDA_ERR_INVALID_ARGUMENT : KDA_ERR_UNSUPPORTED;
    return decode_step_impl(q, k, v, log_alpha, b_erase, w_write, S, o, B, H, d_k, d_v, io_dtype, gate_dtype,
                            stream, false, 0.f, 0);
}

static kda::BwdArgs bwd_sizes(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t num_seqs,
                              int32_t io_dtype) {
    kda::BwdArgs a = {};
    a.varlen = num_seqs > 0;
    a.num_seqs = num_seqs > 0 ? num_seqs : B;
    a.seq_len = T;
    a.total_tokens = (int64_t)B * T;
    a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.io_bf16 = io_dtype == KDA_BF16;
    return a;
}

static bool bwd_sizes_ok(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t num_seqs,
                         int32_t io_dtype) {
    if (B <= 0 || T < 0 || H <= 0 || H > 65535 || !supported_dim(d_k) || !supported_dim(d_v)) return false;
    if (!valid_dtype(io_dtype)) return false;
    if (num_seqs < 0 || (num_seqs > 0 && B != 1)) return false;
    return sizes_fit((int64_t)B * T, H, d_k > d_v ? d_k : d_v) &&
           sizes_fit(num_seqs > 0 ? num_seqs : B, H, (int64_t)d_k * d_v);
}

size_t kda_chunk_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                    int32_t num_seqs, int32_t io_dtype) {
    if (!bwd_sizes_ok(B, T, H, d_k, d_v, num_seqs, io_dtype)) return 0;
    return kda::chunk_bwd_workspace_bytes(bwd_sizes(B, T, H, d_k, d_v, num_seqs, io_dtype));
}

size_t kda_chunk_bwd_prologue_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                             int32_t num_seqs, int32_t io_dtype) {
    if (!bwd_sizes_ok(B, T, H, d_k, d_v, num_seqs, io_dtype)) return 0;
    return kda::pro_chunk_bwd_workspace_bytes(bwd_sizes(B, T, H, d_k, d_v, num_seqs, io_dtype));
}

size_t kda_gdn_chunk_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                        int32_t num_seqs, int32_t io_dtype) {
    if (!bwd_sizes_ok(B, T, H, d_k, d_v, num_seqs, io_dtype)) return 0;
    return kda::gdn_chunk_bwd_workspace_bytes(bwd_sizes(B, T, H, d_k, d_v, num_seqs, io_dtype));
}

}  // extern "C"

namespace {

// gate_mode 0: log_alpha [.., d_k] (KDA); 1: [..] per (token, head); 2: none;
// 3: raw projections through the input prologue (gate_pre [.., d_k]; lo its floor).
kda_status_t chunk_bwd_impl(const void *q, const void *k, const void *v, const void *log_alpha, const void *beta,
                            const float *h0, const int32_t *cu_seqlens, int32_t num_seqs, const void *grad_o,
                            const float *grad_hT, void *grad_q, void *grad_k, void *grad_v, void *grad_log_alpha,
                            void *grad_beta, float *grad_h0, int32_t B, int32_t T, int32_t H, int32_t d_k,
                            int32_t d_v, int32_t io_dtype, int32_t gate_dtype, void *workspace,
                            size_t workspace_bytes, void *stream, int gate_mode, bool decoupled = false,
                            const void *w_write = nullptr, void *grad_w_write = nullptr, float lo = 0.f) {
    if (!valid_dtype(io_dtype) || !valid_dtype(gate_dtype)) return KDA_ERR_UNSUPPORTED;
    if (gate_mode == 3 && !valid_floor(lo)) return KDA_ERR_INVALID_ARGUMENT;
    if (B <= 0 || T < 0 || H <= 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (H > 65535) return KDA_ERR_UNSUPPORTED;   // heads are a grid dimension of the per-chunk kernels
    if (!sizes_fit((int64_t)B * T, H, (d_k > d_v ? d_k : d_v))) return KDA_ERR_INVALID_ARGUMENT;
    int64_t N;
    if (cu_seqlens) {
        if (B != 1 || num_seqs <= 0) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned_to(cu_seqlens, 4)) return KDA_ERR_INVALID_ARGUMENT;
        N = num_seqs;
    } else {
        if (num_seqs != 0 && num_seqs != B) return KDA_ERR_INVALID_ARGUMENT;
        N = B;
    }
    if (!sizes_fit(N, H, (int64_t)d_k * d_v)) return KDA_ERR_INVALID_ARGUMENT;
    const bool have_tokens = (int64_t)B * T > 0;
    if (have_tokens) {
        const void *need16[] = {q, k, v, grad_o, grad_q, grad_k, grad_v};
        for (const void *p : need16)
            if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARGUMENT;
        const uintptr_t gsz = dsize(gate_dtype);
        if (!beta || !grad_beta || !aligned_to(beta, gsz) || !aligned_to(grad_beta, gsz))
            return KDA_ERR_INVALID_ARGUMENT;
        if ((gate_mode == 0 || gate_mode == 3) &&
            (!log_alpha || !aligned16(log_alpha) || !grad_log_alpha || !aligned16(grad_log_alpha)))
            return KDA_ERR_INVALID_ARGUMENT;
        if (gate_mode == 1 && (!grad_log_alpha || !aligned_to(log_alpha, gsz) || !aligned_to(grad_log_alpha, gsz)))
            return KDA_ERR_INVALID_ARGUMENT;
        if (decoupled && (!w_write || !grad_w_write || !aligned_to(w_write, gsz) || !aligned_to(grad_w_write, gsz)))
            return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((h0 && !aligned16(h0)) || (grad_hT && !aligned16(grad_hT)) || (grad_h0 && !aligned16(grad_h0)))
        return KDA_ERR_INVALID_ARGUMENT;
    kda::BwdArgs a = bwd_sizes(B, T, H, d_k, d_v, cu_seqlens ? num_seqs : 0, io_dtype);
    a.gate_bf16 = gate_dtype == KDA_BF16;
    if (!(gate_mode == 3 ? kda::pro_chunk_bwd_grids_fit(a) : kda::chunk_bwd_grids_fit(a)))
        return KDA_ERR_UNSUPPORTED;
    const size_t need = gate_mode == 0   ? kda::chunk_bwd_workspace_bytes(a)
                        : gate_mode == 3 ? kda::pro_chunk_bwd_workspace_bytes(a)
                                         : kda::gdn_chunk_bwd_workspace_bytes(a);
    if (workspace_bytes < need || !workspace) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_INVALID_ARGUMENT;
    if (!have_tokens && !grad_h0) return KDA_OK;  // nothing to compute or write

    a.q = q; a.k = k; a.v = v; a.log_alpha = gate_mode == 2 ? nullptr : log_alpha; a.beta = beta; a.h0 = h0;
    a.cu_seqlens = cu_seqlens;
    a.d_o = grad_o; a.d_hT = grad_hT;
    a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dlog_alpha = gate_mode == 2 ? nullptr : grad_log_alpha;
    a.dbeta = grad_beta; a.dh0 = grad_h0;
    a.w_write = decoupled ? w_write : nullptr;
    a.dw_write = decoupled ? grad_w_write : nullptr;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    g_hip_error[0] = '\0';
    const int rc = gate_mode == 0   ? kda::launch_chunk_bwd(a, stream, g_hip_error, sizeof(g_hip_error))
                   : gate_mode == 3 ? kda::launch_pro_chunk_bwd(a, lo, stream, g_hip_error, sizeof(g_hip_error))
                                    : kda::launch_gdn_chunk_bwd(a, stream, g_hip_error, sizeof(g_hip_error));
    return rc != 0 ? KDA_ERR_HIP : KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *beta, const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                           const void *grad_o, const float *grad_hT, void *grad_q, void *grad_k, void *grad_v,
                           void *grad_log_alpha, void *grad_beta, float *grad_h0, int32_t B, int32_t T, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t io_dtype, int32_t gate_dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_bwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, num_seqs, grad_o, grad_hT, grad_q, grad_k, grad_v,
                          grad_log_alpha, grad_beta, grad_h0, B, T, H, d_k, d_v, io_dtype, gate_dtype, workspace,
                          workspace_bytes, stream, 0);
}

kda_status_t kda_chunk_bwd_prologue(const void *q_raw, const void *k_raw, const void *v, const void *gate_pre,
                                    const void *beta_pre, float log_alpha_min, const float *h0,
                                    const int32_t *cu_seqlens, int32_t num_seqs, const void *grad_o,
                                    const float *grad_hT, void *grad_q_raw, void *grad_k_raw, void *grad_v,
                                    void *grad_gate_pre, void *grad_beta_pre, float *grad_h0, int32_t B, int32_t T,
                                    int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                    int32_t gate_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_bwd_impl(q_raw, k_raw, v, gate_pre, beta_pre, h0, cu_seqlens, num_seqs, grad_o, grad_hT, grad_q_raw,
                          grad_k_raw, grad_v, grad_gate_pre, grad_beta_pre, grad_h0, B, T, H, d_k, d_v, io_dtype,
                          gate_dtype, workspace, workspace_bytes, stream, 3, false, nullptr, nullptr, log_alpha_min);
}

kda_status_t kda_chunk_bwd_decoupled(const void *q, const void *k, const void *v, const void *log_alpha,
                                     const void *b_erase, const void *w_write, const float *h0,
                                     const int32_t *cu_seqlens, int32_t num_seqs, const void *grad_o,
                                     const float *grad_hT, void *grad_q, void *grad_k, void *grad_v,
                                     void *grad_log_alpha, void *grad_b_erase, void *grad_w_write, float *grad_h0,
                                     int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                     int32_t io_dtype, int32_t gate_dtype, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    return chunk_bwd_impl(q, k, v, log_alpha, b_erase, h0, cu_seqlens, num_seqs, grad_o, grad_hT, grad_q, grad_k,
                          grad_v, grad_log_alpha, grad_b_erase, grad_h0, B, T, H, d_k, d_v, io_dtype, gate_dtype,
                          workspace, workspace_bytes, stream, 0, true, w_write, grad_w_write);
}

kda_status_t kda_gdn_chunk_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
                               const void *beta, const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                               const void *grad_o, const float *grad_hT, void *grad_q, void *grad_k, void *grad_v,
                               void *grad_log_alpha, void *grad_beta, float *grad_h0, int32_t B, int32_t T,
                               int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype, int32_t gate_dtype,
                               void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_bwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, num_seqs, grad_o, grad_hT, grad_q, grad_k, grad_v,
                          grad_log_alpha, grad_beta, grad_h0, B, T, H, d_k, d_v, io_dtype, gate_dtype, workspace,
                          workspace_bytes, stream, log_alpha ? 1 : 2);
}

}  // extern "C"

namespace {

kda_status_t chunk_fwd_impl(const void *q, const void *k, const void *v, const void *log_alpha,
                            const void *beta, const void *w_write, const float *h0, const int32_t *cu_seqlens,
                            int32_t num_seqs,
                            void *o, float *h_T, int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                            int32_t io_dtype, int32_t gate_dtype, void *workspace,
                            size_t workspace_bytes, void *stream, bool prologue, float lo, int gate_mode,
                            bool noalloc) {
    if (!valid_dtype(io_dtype) || !valid_dtype(gate_dtype)) return KDA_ERR_UNSUPPORTED;
    if (B <= 0 || T < 0 || H <= 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (!sizes_fit((int64_t)B * T, H, (d_k > d_v ? d_k : d_v))) return KDA_ERR_INVALID_ARGUMENT;
    int64_t N;
    if (cu_seqlens) {
        if (B != 1 || num_seqs <= 0) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned_to(cu_seqlens, 4)) return KDA_ERR_INVALID_ARGUMENT;
        N = num_seqs;
    } else {
        if (num_seqs != 0 && num_seqs != B) return KDA_ERR_INVALID_ARGUMENT;
        N = B;
    }
    if (!sizes_fit(N, H, (int64_t)d_k * d_v)) return KDA_ERR_INVALID_ARGUMENT;
    const bool have_tokens = (int64_t)B * T > 0;
    if (have_tokens) {
        if (!q || !k || !v || !beta || !o) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned_to(beta, dsize(gate_dtype))) return KDA_ERR_INVALID_ARGUMENT;
        if (gate_mode == 0 && (!log_alpha || !aligned16(log_alpha))) return KDA_ERR_INVALID_ARGUMENT;
        if (gate_mode == 1 && !aligned_to(log_alpha, dsize(gate_dtype))) return KDA_ERR_INVALID_ARGUMENT;
    }
    if ((h0 && !aligned16(h0)) || (h_T && !aligned16(h_T))) return KDA_ERR_INVALID_ARGUMENT;
    kda::ChunkArgs a = {};
    a.varlen = cu_seqlens != nullptr;
    a.num_seqs = N; a.seq_len = T; a.total_tokens = (int64_t)B * T;
    a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.io_bf16 = io_dtype == KDA_BF16; a.gate_bf16 = gate_dtype == KDA_BF16;
    a.force_fused = noalloc;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.w_write = w_write;
    a.h0 = h0; a.cu_seqlens = cu_seqlens; a.o = o; a.h_T = h_T;
    a.prologue = prologue; a.log_alpha_min = lo; a.gate_mode = gate_mode;
    if (!kda::chunk_fwd_grids_fit(a)) return KDA_ERR_UNSUPPORTED;
    const size_t need = kda::chunk_fwd_workspace_bytes(a);
    if (noalloc) {
        if (need > kda::kNoAllocScratchBytes) return KDA_ERR_WORKSPACE;
    } else {
        if (need > 0 && (workspace_bytes < need || !workspace)) return KDA_ERR_WORKSPACE;
        if (workspace && !aligned16(workspace)) return KDA_ERR_INVALID_ARGUMENT;
    }
    if (!have_tokens && !h_T) return KDA_OK;  // nothing to compute or write
    g_hip_error[0] = '\0';
    if (noalloc && need > 0) {
        // the library-held scratch of the current device: no allocation
        if (kda::noalloc_scratch(&workspace, g_hip_error, sizeof(g_hip_error)) != 0) return KDA_ERR_HIP;
        workspace_bytes = kda::kNoAllocScratchBytes;
    }

    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    if (kda::launch_chunk_fwd(a, stream, g_hip_error, sizeof(g_hip_error)) != 0)
        return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status_t decode_step_impl(const void *q, const void *k, const void *v, const void *log_alpha,
                              const void *beta, const void *w_write, float *S, void *o, int32_t B, int32_t H, int32_t d_k,
                              int32_t d_v, int32_t io_dtype, int32_t gate_dtype, void *stream,
                              bool prologue, float lo, int gate_mode) {
    if (!valid_dtype(io_dtype) || !valid_dtype(gate_dtype)) return KDA_ERR_UNSUPPORTED;
    if (B <= 0 || H <= 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (!sizes_fit(B, H, (int64_t)d_k * d_v)) return KDA_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !beta || !S || !o) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(o))
        return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned_to(beta, dsize(gate_dtype))) return KDA_ERR_INVALID_ARGUMENT;
    if (gate_mode == 0 && (!log_alpha || !aligned16(log_alpha))) return KDA_ERR_INVALID_ARGUMENT;
    if (gate_mode == 1 && !aligned_to(log_alpha, dsize(gate_dtype))) return KDA_ERR_INVALID_ARGUMENT;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.w_write = w_write; a.S = S; a.o = o;
    a.B = B; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.io_bf16 = io_dtype == KDA_BF16; a.gate_bf16 = gate_dtype == KDA_BF16;
    a.prologue = prologue; a.log_alpha_min = lo; a.gate_mode = gate_mode;
    if (!kda::decode_grids_fit(a)) return KDA_ERR_UNSUPPORTED;
    g_hip_error[0] = '\0';
    if (kda::launch_decode_step(a, stream, g_hip_error, sizeof(g_hip_error)) != 0)
        return KDA_ERR_HIP;
    return KDA_OK;
}

}  // namespace
