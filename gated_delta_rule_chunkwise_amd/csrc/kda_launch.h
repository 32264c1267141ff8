// Internal interface between the host-side C ABI (kda_api.cpp) and the HIP
// launchers (kda_chunk.hip, kda_chunk2.hip, kda_decode.hip).  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct ChunkArgs {
    const void *q, *k, *v, *log_alpha, *beta;
    const void *w_write;        // separate write strengths [.., H], or nullptr (beta writes)
    const float *h0;
    const int32_t *cu_seqlens;  // device, or nullptr (equal-length batch)
    void *o;
    float *h_T;
    int64_t num_seqs;           // N
    int64_t seq_len;            // T when cu_seqlens == nullptr
    int64_t total_tokens;       // B*T
    int32_t H, d_k, d_v;
    int32_t io_bf16, gate_bf16; // 1 = bf16, 0 = fp32
    int32_t varlen;             // cu_seqlens given (sequences packed along T)
    int32_t prologue;           // q, k, log_alpha, beta are raw projections
    float log_alpha_min;        // floor of log alpha under the prologue
    int32_t gate_mode;          // 0: log_alpha [.., d_k]; 1: [..] per (token, head); 2: none
    int32_t force_fused;        // bf16 at d_k = d_v = 128: the fused kernel for every batch shape
    void *workspace;
    size_t workspace_bytes;
};

struct DecodeArgs {
    const void *q, *k, *v, *log_alpha, *beta;
    const void *w_write;        // separate write strengths [B, H], or nullptr (beta writes)
    float *S;
    void *o;
    int64_t B;
    int32_t H, d_k, d_v;
    int32_t io_bf16, gate_bf16;
    int32_t prologue;           // q, k, log_alpha, beta are raw projections
    float log_alpha_min;        // floor of log alpha under the prologue
    int32_t gate_mode;          // 0: log_alpha [B, H, d_k]; 1: [B, H]; 2: none
};

// HIP launch limits: gridDim.x * blockDim.x below 2^32 work-items, and a
// second grid dimension of at most 65535 workgroups.
constexpr int64_t kMaxWorkItems = (int64_t)1 << 32;
constexpr int64_t kMaxGridY = 65535;
inline bool grid_fits(int64_t blocks, int64_t threads) { return blocks >= 0 && blocks * threads < kMaxWorkItems; }

// Both return 0 when the launch was enqueued, or -1 after a HIP error whose
// text is copied into err (err_len bytes, NUL-terminated).
int launch_chunk_fwd(const ChunkArgs &a, void *stream, char *err, size_t err_len);
int launch_decode_step(const DecodeArgs &a, void *stream, char *err, size_t err_len);
// Workspace for these arguments (pointers are not read).
size_t chunk_fwd_workspace_bytes(const ChunkArgs &a);
// Whether every launch of the call stays within the HIP launch limits (host
// check, made before any launch; pointers are not read).
bool chunk_fwd_grids_fit(const ChunkArgs &a);
bool decode_grids_fit(const DecodeArgs &a);

// Size of the library-held device scratch of the forward that allocates nothing.
constexpr size_t kNoAllocScratchBytes = (size_t)80 << 20;
// Device address of the current device's scratch (looked up on the first call
// per device); 0, or -1 after a HIP error whose text is copied into err.
int noalloc_scratch(void **ptr, char *err, size_t err_len);

struct BwdArgs {
    const void *q, *k, *v, *log_alpha, *beta;
    const float *h0;            // [N, H, d_k, d_v] or nullptr (zero state)
    const int32_t *cu_seqlens;  // device, or nullptr (equal-length batch)
    const void *d_o;            // gradient of o, io dtype
    const float *d_hT;          // gradient of h_T, or nullptr (zero)
    void *dq, *dk, *dv;         // io dtype
    void *dlog_alpha, *dbeta;   // gate dtype
    const void *w_write;        // separate write strengths (gate dtype; beta is then the erase
                                // strength), or nullptr: tied to beta
    void *dw_write;             // their gradient (with w_write; dbeta is then the erase strength's)
    float *dh0;                 // or nullptr (not wanted)
    int64_t num_seqs, seq_len, total_tokens;
    int32_t H, d_k, d_v;
    int32_t io_bf16, gate_bf16, varlen;
    int32_t qk_f32;             // q and k (and dq, dk) fp32 with bf16 v and dO (prologue pass)
    int32_t gate_mode;          // 0: log_alpha per key channel; 1: per (token, head); 2: none
    void *workspace;
    size_t workspace_bytes;
};

size_t chunk_bwd_workspace_bytes(const BwdArgs &a);
bool chunk_bwd_grids_fit(const BwdArgs &a);       // also the scalar-gate form
bool pro_chunk_bwd_grids_fit(const BwdArgs &a);
// Raw projections: q, k, log_alpha, beta of a are the raw inputs (and dq, dk,
// dlog_alpha, dbeta their gradients); lo is the gate floor.
size_t pro_chunk_bwd_workspace_bytes(const BwdArgs &a);
int launch_pro_chunk_bwd(const BwdArgs &a, float lo, void *stream, char *err, size_t err_len);
int launch_chunk_bwd(const BwdArgs &a, void *stream, char *err, size_t err_len);
// Scalar-gate form: log_alpha [.., H] (or nullptr: no decay), dlog_alpha likewise.
size_t gdn_chunk_bwd_workspace_bytes(const BwdArgs &a);
int launch_gdn_chunk_bwd(const BwdArgs &a, void *stream, char *err, size_t err_len);

}  // namespace kda
