// Host-only stand-ins for the HIP launchers and size queries behind the C ABI,
// so that kda_api.cpp's argument validation can be built with the address and
// undefined-behaviour sanitizers and driven on the CPU.  Each launch records
// itself and reads every field of its arguments; nothing touches device memory.
#include <stdio.h>
#include <string.h>

#include "kda_launch.h"

namespace kda {

int g_launches = 0;   // launches that reached a launcher
int g_fail_heads = 7; // calls with this head count report a HIP error

namespace {
template <typename A> int record(const A &a, char *err, size_t err_len) {
    volatile unsigned char sink = 0;   // read every byte of the argument block
    const unsigned char *p = reinterpret_cast<const unsigned char *>(&a);
    for (size_t i = 0; i < sizeof(A); ++i) sink ^= p[i];
    (void)sink;
    ++g_launches;
    if (a.H == g_fail_heads) {
        char msg[2048];
        memset(msg, 'x', sizeof(msg) - 1);   // longer than the error buffer
        msg[sizeof(msg) - 1] = '\0';
        snprintf(err, err_len, "%s", msg);
        return -1;
    }
    return 0;
}
}  // namespace

size_t chunk_fwd_workspace_bytes(const ChunkArgs &a) {
    return a.io_bf16 ? (size_t)a.total_tokens * (size_t)a.H * 16 + 256 : 0;
}
bool chunk_fwd_grids_fit(const ChunkArgs &a) { return a.num_seqs * (int64_t)a.H < ((int64_t)1 << 19); }
bool decode_grids_fit(const DecodeArgs &a) { return a.B * (int64_t)a.H < ((int64_t)1 << 24); }
int noalloc_scratch(void **ptr, char *, size_t) {
    alignas(256) static unsigned char scratch_stub[256];
    *ptr = scratch_stub;
    return 0;
}
int launch_chunk_fwd(const ChunkArgs &a, void *, char *err, size_t err_len) { return record(a, err, err_len); }
int launch_decode_step(const DecodeArgs &a, void *, char *err, size_t err_len) { return record(a, err, err_len); }

size_t chunk_bwd_workspace_bytes(const BwdArgs &a) { return (size_t)a.total_tokens * (size_t)a.H * 64 + 256; }
size_t gdn_chunk_bwd_workspace_bytes(const BwdArgs &a) { return chunk_bwd_workspace_bytes(a); }
size_t pro_chunk_bwd_workspace_bytes(const BwdArgs &a) { return 2 * chunk_bwd_workspace_bytes(a); }
bool chunk_bwd_grids_fit(const BwdArgs &a) { return a.num_seqs * (int64_t)a.H < ((int64_t)1 << 20); }
bool pro_chunk_bwd_grids_fit(const BwdArgs &a) { return chunk_bwd_grids_fit(a); }
int launch_chunk_bwd(const BwdArgs &a, void *, char *err, size_t err_len) { return record(a, err, err_len); }
int launch_gdn_chunk_bwd(const BwdArgs &a, void *, char *err, size_t err_len) { return record(a, err, err_len); }
int launch_pro_chunk_bwd(const BwdArgs &a, float, void *, char *err, size_t err_len) {
    return record(a, err, err_len);
}

}  // namespace kda
