// Drives every entry point of the C ABI through valid and invalid arguments,
// built with -fsanitize=address,undefined against host-only launcher stubs:
// checks each status code, that only valid calls reach a launcher, and that
// no check reads out of bounds or overflows (the sanitizers abort on either).
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

namespace kda {
extern int g_launches;
}

namespace {

alignas(256) unsigned char g_buf[1 << 12];   // stands in for device memory; never dereferenced
void *const P = g_buf;
void *at(int off) { return g_buf + off; }
int g_failures = 0;

void expect(int line, const char *what, kda_status_t rc, kda_status_t want, int launches, int want_launches) {
    if (rc != want || launches != want_launches) {
        fprintf(stderr, "line %d: %s -> %d (want %d), launches %d (want %d)\n", line, what, (int)rc, (int)want,
                launches, want_launches);
        ++g_failures;
    }
}
#define EXPECT(call, want, want_launches)                                                \
    do {                                                                                 \
        const int before_ = kda::g_launches;                                             \
        const kda_status_t rc_ = (call);                                                 \
        expect(__LINE__, #call, rc_, (want), kda::g_launches - before_, (want_launches)); \
    } while (0)

struct Fwd {
    const void *q = P, *k = P, *v = P, *la = P, *beta = P, *w = P;
    const float *h0 = nullptr;
    const int32_t *cu = nullptr;
    int32_t N = 0;
    void *o = P;
    float *hT = static_cast<float *>(P);
    int32_t B = 1, T = 256, H = 2, dk = 128, dv = 128;
    int32_t io = KDA_BF16, gt = KDA_BF16;
    void *ws = P;
    size_t wsb = (size_t)1 << 40;
    float lo = -20.f;
};
kda_status_t fwd(const Fwd &f) {
    return kda_chunk_fwd(f.q, f.k, f.v, f.la, f.beta, f.h0, f.cu, f.N, f.o, f.hT, f.B, f.T, f.H, f.dk, f.dv, f.io,
                         f.gt, f.ws, f.wsb, nullptr);
}
kda_status_t fwd_noalloc(const Fwd &f) {
    return kda_chunk_fwd_noalloc(f.q, f.k, f.v, f.la, f.beta, f.h0, f.cu, f.N, f.o, f.hT, f.B, f.T, f.H, f.dk, f.dv,
                                 f.io, f.gt, nullptr);
}
kda_status_t fwd_pro(const Fwd &f) {
    return kda_chunk_fwd_prologue(f.q, f.k, f.v, f.la, f.beta, f.lo, f.h0, f.cu, f.N, f.o, f.hT, f.B, f.T, f.H, f.dk,
                                  f.dv, f.io, f.gt, f.ws, f.wsb, nullptr);
}
kda_status_t fwd_gdn(const Fwd &f) {
    return kda_gdn_chunk_fwd(f.q, f.k, f.v, f.la, f.beta, f.h0, f.cu, f.N, f.o, f.hT, f.B, f.T, f.H, f.dk, f.dv, f.io,
                             f.gt, f.ws, f.wsb, nullptr);
}
kda_status_t fwd_dec(const Fwd &f) {
    return kda_chunk_fwd_decoupled(f.q, f.k, f.v, f.la, f.beta, f.w, f.h0, f.cu, f.N, f.o, f.hT, f.B, f.T, f.H, f.dk,
                                   f.dv, f.io, f.gt, f.ws, f.wsb, nullptr);
}

struct Dec {
    const void *q = P, *k = P, *v = P, *la = P, *beta = P, *w = P;
    float *S = static_cast<float *>(P);
    void *o = P;
    int32_t B = 4, H = 2, dk = 128, dv = 128;
    int32_t io = KDA_BF16, gt = KDA_BF16;
    float lo = -20.f;
};
kda_status_t dec(const Dec &d) {
    return kda_decode_step(d.q, d.k, d.v, d.la, d.beta, d.S, d.o, d.B, d.H, d.dk, d.dv, d.io, d.gt, nullptr);
}
kda_status_t dec_pro(const Dec &d) {
    return kda_decode_step_prologue(d.q, d.k, d.v, d.la, d.beta, d.lo, d.S, d.o, d.B, d.H, d.dk, d.dv, d.io, d.gt,
                                    nullptr);
}
kda_status_t dec_gdn(const Dec &d) {
    return kda_gdn_decode_step(d.q, d.k, d.v, d.la, d.beta, d.S, d.o, d.B, d.H, d.dk, d.dv, d.io, d.gt, nullptr);
}
kda_status_t dec_dec(const Dec &d) {
    return kda_decode_step_decoupled(d.q, d.k, d.v, d.la, d.beta, d.w, d.S, d.o, d.B, d.H, d.dk, d.dv, d.io, d.gt,
                                     nullptr);
}

struct Bwd {
    const void *q = P, *k = P, *v = P, *la = P, *beta = P, *w = P, *go = P;
    const float *h0 = nullptr, *ghT = nullptr;
    const int32_t *cu = nullptr;
    int32_t N = 0;
    void *dq = P, *dk_ = P, *dv_ = P, *dla = P, *db = P, *dw = P;
    float *dh0 = static_cast<float *>(P);
    int32_t B = 1, T = 128, H = 2, dk = 128, dv = 128;
    int32_t io = KDA_BF16, gt = KDA_BF16;
    void *ws = P;
    size_t wsb = (size_t)1 << 40;
    float lo = -20.f;
};
kda_status_t bwd(const Bwd &b) {
    return kda_chunk_bwd(b.q, b.k, b.v, b.la, b.beta, b.h0, b.cu, b.N, b.go, b.ghT, b.dq, b.dk_, b.dv_, b.dla, b.db,
                         b.dh0, b.B, b.T, b.H, b.dk, b.dv, b.io, b.gt, b.ws, b.wsb, nullptr);
}
kda_status_t bwd_gdn(const Bwd &b) {
    return kda_gdn_chunk_bwd(b.q, b.k, b.v, b.la, b.beta, b.h0, b.cu, b.N, b.go, b.ghT, b.dq, b.dk_, b.dv_, b.dla,
                             b.db, b.dh0, b.B, b.T, b.H, b.dk, b.dv, b.io, b.gt, b.ws, b.wsb, nullptr);
}
kda_status_t bwd_pro(const Bwd &b) {
    return kda_chunk_bwd_prologue(b.q, b.k, b.v, b.la, b.beta, b.lo, b.h0, b.cu, b.N, b.go, b.ghT, b.dq, b.dk_, b.dv_,
                                  b.dla, b.db, b.dh0, b.B, b.T, b.H, b.dk, b.dv, b.io, b.gt, b.ws, b.wsb, nullptr);
}
kda_status_t bwd_dec(const Bwd &b) {
    return kda_chunk_bwd_decoupled(b.q, b.k, b.v, b.la, b.beta, b.w, b.h0, b.cu, b.N, b.go, b.ghT, b.dq, b.dk_, b.dv_,
                                   b.dla, b.db, b.dw, b.dh0, b.B, b.T, b.H, b.dk, b.dv, b.io, b.gt, b.ws, b.wsb,
                                   nullptr);
}

template <typename A, typename F> A with(F &&set) {
    A a;
    set(a);
    return a;
}

void forward_cases() {
    typedef kda_status_t (*FwdFn)(const Fwd &);
    const FwdFn fns[] = {fwd, fwd_pro, fwd_gdn, fwd_dec};
    for (FwdFn f : fns) {
        EXPECT(f(Fwd()), KDA_OK, 1);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.q = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.v = at(4); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.o = at(8); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.beta = at(1); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.h0 = static_cast<const float *>(at(4)); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.dk = 96; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.io = 5; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.B = 0; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.T = -1; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.B = INT32_MAX; a.T = INT32_MAX; a.H = INT32_MAX; })),
               KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.cu = static_cast<const int32_t *>(P); a.N = 2; a.B = 2; })),
               KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.cu = static_cast<const int32_t *>(at(2)); a.N = 2; })),
               KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.cu = static_cast<const int32_t *>(P); a.N = 3; })), KDA_OK, 1);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.N = 3; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.B = 1 << 14; a.H = 32; a.T = 64; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.ws = nullptr; })), KDA_ERR_WORKSPACE, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.wsb = 100; })), KDA_ERR_WORKSPACE, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.ws = at(8); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.io = KDA_F32; a.ws = nullptr; a.wsb = 0; })), KDA_OK, 1);
        EXPECT(f(with<Fwd>([](Fwd &a) {
                   a.T = 0; a.q = a.k = a.v = a.la = a.beta = nullptr; a.o = nullptr; a.hT = nullptr;
               })),
               KDA_OK, 0);
        EXPECT(f(with<Fwd>([](Fwd &a) { a.T = 0; a.q = a.k = a.v = a.la = a.beta = nullptr; a.o = nullptr; })),
               KDA_OK, 1);   // h_T = h0 still written
    }
    EXPECT(fwd_pro(with<Fwd>([](Fwd &a) { a.lo = NAN; })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(fwd_pro(with<Fwd>([](Fwd &a) { a.lo = 1.f; })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(fwd_gdn(with<Fwd>([](Fwd &a) { a.la = nullptr; })), KDA_OK, 1);            // DeltaNet
    EXPECT(fwd_gdn(with<Fwd>([](Fwd &a) { a.la = at(2); })), KDA_OK, 1);              // bf16 gate: 2-byte alignment
    EXPECT(fwd_gdn(with<Fwd>([](Fwd &a) { a.la = at(1); })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(fwd_dec(with<Fwd>([](Fwd &a) { a.w = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(fwd_dec(with<Fwd>([](Fwd &a) { a.w = at(1); })), KDA_ERR_INVALID_ARGUMENT, 0);

    // the entry point without allocation: no workspace argument, a bounded scratch
    EXPECT(fwd_noalloc(Fwd()), KDA_OK, 1);
    EXPECT(fwd_noalloc(with<Fwd>([](Fwd &a) { a.q = at(4); })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(fwd_noalloc(with<Fwd>([](Fwd &a) { a.T = 1 << 20; a.H = 8; })), KDA_ERR_WORKSPACE, 0);
    EXPECT(fwd_noalloc(with<Fwd>([](Fwd &a) { a.T = 1 << 20; a.H = 8; a.io = KDA_F32; })), KDA_OK, 1);

    // a HIP error: reported, with its text truncated to the buffer and NUL-terminated
    EXPECT(fwd(with<Fwd>([](Fwd &a) { a.H = 7; })), KDA_ERR_HIP, 1);
    const size_t n = strlen(kda_last_hip_error());
    if (n == 0 || n >= 512) {
        fprintf(stderr, "HIP error text of length %zu\n", n);
        ++g_failures;
    }
    EXPECT(fwd(Fwd()), KDA_OK, 1);
    if (kda_last_hip_error()[0] != '\0') {
        fprintf(stderr, "HIP error text not cleared by a good call\n");
        ++g_failures;
    }
}

void decode_cases() {
    typedef kda_status_t (*DecFn)(const Dec &);
    const DecFn fns[] = {dec, dec_pro, dec_gdn, dec_dec};
    for (DecFn f : fns) {
        EXPECT(f(Dec()), KDA_OK, 1);
        EXPECT(f(with<Dec>([](Dec &a) { a.S = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Dec>([](Dec &a) { a.S = static_cast<float *>(at(4)); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Dec>([](Dec &a) { a.k = at(2); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Dec>([](Dec &a) { a.dv = 256; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Dec>([](Dec &a) { a.B = 0; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Dec>([](Dec &a) { a.B = INT32_MAX; a.H = INT32_MAX; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Dec>([](Dec &a) { a.B = 1 << 19; a.H = 32; })), KDA_ERR_UNSUPPORTED, 0);
    }
    EXPECT(dec_pro(with<Dec>([](Dec &a) { a.lo = INFINITY; })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(dec_gdn(with<Dec>([](Dec &a) { a.la = nullptr; })), KDA_OK, 1);
    EXPECT(dec_dec(with<Dec>([](Dec &a) { a.w = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
}

void backward_cases() {
    typedef kda_status_t (*BwdFn)(const Bwd &);
    const BwdFn fns[] = {bwd, bwd_pro, bwd_gdn, bwd_dec};
    for (BwdFn f : fns) {
        EXPECT(f(Bwd()), KDA_OK, 1);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.go = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.dq = at(4); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.db = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.dh0 = static_cast<float *>(at(8)); })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.dk = 32; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.H = 70000; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.B = INT32_MAX; a.T = INT32_MAX; })), KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.B = 1 << 15; a.H = 32; a.T = 64; })), KDA_ERR_UNSUPPORTED, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.ws = nullptr; })), KDA_ERR_WORKSPACE, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.wsb = 64; })), KDA_ERR_WORKSPACE, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.cu = static_cast<const int32_t *>(P); a.N = 2; })), KDA_OK, 1);
        EXPECT(f(with<Bwd>([](Bwd &a) { a.cu = static_cast<const int32_t *>(P); a.N = 0; })),
               KDA_ERR_INVALID_ARGUMENT, 0);
        EXPECT(f(with<Bwd>([](Bwd &a) {
                   a.T = 0; a.dh0 = nullptr; a.q = a.k = a.v = a.la = a.beta = a.go = nullptr;
               })),
               KDA_OK, 0);
    }
    EXPECT(bwd_pro(with<Bwd>([](Bwd &a) { a.lo = NAN; })), KDA_ERR_INVALID_ARGUMENT, 0);
    EXPECT(bwd_gdn(with<Bwd>([](Bwd &a) { a.la = nullptr; a.dla = nullptr; })), KDA_OK, 1);
    EXPECT(bwd_dec(with<Bwd>([](Bwd &a) { a.dw = nullptr; })), KDA_ERR_INVALID_ARGUMENT, 0);
}

void query_cases() {
    const int32_t big = INT32_MAX;
    const int32_t bf = KDA_BF16;
    // size queries: 0 for invalid or oversized arguments, never an overflow
    size_t (*const queries[])(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) = {
        kda_chunk_fwd_workspace_size, kda_chunk_bwd_workspace_size, kda_chunk_bwd_prologue_workspace_size,
        kda_gdn_chunk_bwd_workspace_size};
    for (auto q : queries) {
        if (q(big, big, big, 128, 128, 0, bf) != 0 || q(1, big, big, 128, 128, big, bf) != 0 ||
            q(0, 64, 2, 128, 128, 0, bf) != 0 || q(1, 64, 2, 96, 128, 0, bf) != 0 ||
            q(1, 64, 2, 128, 128, 0, 9) != 0 || q(1, 256, 2, 128, 128, 0, bf) == 0) {
            fprintf(stderr, "size query misbehaves\n");
            ++g_failures;
        }
    }
    if (kda_abi_version() != 1 || strcmp(kda_status_string(42), "KDA_ERR_UNKNOWN") != 0) {
        fprintf(stderr, "version or status string\n");
        ++g_failures;
    }
}

}  // namespace

int main() {
    forward_cases();
    decode_cases();
    backward_cases();
    query_cases();
    if (g_failures) {
        fprintf(stderr, "%d failure(s)\n", g_failures);
        return 1;
    }
    printf("abi driver: ok (%d launches)\n", kda::g_launches);
    return 0;
}
