// Varlen chunk plan shared by the chunkwise kernels: chunks are aligned to
// each sequence's start (the last chunk of a sequence may be partial), and a
// flat chunk index runs over the chunks of all sequences in order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {
namespace {

constexpr int kPlanChunk = 64;   // chunk length (tokens)

size_t plan_bytes(int64_t num_seqs) { return ((size_t)(num_seqs + 1) * 4 + 255) / 256 * 256; }


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
        if (n < N) cnt = (cu[n + 1] - cu[n] + kPlanChunk - 1) / kPlanChunk;
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
        t0 = cu[n] + (int64_t)kPlanChunk * (chunk - chunk_off[n]);
        const int64_t rem = cu[n + 1] - t0;
        nv = (int)(rem < kPlanChunk ? rem : kPlanChunk);
        return true;
    }
    const int64_t cps = (T + kPlanChunk - 1) / kPlanChunk;
    n = chunk / cps;
    const int64_t c = chunk % cps;
    t0 = n * T + (int64_t)kPlanChunk * c;
    const int64_t rem = T - (int64_t)kPlanChunk * c;
    nv = (int)(rem < kPlanChunk ? rem : kPlanChunk);
    return true;
}

}  // namespace
}  // namespace kda
