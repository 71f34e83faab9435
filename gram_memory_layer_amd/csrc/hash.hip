// Stage 1: the n-gram hash ("Module engram" docs, stage 1 and NgramHashState).
//
// One thread per (sequence, position, column): consecutive threads write
// consecutive int32 hash ids, so the output is fully coalesced; the few
// token-id and token_map reads per thread are shared through L1/L2 by the
// n_cols threads of a position.  Arithmetic is unsigned 64-bit: the wrapping
// multiply is built from 32-bit pieces by the compiler, the modulus is the
// exact 64-bit unsigned remainder.
#include "internal.h"

namespace engram {
namespace {

// Compressed id at position p (relative to this call) of sequence b.
// p < 0 reaches into the carried state (oldest first), or the pad id.
__device__ __forceinline__ uint32_t compressed_at(int p, int b, int T, int n_state,
                                                  const int32_t* __restrict__ ids,
                                                  const int32_t* __restrict__ token_map,
                                                  const int32_t* __restrict__ state, int vocab,
                                                  int pad_id, uint32_t* bad) {
    if (p < 0) {
        if (state == nullptr) return (uint32_t)pad_id;
        return (uint32_t)state[(int64_t)b * n_state + (n_state + p)];
    }
    int32_t tok = ids[(int64_t)b * T + p];
    if (tok < 0 || tok >= vocab) {
        *bad |= ENGRAM_ERRBIT_TOKEN;
        return (uint32_t)pad_id;
    }
    return (uint32_t)token_map[tok];
}

__global__ void __launch_bounds__(256) hash_kernel(
    const int32_t* __restrict__ token_map, const uint64_t* __restrict__ mult,
    const uint64_t* __restrict__ prime, const uint64_t* __restrict__ offset,
    const int32_t* __restrict__ state, const int32_t* __restrict__ ids, int B, int T,
    int n_cols, int n_heads, int max_ngram, int vocab, int pad_id, int64_t num_embeddings,
    int32_t* __restrict__ hash_ids, uint32_t* __restrict__ err) {
    const int64_t total = (int64_t)B * T * n_cols;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int col = (int)(i % n_cols);
    const int64_t bt = i / n_cols;
    const int b = (int)(bt / T);
    const int t = (int)(bt % T);
    const int n = 2 + col / n_heads;
    const int n_state = max_ngram - 1;
    uint32_t bad = 0;
    uint64_t mix = 0;
    for (int k = 0; k < n; ++k) {
        uint32_t c = compressed_at(t - k, b, T, n_state, ids, token_map, state, vocab, pad_id, &bad);
        mix ^= (uint64_t)c * mult[(int64_t)col * max_ngram + k];
    }
    uint64_t h = mix % prime[col] + offset[col];
    int32_t out;
    if (h < (uint64_t)num_embeddings) {
        out = (int32_t)h;
    } else {
        out = -1;
        bad |= ENGRAM_ERRBIT_HASH;
    }
    hash_ids[i] = out;
    if (bad && err) atomicOr(err, bad);
}

// New state = the last n_state compressed ids after this call's T positions.
// One thread per sequence reads everything it needs before writing, so the
// in-place shift is race-free.
__global__ void __launch_bounds__(64) state_kernel(const int32_t* __restrict__ token_map,
                                                   const int32_t* __restrict__ ids, int B, int T,
                                                   int n_state, int vocab, int pad_id,
                                                   int32_t* state) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    uint32_t v[16];
    uint32_t bad = 0;
    for (int j = 0; j < n_state; ++j)
        v[j] = compressed_at(T - n_state + j, b, T, n_state, ids, token_map, state, vocab,
                             pad_id, &bad);
    for (int j = 0; j < n_state; ++j) state[(int64_t)b * n_state + j] = (int32_t)v[j];
}

}  // namespace

hipError_t launch_hash(const Geom& g, const engram_hash_tables& t, int32_t* state,
                       const int32_t* ids, int B, int T, int32_t* hash_ids, uint32_t* err,
                       hipStream_t s) {
    const int64_t total = (int64_t)B * T * g.n_cols;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hash_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(
        t.token_map, t.mult, t.prime, t.offset, state, ids, B, T, g.n_cols, g.n_heads,
        g.max_ngram, g.vocab, g.pad_id, g.num_embeddings, hash_ids, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || state == nullptr) return e;
    state_kernel<<<dim3((B + 63) / 64), dim3(64), 0, s>>>(t.token_map, ids, B, T, g.max_ngram - 1,
                                                          g.vocab, g.pad_id, state);
    return hipGetLastError();
}

}  // namespace engram
