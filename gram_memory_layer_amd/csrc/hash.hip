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

// Hash id of column col at position t of sequence b (the unsigned 64-bit
// mix, reduced modulo the column's prime and moved by its offset); sets
// ENGRAM_ERRBIT_HASH and gives -1 when that lands outside the table.
__device__ __forceinline__ int32_t hash_at(int b, int t, int col, int T, int n_heads,
                                           int max_ngram, const int32_t* __restrict__ ids,
                                           const int32_t* __restrict__ token_map,
                                           const uint64_t* __restrict__ mult,
                                           const uint64_t* __restrict__ prime,
                                           const uint64_t* __restrict__ offset,
                                           const int32_t* __restrict__ state, int vocab,
                                           int pad_id, int64_t num_embeddings, uint32_t* bad) {
    const int n = 2 + col / n_heads;
    const int n_state = max_ngram - 1;
    uint64_t mix = 0;
    for (int k = 0; k < n; ++k) {
        uint32_t c = compressed_at(t - k, b, T, n_state, ids, token_map, state, vocab, pad_id, bad);
        mix ^= (uint64_t)c * mult[(int64_t)col * max_ngram + k];
    }
    const uint64_t h = mix % prime[col] + offset[col];
    if (h < (uint64_t)num_embeddings) return (int32_t)h;
    *bad |= ENGRAM_ERRBIT_HASH;
    return -1;
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
    uint32_t bad = 0;
    hash_ids[i] = hash_at(b, t, col, T, n_heads, max_ngram, ids, token_map, mult, prime, offset,
                          state, vocab, pad_id, num_embeddings, &bad);
    if (bad && err) atomicOr(err, bad);
}

// The hash, written straight in the form the fused projections read: one
// thread per (column c, padded row m), m fastest, so the offset and scale
// stores are coalesced.  Row m = b*T + t; rows past B*T are padding.  A hash
// outside the table also counts as a bad row, as it does when the ids pass
// through memory.  When wqk is given, q*k in fp32 as well.
__global__ void __launch_bounds__(256) hash_prep_kernel(
    const int32_t* __restrict__ token_map, const uint64_t* __restrict__ mult,
    const uint64_t* __restrict__ prime, const uint64_t* __restrict__ offset,
    const int32_t* __restrict__ state, const int32_t* __restrict__ ids, int B, int T,
    int n_cols, int n_heads, int max_ngram, int vocab, int pad_id, int64_t num_embeddings,
    const uint8_t* __restrict__ scales, int64_t m_pad, uint32_t* __restrict__ aoff,
    float2* __restrict__ scl, uint32_t* __restrict__ err, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, float* __restrict__ wqk, int nqk) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wqk)
        for (int64_t j = i; j < nqk; j += (int64_t)gridDim.x * blockDim.x)
            wqk[j] = __uint_as_float((uint32_t)q[j] << 16) * __uint_as_float((uint32_t)k[j] << 16);
    if (i >= (int64_t)n_cols * m_pad) return;
    const int col = (int)(i / m_pad);
    const int64_t m = i - (int64_t)col * m_pad;
    uint32_t off = kBadRowOffset;
    float2 sc = make_float2(0.0f, 0.0f);
    uint32_t bad = 0;
    if (m < (int64_t)B * T) {
        const int b = (int)(m / T);
        const int t = (int)(m - (int64_t)b * T);
        const int32_t id = hash_at(b, t, col, T, n_heads, max_ngram, ids, token_map, mult, prime,
                                   offset, state, vocab, pad_id, num_embeddings, &bad);
        if (id >= 0) {
            off = (uint32_t)id * 64u;
            sc = make_float2(e8m0_scale(scales[2 * (int64_t)id]),
                             e8m0_scale(scales[2 * (int64_t)id + 1]));
        } else {
            bad |= ENGRAM_ERRBIT_ROW;
        }
    }
    aoff[i] = off;
    scl[i] = sc;
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

void launch_state(const Geom& g, const engram_hash_tables& t, int32_t* state, const int32_t* ids,
                  int B, int T, hipStream_t s) {
    state_kernel<<<dim3((B + 63) / 64), dim3(64), 0, s>>>(t.token_map, ids, B, T, g.max_ngram - 1,
                                                          g.vocab, g.pad_id, state);
}

}  // namespace

hipError_t launch_hash_prep(const Geom& g, const engram_hash_tables& t, int32_t* state,
                            const int32_t* ids, int B, int T, const uint8_t* scales,
                            const uint16_t* q, const uint16_t* k, void* scratch, uint32_t* err,
                            hipStream_t s) {
    const int64_t M = (int64_t)B * T;
    if (M == 0) return hipSuccess;
    const GatheredScratch gs = gathered_scratch(g, M, scratch);
    const int64_t total = (int64_t)g.n_cols * gs.m_pad;
    hash_prep_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(
        t.token_map, t.mult, t.prime, t.offset, state, ids, B, T, g.n_cols, g.n_heads,
        g.max_ngram, g.vocab, g.pad_id, g.num_embeddings, scales, gs.m_pad, gs.aoff, gs.scl, err,
        q, k, q ? gs.wqk : nullptr, g.hc * g.dim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || state == nullptr) return e;
    launch_state(g, t, state, ids, B, T, s);
    return hipGetLastError();
}

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
    launch_state(g, t, state, ids, B, T, s);
    return hipGetLastError();
}

}  // namespace engram
