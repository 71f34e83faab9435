// Stage 1: the n-gram hash ("Module engram" docs, stage 1 and NgramHashState).
//
// Arithmetic is unsigned 64-bit: the wrapping multiply is built from 32-bit
// pieces by the compiler, the modulus is the exact 64-bit unsigned remainder.
//
// One kernel hashes and updates the carried state.  Only the first
// n_state = max_ngram_size-1 positions of a sequence read the state, so the
// work is split in two kinds of workgroups:
//  * body workgroups take every (position, column) item at t >= n_state, one
//    thread each, laid out so that the output stores are coalesced; they
//    never touch the state;
//  * head workgroups each own a few whole sequences: they hash those
//    sequences' first min(T, n_state) positions (every column), then, after
//    a workgroup barrier that orders all of this workgroup's state reads
//    before any write, one thread per sequence writes the new state (the
//    last n_state compressed ids).  No other workgroup reads those
//    sequences' state, so the in-place update is race-free.
// Without a state, every position reads the pad id and there are no head
// workgroups.
//
// Two output forms: hash ids [M][n_cols] (column fastest), or the fused
// projections' rows and scales [n_cols][m_pad] (row fastest: each item
// copies its table row's 64 codes there, or for decode-sized batches writes
// the row's table offset, with q*k beside them when asked).
#include "internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;

// Compressed id at position p (relative to this call) of sequence b.
// p < 0 reaches into the carried state (oldest first), or the pad id.
__device__ __forceinline__ uint32_t compressed_at(int p, int b, int T, int n_state,
                                                  const int32_t* __restrict__ ids,
                                                  const int32_t* __restrict__ token_map,
                                                  const int32_t* state, int vocab, int pad_id,
                                                  uint32_t* bad) {
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

struct HashArgs {
    const int32_t* token_map;
    const uint64_t* mult;
    const uint64_t* prime;
    const uint64_t* offset;
    int32_t* state;  // [B][n_state] or null
    const int32_t* ids;
    int B, T, n_cols, n_heads, max_ngram, vocab, pad_id;
    int64_t num_embeddings;
    uint32_t* err;
    // head workgroups: seq_per_head sequences each, after n_body body workgroups
    int n_body, seq_per_head;
    // hash-id form
    int32_t* hash_ids;
    // rows-and-scales form (arows, or aoff for decode-sized batches)
    const uint8_t* table;
    const uint8_t* scales;
    int64_t m_pad;
    uint8_t* arows;
    uint32_t* aoff;
    float2* scl;
    const uint16_t* q;
    const uint16_t* k;
    float* wqk;
    int nqk;
    // compacted rows (masked prefill): live positions go to row live_idx[m]
    const int32_t* live_idx;
    const int* m_live;
    // or the compaction done here (fuse_mask): each workgroup counts the live
    // positions before its rows itself; the maps are written as by
    // launch_live_rows
    const uint8_t* mask;
    int32_t* live_out;
    int32_t* rowmap_out;
    int* m_live_out;
    int fuse_mask, mask16;
};

// Hash id of column col at position t of sequence b (the unsigned 64-bit
// mix, reduced modulo the column's prime and moved by its offset); sets
// ENGRAM_ERRBIT_HASH and gives -1 when that lands outside the table.
__device__ __forceinline__ int32_t hash_at(const HashArgs& a, int b, int t, int col,
                                           uint32_t* bad) {
    const int n = 2 + col / a.n_heads;
    const int n_state = a.max_ngram - 1;
    uint64_t mix = 0;
    for (int k = 0; k < n; ++k) {
        uint32_t c = compressed_at(t - k, b, a.T, n_state, a.ids, a.token_map, a.state, a.vocab,
                                   a.pad_id, bad);
        mix ^= (uint64_t)c * a.mult[(int64_t)col * a.max_ngram + k];
    }
    const uint64_t h = mix % a.prime[col] + a.offset[col];
    if (h < (uint64_t)a.num_embeddings) return (int32_t)h;
    *bad |= ENGRAM_ERRBIT_HASH;
    return -1;
}

// A zero row (or a bad row offset) and zero scales at projection row r of
// column col: a bad id, or a padding row the projection reads past the last
// position.
__device__ __forceinline__ void zero_row(const HashArgs& a, int64_t r, int col) {
    const int64_t i = (int64_t)col * a.m_pad + r;
    if (a.arows) {
        uint4* dst = reinterpret_cast<uint4*>(a.arows + i * 64);
        const uint4 z = make_uint4(0, 0, 0, 0);
        dst[0] = z;
        dst[1] = z;
        dst[2] = z;
        dst[3] = z;
    } else {
        a.aoff[i] = kBadRowOffset;
    }
    a.scl[i] = make_float2(0.0f, 0.0f);
}

// Store the result of item (position m, column col) in the output form.  In
// the rows-and-scales form a hash outside the table is also a bad row, as
// it is when the ids pass through memory to the projection; with compacted
// rows a masked position is not placed (and its row never read).
// The table row (or its offset) and scales of hash id `id` at projection
// row r (the row's loads and the scales' go out together).
__device__ __forceinline__ void place(const HashArgs& a, int64_t r, int col, int32_t id,
                                      uint32_t* bad) {
    if (id < 0) {
        *bad |= ENGRAM_ERRBIT_ROW;
        zero_row(a, r, col);
        return;
    }
    const int64_t i = (int64_t)col * a.m_pad + r;
    const float2 sc = make_float2(e8m0_scale(a.scales[2 * (int64_t)id]),
                                  e8m0_scale(a.scales[2 * (int64_t)id + 1]));
    if (a.arows) {
        // four named values, all loads before the stores (a local array of
        // them ends up in scratch memory)
        const uint4* src = reinterpret_cast<const uint4*>(a.table + (int64_t)id * 64);
        const uint4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
        uint4* dst = reinterpret_cast<uint4*>(a.arows + i * 64);
        dst[0] = v0;
        dst[1] = v1;
        dst[2] = v2;
        dst[3] = v3;
    } else {
        a.aoff[i] = (uint32_t)id * 64u;
    }
    a.scl[i] = sc;
}

template <bool PREP>
__device__ __forceinline__ void emit(const HashArgs& a, int64_t m, int col, int32_t id,
                                     uint32_t* bad) {
    if (!PREP) {
        a.hash_ids[m * a.n_cols + col] = id;
        return;
    }
    int64_t r = m;
    if (a.live_idx && *a.m_live < a.B * (int64_t)a.T) {  // (all live: the identity)
        r = a.live_idx[m];
        if (r < 0) return;
    }
    place(a, r, col, id, bad);
}

// Nonzero bytes in a word.
__device__ __forceinline__ int live_bytes(uint32_t w) {
    const uint32_t z = ~(((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w | 0x7F7F7F7Fu);  // 0x80 per zero byte
    return 4 - __popc(z);
}

// Body workgroup of the fused compaction: rows m0 .. m0+255 of one column.
// Every thread takes part (two workgroup barriers), so nothing returns early.
__device__ __forceinline__ void body_fused(const HashArgs& a, int body_from, uint32_t* bad) {
    __shared__ int red[kThreads / 64], wl[kThreads / 64];
    const int64_t M = (int64_t)a.B * a.T;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t g0 = (int64_t)blockIdx.x * kThreads;
    const int col = (int)(g0 / a.m_pad);
    const int64_t m0 = g0 - (int64_t)col * a.m_pad;  // a multiple of 256, below M
    const int64_t m = m0 + tid;
    // live positions before this block (m0 is a multiple of 16)
    int cnt = 0;
    if (a.mask16) {
        for (int64_t j = 16 * (int64_t)tid; j < m0; j += 16 * kThreads) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.mask + j);
            cnt += live_bytes(v.x) + live_bytes(v.y) + live_bytes(v.z) + live_bytes(v.w);
        }
    } else {
        for (int64_t j = 4 * (int64_t)tid; j < m0; j += 4 * kThreads)
            cnt += live_bytes(*reinterpret_cast<const uint32_t*>(a.mask + j));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    const bool live = m < M && a.mask[m] != 0;
    const uint64_t bal = __ballot(live);
    if (lane == 0) {
        red[wv] = cnt;
        wl[wv] = __popcll(bal);
    }
    __syncthreads();
    int64_t pre = 0, blk = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        pre += red[w];
        blk += wl[w];
        before += w < wv ? wl[w] : 0;
    }
    const int64_t slot = pre + before + __popcll(bal & ((1ull << lane) - 1ull));
    if (col == 0) {
        if (m < M) a.live_out[m] = live ? (int32_t)slot : -1;
        if (live) a.rowmap_out[slot] = (int32_t)m;
    }
    if (m0 + kThreads >= M) {
        // the block holding the last position: the live count is known here;
        // rows tot .. ceil256(tot)-1 are the only rows past it the projection
        // reads, so they are the ones marked bad
        const int64_t tot = pre + blk;
        const int64_t r = tot + tid;
        if (r < (tot + 255) / 256 * 256) {
            zero_row(a, r, col);
            if (col == 0) a.rowmap_out[r] = (int32_t)M;
        }
        if (col == 0 && tid == 0) *a.m_live_out = (int)tot;
    }
    if (m < M) {
        const int b = (int)(m / a.T);
        const int t = (int)(m - (int64_t)b * a.T);
        if (t >= body_from) {
            const int32_t id = hash_at(a, b, t, col, bad);
            if (live) place(a, slot, col, id, bad);
        }
    }
}

template <bool PREP>
__device__ __forceinline__ void hash_work(const HashArgs& a) {
    const int n_state = a.max_ngram - 1;
    const int64_t M = (int64_t)a.B * a.T;
    // with a state, positions t < n_state belong to the head workgroups
    const int body_from = a.state ? n_state : 0;
    uint32_t bad = 0;
    if ((int)blockIdx.x < a.n_body) {
        const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        if (PREP && a.wqk)
            for (int64_t j = i; j < a.nqk; j += (int64_t)a.n_body * kThreads)
                a.wqk[j] = __uint_as_float((uint32_t)a.q[j] << 16) *
                           __uint_as_float((uint32_t)a.k[j] << 16);
        if constexpr (PREP) {
            if (a.fuse_mask) {
                body_fused(a, body_from, &bad);
                if (bad && a.err) atomicOr(a.err, bad);
                return;
            }
        }
        int64_t m;
        int col;
        if (PREP) {  // rows fastest, padded rows included
            if (i >= (int64_t)a.n_cols * a.m_pad) return;
            col = (int)(i / a.m_pad);
            m = i - (int64_t)col * a.m_pad;
            // row m holds no position from the row count on (M, or the live
            // count when compacted): a bad row
            if (m >= (a.live_idx ? (int64_t)*a.m_live : M)) zero_row(a, m, col);
            if (m >= M) return;
        } else {  // columns fastest
            if (i >= M * a.n_cols) return;
            col = (int)(i % a.n_cols);
            m = i / a.n_cols;
        }
        const int b = (int)(m / a.T);
        const int t = (int)(m - (int64_t)b * a.T);
        if (t < body_from) return;
        const int32_t id = hash_at(a, b, t, col, &bad);
        emit<PREP>(a, m, col, id, &bad);
    } else {
        const int b0 = ((int)blockIdx.x - a.n_body) * a.seq_per_head;
        const int nb = min(a.seq_per_head, a.B - b0);
        const int hh = min(a.T, n_state);
        const int items = nb * hh * a.n_cols;
        // the new state, read first so that its loads overlap the hash work
        // (n_state <= 15; the fully unrolled loops keep v in registers)
        uint32_t v[16];
        const bool writer = (int)threadIdx.x < nb;
        if (writer) {
            const int b = b0 + threadIdx.x;
            uint32_t ignored = 0;  // bad tokens are flagged by the hash itself
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j < n_state)
                    v[j] = compressed_at(a.T - n_state + j, b, a.T, n_state, a.ids, a.token_map,
                                         a.state, a.vocab, a.pad_id, &ignored);
        }
        for (int j = threadIdx.x; j < items; j += kThreads) {
            const int col = j % a.n_cols;
            const int r = j / a.n_cols;
            const int b = b0 + r / hh;
            const int t = r % hh;
            const int32_t id = hash_at(a, b, t, col, &bad);
            if (PREP && a.fuse_mask) {
                // one sequence (B = 1): the compact row of position t counts
                // the live positions before it
                if (a.mask[t] != 0) {
                    int slot = 0;
                    for (int u = 0; u < t; ++u) slot += a.mask[u] != 0;
                    place(a, slot, col, id, &bad);
                }
            } else {
                emit<PREP>(a, (int64_t)b * a.T + t, col, id, &bad);
            }
        }
        // every state read of these sequences is above this barrier
        __syncthreads();
        if (writer) {
            const int b = b0 + threadIdx.x;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j < n_state) a.state[(int64_t)b * n_state + j] = (int32_t)v[j];
        }
    }
    if (bad && a.err) atomicOr(a.err, bad);
}

template <bool PREP>
__global__ void __launch_bounds__(kThreads) hash_kernel(HashArgs a) {
    hash_work<PREP>(a);
}

// Several layers' hashes in one launch: blockIdx.y picks the layer, whose
// tables, state, table size and output replace the shared arguments'.
struct LayerTables {
    const int32_t* token_map;
    const uint64_t* mult;
    const uint64_t* prime;
    const uint64_t* offset;
    int32_t* state;
    int32_t* hash_ids;
    int64_t num_embeddings;
};
struct LayersArgs {
    HashArgs shared;
    LayerTables layer[kMaxHashLayers];
};
static_assert(sizeof(LayersArgs) <= 4096, "kernel argument budget");

__global__ void __launch_bounds__(kThreads) hash_layers_kernel(LayersArgs la) {
    HashArgs a = la.shared;
    const LayerTables& l = la.layer[blockIdx.y];
    a.token_map = l.token_map;
    a.mult = l.mult;
    a.prime = l.prime;
    a.offset = l.offset;
    a.state = l.state;
    a.hash_ids = l.hash_ids;
    a.num_embeddings = l.num_embeddings;
    hash_work<false>(a);
}

HashArgs base_args(const Geom& g, const engram_hash_tables& t, int32_t* state, const int32_t* ids,
                   int B, int T, uint32_t* err) {
    HashArgs a{};
    a.token_map = t.token_map;
    a.mult = t.mult;
    a.prime = t.prime;
    a.offset = t.offset;
    a.state = state;
    a.ids = ids;
    a.B = B;
    a.T = T;
    a.n_cols = g.n_cols;
    a.n_heads = g.n_heads;
    a.max_ngram = g.max_ngram;
    a.vocab = g.vocab;
    a.pad_id = g.pad_id;
    a.num_embeddings = g.num_embeddings;
    a.err = err;
    return a;
}

// Head workgroups: a few sequences each (up to one pass of the workgroup
// over their head items), so that decode-sized calls spread over several CUs.
int head_blocks(const Geom& g, int B, int T, int* seq_per_head) {
    const int hh = std::min(T, g.max_ngram - 1);
    const int per_seq = hh * g.n_cols;
    *seq_per_head = std::max(1, std::min(4, kThreads / std::max(per_seq, 1)));
    return (B + *seq_per_head - 1) / *seq_per_head;
}

}  // namespace

hipError_t launch_hash_prep(const Geom& g, const engram_hash_tables& t, int32_t* state,
                            const int32_t* ids, int B, int T, const uint8_t* table,
                            const uint8_t* scales,
                            const uint16_t* q, const uint16_t* k, void* scratch, uint32_t* err,
                            hipStream_t s, const uint8_t* mask, int32_t* live_idx,
                            int32_t* rowmap, int* m_live) {
    const int64_t M = (int64_t)B * T;
    if (M == 0) return hipSuccess;
    if (mask && (!live_idx || !rowmap || !m_live)) return hipErrorInvalidValue;
    const GatheredScratch gs = gathered_scratch(g, M, scratch);
    HashArgs a = base_args(g, t, state, ids, B, T, err);
    if (mask) {
        // Short sequences count the live positions in every workgroup (each
        // reads the mask up to its own rows); longer ones, several sequences
        // with a state, or a mask not 4-byte aligned take the one-workgroup
        // scan first.
        const bool fuse = M <= kFusedCompactionMax && (state == nullptr || B == 1) &&
                          ((uintptr_t)mask & 3u) == 0;
        if (fuse) {
            a.fuse_mask = 1;
            a.mask16 = ((uintptr_t)mask & 15u) == 0;
            a.mask = mask;
            a.live_out = live_idx;
            a.rowmap_out = rowmap;
            a.m_live_out = m_live;
        } else {
            const hipError_t e = launch_live_rows(mask, M, gs.m_pad, live_idx, rowmap, m_live, s);
            if (e != hipSuccess) return e;
            a.live_idx = live_idx;
            a.m_live = m_live;
        }
    }
    a.table = table;
    a.scales = scales;
    a.m_pad = gs.m_pad;
    a.arows = gs.arows;
    a.aoff = gs.aoff;
    a.scl = gs.scl;
    a.q = q;
    a.k = k;
    a.wqk = q ? gs.wqk : nullptr;
    a.nqk = g.hc * g.dim;
    const int64_t total = (int64_t)g.n_cols * gs.m_pad;
    a.n_body = (int)((total + kThreads - 1) / kThreads);
    const int heads = state ? head_blocks(g, B, T, &a.seq_per_head) : 0;
    hash_kernel<true><<<dim3((unsigned)(a.n_body + heads)), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_hash_layers(const Geom& g, const engram_hash_tables* tables,
                              const int64_t* num_embeddings, int n_layers, int32_t* const* states,
                              const int32_t* ids, int B, int T, int32_t* hash_ids, uint32_t* err,
                              hipStream_t s) {
    const int64_t total = (int64_t)B * T * g.n_cols;
    if (total == 0) return hipSuccess;
    if (n_layers < 1 || n_layers > kMaxHashLayers) return hipErrorInvalidValue;
    LayersArgs la{};
    la.shared = base_args(g, tables[0], nullptr, ids, B, T, err);
    la.shared.n_body = (int)((total + kThreads - 1) / kThreads);
    const int heads = states ? head_blocks(g, B, T, &la.shared.seq_per_head) : 0;
    for (int l = 0; l < n_layers; ++l) {
        la.layer[l] = LayerTables{tables[l].token_map, tables[l].mult,    tables[l].prime,
                                  tables[l].offset,    states ? states[l] : nullptr,
                                  hash_ids + (int64_t)l * total, num_embeddings[l]};
    }
    hash_layers_kernel<<<dim3((unsigned)(la.shared.n_body + heads), (unsigned)n_layers),
                         dim3(kThreads), 0, s>>>(la);
    return hipGetLastError();
}

hipError_t launch_hash(const Geom& g, const engram_hash_tables& t, int32_t* state,
                       const int32_t* ids, int B, int T, int32_t* hash_ids, uint32_t* err,
                       hipStream_t s) {
    const int64_t total = (int64_t)B * T * g.n_cols;
    if (total == 0) return hipSuccess;
    HashArgs a = base_args(g, t, state, ids, B, T, err);
    a.hash_ids = hash_ids;
    a.n_body = (int)((total + kThreads - 1) / kThreads);
    const int heads = state ? head_blocks(g, B, T, &a.seq_per_head) : 0;
    hash_kernel<false><<<dim3((unsigned)(a.n_body + heads)), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace engram
