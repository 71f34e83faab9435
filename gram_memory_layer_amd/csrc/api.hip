// The C ABI of libengram: argument validation, launch dispatch and the fused
// forward.  All checks happen on the host before anything is enqueued.
#include <math.h>
#include <string.h>

#include "internal.h"

namespace engram {

Geom make_geom(const engram_geometry& g) {
    Geom o;
    o.dim = g.dim;
    o.hc = g.hc_mult;
    o.max_ngram = g.max_ngram_size;
    o.n_heads = g.n_heads;
    o.head_dim = g.head_dim;
    o.n_cols = (g.max_ngram_size - 1) * g.n_heads;
    o.K = o.n_cols * g.head_dim;
    o.N = g.dim * (g.hc_mult + 1);
    o.vocab = g.vocab;
    o.pad_id = g.pad_id;
    o.num_embeddings = g.num_embeddings;
    o.eps = g.norm_eps;
    return o;
}

}  // namespace engram

using engram::Geom;

namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 31;

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

engram_status from_hip(hipError_t e) { return e == hipSuccess ? ENGRAM_OK : ENGRAM_ERR_HIP; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The forward's workspace, in order: hash ids; gathered rows or the fused
// projection's scratch (whichever is larger); kv (or v and the partial
// sums); the live-position maps.  engram_forward_workspace_size adds these up.
struct FwdWorkspace {
    int32_t* hash_ids;
    uint16_t* rows;
    uint16_t* kv;
    int32_t* live_idx;
    int32_t* rowmap;
    int* m_live;
};

FwdWorkspace carve(const Geom& gg, int64_t n_tok, void* workspace) {
    FwdWorkspace f;
    char* ws = (char*)workspace;
    f.hash_ids = (int32_t*)ws;
    ws += align256((size_t)n_tok * gg.n_cols * sizeof(int32_t));
    f.rows = (uint16_t*)ws;
    const size_t rb = (size_t)n_tok * gg.K * sizeof(uint16_t);
    const size_t sb = engram::gathered_scratch_bytes(gg, n_tok);
    ws += align256(rb > sb ? rb : sb);
    f.kv = (uint16_t*)ws;
    ws += align256((size_t)n_tok * gg.N * sizeof(uint16_t));
    f.live_idx = (int32_t*)ws;
    ws += align256((size_t)n_tok * sizeof(int32_t));
    f.rowmap = (int32_t*)ws;
    ws += align256((size_t)engram::padded_rows(n_tok) * sizeof(int32_t));
    f.m_live = (int*)ws;
    return f;
}

}  // namespace

namespace engram {

// Every argument check of engram_forward except the workspace's.
engram_status forward_check(const engram_geometry* g, const engram_hash_tables* t,
                            const uint8_t* table, const uint8_t* scales, const uint16_t* w,
                            const uint16_t* q, const uint16_t* k, const uint16_t* x,
                            const int32_t* ids, int32_t B, int32_t T, const uint16_t* out) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (t == nullptr || B < 0 || T < 0) return ENGRAM_ERR_INVALID_ARG;
    const int64_t n_tok = (int64_t)B * T;
    if (n_tok >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (n_tok == 0) return ENGRAM_OK;
    if (!t->token_map || !t->mult || !t->prime || !t->offset || !ids) return ENGRAM_ERR_INVALID_ARG;
    if (!table || !scales || !w || !q || !k || !x || !out) return ENGRAM_ERR_INVALID_ARG;
    if (((uintptr_t)table & 7u) != 0 || !aligned16(w) || !aligned16(q) || !aligned16(k) ||
        !aligned16(x) || !aligned16(out))
        return ENGRAM_ERR_INVALID_ARG;
    return ENGRAM_OK;
}

// The forward's launches on a checked call, with its workspace (at least
// engram_forward_workspace_size bytes, 256-byte aligned; nothing in it needs
// to hold anything on entry).
engram_status forward_launch(const engram_geometry* g, const engram_hash_tables* t,
                             const uint8_t* table, const uint8_t* scales, const uint16_t* w,
                             const uint16_t* q, const uint16_t* k, int32_t* state,
                             const uint16_t* x, const int32_t* ids, const uint8_t* mask,
                             int32_t B, int32_t T, uint16_t* out, float* gate, void* workspace,
                             uint32_t* err, void* stream) {
    const int64_t n_tok = (int64_t)B * T;
    const Geom gg = engram::make_geom(*g);
    const FwdWorkspace f = carve(gg, n_tok, workspace);
    int32_t* hash_ids = f.hash_ids;
    uint16_t* rows = f.rows;  // or the fused projection's scratch
    uint16_t* kv = f.kv;
    int32_t* live_idx = f.live_idx;
    int32_t* rowmap = f.rowmap;
    int* m_live = f.m_live;
    hipStream_t s = (hipStream_t)stream;
    // the fused gather + projection wherever its layout applies (64-wide
    // tiles up to 256 positions, 256-wide ones above); gather then the bf16
    // projection otherwise
    const bool fused = aligned16(table) && engram::gathered_supported(gg, n_tok);
    if (fused && engram::gate_partials_supported(gg, n_tok)) {
        // fully fused: the hash writes the projection's copied rows and
        // scales directly; the projection reduces the key columns into the
        // gate's partial sums and stores only the value; kv's region holds both
        // With a mask, only live positions are projected: they are packed
        // in order into the first rows (v and part then hold compact rows).
        uint16_t* v = kv;
        float2* part = reinterpret_cast<float2*>(
            reinterpret_cast<char*>(kv) + align256((size_t)n_tok * gg.dim * sizeof(uint16_t)));
        engram::GatePartials gp{x, q, k, part, gg.dim, gg.hc};
        if (mask) {
            gp.m_live = m_live;
            gp.rowmap = rowmap;
        }
        hipError_t e = engram::launch_hash_prep(gg, *t, state, ids, B, T, table, scales, q, k,
                                                rows, err, s, mask, live_idx, rowmap, m_live);
        if (e == hipSuccess)
            e = engram::launch_wkv_gate_partials(gg, nullptr, table, scales, w, n_tok, gp, v, rows,
                                                 err, s, /*prepared=*/true);
        if (e == hipSuccess)
            e = engram::launch_gate_from_partials(gg, x, v, part, mask, n_tok, out, gate, s,
                                                  mask ? live_idx : nullptr);
        return from_hip(e);
    }
    hipError_t e;
    if (fused) {
        e = engram::launch_hash_prep(gg, *t, state, ids, B, T, table, scales, nullptr, nullptr,
                                     rows, err, s);
        if (e == hipSuccess)
            e = engram::launch_wkv_gathered(gg, nullptr, table, scales, w, n_tok, kv, rows, err, s,
                                            /*prepared=*/true);
    } else {
        e = engram::launch_hash(gg, *t, state, ids, B, T, hash_ids, err, s);
        if (e == hipSuccess)
            e = engram::launch_gather(gg, table, scales, hash_ids, n_tok, rows, err, s);
        if (e == hipSuccess) e = engram::launch_wkv(rows, w, n_tok, gg.N, gg.K, kv, s);
    }
    if (e == hipSuccess) e = engram::launch_gate_add(gg, x, kv, q, k, mask, n_tok, out, gate, s);
    return from_hip(e);
}

}  // namespace engram

extern "C" {

const char* engram_status_string(engram_status s) {
    switch (s) {
        case ENGRAM_OK: return "ok";
        case ENGRAM_ERR_INVALID_ARG: return "invalid argument";
        case ENGRAM_ERR_UNSUPPORTED: return "unsupported geometry";
        case ENGRAM_ERR_WORKSPACE: return "workspace missing or too small";
        case ENGRAM_ERR_HIP: return "HIP runtime error";
        case ENGRAM_ERR_TOO_LARGE: return "call needs more than the fixed scratch array holds";
    }
    return "unknown status";
}

engram_status engram_check_geometry(const engram_geometry* g) {
    if (g == nullptr) return ENGRAM_ERR_INVALID_ARG;
    if (g->reserved != 0 || g->reserved2 != 0) return ENGRAM_ERR_INVALID_ARG;
    if (g->dim < 8 || g->dim > 32768 || g->dim % 8 != 0) return ENGRAM_ERR_UNSUPPORTED;
    if (g->hc_mult < 1 || g->hc_mult > 8) return ENGRAM_ERR_UNSUPPORTED;
    if (g->max_ngram_size < 2 || g->max_ngram_size > 16) return ENGRAM_ERR_UNSUPPORTED;
    if (g->n_heads < 1 || (int64_t)(g->max_ngram_size - 1) * g->n_heads > 1024)
        return ENGRAM_ERR_UNSUPPORTED;
    if (g->head_dim < 32 || g->head_dim > 1024 || g->head_dim % 32 != 0)
        return ENGRAM_ERR_UNSUPPORTED;
    if (g->num_embeddings < 1 || g->num_embeddings > INT32_MAX) return ENGRAM_ERR_UNSUPPORTED;
    if (g->vocab < 1) return ENGRAM_ERR_INVALID_ARG;
    if (!(g->norm_eps >= 0.0f) || !isfinite(g->norm_eps)) return ENGRAM_ERR_INVALID_ARG;
    return ENGRAM_OK;
}

engram_status engram_hash(const engram_geometry* g, const engram_hash_tables* t, int32_t* state,
                          const int32_t* ids, int32_t B, int32_t T, int32_t* hash_ids,
                          uint32_t* err, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (t == nullptr || B < 0 || T < 0) return ENGRAM_ERR_INVALID_ARG;
    if ((int64_t)B * T >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if ((int64_t)B * T == 0) return ENGRAM_OK;
    if (!t->token_map || !t->mult || !t->prime || !t->offset || !ids || !hash_ids)
        return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(*g);
    return from_hip(engram::launch_hash(gg, *t, state, ids, B, T, hash_ids, err,
                                        (hipStream_t)stream));
}

engram_status engram_hash_layers(const engram_geometry* geoms, const engram_hash_tables* tables,
                                 int32_t n_layers, int32_t* const* states, const int32_t* ids,
                                 int32_t B, int32_t T, int32_t* hash_ids, uint32_t* err,
                                 void* stream) {
    if (geoms == nullptr || tables == nullptr) return ENGRAM_ERR_INVALID_ARG;
    if (n_layers < 1 || n_layers > engram::kMaxHashLayers) return ENGRAM_ERR_INVALID_ARG;
    int64_t num_emb[engram::kMaxHashLayers];
    for (int l = 0; l < n_layers; ++l) {
        const engram_status st = engram_check_geometry(&geoms[l]);
        if (st != ENGRAM_OK) return st;
        // every field the hash reads, except the table size, is shared
        const engram_geometry& a = geoms[0];
        const engram_geometry& b = geoms[l];
        if (b.max_ngram_size != a.max_ngram_size || b.n_heads != a.n_heads ||
            b.vocab != a.vocab || b.pad_id != a.pad_id)
            return ENGRAM_ERR_INVALID_ARG;
        const engram_hash_tables& t = tables[l];
        if (!t.token_map || !t.mult || !t.prime || !t.offset) return ENGRAM_ERR_INVALID_ARG;
        num_emb[l] = b.num_embeddings;
        if (states) {
            if (states[l] == nullptr) return ENGRAM_ERR_INVALID_ARG;
            for (int j = 0; j < l; ++j)
                if (states[j] == states[l]) return ENGRAM_ERR_INVALID_ARG;  // updated in place
        }
    }
    if (B < 0 || T < 0) return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(geoms[0]);
    const int64_t per_layer = (int64_t)B * T * gg.n_cols;
    if ((int64_t)B * T >= kMaxTokens || per_layer * n_layers >= ((int64_t)1 << 40))
        return ENGRAM_ERR_INVALID_ARG;
    if (per_layer == 0) return ENGRAM_OK;
    if (!ids || !hash_ids) return ENGRAM_ERR_INVALID_ARG;
    return from_hip(engram::launch_hash_layers(gg, tables, num_emb, n_layers, states, ids, B, T,
                                               hash_ids, err, (hipStream_t)stream));
}

engram_status engram_gather(const engram_geometry* g, const uint8_t* table, const uint8_t* scales,
                            const int32_t* hash_ids, int64_t n_tok, uint16_t* rows,
                            uint32_t* err, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (n_tok < 0 || n_tok >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (n_tok == 0) return ENGRAM_OK;
    if (!table || !scales || !hash_ids || !rows) return ENGRAM_ERR_INVALID_ARG;
    if (((uintptr_t)table & 7u) != 0 || !aligned16(rows)) return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(*g);
    return from_hip(engram::launch_gather(gg, table, scales, hash_ids, n_tok, rows, err,
                                          (hipStream_t)stream));
}

engram_status engram_wkv(const engram_geometry* g, const uint16_t* a, const uint16_t* w,
                         int64_t M, uint16_t* kv, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (M < 0 || M >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (M == 0) return ENGRAM_OK;
    if (!a || !w || !kv) return ENGRAM_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(w) || ((uintptr_t)kv & 7u) != 0) return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(*g);
    return from_hip(engram::launch_wkv(a, w, M, gg.N, gg.K, kv, (hipStream_t)stream));
}

size_t engram_wkv_gathered_scratch_size(const engram_geometry* g, int64_t M) {
    if (engram_check_geometry(g) != ENGRAM_OK || M < 0) return 0;
    return engram::gathered_scratch_bytes(engram::make_geom(*g), M);
}

engram_status engram_wkv_gathered(const engram_geometry* g, const uint8_t* table,
                                  const uint8_t* scales, const int32_t* hash_ids, int64_t M,
                                  const uint16_t* w, uint16_t* kv, void* scratch,
                                  size_t scratch_bytes, uint32_t* err, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (M < 0 || M >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(*g);
    if (!engram::gathered_supported(gg, M)) return ENGRAM_ERR_UNSUPPORTED;
    if (M == 0) return ENGRAM_OK;
    if (!table || !scales || !hash_ids || !w || !kv) return ENGRAM_ERR_INVALID_ARG;
    if (!aligned16(table) || !aligned16(w) || !aligned16(kv) || ((uintptr_t)hash_ids & 3u) != 0)
        return ENGRAM_ERR_INVALID_ARG;
    if (scratch == nullptr || scratch_bytes < engram::gathered_scratch_bytes(gg, M) ||
        ((uintptr_t)scratch & 255u) != 0)
        return ENGRAM_ERR_WORKSPACE;
    return from_hip(engram::launch_wkv_gathered(gg, hash_ids, table, scales, w, M, kv, scratch,
                                                err, (hipStream_t)stream));
}

engram_status engram_gate_add(const engram_geometry* g, const uint16_t* x, const uint16_t* kv,
                              const uint16_t* q, const uint16_t* k, const uint8_t* mask,
                              int64_t n_tok, uint16_t* out, float* gate, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (n_tok < 0 || n_tok >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (n_tok == 0) return ENGRAM_OK;
    if (!x || !kv || !q || !k || !out) return ENGRAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(kv) || !aligned16(q) || !aligned16(k) || !aligned16(out))
        return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(*g);
    return from_hip(engram::launch_gate_add(gg, x, kv, q, k, mask, n_tok, out, gate,
                                            (hipStream_t)stream));
}

int engram_gate_partials_supported(const engram_geometry* g, int64_t M) {
    if (engram_check_geometry(g) != ENGRAM_OK || M < 1 || M >= kMaxTokens) return 0;
    return engram::gate_partials_supported(engram::make_geom(*g), M) ? 1 : 0;
}

engram_status engram_wkv_gate_partials(const engram_geometry* g, const uint8_t* table,
                                       const uint8_t* scales, const int32_t* hash_ids,
                                       int64_t M, const uint16_t* w, const uint16_t* x,
                                       const uint16_t* q, const uint16_t* k, uint16_t* v,
                                       float* part, void* scratch, size_t scratch_bytes,
                                       uint32_t* err, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (M < 0 || M >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (M == 0) return ENGRAM_OK;
    const Geom gg = engram::make_geom(*g);
    if (!engram::gate_partials_supported(gg, M)) return ENGRAM_ERR_UNSUPPORTED;
    if (!table || !scales || !hash_ids || !w || !x || !q || !k || !v || !part)
        return ENGRAM_ERR_INVALID_ARG;
    if (!aligned16(table) || !aligned16(w) || !aligned16(x) || !aligned16(q) || !aligned16(k) ||
        !aligned16(v) || ((uintptr_t)part & 7u) != 0 || ((uintptr_t)hash_ids & 3u) != 0)
        return ENGRAM_ERR_INVALID_ARG;
    if (scratch == nullptr || scratch_bytes < engram::gathered_scratch_bytes(gg, M) ||
        ((uintptr_t)scratch & 255u) != 0)
        return ENGRAM_ERR_WORKSPACE;
    const engram::GatePartials gp{x, q, k, reinterpret_cast<float2*>(part), gg.dim, gg.hc};
    return from_hip(engram::launch_wkv_gate_partials(gg, hash_ids, table, scales, w, M, gp, v,
                                                     scratch, err, (hipStream_t)stream));
}

engram_status engram_gate_from_partials(const engram_geometry* g, const uint16_t* x,
                                        const uint16_t* v, const float* part,
                                        const uint8_t* mask, int64_t n_tok, uint16_t* out,
                                        float* gate, void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (n_tok < 0 || n_tok >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (g->dim % 128 != 0) return ENGRAM_ERR_UNSUPPORTED;
    if (n_tok == 0) return ENGRAM_OK;
    if (!x || !v || !part || !out) return ENGRAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(v) || !aligned16(out) || ((uintptr_t)part & 7u) != 0)
        return ENGRAM_ERR_INVALID_ARG;
    const Geom gg = engram::make_geom(*g);
    return from_hip(engram::launch_gate_from_partials(gg, x, v,
                                                      reinterpret_cast<const float2*>(part), mask,
                                                      n_tok, out, gate, (hipStream_t)stream));
}

size_t engram_forward_workspace_size(const engram_geometry* g, int64_t n_tok) {
    if (engram_check_geometry(g) != ENGRAM_OK || n_tok <= 0) return 0;
    const Geom gg = engram::make_geom(*g);
    const size_t rows = (size_t)n_tok * gg.K * sizeof(uint16_t);
    const size_t scl = engram::gathered_scratch_bytes(gg, n_tok);
    // + the live-row maps of the masked fully fused path
    const size_t live = align256((size_t)n_tok * sizeof(int32_t)) +
                        align256((size_t)engram::padded_rows(n_tok) * sizeof(int32_t)) + 256;
    return align256((size_t)n_tok * gg.n_cols * sizeof(int32_t)) +
           align256(rows > scl ? rows : scl) + align256((size_t)n_tok * gg.N * sizeof(uint16_t)) +
           live;
}

engram_status engram_forward(const engram_geometry* g, const engram_hash_tables* t,
                             const uint8_t* table, const uint8_t* scales, const uint16_t* w,
                             const uint16_t* q, const uint16_t* k, int32_t* state,
                             const uint16_t* x, const int32_t* ids, const uint8_t* mask,
                             int32_t B, int32_t T, uint16_t* out, float* gate, void* workspace,
                             size_t workspace_bytes, uint32_t* err, void* stream) {
    const engram_status st =
        engram::forward_check(g, t, table, scales, w, q, k, x, ids, B, T, out);
    if (st != ENGRAM_OK || (int64_t)B * T == 0) return st;
    const size_t need = engram_forward_workspace_size(g, (int64_t)B * T);
    if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return ENGRAM_ERR_WORKSPACE;
    return engram::forward_launch(g, t, table, scales, w, q, k, state, x, ids, mask, B, T, out,
                                  gate, workspace, err, stream);
}

engram_status engram_forward_hashed(const engram_geometry* g, const uint8_t* table,
                                    const uint8_t* scales, const uint16_t* w, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* x, const int32_t* hash_ids,
                                    const uint8_t* mask, int64_t n_tok, uint16_t* out, float* gate,
                                    void* workspace, size_t workspace_bytes, uint32_t* err,
                                    void* stream) {
    engram_status st = engram_check_geometry(g);
    if (st != ENGRAM_OK) return st;
    if (n_tok < 0 || n_tok >= kMaxTokens) return ENGRAM_ERR_INVALID_ARG;
    if (n_tok == 0) return ENGRAM_OK;
    if (!hash_ids || !table || !scales || !w || !q || !k || !x || !out)
        return ENGRAM_ERR_INVALID_ARG;
    if (((uintptr_t)table & 7u) != 0 || !aligned16(w) || !aligned16(q) || !aligned16(k) ||
        !aligned16(x) || !aligned16(out))
        return ENGRAM_ERR_INVALID_ARG;
    const size_t need = engram_forward_workspace_size(g, n_tok);
    if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return ENGRAM_ERR_WORKSPACE;
    const Geom gg = engram::make_geom(*g);
    // the same workspace as engram_forward (its hash-id region unused)
    const FwdWorkspace f = carve(gg, n_tok, workspace);
    uint16_t* rows = f.rows;
    uint16_t* kv = f.kv;
    int32_t* live_idx = f.live_idx;
    int32_t* rowmap = f.rowmap;
    int* m_live = f.m_live;
    hipStream_t s = (hipStream_t)stream;
    const bool fused = aligned16(table) && engram::gathered_supported(gg, n_tok);
    hipError_t e = hipSuccess;
    if (fused && engram::gate_partials_supported(gg, n_tok)) {
        uint16_t* v = kv;
        float2* part = reinterpret_cast<float2*>(
            reinterpret_cast<char*>(kv) + align256((size_t)n_tok * gg.dim * sizeof(uint16_t)));
        engram::GatePartials gp{x, q, k, part, gg.dim, gg.hc};
        if (mask) {
            e = engram::launch_live_rows(mask, n_tok, engram::padded_rows(n_tok), live_idx,
                                         rowmap, m_live, s);
            gp.m_live = m_live;
            gp.rowmap = rowmap;
        }
        if (e == hipSuccess)
            e = engram::launch_prep_scratch(gg, hash_ids, table, scales, n_tok, rows, err, s, q, k,
                                            mask ? live_idx : nullptr, mask ? m_live : nullptr);
        if (e == hipSuccess)
            e = engram::launch_wkv_gate_partials(gg, nullptr, table, scales, w, n_tok, gp, v, rows,
                                                 err, s, /*prepared=*/true);
        if (e == hipSuccess)
            e = engram::launch_gate_from_partials(gg, x, v, part, mask, n_tok, out, gate, s,
                                                  mask ? live_idx : nullptr);
        return from_hip(e);
    }
    if (fused) {
        e = engram::launch_wkv_gathered(gg, hash_ids, table, scales, w, n_tok, kv, rows, err, s);
    } else {
        e = engram::launch_gather(gg, table, scales, hash_ids, n_tok, rows, err, s);
        if (e == hipSuccess) e = engram::launch_wkv(rows, w, n_tok, gg.N, gg.K, kv, s);
    }
    if (e == hipSuccess) e = engram::launch_gate_add(gg, x, kv, q, k, mask, n_tok, out, gate, s);
    return from_hip(e);
}

}  // extern "C"
