/*
 * libengram -- the Engram forward path on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a DEVICE pointer owned by the caller; the
 * library allocates nothing, keeps no pointer after a call returns and never
 * synchronises.  Every call validates its arguments on the host first: on an
 * error it returns a status and launches nothing.  Work is enqueued on
 * `stream` (a hipStream_t; NULL means the legacy default stream) and runs
 * asynchronously; a HIP launch failure is reported as ENGRAM_ERR_HIP.
 *
 * Data-dependent errors (a token id outside [0, vocab), a hash id outside
 * [0, num_embeddings)) cannot be seen on the host.  The kernels OR the
 * ENGRAM_ERRBIT_* flags into the optional device word `err` (uint32, caller
 * zeroes it; NULL = do not report) and still write well-defined output: a bad
 * token is treated as the pad id, and a bad row id gathers a row of zeros.
 * No kernel ever reads outside its inputs.
 *
 * Layouts are row-major and dense.  bf16 tensors are passed as uint16_t bit
 * patterns.  Names follow the pages that describe the method:
 *   [block] the DeepSeek V4.1 Engram block listing (constructor and forward);
 *   [gate]  the "Gate per stream" page (equations for a_k and g, in/out box);
 *   [docs]  the "Module engram" CPU-reference docs (four stages, structs,
 *           functions).
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum engram_status {
    ENGRAM_OK = 0,
    ENGRAM_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad shape */
    ENGRAM_ERR_UNSUPPORTED = 2,   /* geometry outside what the kernels handle */
    ENGRAM_ERR_WORKSPACE = 3,     /* workspace missing or too small */
    ENGRAM_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
    ENGRAM_ERR_TOO_LARGE = 5      /* the call needs more than the fixed scratch array */
} engram_status;

/* Bits OR-ed into the optional device error word. */
#define ENGRAM_ERRBIT_TOKEN 0x1u  /* a token id outside [0, vocab) (used as pad) */
#define ENGRAM_ERRBIT_HASH  0x2u  /* a computed hash id outside [0, num_embeddings) */
#define ENGRAM_ERRBIT_ROW   0x4u  /* gather saw a row id outside [0, num_embeddings) */

/* Geometry of one Engram layer ([block] constructor: ModelArgs dim, hc_mult,
 * norm_eps; EngramLayout num_embeddings, head_dim, max_ngram_size, n_heads).
 * Derived: n_hash_cols = (max_ngram_size - 1) * n_heads;
 *          K = n_hash_cols * head_dim (wkv input width);
 *          N = dim * (hc_mult + 1)     (wkv output width).
 * Supported: dim % 8 == 0 and 8 <= dim <= 32768; 1 <= hc_mult <= 8;
 * 2 <= max_ngram_size <= 16; n_heads >= 1 and n_hash_cols <= 1024;
 * head_dim % 32 == 0 and 32 <= head_dim <= 1024; 1 <= num_embeddings < 2^31;
 * vocab >= 1; norm_eps finite and >= 0. */
typedef struct engram_geometry {
    int32_t dim;             /* model width */
    int32_t hc_mult;         /* hyper-connection streams */
    int32_t max_ngram_size;  /* n-gram sizes 2..max_ngram_size */
    int32_t n_heads;         /* hash heads per n-gram size */
    int32_t head_dim;        /* table row width */
    int32_t vocab;           /* raw token ids are in [0, vocab) */
    int32_t pad_id;          /* compressed id used before position 0 */
    int32_t reserved;        /* must be 0 */
    int64_t num_embeddings;  /* table rows */
    float norm_eps;          /* eps inside each rsqrt of the gate */
    int32_t reserved2;       /* must be 0 */
} engram_geometry;

/* The hash tables, used exactly as given ([docs] EngramTables: token_map,
 * multipliers, primes, offsets; never recomputed).  Device pointers. */
typedef struct engram_hash_tables {
    const int32_t* token_map;  /* [vocab] raw id -> compressed id */
    const uint64_t* mult;      /* [n_hash_cols][max_ngram_size] per-lookback multipliers */
    const uint64_t* prime;     /* [n_hash_cols] modulus of each column */
    const uint64_t* offset;    /* [n_hash_cols] first table row of each column */
} engram_hash_tables;

const char* engram_status_string(engram_status s);

/* Checks a geometry against the supported ranges above. */
engram_status engram_check_geometry(const engram_geometry* g);

/* Stage 1: the n-gram hash ([docs] stage 1 and NgramHashState; [block]
 * forward's hash_ids argument).
 *   ids      int32 [B, T]   raw token ids of T new positions per sequence.
 *   state    int32 [B, max_ngram_size - 1] or NULL.  The compressed ids of the
 *            last max_ngram_size-1 positions seen, oldest first; a fresh
 *            sequence holds pad_id.  Read for the look-back before position 0
 *            of this call, then overwritten with the last max_ngram_size-1
 *            compressed ids (so prefill then decode equals one long prefill).
 *            NULL = fresh pad history and no update.
 *   hash_ids int32 [B, T, n_hash_cols] out.  Column col = (n-2)*n_heads + head
 *            for n-gram size n:  c_j = token_map[ids] (compressed, unsigned
 *            32-bit), mix = XOR_{k=0..n-1} c_{t-k} * mult[col][k] (mod 2^64),
 *            hash = mix % prime[col] + offset[col]  (unsigned 64-bit).
 *            A hash outside [0, num_embeddings) is written as -1 and flagged.
 * Bit-exact (integer). */
engram_status engram_hash(const engram_geometry* g, const engram_hash_tables* t,
                          int32_t* state, const int32_t* ids, int32_t B, int32_t T,
                          int32_t* hash_ids, uint32_t* err, void* stream);

/* Stage 1 for several Engram layers in one launch.  Each layer hashes with
 * its own tables and table size ([block] constructor: the layer's
 * layer_hash_index selects its num_embeddings; [docs] stage 1), while the
 * token ids, and so all the index arithmetic, are shared.
 *   geoms    n_layers geometries, equal in max_ngram_size, n_heads, vocab and
 *            pad_id (num_embeddings may differ; the other fields are unused).
 *   tables   n_layers table sets.
 *   states   NULL, or a host array of n_layers distinct device pointers, each
 *            as engram_hash's state for that layer.
 *   hash_ids int32 [n_layers, B, T, n_hash_cols] out; layer l's block is what
 *            engram_hash(geoms[l], tables[l], states[l], ...) writes.
 * 1 <= n_layers <= 32.  Bit-exact (integer); the error word collects every
 * layer's flags. */
engram_status engram_hash_layers(const engram_geometry* geoms,
                                 const engram_hash_tables* tables, int32_t n_layers,
                                 int32_t* const* states, const int32_t* ids, int32_t B,
                                 int32_t T, int32_t* hash_ids, uint32_t* err, void* stream);

/* Stage 2: gather and dequantise table rows ([docs] stage 2, embed_rows,
 * regen_table; [block] self.embed).
 *   table    uint8 [num_embeddings, head_dim]      fp8 e4m3fn codes.
 *   scales   uint8 [num_embeddings, head_dim / 32] e8m0 codes, one per 32-block.
 *   hash_ids int32 [n_tok, n_hash_cols].
 *   rows     bf16  [n_tok, n_hash_cols * head_dim] out: the fp32 product
 *            e4m3(v) * 2^(s-127) rounded to bf16 (nearest-even; NaN -> 0x7FC0).
 * Bit-exact. */
engram_status engram_gather(const engram_geometry* g, const uint8_t* table,
                            const uint8_t* scales, const int32_t* hash_ids, int64_t n_tok,
                            uint16_t* rows, uint32_t* err, void* stream);

/* Stage 3: the wkv projection ([docs] stage 3, linear_bf16; [block] self.wkv):
 * kv[m][n] = bf16( sum_k a[m][k] * w[n][k] ), fp32 accumulation on bf16 MFMA,
 * no bias; the final rounding is to nearest even, and a NaN result is a NaN
 * of unspecified sign and payload.
 *   a  bf16 [M, K];  w  bf16 [N, K] ([out, in]);  kv bf16 [M, N] out.
 * Columns [s*dim, (s+1)*dim) of kv are the key of stream s; the last dim
 * columns are the shared value. */
engram_status engram_wkv(const engram_geometry* g, const uint16_t* a, const uint16_t* w,
                         int64_t M, uint16_t* kv, void* stream);

/* Stages 2 and 3 fused ([docs] stages 2 and 3; [block]
 * self.wkv(self.embed(hash_ids).flatten(-2))): the projection with the row
 * gather as its A operand, kv = bf16( rows(hash_ids) @ w^T ), where rows is
 * exactly what engram_gather writes (each dequantised element is the same
 * bf16 value) and the sum is the one engram_wkv takes.  The bf16 rows never
 * reach memory.  Requires head_dim == 64 (one table row per 64-wide k-tile)
 * and, with P = n_hash_cols * roundup(M, 256): for M > 256, P * 64 < 2^31;
 * for M <= 256, P * 8 < 2^31 and num_embeddings * 64 < 2^32; otherwise
 * ENGRAM_ERR_UNSUPPORTED (use engram_gather + engram_wkv).
 *   table, scales, hash_ids as in engram_gather; w, kv as in engram_wkv.
 *   scratch  device memory of engram_wkv_gathered_scratch_size(g, M) bytes,
 *            256-byte aligned: per hash column and position (rounded up to
 *            256 positions), for M > 256 the row's 64 fp8 codes copied from
 *            the table, for M <= 256 its byte offset in the table (4 bytes),
 *            then its two scales as fp32 (8 bytes); then q*k in fp32;
 *            contents on entry do not matter.
 * An id outside [0, num_embeddings) reads as a zero row and sets
 * ENGRAM_ERRBIT_ROW in *err (if err is not NULL). */
size_t engram_wkv_gathered_scratch_size(const engram_geometry* g, int64_t M);
engram_status engram_wkv_gathered(const engram_geometry* g, const uint8_t* table,
                                  const uint8_t* scales, const int32_t* hash_ids, int64_t M,
                                  const uint16_t* w, uint16_t* kv, void* scratch,
                                  size_t scratch_bytes, uint32_t* err, void* stream);

/* Stage 4: gate and add ([docs] gate_and_add; [block] forward after the
 * projection; [gate] equations for a_k and g).  Per token and stream s:
 *   w = q[s]*k[s];  rstd = rsqrt(mean(h^2)+eps) * rsqrt(mean(key^2)+eps);
 *   a = sum(h*w*key) * rstd * dim^-0.5;
 *   g = sigmoid(copysign(sqrt(max(|a|, 1e-6)), a)),  0 where mask is 0;
 *   out = bf16(h + g*value); a masked position returns x bit-exactly.
 *   x    bf16 [n_tok, hc_mult, dim];  kv bf16 [n_tok, dim*(hc_mult+1)];
 *   q, k bf16 [hc_mult, dim];  mask uint8 [n_tok] or NULL (all live);
 *   out  bf16 [n_tok, hc_mult, dim] (may be the same buffer as x: then a
 *        masked position is not touched at all);
 *   gate fp32 [n_tok, hc_mult] or NULL.
 * fp32 arithmetic with fixed-order reductions (run-to-run deterministic).
 * The max in g keeps a NaN (as the block's elementwise clamp does): a NaN
 * or an infinity in a stream or its key that makes a NaN gives that stream
 * a NaN gate and an all-NaN out; every NaN written is 0x7FC0. */
engram_status engram_gate_add(const engram_geometry* g, const uint16_t* x, const uint16_t* kv,
                              const uint16_t* q, const uint16_t* k, const uint8_t* mask,
                              int64_t n_tok, uint16_t* out, float* gate, void* stream);

/* Fully fused prefill, stages 2-3 ([docs] stages 2-4; [block] forward; [gate]
 * equation for a_k): engram_wkv_gathered whose key columns are not stored but
 * reduced, per position m, stream s and 128-column block b of the stream, to
 *   part[m][s][b] = ( sum key^2, sum (h*w)*key ),  w = q*k,
 * over the block's columns, with key the bf16 value engram_wkv_gathered would
 * store and h = x[m][s]; fp32, products rounded before they are added.  The
 * value columns go to v.
 *   x bf16 [M, hc_mult, dim]; q, k bf16 [hc_mult, dim];
 *   v bf16 [M, dim] out;  part float2 [M, hc_mult, dim/128] out (8-byte aligned);
 *   scratch as in engram_wkv_gathered.
 * Supported for prefill-sized batches only: head_dim 64, dim % 256 == 0,
 * n_hash_cols % 3 == 0, at least two 256x256 key/value tiles per compute
 * unit, M*hc_mult*dim*2 < 2^32; otherwise ENGRAM_ERR_UNSUPPORTED
 * (engram_gate_partials_supported says which). */
int engram_gate_partials_supported(const engram_geometry* g, int64_t M);
engram_status engram_wkv_gate_partials(const engram_geometry* g, const uint8_t* table,
                                       const uint8_t* scales, const int32_t* hash_ids,
                                       int64_t M, const uint16_t* w, const uint16_t* x,
                                       const uint16_t* q, const uint16_t* k, uint16_t* v,
                                       float* part, void* scratch, size_t scratch_bytes,
                                       uint32_t* err, void* stream);

/* Stage 4 from the partial sums of engram_wkv_gate_partials: S_hh from x, S_kk
 * and S_hwk as the in-order sum over b of part[m][s][b], then a, g and out as
 * in engram_gate_add.  v bf16 [n_tok, dim]; other arguments as there. */
engram_status engram_gate_from_partials(const engram_geometry* g, const uint16_t* x,
                                        const uint16_t* v, const float* part,
                                        const uint8_t* mask, int64_t n_tok, uint16_t* out,
                                        float* gate, void* stream);

/* Bytes of workspace engram_forward needs for n_tok = B*T positions
 * (hash ids, gathered rows or the fused projection's scratch, kv, and the
 * live-position maps of a masked call). */
size_t engram_forward_workspace_size(const engram_geometry* g, int64_t n_tok);

/* The whole forward ([block] Engram.forward with the hash in front):
 * stage 1 -> 2 -> 3 -> 4 on one stream, stages 2 and 3 fused as in
 * engram_wkv_gathered where it applies.  Arguments as in the stage calls;
 * x, out: [B, T, hc_mult, dim]; ids, mask: [B, T]; gate: [B, T, hc_mult].
 * workspace: device memory of at least engram_forward_workspace_size bytes,
 * 256-byte aligned.
 * With a mask, where the fully fused path applies (see
 * engram_gate_partials_supported) only the live positions are hashed into
 * the projection: they are packed in order, and the projection's tiles past
 * the live count are skipped.  Masked positions still have their token ids
 * and hashes checked (ENGRAM_ERRBIT_TOKEN, ENGRAM_ERRBIT_HASH); as their rows
 * are never read they do not set ENGRAM_ERRBIT_ROW.  Every output is the same
 * as without the packing. */
engram_status engram_forward(const engram_geometry* g, const engram_hash_tables* t,
                             const uint8_t* table, const uint8_t* scales, const uint16_t* w,
                             const uint16_t* q, const uint16_t* k, int32_t* state,
                             const uint16_t* x, const int32_t* ids, const uint8_t* mask,
                             int32_t B, int32_t T, uint16_t* out, float* gate,
                             void* workspace, size_t workspace_bytes, uint32_t* err,
                             void* stream);

/* The forward from given hash ids, as [block] Engram.forward takes them
 * (x, hash_ids, token_mask): stages 2 -> 3 -> 4 with the same paths as
 * engram_forward (hash ids computed once for several layers by
 * engram_hash_layers can be fed to each layer's call).
 *   hash_ids int32 [n_tok, n_hash_cols]; x, out [n_tok, hc_mult, dim];
 *   mask uint8 [n_tok] or NULL; gate fp32 [n_tok, hc_mult] or NULL.
 * A hash id outside [0, num_embeddings) reads a zero row and sets
 * ENGRAM_ERRBIT_ROW (for a projected position).  The workspace is sized by
 * engram_forward_workspace_size.  Every output equals engram_forward's for
 * the ids engram_hash gives. */
engram_status engram_forward_hashed(const engram_geometry* g, const uint8_t* table,
                                    const uint8_t* scales, const uint16_t* w, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* x,
                                    const int32_t* hash_ids, const uint8_t* mask, int64_t n_tok,
                                    uint16_t* out, float* gate, void* workspace,
                                    size_t workspace_bytes, uint32_t* err, void* stream);

/* For callers that cannot allocate device memory, or pass none (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * engram_forward with its workspace taken from a fixed array the library
 * holds in device memory (ENGRAM_FIXED_SCRATCH_BYTES, 32 MiB, one copy per
 * GPU the library runs on, kept until the process ends).  The call allocates
 * nothing and frees nothing.  Arguments, outputs and errors are as in
 * engram_forward; every output equals engram_forward's for the same inputs.
 * A call whose engram_forward_workspace_size(g, B*T) exceeds the array
 * returns ENGRAM_ERR_TOO_LARGE and launches nothing (at dim 5120, hc 4 and 24
 * hash columns that is more than 600 positions: decode-sized batches fit).
 * The device that is current must be the stream's device.  Every call on a
 * GPU uses that GPU's one array, which keeps the last call's contents (the
 * forward needs none of them): calls that overlap on one GPU (other threads,
 * other streams) race and must be serialised by the caller. */
#define ENGRAM_FIXED_SCRATCH_BYTES (32u * 1024u * 1024u)
size_t engram_fixed_scratch_bytes(void);
engram_status engram_forward_noalloc(const engram_geometry* g, const engram_hash_tables* t,
                                     const uint8_t* table, const uint8_t* scales,
                                     const uint16_t* w, const uint16_t* q, const uint16_t* k,
                                     int32_t* state, const uint16_t* x, const int32_t* ids,
                                     const uint8_t* mask, int32_t B, int32_t T, uint16_t* out,
                                     float* gate, uint32_t* err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
