// Internal interfaces between the C ABI (api.hip) and the kernels.
// gfx950 only: wave64, bf16 MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

// bf16 <-> fp32 bit helpers (bf16 is the top half of an IEEE binary32).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even; NaN -> canonical 0x7FC0.  The add of
// 0x7FFF plus the kept LSB rounds ties to even, carries into the exponent
// when the mantissa overflows and reaches infinity past the largest finite
// value; subnormals round on the same integer grid.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct Geom {
    int dim, hc, max_ngram, n_heads, head_dim, n_cols, K, N;
    int vocab, pad_id;
    int64_t num_embeddings;
    float eps;
};

Geom make_geom(const engram_geometry& g);

hipError_t launch_hash(const Geom& g, const engram_hash_tables& t, int32_t* state,
                       const int32_t* ids, int B, int T, int32_t* hash_ids, uint32_t* err,
                       hipStream_t s);

// Several layers' stage 1 in one launch: layer l uses tables[l],
// num_embeddings[l] and states[l] (states NULL, or every entry set and
// distinct) and writes hash_ids + l * B*T*n_cols; the other geometry
// fields are shared.
constexpr int kMaxHashLayers = 32;
hipError_t launch_hash_layers(const Geom& g, const engram_hash_tables* tables,
                              const int64_t* num_embeddings, int n_layers, int32_t* const* states,
                              const int32_t* ids, int B, int T, int32_t* hash_ids, uint32_t* err,
                              hipStream_t s);

hipError_t launch_gather(const Geom& g, const uint8_t* table, const uint8_t* scales,
                         const int32_t* hash_ids, int64_t n_tok, uint16_t* rows, uint32_t* err,
                         hipStream_t s);

hipError_t launch_wkv(const uint16_t* a, const uint16_t* w, int64_t M, int N, int K,
                      uint16_t* kv, hipStream_t s);

// The gate's key-side reductions done in the projection's epilogue (fully
// fused prefill): for key columns the projection writes, per (position m,
// stream s, 128-column block b of the stream), the partial sums over that
// block of key^2 and (h*w)*key, w = q*k, with the key rounded to bf16 as it
// would be stored; key columns never reach memory.  The value columns go to
// C = v [M, dim].
struct GatePartials {
    const uint16_t* x;  // [M, hc, dim] bf16
    const uint16_t* q;  // [hc, dim] bf16
    const uint16_t* k;  // [hc, dim] bf16
    float2* part;       // [M, hc, dim / 128] (sum key^2, sum (h*w)*key)
    int dim, hc;
    const float* wqk;   // [hc, dim] q*k in fp32 (filled by the launcher)
    // Compacted rows (positions whose mask is False are left out): row r of
    // the projection is position rowmap[r] of x; only the first *m_live rows
    // hold positions, tiles past them are skipped.  Both null: dense.
    const int* m_live = nullptr;
    const int32_t* rowmap = nullptr;
};

// Compaction of the live (mask True) positions, in order: live_idx[m] = the
// position's compact row (or -1 when masked), rowmap[r] = the position of
// compact row r (M for r >= the live count, up to m_pad), *m_live = the
// live count.  One workgroup.
hipError_t launch_live_rows(const uint8_t* mask, int64_t M, int64_t m_pad, int32_t* live_idx,
                            int32_t* rowmap, int* m_live, hipStream_t s);

// Scratch of the fused projections, per (hash column c, padded row m):
//  * batches of more than 256 positions (256- and 128-wide tiles, each A row
//    read by many workgroups): the 64 fp8 codes of table row hash_ids[m][c],
//    copied there by the hash or prep kernel (zeros for a bad id and for the
//    padding rows past the last position), so that k-tile c of rows m0.. is
//    one contiguous run at a computed address;
//  * decode-sized batches (64-wide tiles): the table byte offset of that row
//    instead (kBadRowOffset, past any table, for a bad id or a padding row:
//    the buffer load then reads zeros); the projection fetches the row itself,
//    beside its weight stream;
// then the row's two block scales as fp32 (zero for a zero row), and q*k in
// fp32 per (stream, feature).
constexpr uint32_t kBadRowOffset = 0xFFFFFFC0u;
constexpr int64_t kOffsetRowsMax = 256;  // batches up to this size use row offsets
__host__ __device__ inline int64_t padded_rows(int64_t M) { return (M + 255) / 256 * 256; }
struct GatheredScratch {
    uint8_t* arows;  // [n_cols][m_pad][64], when M > kOffsetRowsMax
    uint32_t* aoff;  // [n_cols][m_pad], when M <= kOffsetRowsMax
    float2* scl;     // [n_cols][m_pad]
    float* wqk;      // [hc * dim]
    int64_t m_pad;
};
GatheredScratch gathered_scratch(const Geom& g, int64_t M, void* base);

// e8m0 code -> fp32 scale 2^(c-127), branch-free (code 0 is the subnormal
// 2^-127, 255 is NaN)
__device__ __forceinline__ float e8m0_scale(uint32_t c) {
    uint32_t b = c << 23;
    b = c == 0u ? 0x00400000u : b;
    b = c == 0xFFu ? 0x7FC00000u : b;
    return __uint_as_float(b);
}

// Stage 1 straight into the fused projections' scratch (the hash ids
// themselves are not written): for every position and hash column, the
// table row's codes (or its offset) and scales; q*k as well when q is given;
// the state updated as in launch_hash.
// With a mask, the live positions are packed in order: live_idx, rowmap and
// *m_live are written as by launch_live_rows (by that kernel first, or, for
// short single sequences, by the hash kernel itself), live positions go to
// their compact rows, masked ones are hashed (their token and hash checks
// still flag) but not placed, and the compact rows past the live count that
// the projection reads are zero (or bad) rows.
constexpr int64_t kFusedCompactionMax = 32768;
hipError_t launch_hash_prep(const Geom& g, const engram_hash_tables& t, int32_t* state,
                            const int32_t* ids, int B, int T, const uint8_t* table,
                            const uint8_t* scales,
                            const uint16_t* q, const uint16_t* k, void* scratch, uint32_t* err,
                            hipStream_t s, const uint8_t* mask = nullptr,
                            int32_t* live_idx = nullptr, int32_t* rowmap = nullptr,
                            int* m_live = nullptr);

// The fused projections' scratch from given hash ids [M][n_cols] (what the
// stage calls' own prep does); with q, also q*k; with live_idx and m_live
// (from launch_live_rows), live positions at their compact rows as in
// launch_hash_prep.
hipError_t launch_prep_scratch(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                               const uint8_t* scales, int64_t M, void* scratch, uint32_t* err, hipStream_t s,
                               const uint16_t* q = nullptr, const uint16_t* k = nullptr,
                               const int32_t* live_idx = nullptr, const int* m_live = nullptr);

// number of compute units of the current device (cached)
int cu_count();

// projection straight from hash ids (rows gathered as the GEMM's A operand)
bool gathered_supported(const Geom& g, int64_t M);
size_t gathered_scratch_bytes(const Geom& g, int64_t M);
// prepared: the scratch already holds the rows and scales (launch_hash_prep)
hipError_t launch_wkv_gathered(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                               const uint8_t* scales, const uint16_t* w, int64_t M, uint16_t* kv,
                               void* scratch, uint32_t* err, hipStream_t s,
                               bool prepared = false);

// The same projection with the gate's key reductions in its epilogue (see
// GatePartials); writes v [M, dim] and gp.part.  Only where
// gate_partials_supported(g, M).
bool gate_partials_supported(const Geom& g, int64_t M);
hipError_t launch_wkv_gate_partials(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                                    const uint8_t* scales, const uint16_t* w, int64_t M,
                                    const GatePartials& gp, uint16_t* v, void* scratch,
                                    uint32_t* err, hipStream_t s, bool prepared = false);

// Stage 4 from the partial sums: per (token, stream) S_hh from x, S_kk and
// S_hwk as the fixed-order sum of the dim/128 partials, then g and
// out = bf16(h + g*v).
// live_idx (with mask): v and part hold compacted rows, position m's at row
// live_idx[m]
hipError_t launch_gate_from_partials(const Geom& g, const uint16_t* x, const uint16_t* v,
                                     const float2* part, const uint8_t* mask, int64_t n_tok,
                                     uint16_t* out, float* gate, hipStream_t s,
                                     const int32_t* live_idx = nullptr);

hipError_t launch_gate_add(const Geom& g, const uint16_t* x, const uint16_t* kv,
                           const uint16_t* q, const uint16_t* k, const uint8_t* mask,
                           int64_t n_tok, uint16_t* out, float* gate, hipStream_t s);

// engram_forward split at its workspace: every other argument check, and the
// launches given a workspace of engram_forward_workspace_size bytes.
engram_status forward_check(const engram_geometry* g, const engram_hash_tables* t,
                            const uint8_t* table, const uint8_t* scales, const uint16_t* w,
                            const uint16_t* q, const uint16_t* k, const uint16_t* x,
                            const int32_t* ids, int32_t B, int32_t T, const uint16_t* out);
engram_status forward_launch(const engram_geometry* g, const engram_hash_tables* t,
                             const uint8_t* table, const uint8_t* scales, const uint16_t* w,
                             const uint16_t* q, const uint16_t* k, int32_t* state,
                             const uint16_t* x, const int32_t* ids, const uint8_t* mask,
                             int32_t B, int32_t T, uint16_t* out, float* gate, void* workspace,
                             uint32_t* err, void* stream);

}  // namespace engram
