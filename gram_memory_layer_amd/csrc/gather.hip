// Stage 2: gather and dequantise table rows ("Module engram" docs, stage 2 /
// embed_rows; the Engram block's self.embed).
//
// One thread per 8 output values: it reads 8 fp8 codes (8 bytes) of one
// table row plus that 32-block's scale byte and writes 16 bytes of bf16.
// Eight consecutive threads cover one 64-byte table row and one 128-byte
// output row, and consecutive rows (hash columns of a position) are adjacent
// in the output, so stores are fully coalesced (nontemporal: 2% faster at
// the T=32,768 shape).  The table reads are random 64-byte rows by
// construction.
#include "dequant.h"

namespace engram {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* __restrict__ table,
                                                     const uint8_t* __restrict__ scales,
                                                     const int32_t* __restrict__ hash_ids,
                                                     int64_t n_rows_out, int head_dim,
                                                     int64_t num_embeddings,
                                                     uint16_t* __restrict__ rows,
                                                     uint32_t* __restrict__ err) {
    const int per_row = head_dim / 8;  // threads per table row
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_rows_out * per_row) return;
    const int64_t r = i / per_row;
    const int j0 = (int)(i % per_row) * 8;
    const int64_t id = hash_ids[r];
    uint4 o;
    if (id < 0 || id >= num_embeddings) {
        o = make_uint4(0, 0, 0, 0);
        if (err) atomicOr(err, ENGRAM_ERRBIT_ROW);
    } else {
        const uint2 codes = *reinterpret_cast<const uint2*>(table + id * head_dim + j0);
        const float sc = e8m0_to_f32(scales[id * (head_dim / 32) + j0 / 32]);
        uint32_t p[4];
        dequant8(codes.x, codes.y, sc, p);
        o = make_uint4(p[0], p[1], p[2], p[3]);
    }
    const u32x4 u = {o.x, o.y, o.z, o.w};  // written once: nontemporal hint
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(rows + r * head_dim + j0));
}

}  // namespace

hipError_t launch_gather(const Geom& g, const uint8_t* table, const uint8_t* scales,
                         const int32_t* hash_ids, int64_t n_tok, uint16_t* rows, uint32_t* err,
                         hipStream_t s) {
    const int64_t n_rows_out = n_tok * g.n_cols;
    const int64_t total = n_rows_out * (g.head_dim / 8);
    if (total == 0) return hipSuccess;
    const int threads = 256;
    gather_kernel<<<dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s>>>(
        table, scales, hash_ids, n_rows_out, g.head_dim, g.num_embeddings, rows, err);
    return hipGetLastError();
}

}  // namespace engram
