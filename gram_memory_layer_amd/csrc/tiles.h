// Shared pieces of the MFMA GEMM kernels (gfx950): operand vector types,
// buffer descriptors, the LDS row swizzle and the XCD-aware tile order.
#pragma once

#include "internal.h"

namespace engram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int N_XCD = 8;    // MI355X: 8 XCDs; workgroups go round-robin over them
constexpr int GROUP_M = 4;  // M-tiles per group in the tile order

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // raw buffer: stride 0, num_records = bytes (reads past it return 0);
    // word 3 = 0x00020000, the gfx9 data format for raw dword access
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16-byte slot of logical chunk c (0..7) in a 128-byte LDS row: XOR with a
// row function that is a permutation on any 8 consecutive rows and maps the
// even and the odd rows of any 16 consecutive rows onto all 8 slots, so a
// fragment read (32 consecutive rows, one logical chunk) is free of bank
// conflicts for both 8- and 16-lane LDS issue groups.
__device__ __forceinline__ int slot128(int row, int c) {
    return c ^ ((row & 7) ^ ((row >> 3) & 1));
}

// K order inside a 64-wide k-tile.  K-step ks (0..3) of the 32x32x16 MFMA
// takes, in lane half h (lanes 32h .. 32h+31), the 8 values of 16-byte bf16
// chunk kchunk(ks, h) = 4*(ks/2) + 2h + ks%2, a permutation of the natural
// 2*ks + h.  The two k-steps 2j and 2j+1 of lane half h then cover the 16
// consecutive values 32j + 16h .. 32j + 16h + 15, which an fp8 operand holds
// in one 16-byte LDS chunk: a single 128-bit LDS read feeds two k-steps.
// Every projection kernel with 64-wide k-tiles uses this order, so they all
// form each output's sum in the same order.
__device__ __forceinline__ int kchunk(int ks, int h) { return 4 * (ks >> 1) + 2 * h + (ks & 1); }

// Two fp32 -> a packed bf16 pair (lo in the low half), round to nearest even,
// by the hardware convert (v_cvt_pk_bf16_f32): one instruction per pair.  It
// equals the integer rounding of f32_to_bf16 for every non-NaN input
// (checked over all 2^32 patterns, subnormals and infinities included); a NaN
// stays a NaN but keeps its sign and payload bits instead of becoming 0x7FC0.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Tile number L (in the XCD-contiguous order) -> output tile (mt, nt): the
// tiles are ordered in groups of GM M-tiles so that concurrent workgroups
// share A and W panels in their XCD's L2.
template <int GM = GROUP_M>
__device__ __forceinline__ void tile_at(int L, int tiles_m, int tiles_n, int* mt, int* nt) {
    const int group_size = GM * tiles_n;
    const int first_m = (L / group_size) * GM;
    const int gm = min(tiles_m - first_m, GM);
    *mt = first_m + (L % group_size) % gm;
    *nt = (L % group_size) / gm;
}

// Workgroup b -> output tile (mt, nt).  Workgroups are dealt to the 8 XCDs
// round-robin; each XCD takes a contiguous range of per_xcd tile numbers.
// Returns false for the padding workgroups.
template <int GM = GROUP_M>
__device__ __forceinline__ bool tile_of(int b, int per_xcd, int tiles_m, int tiles_n, int* mt,
                                        int* nt) {
    const int L = (b % N_XCD) * per_xcd + b / N_XCD;
    if (L >= tiles_m * tiles_n) return false;
    tile_at<GM>(L, tiles_m, tiles_n, mt, nt);
    return true;
}

}  // namespace engram
