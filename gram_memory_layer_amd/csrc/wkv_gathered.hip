// Stages 2 + 3 fused: the wkv projection with the row gather as its A loader
// ("Module engram" docs, stages 2 and 3; the Engram block's
// `self.wkv(self.embed(hash_ids).flatten(-2))`).
//
// With head_dim = 64, k-tile kt of the projection is exactly hash column kt:
// A[m][64 kt .. 64 kt + 63] is table row hash_ids[m][kt], dequantised.  So the
// A tile is fetched as fp8 rows straight into LDS by buffer DMA (one 64-byte
// row per output row) and converted to bf16 only after the LDS read, with the
// scaled fp8->bf16 convert instruction (bit-identical to the standalone
// dequant for every value and scale code).  Compared with a materialised bf16
// A this halves A's LDS writes and reads, drops the rows round trip through
// HBM, and leaves room for a 3-stage ring (loads two k-tiles ahead).
//
// A small prep kernel first regroups the rows per hash column:
//   arows[c][m]  the 64 fp8 codes of table row hash_ids[m][c] (zeros for a
//                bad id or a padding row), for batches of more than 256
//                positions: the 256- and 128-wide tiles then fetch each
//                k-tile's rows as contiguous runs at computed addresses (no
//                row offsets to load first, two rows per cache line);
//   aoff[c][m]   for decode-sized batches, the row's byte offset in the table
//                instead (past the table for a bad id or a padding row: reads
//                as 0): the 64-wide tiles fetch the rows themselves, beside
//                the weight stream, rather than wait for a copy;
//   scl[c][m]    the row's two 32-block scales 2^(s-127) as fp32,
// so that the projection does no id checks or scale decoding in its inner
// loop.  (The forward skips it: its hash kernel writes these arrays.)
//
// LDS: each of the three ring stages is made of 1 KiB blocks (one buffer DMA
// instruction each: 16 fp8 A rows, or 8 W rows of 128 bytes) plus 256 bytes
// of scales per wave; block b of stage s sits at (3b + s) KiB within its
// region, so a fragment's address in every stage and every fragment of a
// wave differ by constants and the inner loop computes almost no addresses.
// Within a block, 16-byte chunks are XOR-swizzled per row (slot64, slot128).
// Everything else (tile order, 32x32x16 MFMA, fenced k-steps, LDS-staged
// epilogue) is as in the bf16 kernel.
#include <type_traits>

#include "tiles.h"

namespace engram {
namespace {

constexpr int G_NS = 3;                   // stages in the LDS ring
// M-tiles per group in the tile order: 8 for the fully fused projection
// (fewer bytes fetched, same speed), 4 elsewhere (the plain persistent
// projection measured 5 us slower with 8)
constexpr int G_GROUP_M_FUSED = 8, G_GROUP_M = 4;

// 16-byte slot of logical chunk c (0..3) in a 64-byte LDS row.  A fragment
// read is one 16-byte chunk of 32 consecutive rows; the XOR term is a
// permutation of 0..3 over the even and over the odd rows of any aligned 8
// rows, and over each residue class mod 4 of any aligned 16 rows, so both
// 8- and 16-lane LDS issue groups of a 128-bit read hit distinct banks.
__device__ __forceinline__ int slot64(int row, int c) {
    return c ^ (((row >> 1) & 3) ^ ((row >> 3) & 1));
}


// One thread per (column c, padded row m), m fastest.  Padding rows m >= M
// get zero codes (or a bad offset) and zero scales.  With q and k given, the
// threads also write wqk = q*k in fp32 (exact: two 8-bit significands) for
// the gate partials.
__global__ void __launch_bounds__(256) prep_kernel(const int32_t* __restrict__ hash_ids,
                                                   int n_cols, int64_t M, int64_t m_pad,
                                                   const uint8_t* __restrict__ table,
                                                   const uint8_t* __restrict__ scales,
                                                   int64_t num_rows, uint8_t* __restrict__ arows,
                                                   uint32_t* __restrict__ aoff,
                                                   float2* __restrict__ scl,
                                                   uint32_t* __restrict__ err,
                                                   const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   float* __restrict__ wqk, int nqk,
                                                   const int32_t* __restrict__ live_idx,
                                                   const int* __restrict__ m_live) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wqk)
        for (int64_t j = i; j < nqk; j += (int64_t)gridDim.x * blockDim.x)
            wqk[j] = __uint_as_float((uint32_t)q[j] << 16) * __uint_as_float((uint32_t)k[j] << 16);
    if (i >= (int64_t)n_cols * m_pad) return;
    const int c = (int)(i / m_pad);
    const int64_t m = i - (int64_t)c * m_pad;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    // compacted rows: row r holds no position from the live count on
    if (live_idx && m >= *m_live) {
        if (arows) {
            uint4* dst = reinterpret_cast<uint4*>(arows + i * 64);
            dst[0] = zero;
            dst[1] = zero;
            dst[2] = zero;
            dst[3] = zero;
        } else {
            aoff[i] = kBadRowOffset;
        }
        scl[i] = make_float2(0.0f, 0.0f);
    }
    // the row as four named values (a local array of them ends up in
    // scratch memory)
    uint4 v0 = zero, v1 = zero, v2 = zero, v3 = zero;
    uint32_t off = kBadRowOffset;
    float2 sc = make_float2(0.0f, 0.0f);
    int64_t r = m;  // the projection row of position m
    if (m < M) {
        if (live_idx) {
            r = live_idx[m];
            if (r < 0) return;  // masked: not projected, its row never read
        }
        const int32_t id = hash_ids[m * n_cols + c];
        if (id >= 0 && id < num_rows) {
            if (arows) {
                const uint4* src = reinterpret_cast<const uint4*>(table + (int64_t)id * 64);
                v0 = src[0];
                v1 = src[1];
                v2 = src[2];
                v3 = src[3];
            }
            off = (uint32_t)id * 64u;
            sc = make_float2(e8m0_scale(scales[2 * (int64_t)id]),
                             e8m0_scale(scales[2 * (int64_t)id + 1]));
        } else if (err) {
            atomicOr(err, ENGRAM_ERRBIT_ROW);
        }
    } else if (live_idx) {
        return;  // (padding rows are filled above, as rows past the live count)
    }
    const int64_t o = (int64_t)c * m_pad + r;
    if (arows) {
        uint4* dst = reinterpret_cast<uint4*>(arows + o * 64);
        dst[0] = v0;
        dst[1] = v1;
        dst[2] = v2;
        dst[3] = v3;
    } else {
        aoff[o] = off;
    }
    scl[o] = sc;
}

// Ring hand-over: wait until at most N of this wave's vector loads are in
// flight and its LDS reads have returned, then a workgroup barrier.  The
// barrier is issued without a memory fence: a fence would also wait for the
// DMA of the k-tile two ahead, which is still allowed to be in flight; the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void handover() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

template <int V>
using IC = std::integral_constant<int, V>;

// Where a projection finds its fp8 A rows: the rows copied per hash column
// (256- and 128-wide tiles; aoff null), or the table itself at the row
// offsets aoff (64-wide tiles).  Buffer loads past src_bytes read zeros.
struct ASource {
    const uint8_t* src;    // arows [n_cols][m_pad][64], or the table
    const uint32_t* aoff;  // [n_cols][m_pad] table byte offsets, or null
    uint32_t src_bytes;
};

// One workgroup's work.
//   P = false: one output tile; L is the number of k-tiles after the steady
//     loop (nk <= 2 ? nk : 3 + nk % 3), a template parameter so that each
//     kernel ends in one straight-line sequence of k-tiles (branching between
//     several leaves the register allocator spilling).
//   P = true (persistent): a sequence of tiles, every one full-width in N and
//     nk a multiple of 3.  The k-tile pipeline runs on across tiles: the
//     last k-tiles of a tile already load the first ones of the next, and a
//     tile's output is staged through the ring stage that is free at that
//     point, so neither the start-up latency of a tile nor its stores stall
//     the matrix pipe for long.  The last tile loads its own first k-tiles a
//     second time (harmless; they land before the workgroup ends).
//   G (persistent only, gp set): tiles of key columns (n0 < hc*dim)
//     end in the gate's partial sums instead of a store; value columns go to
//     C at column n - hc*dim.
// A rows: copied rows for BT >= 128, table rows at loaded offsets for BT = 64
// (ASource).
template <int BT, int WMV, int WNV, int L, bool P, bool G = false>
__device__ __forceinline__ void gathered_tile(const ASource as,
                                              const float2* __restrict__ scl, int n_cols,
                                              int64_t m_pad, const uint16_t* __restrict__ W,
                                              int64_t M, int N, uint16_t* __restrict__ C,
                                              int64_t ldc, int tiles_m, int tiles_n, int per_xcd,
                                              const GatePartials& gp, uint8_t* smem) {
    constexpr int NW = WMV * WNV;
    constexpr int WM = BT / WMV, WN = BT / WNV;
    constexpr int TI = WM / 32, TJ = WN / 32;
    constexpr int NA = BT / 16 / NW;  // fp8 A DMA instructions per wave (16 rows each)
    constexpr int NB = BT / 8 / NW;   // W DMA instructions per wave (8 rows each)
    static_assert(BT / NW == 32, "one scale DMA of 32 rows per wave");
    static_assert(NA >= 1 && NB >= 1 && TI >= 1 && TJ % 2 == 0, "tile shape");
    constexpr int OFF_SC = (BT / 16) * G_NS * 1024;
    constexpr int OFF_W = OFF_SC + NW * G_NS * 256;
    constexpr int OFF_WQK = OFF_W + (BT / 8) * G_NS * 1024;  // q*k, 512 bytes per wave (G only)
    constexpr int NLOAD = NA + 1 + NB;  // DMA per wave per k-tile
    constexpr bool CA = BT >= 128;      // copied rows (else table rows at offsets)
    constexpr int NIDS = CA ? 0 : NA;   // row-offset loads per wave per k-tile

    const int K = n_cols * 64;
    const int nk = n_cols;
    // current tile (m0c, n0c) and the next one of this workgroup (itself at
    // the end of the sequence)
    const int xcd = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD;
    const int nwg = gridDim.x / N_XCD;
    // Persistent order.  Plain projection: each XCD walks its contiguous range
    // of tile numbers.  With the gate partials (key tiles cost more than value
    // tiles): round q of the machine takes tile numbers q*grid .. q*grid+grid-1,
    // the key tiles first, so every workgroup gets the same mix; within a
    // round an XCD's workgroups take consecutive numbers (shared panels).
    const int n_key = G ? (gp.hc * gp.dim) / BT : 0;  // key column tiles
    auto tile_num = [&](int q) {
        return G ? q * (int)gridDim.x + xcd * nwg + slot : xcd * per_xcd + slot + q * nwg;
    };
    auto tile_valid = [&](int q) {
        if constexpr (G) return tile_num(q) < tiles_m * tiles_n;
        const int idx = slot + q * nwg;
        return idx < per_xcd && xcd * per_xcd + idx < tiles_m * tiles_n;
    };
    auto tile_coords = [&](int q, int* mt, int* nt) {
        const int t = tile_num(q);
        if (G && t < tiles_m * n_key) {
            tile_at<G_GROUP_M_FUSED>(t, tiles_m, n_key, mt, nt);
        } else if (G) {
            tile_at<G_GROUP_M_FUSED>(t - tiles_m * n_key, tiles_m, tiles_n - n_key, mt, nt);
            *nt += n_key;
        } else {
            tile_at<G_GROUP_M>(t, tiles_m, tiles_n, mt, nt);
        }
    };
    // compacted rows: only the first *gp.m_live rows hold positions; the
    // persistent order is laid over just the tiles that reach them, a single
    // tile past them ends at once
    const int m_live = gp.m_live ? *gp.m_live : 0;
    if (P && gp.m_live) tiles_m = min(tiles_m, (m_live + BT - 1) / BT);
    // every position live: the row map is the identity, skip its loads
    const int32_t* rowmap = (gp.rowmap && m_live < M) ? gp.rowmap : nullptr;
    int m0c, n0c, m0n, n0n;
    {
        int mt, nt;
        if constexpr (P) {
            if (!tile_valid(0)) return;
            tile_coords(0, &mt, &nt);
        } else {
            if (!tile_of<G_GROUP_M>(blockIdx.x, per_xcd, tiles_m, tiles_n, &mt, &nt)) return;
            if (gp.m_live && mt * BT >= m_live) return;
        }
        m0c = m0n = mt * BT;
        n0c = n0n = nt * BT;
    }
    auto set_next = [&](int q) {
        if (tile_valid(q)) {
            int mt, nt;
            tile_coords(q, &mt, &nt);
            m0n = mt * BT;
            n0n = nt * BT;
        } else {
            m0n = m0c;
            n0n = n0c;
        }
    };
    if constexpr (P) set_next(1);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WNV, wn = wave % WNV;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(as.src, as.src_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(as.aoff, CA ? 0u : (uint32_t)(n_cols * m_pad * 4));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(scl, (uint32_t)(n_cols * m_pad * 8));
    // W rows n0 .. n0+BT-1 (rows past N read as zeros)
    auto w_rsrc = [&](int n0x) {
        return make_rsrc(W + (int64_t)n0x * K, (uint32_t)(min(BT, N - n0x) * K * 2));
    };
    const int col_a = (int)(m_pad * 64);  // arows bytes per hash column
    const int col_o = (int)(m_pad * 4);   // aoff bytes per hash column
    const int col_s = (int)(m_pad * 8);   // scl bytes per hash column

    // DMA lanes.  fp8 A instruction i fills block NW*i + wave: rows
    // 16*(NW*i + wave) + lane/4, lane%4 picking the 16-byte slot (which holds
    // logical chunk slot64(row, lane%4)).  The scale instruction moves the 32
    // rows x 2 fp32 of rows 32*wave .. 32*wave+31.  W instruction i fills
    // block NW*i + wave: rows 8*(NW*i + wave) + lane/8.
    // av: copied rows, the lane's byte within the k-tile's rows (+ (kt * m_pad
    // + m0) * 64 in the scalar offset); table rows, the lane's aoff entry
    // (+ kt * m_pad * 4 + m0 * 4 likewise) and ach its 16-byte chunk
    uint32_t av[NA], ach[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int row = 16 * (NW * i + wave) + (lane >> 2);
        ach[i] = (uint32_t)slot64(row, lane & 3) * 16u;
        av[i] = CA ? (uint32_t)(row * 64) + ach[i] : (uint32_t)(row * 4);
    }
    const uint32_t sc_v = (uint32_t)(32 * wave * 8 + lane * 4);  // + m0*8 likewise
    uint32_t wvoff[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int row = (NW * i + wave) * 8 + (lane >> 3);
        wvoff[i] = (uint32_t)(row * K * 2 + slot128(row, lane & 7) * 16);
    }

    uint32_t id_a[NA];  // table rows: byte offsets of the next k-tile to fetch
    auto load_offs = [&](int kt, int m0x) {
        if constexpr (!CA)
#pragma unroll
            for (int i = 0; i < NA; ++i)
                id_a[i] = __builtin_amdgcn_raw_buffer_load_b32(ro, av[i], kt * col_o + m0x * 4, 0);
    };
    // part 0: the fp8 rows and the scales; parts 1 and 2: the two halves of
    // the W rows (spread over the k-tile's first three k-steps).  ia: the
    // rows' table offsets (table rows only)
    auto issue_dma = [&](int kt, auto sd, const uint32_t* ia, int m0x, int n0x, auto partc) {
        constexpr int SD = decltype(sd)::value;
        constexpr int PART = decltype(partc)::value;
        if constexpr (PART == 0) {
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                lds_void* dst = (lds_void*)(smem + ((NW * i + wave) * G_NS + SD) * 1024);
                if constexpr (CA)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, av[i],
                                                             kt * col_a + m0x * 64, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, ia[i] + ach[i], 0, 0, 0);
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_void*)(smem + OFF_SC + (wave * G_NS + SD) * 256), 4, sc_v,
                kt * col_s + m0x * 8, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rw = w_rsrc(n0x);
            constexpr int I0 = PART == 1 ? 0 : NB / 2, I1 = PART == 1 ? NB / 2 : NB;
#pragma unroll
            for (int i = I0; i < I1; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_void*)(smem + OFF_W + ((NW * i + wave) * G_NS + SD) * 1024), 16,
                    wvoff[i], kt * 128, 0, 0);
        }
    };

    // Fragment reads.  Row wm*WM + 32i + lrow of A lies in block
    // (wm*WM + lrow)/16 + 2i, W row wn*WN + 32j + lrow in block
    // (wn*WN + lrow)/8 + 4j; both swizzles depend on the row mod 16 only, so
    // one base address per lane serves every fragment and stage.  K order
    // (kchunk): lane half h takes, over k-steps 2j' and 2j'+1, fp8 values
    // 32j' + 16h .. +15 = logical chunk 2j' + h of its row, read once; both
    // lie in 32-block j', whose scale comes with them.
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int r16 = lrow & 15;
    const uint32_t a_base =
        (uint32_t)(((wm * WM + lrow) >> 4) * G_NS * 1024 + r16 * 64 + slot64(r16, lhalf) * 16);
    const uint32_t s_base = (uint32_t)(OFF_SC + ((wm * WM) >> 5) * G_NS * 256 + lrow * 8);
    const uint32_t w_base = (uint32_t)(OFF_W + ((wn * WN + lrow) >> 3) * G_NS * 1024 +
                                       (lrow & 7) * 128 + slot128(r16, 2 * lhalf) * 16);

    uint4 raw[TI];             // fp8 A: 16 values per fragment row (two k-steps)
    float scf[TI];             // their 32-block scale
    bf16x8 fa[TI], fw[2][TJ];  // converted A fragments, W fragments
    auto read_a = [&](auto st, auto jc) {
        constexpr int S = decltype(st)::value, J = decltype(jc)::value;
        // chunk 2J + lhalf: flipping logical bit 1 flips address bit 5
        const uint32_t ab = J ? (a_base ^ 32u) : a_base;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            raw[i] = *reinterpret_cast<const uint4*>(smem + ab + i * 2 * G_NS * 1024 + S * 1024);
            scf[i] = *reinterpret_cast<const float*>(smem + s_base + i * G_NS * 256 + S * 256 + J * 4);
        }
    };
    auto read_w = [&](auto st, auto ksc, int buf) {
        constexpr int S = decltype(st)::value, KS = decltype(ksc)::value;
        // kchunk(KS, lhalf) = A | 2*lhalf with A = 4*(KS/2) + KS%2: XOR its
        // bits 0 and 2 into the swizzled slot held in w_base (bits 4..6)
        constexpr uint32_t AX = (uint32_t)(4 * (KS >> 1) + (KS & 1)) * 16u;
        const uint32_t wb = AX ? (w_base ^ AX) : w_base;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            fw[buf][j] = *reinterpret_cast<const bf16x8*>(smem + wb + j * 4 * G_NS * 1024 + S * 1024);
    };
    // A fragment of k-step ks: the first (even ks) or second (odd ks) 8 values
    auto convert = [&](int odd) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const float s = scf[i];
            const uint32_t w0 = odd ? raw[i].z : raw[i].x;
            const uint32_t w1 = odd ? raw[i].w : raw[i].y;
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
            fa[i] = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                            __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2,
                                            3, 4, 5, 6, 7);
        }
    };

    f32x16 acc[TJ][TI];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
    auto mfma_half = [&](int cur, int half) {
#pragma unroll
        for (int j = half * (TJ / 2); j < (half + 1) * (TJ / 2); ++j)
#pragma unroll
            for (int i = 0; i < TI; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[cur][j], fa[i], acc[j][i],
                                                                    0, 0, 0);
    };

    // One k-tile (in ring stage S): 4 k-steps, each converts its A fragments
    // from the fp8 read (k-steps 0 and 2 read nothing new for A, 1 and 3 read
    // the next pair's after converting), reads the next k-step's W fragments
    // and issues TI*TJ MFMAs (a fenced scheduling region).  At k-step 0 the
    // DMA of k-tile kt+2's fp8 rows and scales is issued (copied rows: at
    // computed addresses; table rows: at the offsets that arrived one k-tile
    // ago, after loading k-tile kt+3's, so that waiting for the offsets
    // never waits for the newer DMA), and k-steps 1 and 2 issue one half of
    // its W rows each (every load of the
    // k-tile is still issued before its hand-over, and the two waves of a
    // SIMD do not both burst all their loads into one k-step).  The hand-over
    // barrier comes before the last k-step's MFMAs, once its fragments have
    // arrived, so that all eight of them cover the next k-tile's first
    // fragment reads (measured: 1% on the prefill forward against splitting
    // that k-step around the barrier; issuing a k-step's reads ahead of its
    // MFMAs instead of between them was slower).
    //   WAITN: loads issued after k-tile kt+1's DMA that may stay in flight;
    //          -1 for the last k-tile (no hand-over).
    //   LOAD_IDS (table rows): load the row offsets of k-tile kt+3.
    auto k_tile = [&](int kt, auto st, auto ldids, auto dma, auto waitn) {
        constexpr int S = decltype(st)::value;
        constexpr bool LOAD_IDS = decltype(ldids)::value && !CA;
        constexpr bool DMA = decltype(dma)::value;
        constexpr int WAITN = decltype(waitn)::value;
        auto step = [&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            constexpr int cur = ks & 1;
            convert(cur);
            if constexpr (ks == 0 && DMA) {
                uint32_t ia[NA];
                if constexpr (!CA)
#pragma unroll
                    for (int i = 0; i < NA; ++i) ia[i] = id_a[i];
                // persistent: past this tile's last k-tile, load the next tile's
                const bool nx3 = P && kt + 3 >= nk, nx2 = P && kt + 2 >= nk;
                if constexpr (LOAD_IDS) load_offs(nx3 ? kt + 3 - nk : kt + 3, nx3 ? m0n : m0c);
                issue_dma(nx2 ? kt + 2 - nk : kt + 2, IC<(S + 2) % G_NS>{}, ia, nx2 ? m0n : m0c,
                          nx2 ? n0n : n0c, IC<0>{});
            }
            if constexpr ((ks == 1 || ks == 2) && DMA) {
                const bool nx2 = P && kt + 2 >= nk;
                issue_dma(nx2 ? kt + 2 - nk : kt + 2, IC<(S + 2) % G_NS>{}, nullptr,
                          nx2 ? m0n : m0c, nx2 ? n0n : n0c, IC<ks>{});
            }
            read_w(IC<S>{}, IC<ks + 1>{}, cur ^ 1);
            if constexpr (ks == 1) read_a(IC<S>{}, IC<1>{});
            mfma_half(cur, 0);
            mfma_half(cur, 1);
            // spread the converts, the loads of k-tile kt+2 and the fragment
            // reads over the MFMAs so the matrix pipe never waits on issue
#pragma unroll
            for (int r = 0; r < TI * TJ; ++r) {
                if (r < TI) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (ks == 0 && DMA && r < 2)
                    __builtin_amdgcn_sched_group_barrier(0x020, CA ? 1 : 2, 0);
                if (ks == 0 && DMA && r == 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if ((ks == 1 || ks == 2) && DMA && r < NB / 2)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if (ks == 1 && r < 5) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                if (ks != 1 && r < TJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        step(IC<0>{});
        step(IC<1>{});
        step(IC<2>{});
        convert(1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (WAITN >= 0) {
            // k-tile kt+1 is in LDS for everyone; stage S is free
            handover<WAITN>();
            __builtin_amdgcn_sched_barrier(0);
            read_a(IC<(S + 1) % G_NS>{}, IC<0>{});
            read_w(IC<(S + 1) % G_NS>{}, IC<0>{}, 0);
        }
        mfma_half(1, 0);
        mfma_half(1, 1);
#pragma unroll
        for (int r = 0; r < TI * TJ; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (r < 5) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    using T = std::true_type;
    using F = std::false_type;
    // loads issued after k-tile kt+1's DMA when k-tile kt hands over: k-tile
    // kt+3's offsets and kt+2's whole DMA (steady), kt+2's DMA alone (no
    // offsets left to load), none (the last DMA'd k-tile), no hand-over after
    // the last k-tile
    using Wsteady = IC<NIDS + NLOAD>;
    using W7 = IC<NLOAD>;
    using W0 = IC<0>;
    using Wn = IC<-1>;

    // prologue: k-tiles 0 and 1 in flight (and for table rows the offsets of
    // k-tile 2 loaded).  The W rows of both go first: they need no row
    // offsets, so they stream while any offsets make their round trip.
    {
        issue_dma(0, IC<0>{}, nullptr, m0c, n0c, IC<1>{});
        issue_dma(0, IC<0>{}, nullptr, m0c, n0c, IC<2>{});
        if (nk > 1) {
            issue_dma(1, IC<1>{}, nullptr, m0c, n0c, IC<1>{});
            issue_dma(1, IC<1>{}, nullptr, m0c, n0c, IC<2>{});
        }
        uint32_t ia[NA];
        load_offs(0, m0c);
        if constexpr (!CA)
#pragma unroll
            for (int i = 0; i < NA; ++i) ia[i] = id_a[i];
        if (nk > 1) load_offs(1, m0c);
        issue_dma(0, IC<0>{}, ia, m0c, n0c, IC<0>{});
        if (nk > 1) {
            if constexpr (!CA)
#pragma unroll
                for (int i = 0; i < NA; ++i) ia[i] = id_a[i];
            if (nk > 2) load_offs(2, m0c);
            issue_dma(1, IC<1>{}, ia, m0c, n0c, IC<0>{});
        }
        // k-tile 0 has landed once at most the loads issued after its fp8
        // rows are in flight (the offsets of k-tile 2, k-tile 1's rows)
        if (nk > 2) handover<NIDS + NA + 1>();
        else if (nk > 1) handover<NA + 1>();
        else handover<0>();
        read_a(IC<0>{}, IC<0>{});
        read_w(IC<0>{}, IC<0>{}, 0);
    }
    if constexpr (P) {
        // Output of the tile just finished, staged through ring stage 2: once
        // every wave is past the hand-over of the tile's last k-tile (stage
        // 2), stage 2 is unused until the next tile's first k-tile refills
        // it, while stages 0 and 1 hold or receive the next tile's first two
        // k-tiles.  Its 1 KiB blocks give each wave PB private blocks, two per
        // 32x32 fragment (16 rows of 64 bytes each), so the fragments go out
        // in passes of PB/2 with no workgroup barrier in between.
        constexpr int NBLK = BT / 16 + BT / 8;
        constexpr int PB = NBLK / NW, FP = PB / 2, NF = TI * TJ;
        static_assert(NBLK % NW == 0 && FP >= 1, "staging blocks");
        auto blk = [&](int q) -> uint32_t {  // this wave's staging block q (0 .. PB-1)
            const int gq = wave * PB + q;
            return gq < BT / 16 ? (uint32_t)((gq * G_NS + 2) * 1024)
                                : (uint32_t)(OFF_W + ((gq - BT / 16) * G_NS + 2) * 1024);
        };
        const int kcols = G ? gp.hc * gp.dim : 0;  // key columns: reduced, not stored
        // Key tile: per row, the sums over this wave's 128 columns of key^2
        // and (h*w)*key, the key rounded to bf16 first; products are rounded
        // before they are added (no fused multiply-add), each lane sums its
        // 64 values in a fixed order and adds the other lane half's.
        auto gate_partials = [&]() {
#pragma clang fp contract(off)
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            constexpr int NQ = TI * TJ;  // quarters: 32 rows x 32 columns each
            const int s = n0c / gp.dim, f0 = n0c - s * gp.dim + wn * WN;
            const int nq = gp.dim >> 7;
            const __amdgpu_buffer_rsrc_t rx =
                make_rsrc(gp.x, (uint32_t)(M * gp.hc * gp.dim * 2));  // rows past M read 0
            // this wave's 128 values of q*k
            const uint32_t wl = (uint32_t)(OFF_WQK + wave * 512);
            if (lane < 32)
                *reinterpret_cast<uint4*>(smem + wl + lane * 16) =
                    *reinterpret_cast<const uint4*>(gp.wqk + s * gp.dim + f0 + lane * 4);
            // x arrives by DMA in quarters (the 32 rows of one i, the 32
            // columns of one j: 64 bytes per row), each in two of this wave's
            // stage-2 blocks, three quarters in flight.  DMA lane L of block t
            // moves 16 bytes of row 16t + L/4 of the quarter: logical chunk
            // (L%4) ^ (row/4 % 4), stored at slot L%4 of the row's 64 bytes,
            // so that the fragment-layout reads below spread over the banks.
            // Each DMA instruction reads whole 64-byte row pieces of 16 rows;
            // loading x straight into the fragment layout (8 bytes per lane,
            // 32 rows per instruction) kept the address unit busy on 32 cache
            // lines per instruction, four times as many per byte, and cost
            // 17 us more per prefill forward at T=4096.  (Padding rows past M,
            // whose sums are not stored, may wrap the 32-bit offset: the read
            // then stays inside x.)
            uint32_t xo[TI][2];
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int rr = 16 * t + (lane >> 2);
                    const int64_t m = (int64_t)m0c + wm * WM + i * 32 + rr;
                    // the position of row m (compacted: from the row map, which
                    // points rows past the live count past x, where loads read 0)
                    const int64_t xm = rowmap ? (int64_t)rowmap[m] : m;
                    const int c = (lane & 3) ^ ((rr >> 2) & 3);
                    xo[i][t] = (uint32_t)(((xm * gp.hc + s) * gp.dim + f0) * 2) + (uint32_t)(c * 16);
                }
            auto issue_q = [&](int q) {
                const int i = q / TJ, j = q % TJ, b = q % 3;
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (lds_void*)(smem + blk(2 * b + t)), 16, xo[i][t], j * 64, 0, 0);
            };
            const int sw = (lrow >> 2) & 3;
            issue_q(0);
            issue_q(1);
            issue_q(2);
            float skk = 0.0f, shwk = 0.0f;
            float2 res[TI];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int i = q / TJ, j = q % TJ, b = q % 3;
                // quarter q has landed once only the quarters issued after it
                // (two DMA instructions each) may still be in flight
                if (NQ - 1 - q >= 2) __builtin_amdgcn_s_waitcnt(0x0F74);       // vmcnt(4)
                else if (NQ - 1 - q == 1) __builtin_amdgcn_s_waitcnt(0x0F72);  // vmcnt(2)
                else __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0)
                const uint32_t rb = blk(2 * b + (lrow >> 4)) + (lrow & 15) * 64 + lhalf * 8;
                u32x2 h4[4];
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    h4[g4] = *reinterpret_cast<const u32x2*>(smem + rb + ((g4 ^ sw) << 4));
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the buffer is free again
                if (q + 3 < NQ) issue_q(q + 3);
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int nl = j * 32 + 8 * g4 + 4 * lhalf;
                    const f32x4 ww = *reinterpret_cast<const f32x4*>(smem + wl + nl * 4);
                    const uint32_t kb[2] = {
                        pack_bf16(acc[j][i][4 * g4 + 0], acc[j][i][4 * g4 + 1]),
                        pack_bf16(acc[j][i][4 * g4 + 2], acc[j][i][4 * g4 + 3])};
                    const u32x2 h2 = h4[g4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sh = (e & 1) ? 0 : 16;  // low half first
                        const float key = __uint_as_float((kb[e >> 1] << sh) & 0xFFFF0000u);
                        const float h = __uint_as_float((h2[e >> 1] << sh) & 0xFFFF0000u);
                        // key^2 is exact in fp32, so the fused form rounds the
                        // same sum; (h*w)*key is rounded before the add
                        skk = __builtin_fmaf(key, key, skk);
                        shwk += (h * ww[e]) * key;
                    }
                }
                if (j == TJ - 1) {
                    skk += __shfl_xor(skk, 32, 64);
                    shwk += __shfl_xor(shwk, 32, 64);
                    res[i] = make_float2(skk, shwk);
                    skk = 0.0f;
                    shwk = 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int64_t m = (int64_t)m0c + wm * WM + i * 32 + lrow;
                if (lhalf == 0 && m < M) gp.part[(m * gp.hc + s) * nq + (f0 >> 7)] = res[i];
            }
            // the next tile's DMA may refill stage 2 only after every wave is
            // done with its x quarters there
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("s_barrier" ::: "memory");
        };
        auto epilogue = [&]() {
            if (G && n0c < kcols) {
                gate_partials();
                return;
            }
#pragma unroll
            for (int f0 = 0; f0 < NF; f0 += FP) {
#pragma unroll
                for (int s = 0; s < FP; ++s) {
                    if (f0 + s >= NF) break;
                    const int j = (f0 + s) / TI, i = (f0 + s) % TI;
                    const uint32_t b = blk(2 * s + (lrow >> 4)) + (lrow & 15) * 64 + lhalf * 8;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const uint32_t lo = pack_bf16(acc[j][i][4 * g4 + 0], acc[j][i][4 * g4 + 1]);
                        const uint32_t hi = pack_bf16(acc[j][i][4 * g4 + 2], acc[j][i][4 * g4 + 3]);
                        *reinterpret_cast<uint2*>(smem + b + ((g4 ^ (lrow & 3)) << 4)) =
                            make_uint2(lo, hi);
                    }
                }
#pragma unroll
                for (int s = 0; s < FP; ++s) {
                    if (f0 + s >= NF) break;
                    const int j = (f0 + s) / TI, i = (f0 + s) % TI;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int rr = (lane >> 2) + 16 * hh, sl = lane & 3;
                        const uint4 v = *reinterpret_cast<const uint4*>(
                            smem + blk(2 * s + hh) + (rr & 15) * 64 + sl * 16);
                        const int64_t m = (int64_t)m0c + wm * WM + i * 32 + rr;
                        const int n = n0c + wn * WN + j * 32 + ((sl ^ (rr & 3)) << 3);
                        if (m < M && n < N) *reinterpret_cast<uint4*>(C + m * ldc + (n - kcols)) = v;
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): staging reads returned
            asm volatile("s_barrier" ::: "memory");  // stage 2 free for the next DMA
        };
        for (int q = 1;; ++q) {
            for (int kt = 0; kt < nk; kt += 3) {
                k_tile(kt, IC<0>{}, T{}, T{}, Wsteady{});
                k_tile(kt + 1, IC<1>{}, T{}, T{}, Wsteady{});
                k_tile(kt + 2, IC<2>{}, T{}, T{}, Wsteady{});
            }
            epilogue();
            if (!tile_valid(q)) break;
            m0c = m0n;
            n0c = n0n;
            set_next(q + 1);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no DMA into LDS left at exit
        return;
    } else {
        // steady state, three k-tiles (one per stage) per iteration
        int kt = 0;
        for (; kt < nk - L; kt += 3) {
            k_tile(kt, IC<0>{}, T{}, T{}, Wsteady{});
            k_tile(kt + 1, IC<1>{}, T{}, T{}, Wsteady{});
            k_tile(kt + 2, IC<2>{}, T{}, T{}, Wsteady{});
        }
        // the last L k-tiles; kt is a multiple of 3, so tile kt+p uses stage p%3
        if constexpr (L == 1) {
            k_tile(kt, IC<0>{}, F{}, F{}, Wn{});
        } else if constexpr (L == 2) {
            k_tile(kt, IC<0>{}, F{}, F{}, W0{});
            k_tile(kt + 1, IC<1>{}, F{}, F{}, Wn{});
        } else {
            if constexpr (L >= 4) k_tile(kt, IC<0>{}, T{}, T{}, Wsteady{});
            if constexpr (L == 5) k_tile(kt + 1, IC<1>{}, T{}, T{}, Wsteady{});
            k_tile(kt + L - 3, IC<(L - 3) % G_NS>{}, F{}, T{}, W7{});
            k_tile(kt + L - 2, IC<(L - 2) % G_NS>{}, F{}, F{}, W0{});
            k_tile(kt + L - 1, IC<(L - 1) % G_NS>{}, F{}, F{}, Wn{});
        }
        __syncthreads();  // every wave is done with the ring before the epilogue reuses it

        // ---- epilogue through LDS (as in the bf16 kernel)
        constexpr int RB = WN * 2, CHW = RB / 16, RPI = 64 / CHW;
        uint8_t* ep = smem + wave * (WM * RB);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int r = i * 32 + lrow;
                    const int nn = j * 32 + 8 * g4 + 4 * lhalf;
                    const int ch = (nn >> 3) ^ (r & (CHW - 1));
                    const uint32_t lo = pack_bf16(acc[j][i][4 * g4 + 0], acc[j][i][4 * g4 + 1]);
                    const uint32_t hi = pack_bf16(acc[j][i][4 * g4 + 2], acc[j][i][4 * g4 + 3]);
                    *reinterpret_cast<uint2*>(ep + r * RB + ch * 16 + (nn & 4) * 2) =
                        make_uint2(lo, hi);
                }
        const int rsub = lane / CHW, csub = lane % CHW;
#pragma unroll 4
        for (int it = 0; it < WM / RPI; ++it) {
            const int r = it * RPI + rsub;
            const uint4 v =
                *reinterpret_cast<const uint4*>(ep + r * RB + ((csub ^ (r & (CHW - 1))) << 4));
            const int64_t m = (int64_t)m0c + wm * WM + r;
            const int n = n0c + wn * WN + csub * 8;
            if (m < M && n < N) *reinterpret_cast<uint4*>(C + m * ldc + n) = v;
        }
    }
}

constexpr int SMEM256 = (256 / 16) * G_NS * 1024 + 8 * G_NS * 256 + (256 / 8) * G_NS * 1024 +
                        8 * 512;  // + the gate partials' q*k
constexpr int SMEM128 = (128 / 16) * G_NS * 1024 + 4 * G_NS * 256 + (128 / 8) * G_NS * 1024;
static_assert(SMEM256 <= 160 * 1024, "LDS budget");
static_assert(8 * 128 * 128 <= SMEM256 && 4 * 64 * 128 <= SMEM128, "epilogue staging fits the ring");

template <int L, bool P, bool G>
__global__ void __launch_bounds__(512, 1)
wkv_gathered_256(const ASource as, const float2* __restrict__ scl, int n_cols, int64_t m_pad,
                 const uint16_t* __restrict__ W, int64_t M, int N, uint16_t* __restrict__ C,
                 int64_t ldc, int tiles_m, int tiles_n, int per_xcd, GatePartials gp) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM256];
    gathered_tile<256, 4, 2, L, P, G>(as, scl, n_cols, m_pad, W, M, N, C, ldc,
                                      tiles_m, tiles_n, per_xcd, gp, smem);
}

template <int L>
__global__ void __launch_bounds__(256, 1)
wkv_gathered_128(const ASource as, const float2* __restrict__ scl, int n_cols, int64_t m_pad,
                 const uint16_t* __restrict__ W, int64_t M, int N, uint16_t* __restrict__ C,
                 int64_t ldc, int tiles_m, int tiles_n, int per_xcd, const int* m_live) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM128];
    GatePartials lim{};
    lim.m_live = m_live;
    gathered_tile<128, 2, 2, L, false>(as, scl, n_cols, m_pad, W, M, N, C, ldc,
                                       tiles_m, tiles_n, per_xcd, lim, smem);
}

// decode-sized batches: 64 x 64 tiles, two waves of 32 x 64, so that a
// 64-position step still spreads the weight stream over 400 workgroups
constexpr int SMEM64 = (64 / 16) * G_NS * 1024 + 2 * G_NS * 256 + (64 / 8) * G_NS * 1024;

template <int L>
__global__ void __launch_bounds__(128)
wkv_gathered_64(const ASource as, const float2* __restrict__ scl, int n_cols, int64_t m_pad,
                const uint16_t* __restrict__ W, int64_t M, int N, uint16_t* __restrict__ C,
                int64_t ldc, int tiles_m, int tiles_n, int per_xcd) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM64];
    const GatePartials none{};
    gathered_tile<64, 2, 1, L, false>(as, scl, n_cols, m_pad, W, M, N, C, ldc,
                                      tiles_m, tiles_n, per_xcd, none, smem);
}

template <int L>
hipError_t run_gathered_l(int bt, const ASource& as, const float2* scl, int n_cols,
                          int64_t m_pad, const uint16_t* w, int64_t M, int N, uint16_t* c, int64_t ldc,
                          hipStream_t s, const int* m_live) {
    const int tiles_m = (int)((M + bt - 1) / bt);
    const int tiles_n = (N + bt - 1) / bt;
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + N_XCD - 1) / N_XCD;
    if (bt == 256)
        wkv_gathered_256<L, false, false><<<dim3(per_xcd * N_XCD), dim3(512), 0, s>>>(
            as, scl, n_cols, m_pad, w, M, N, c, ldc, tiles_m, tiles_n, per_xcd,
            GatePartials{});
    else if (bt == 64)
        wkv_gathered_64<L><<<dim3(per_xcd * N_XCD), dim3(128), 0, s>>>(
            as, scl, n_cols, m_pad, w, M, N, c, ldc, tiles_m, tiles_n, per_xcd);
    else
        wkv_gathered_128<L><<<dim3(per_xcd * N_XCD), dim3(256), 0, s>>>(
            as, scl, n_cols, m_pad, w, M, N, c, ldc, tiles_m, tiles_n, per_xcd,
            m_live);
    return hipGetLastError();
}

hipError_t run_gathered(int bt, const ASource& as, const float2* scl, int n_cols,
                        int64_t m_pad, const uint16_t* w,
                        int64_t M, int N, uint16_t* c, int64_t ldc, hipStream_t s,
                        const int* m_live = nullptr) {
    // m_live (compacted rows) is honoured by the 128-wide tiles only
    if (m_live && bt != 128) return hipErrorInvalidValue;
    const int L = n_cols <= 2 ? n_cols : 3 + n_cols % 3;
#define ENGRAM_RUN_L(V) \
    run_gathered_l<V>(bt, as, scl, n_cols, m_pad, w, M, N, c, ldc, s, m_live)
    switch (L) {
        case 1: return ENGRAM_RUN_L(1);
        case 2: return ENGRAM_RUN_L(2);
        case 3: return ENGRAM_RUN_L(3);
        case 4: return ENGRAM_RUN_L(4);
        default: return ENGRAM_RUN_L(5);
    }
#undef ENGRAM_RUN_L
}

// Persistent 256x256 launch: one workgroup per compute unit (a multiple of 8,
// so every XCD gets the same number), each running its XCD's tiles
// slot, slot + nwg, ...  Needs nk % 3 == 0 and N a multiple of 256.
hipError_t run_persistent(const ASource& as, const float2* scl, int n_cols, int64_t m_pad,
                          const uint16_t* w, int64_t M,
                          int N, uint16_t* c, int64_t ldc, int cus, const GatePartials& gp,
                          hipStream_t s) {
    const int tiles_m = (int)((M + 255) / 256);
    const int tiles_n = N / 256;
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + N_XCD - 1) / N_XCD;
    int grid = cus / N_XCD * N_XCD;
    if (grid > per_xcd * N_XCD) grid = per_xcd * N_XCD;
    if (gp.x)
        wkv_gathered_256<3, true, true><<<dim3(grid), dim3(512), 0, s>>>(
            as, scl, n_cols, m_pad, w, M, N, c, ldc, tiles_m, tiles_n, per_xcd,
            gp);
    else
        wkv_gathered_256<3, true, false><<<dim3(grid), dim3(512), 0, s>>>(
            as, scl, n_cols, m_pad, w, M, N, c, ldc, tiles_m, tiles_n, per_xcd,
            gp);
    return hipGetLastError();
}

hipError_t launch_prep(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                       const uint8_t* scales, int64_t M, int64_t m_pad, uint8_t* arows,
                       uint32_t* aoff, float2* scl, uint32_t* err, hipStream_t s,
                       const uint16_t* q = nullptr, const uint16_t* k = nullptr,
                       float* wqk = nullptr, const int32_t* live_idx = nullptr,
                       const int* m_live = nullptr) {
    const int64_t total = (int64_t)g.n_cols * m_pad;
    prep_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(
        hash_ids, g.n_cols, M, m_pad, table, scales, g.num_embeddings, arows, aoff, scl, err, q,
        k, wqk,
        g.hc * g.dim, live_idx, m_live);
    return hipGetLastError();
}

// Columns [0, nbig) run in 256x256 tiles, the rest in 128x128 tiles: nbig is
// the widest multiple of 256 whose tile count fills whole rounds of the
// machine, provided the 128x128 rest fits in one round (else all of N).
int big_columns(int64_t M, int N, int cus) {
    const int tiles_m = (int)((M + 255) / 256);
    const int tiles_n = (N + 255) / 256;
    int nb = tiles_n;
    if ((int64_t)tiles_m * tiles_n % cus != 0) {
        int cand = tiles_n - 1;
        while (cand > 0 && (int64_t)tiles_m * cand % cus != 0) --cand;
        if (cand > 0) {
            const int64_t small = ((M + 127) / 128) * ((N - cand * 256 + 127) / 128);
            if (small <= cus) nb = cand;
        }
    }
    return nb * 256 < N ? nb * 256 : N;
}

// the persistent kernel: nk a multiple of 3, whole 256-column tiles, and at
// least two tiles per compute unit
bool persistent_ok(const Geom& g, int64_t M, int nbig, int cus) {
    return g.n_cols % 3 == 0 && nbig % 256 == 0 && cus >= N_XCD &&
           ((M + 255) / 256) * (nbig / 256) >= 2 * (int64_t)cus;
}

}  // namespace

// 32-bit buffer offsets: copied rows stay below 2 GiB (their offsets within
// the array are 32-bit signed scalars; the copies read the table with 64-bit
// addresses); with row offsets the table stays below 4 GiB and each array
// below 2 GiB
bool gathered_supported(const Geom& g, int64_t M) {
    if (g.head_dim != 64) return false;
    const int64_t rows = (int64_t)g.n_cols * padded_rows(M);
    if (M > kOffsetRowsMax) return rows * 64 < ((int64_t)1 << 31);
    return g.num_embeddings * 64 < ((int64_t)1 << 32) && rows * 8 < ((int64_t)1 << 31);
}

// per (hash column, padded row): the copied row (64 bytes) or its offset
// (4), then its scales (8); then q*k in fp32 per (stream, feature) for the
// gate partials
size_t gathered_scratch_bytes(const Geom& g, int64_t M) {
    const size_t per = M > kOffsetRowsMax ? 72 : 12;
    return (size_t)g.n_cols * (size_t)padded_rows(M) * per + (size_t)g.hc * g.dim * 4;
}

// Same tiling policy as the bf16 projection: 256 x 256 tiles over the widest
// column range that fills whole rounds of the machine, 128 x 128 tiles over
// the rest when they fit in one round.  `scratch` holds
// gathered_scratch_bytes(g, M) bytes, 256-byte aligned.
GatheredScratch gathered_scratch(const Geom& g, int64_t M, void* base) {
    GatheredScratch r;
    r.m_pad = padded_rows(M);
    const int64_t rows = (int64_t)g.n_cols * r.m_pad;
    if (M > kOffsetRowsMax) {
        r.arows = reinterpret_cast<uint8_t*>(base);
        r.aoff = nullptr;
        r.scl = reinterpret_cast<float2*>(r.arows + rows * 64);
    } else {
        r.arows = nullptr;
        r.aoff = reinterpret_cast<uint32_t*>(base);
        r.scl = reinterpret_cast<float2*>(r.aoff + rows);
    }
    r.wqk = reinterpret_cast<float*>(r.scl + (int64_t)g.n_cols * r.m_pad);
    return r;
}

// The projection's A source for scratch gs: the copied rows, or the table
// at the row offsets.
ASource a_source(const Geom& g, const GatheredScratch& gs, const uint8_t* table) {
    if (gs.arows) return ASource{gs.arows, nullptr, (uint32_t)(g.n_cols * gs.m_pad * 64)};
    return ASource{table, gs.aoff, (uint32_t)(g.num_embeddings * 64)};
}

hipError_t launch_prep_scratch(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                               const uint8_t* scales, int64_t M, void* scratch, uint32_t* err,
                               hipStream_t s,
                               const uint16_t* q, const uint16_t* k, const int32_t* live_idx,
                               const int* m_live) {
    if (M == 0) return hipSuccess;
    const GatheredScratch gs = gathered_scratch(g, M, scratch);
    return launch_prep(g, hash_ids, table, scales, M, gs.m_pad, gs.arows, gs.aoff, gs.scl, err,
                       s, q, k,
                       q ? gs.wqk : nullptr, live_idx, m_live);
}

hipError_t launch_wkv_gathered(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                               const uint8_t* scales, const uint16_t* w, int64_t M, uint16_t* kv,
                               void* scratch, uint32_t* err, hipStream_t s, bool prepared) {
    if (M == 0) return hipSuccess;
    const GatheredScratch gs = gathered_scratch(g, M, scratch);
    const int64_t m_pad = gs.m_pad;
    float2* scl = gs.scl;
    if (!prepared) {
        hipError_t e = launch_prep(g, hash_ids, table, scales, M, m_pad, gs.arows, gs.aoff, scl,
                                   err, s);
        if (e != hipSuccess) return e;
    }
    const ASource as = a_source(g, gs, table);
    if (M <= kOffsetRowsMax)  // decode-sized: the weight stream dominates; small tiles
        return run_gathered(64, as, scl, g.n_cols, m_pad, w, M, g.N, kv, g.N, s);
    const int N = g.N;
    const int cus = cu_count();
    const int nbig = big_columns(M, N, cus);
    hipError_t e;
    if (persistent_ok(g, M, nbig, cus))
        e = run_persistent(as, scl, g.n_cols, m_pad, w, M, nbig, kv, N, cus, GatePartials{}, s);
    else
        e = run_gathered(256, as, scl, g.n_cols, m_pad, w, M, nbig, kv, N, s);
    if (e != hipSuccess || nbig >= N) return e;
    return run_gathered(128, as, scl, g.n_cols, m_pad, w + (int64_t)nbig * g.K, M, N - nbig,
                        kv + nbig, N, s);
}

bool gate_partials_supported(const Geom& g, int64_t M) {
    if (!gathered_supported(g, M) || g.dim % 256 != 0) return false;
    if (M * g.hc * g.dim * 2 >= ((int64_t)1 << 32)) return false;  // x under one descriptor
    const int cus = cu_count();
    const int nbig = big_columns(M, g.N, cus);
    return nbig >= g.hc * g.dim && persistent_ok(g, M, nbig, cus);
}

// The persistent 256x256 kernel covers every key column (and the first value
// columns); the 128x128 tail, if any, holds value columns only.
hipError_t launch_wkv_gate_partials(const Geom& g, const int32_t* hash_ids, const uint8_t* table,
                                    const uint8_t* scales, const uint16_t* w, int64_t M,
                                    const GatePartials& gp, uint16_t* v, void* scratch,
                                    uint32_t* err, hipStream_t s, bool prepared) {
    if (M == 0) return hipSuccess;
    if (!gate_partials_supported(g, M) || gp.dim != g.dim || gp.hc != g.hc) return hipErrorInvalidValue;
    // compacted rows come only from the hash's own placement
    if ((gp.m_live == nullptr) != (gp.rowmap == nullptr) || (gp.m_live && !prepared))
        return hipErrorInvalidValue;
    const GatheredScratch gs = gathered_scratch(g, M, scratch);
    const int64_t m_pad = gs.m_pad;
    float2* scl = gs.scl;
    float* wqk = gs.wqk;
    hipError_t e = prepared ? hipSuccess
                            : launch_prep(g, hash_ids, table, scales, M, m_pad, gs.arows, gs.aoff,
                                          scl, err, s, gp.q, gp.k, wqk);
    if (e != hipSuccess) return e;
    const int cus = cu_count();
    const int nbig = big_columns(M, g.N, cus);
    const int kcols = g.hc * g.dim;
    GatePartials gpw = gp;
    gpw.wqk = wqk;
    const ASource as = a_source(g, gs, table);
    e = run_persistent(as, scl, g.n_cols, m_pad, w, M, nbig, v, g.dim, cus, gpw, s);
    if (e != hipSuccess || nbig >= g.N) return e;
    return run_gathered(128, as, scl, g.n_cols, m_pad, w + (int64_t)nbig * g.K, M, g.N - nbig,
                        v + (nbig - kcols), g.dim, s, gp.m_live);
}

}  // namespace engram
