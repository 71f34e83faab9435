// Stage 3: the wkv projection ("Module engram" docs, stage 3 / linear_bf16;
// the Engram block's self.wkv): kv[m][n] = bf16(sum_k a[m][k] * w[n][k]).
//
// bf16 MFMA GEMM for gfx950.  Both operands are K-contiguous ([M, K] and
// [N, K]), which is exactly the per-lane operand layout of
// v_mfma_f32_32x32x16_bf16 (each lane holds 8 consecutive k of one row), so
// tiles go global -> registers -> LDS unchanged and come back out of LDS as
// one 16-byte read per fragment.
//
//  * Macro tile BM x BN x 64, double-buffered in LDS; the next k-tile's global
//    loads are issued before the current tile's MFMAs.
//  * LDS rows are 128 bytes (64 bf16); the 16-byte chunk index is XOR-swizzled
//    with the row so that the 32 rows of a fragment read hit distinct banks.
//  * The MFMA computes the transposed product W.A^T, so each lane ends up with
//    4 consecutive output columns per register group and writes 8-byte bf16
//    runs (instead of 2-byte scatters).
//  * Tiles are numbered so that the tiles one XCD runs are contiguous and, in
//    groups of 4 M-tiles, share A and W panels in that XCD's L2.
//  * Edges (M, N, K not multiples of the tile) are zero-filled on load and
//    masked on store; no access leaves the operands.
#include "internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;      // k per LDS tile: 64 bf16 = 128 bytes per row
constexpr int CH = BK / 8;  // 16-byte chunks per row
constexpr int N_XCD = 8;    // MI355X: 8 XCDs; workgroups go round-robin over them
constexpr int GROUP_M = 4;  // M-tiles per group in the tile order

__device__ __forceinline__ int swz(int row, int ch) {
    return ch ^ ((row & 7) ^ ((row >> 3) & 1));
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64, 1)
wkv_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, int64_t M, int N,
           int K, uint16_t* __restrict__ C, int tiles_m, int tiles_n, int per_xcd) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_LD = BM * CH / NT;
    constexpr int B_LD = BN * CH / NT;
    static_assert(BM * CH % NT == 0 && BN * CH % NT == 0, "tile/thread mismatch");
    __shared__ uint4 lds[2][(BM + BN) * CH];

    // ---- tile of this workgroup
    const int b = blockIdx.x;
    const int L = (b % N_XCD) * per_xcd + b / N_XCD;
    if (L >= tiles_m * tiles_n) return;
    const int group_size = GROUP_M * tiles_n;
    const int first_m = (L / group_size) * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int mt = first_m + (L % group_size) % gm;
    const int nt = (L % group_size) / gm;
    const int64_t m0 = (int64_t)mt * BM;
    const int n0 = nt * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // ---- global load slots: chunk q = tid + i*NT -> (row q/CH, chunk q%CH)
    const uint16_t* a_src[A_LD];
    const uint16_t* b_src[B_LD];
    int a_dst[A_LD], b_dst[B_LD];
    bool a_ok[A_LD], b_ok[B_LD];
    int a_ch[A_LD], b_ch[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int q = tid + i * NT, row = q / CH, ch = q % CH;
        a_ok[i] = (m0 + row) < M;
        a_src[i] = A + (a_ok[i] ? (m0 + row) : 0) * (int64_t)K + ch * 8;
        a_dst[i] = row * CH + swz(row, ch);
        a_ch[i] = ch * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int q = tid + i * NT, row = q / CH, ch = q % CH;
        b_ok[i] = (n0 + row) < N;
        b_src[i] = W + (int64_t)(b_ok[i] ? (n0 + row) : 0) * K + ch * 8;
        b_dst[i] = (BM + row) * CH + swz(row, ch);
        b_ch[i] = ch * 8;
    }

    uint4 ra[A_LD], rb[B_LD];
    auto load = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = (a_ok[i] && k0 + a_ch[i] < K)
                        ? *reinterpret_cast<const uint4*>(a_src[i] + k0)
                        : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[i] = (b_ok[i] && k0 + b_ch[i] < K)
                        ? *reinterpret_cast<const uint4*>(b_src[i] + k0)
                        : make_uint4(0, 0, 0, 0);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) lds[buf][a_dst[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) lds[buf][b_dst[i]] = rb[i];
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;

    const int nk = (K + BK - 1) / BK;
    load(0);
    store(0);
    __syncthreads();

    const int lrow = lane & 31;
    const int lhalf = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + lhalf;
            bf16x8 fa[TM], fw[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 32 + lrow;
                uint4 u = lds[cur][row * CH + swz(row, ch)];
                fa[i] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 32 + lrow;
                uint4 u = lds[cur][(BM + row) * CH + swz(row, ch)];
                fw[j] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], fa[i], acc[j][i],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) store(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: D[n][m]; lane holds m = lane%32, n = 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = m0 + wm * WM + i * 32 + lrow;
            if (m >= M) continue;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int n = n0 + wn * WN + j * 32 + 8 * g4 + 4 * lhalf;
                if (n >= N) continue;
                const uint32_t lo = f32_to_bf16(acc[j][i][4 * g4 + 0]) |
                                    (f32_to_bf16(acc[j][i][4 * g4 + 1]) << 16);
                const uint32_t hi = f32_to_bf16(acc[j][i][4 * g4 + 2]) |
                                    (f32_to_bf16(acc[j][i][4 * g4 + 3]) << 16);
                *reinterpret_cast<uint2*>(C + m * N + n) = make_uint2(lo, hi);
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t run(const uint16_t* a, const uint16_t* w, int64_t M, int N, int K, uint16_t* kv,
               hipStream_t s) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + N_XCD - 1) / N_XCD;
    wkv_kernel<BM, BN, WM, WN>
        <<<dim3(per_xcd * N_XCD), dim3(NT), 0, s>>>(a, w, M, N, K, kv, tiles_m, tiles_n, per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv(const uint16_t* a, const uint16_t* w, int64_t M, int N, int K,
                      uint16_t* kv, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (M >= 1024) return run<256, 256, 128, 128>(a, w, M, N, K, kv, s);
    return run<64, 64, 32, 32>(a, w, M, N, K, kv, s);
}

}  // namespace engram
