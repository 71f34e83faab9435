// Live-row compaction for masked prefill.  A position whose mask is False
// leaves x unchanged (Engram block forward; "Gate per stream" in/out box),
// so the projection need not compute its row: the live positions are packed,
// in order, into the first rows of the projection's operand.
//
// One workgroup of 1024 threads walks the positions in blocks of 4096, four
// consecutive positions per thread (coalesced mask reads and live_idx
// stores): an inclusive shuffle scan within each wave, the 16 wave totals
// through LDS, and a running count across blocks give each live position its
// compact row.  The maps are a few bytes per position against the
// projection's 78.6 Mflop per position, so one workgroup suffices.
#include "internal.h"

namespace engram {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kPerThread = 4;
constexpr int kBlock = kScanThreads * kPerThread;

__global__ void __launch_bounds__(kScanThreads) live_rows_kernel(
    const uint8_t* __restrict__ mask, int64_t M, int64_t m_pad, int32_t* __restrict__ live_idx,
    int32_t* __restrict__ rowmap, int* __restrict__ m_live) {
    __shared__ int wsum[kScanThreads / 64];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int carry = 0;  // live positions before this block
    for (int64_t base = 0; base < M; base += kBlock) {
        const int64_t r = base + (int64_t)kPerThread * t;
        int live[kPerThread];
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            live[j] = (r + j < M) && mask[r + j] != 0;
            cnt += live[j];
        }
        int incl = cnt;  // inclusive scan over the wave's lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kScanThreads / 64; ++w) {
            const int x = wsum[w];
            before += w < wv ? x : 0;
            total += x;
        }
        int slot = carry + before + incl - cnt;
        int idx[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            idx[j] = -1;
            if (live[j]) {
                idx[j] = slot;
                rowmap[slot] = (int32_t)(r + j);
                ++slot;
            }
        }
        if (r + kPerThread <= M) {
            *reinterpret_cast<int4*>(live_idx + r) = make_int4(idx[0], idx[1], idx[2], idx[3]);
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j)
                if (r + j < M) live_idx[r + j] = idx[j];
        }
        carry += total;
        __syncthreads();  // wsum is rewritten by the next block
    }
    for (int64_t j = carry + t; j < m_pad; j += kScanThreads) rowmap[j] = (int32_t)M;
    if (t == 0) *m_live = carry;
}

}  // namespace

hipError_t launch_live_rows(const uint8_t* mask, int64_t M, int64_t m_pad, int32_t* live_idx,
                            int32_t* rowmap, int* m_live, hipStream_t s) {
    // live_idx is stored four at a time
    if (M <= 0 || M > INT32_MAX || m_pad < M || ((uintptr_t)live_idx & 15) != 0)
        return hipErrorInvalidValue;
    live_rows_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(mask, M, m_pad, live_idx, rowmap,
                                                            m_live);
    return hipGetLastError();
}

}  // namespace engram
