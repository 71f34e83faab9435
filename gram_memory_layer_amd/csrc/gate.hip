// Stage 4: gate and add ("Module engram" docs, gate_and_add; the Engram
// block's forward after the projection; "Gate per stream" equations for a_k
// and g).  Two forms: from the full kv (keys and value), or, in the fully
// fused prefill, from the value alone plus the key-side partial sums the
// projection's epilogue produced (S_kk and S_hwk per 128 columns).
//
// One workgroup per token.  Each thread owns NCH 16-byte chunks (8 features)
// of every stream and of the shared value: it loads them once, keeps x and
// the value in registers, accumulates its share of the 3*HC sums
//   S_hh[s] = sum h^2,  S_kk[s] = sum key^2,  S_hwk[s] = sum (h*w)*key,
// and after a fixed-order block reduction writes out = bf16(h + g[s]*v) from
// the registers it already holds.  HBM traffic is the algorithmic minimum:
// x and kv read once, out written once (nontemporal); q and k are
// L2-resident.  In the full-kv form with one workgroup per token, x, the
// keys and the value are also loaded with the nontemporal hint, so that the
// streamed lines do not displace q and k (65,536 tokens: 5.51 -> 5.62 TB/s;
// T=4096: 4.93 -> 5.11 TB/s); the form from partial sums and the
// per-(token, stream) form measured slower with it and keep plain loads.
// (Persistent workgroups holding q and k in registers, DPP reductions with
// one barrier per token, and fewer threads with more chunks each all
// measured slower on the T=4096 prefill shape; so did one workgroup per
// (token, stream) with a token's streams in consecutive workgroups: full kv
// 5.24 -> 4.52 TB/s at T=4096, 5.65 -> 4.63 TB/s over 65,536 tokens.)
//
// x and out may be the same buffer: every thread writes only the chunks it
// has itself read, after reading them (so neither pointer is __restrict__).
//
// Numerics: fp32.  h*w is exact in fp32 (8 + 16 significand bits); the
// product with key is rounded and then added (no fused multiply-add), as an
// elementwise product followed by a sum does, so an exactly cancelling pair
// of terms sums to exactly +0.  Reductions are in a fixed tree order, so the
// result is the same on every run.
#include "internal.h"

namespace engram {
namespace {

__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// write-once output: 16-byte store with the nontemporal hint
__device__ __forceinline__ void st_nt(uint16_t* p, uint4 v) {
    const u32x4 u = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
}

// 16-byte load, with the nontemporal hint when NT
template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
    if constexpr (NT) {
        const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(u.x, u.y, u.z, u.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

// Two fp32 -> packed bf16 (lo in the low half), round to nearest even, by
// the hardware convert (v_cvt_pk_bf16_f32, one instruction per pair): for
// every non-NaN input, infinities and overflow included, it equals the
// integer rounding of f32_to_bf16; a NaN is then made the canonical 0x7FC0
// that f32_to_bf16 gives.  (Measured: 65,536 tokens 5.63 -> 5.68 TB/s, the
// form from partial sums 59.9 -> 58.8 us.)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    uint32_t o = __builtin_bit_cast(uint32_t, v);
    o = (lo != lo) ? ((o & 0xFFFF0000u) | 0x7FC0u) : o;
    o = (hi != hi) ? ((o & 0x0000FFFFu) | 0x7FC00000u) : o;
    return o;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// PART: the key-side sums come as per-128-column partials from the
// projection's epilogue (kv then points at the value [n_tok, dim] alone, q and
// kw are unused); only S_hh is reduced here.
// SPLIT: one workgroup per (token, stream), stream = blockIdx.y, for batches
// too small to fill the machine with one workgroup per token.  Each stream's
// sums are formed by the same threads in the same order either way, so the
// results are identical.
template <int HC, int NCH, bool PART, bool SPLIT = false>
__global__ void __launch_bounds__(1024) gate_kernel(
    const uint16_t* x, const uint16_t* __restrict__ kv,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kw,
    const float2* __restrict__ part, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ live_idx, int dim, float eps, float inv_sqrt_dim, uint16_t* out,
    float* __restrict__ gate) {
#pragma clang fp contract(off)
    constexpr int HS = SPLIT ? 1 : HC;  // streams of this workgroup
    constexpr int NS = PART ? HS : 3 * HS;
    constexpr bool NT = !PART && !SPLIT;  // streamed loads with the nontemporal hint
    __shared__ float red[16][NS];
    __shared__ float gsh[HS];

    const int64_t tok = blockIdx.x;
    const int s0 = SPLIT ? (int)blockIdx.y : 0;  // first stream of this workgroup
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int d8 = dim / 8;
    const int64_t row = PART ? (int64_t)dim : (int64_t)dim * (HC + 1);
    const int64_t voff = PART ? 0 : (int64_t)HC * dim;  // value within the kv row
    const uint16_t* xt = x + (tok * HC + s0) * dim;
    uint16_t* ot = out + (tok * HC + s0) * dim;
    // compacted rows (fully fused prefill under a mask): the value and the
    // partial sums of a live position sit at its compact row (loaded
    // alongside the mask byte, not after it)
    const int32_t crow = (PART && live_idx) ? live_idx[tok] : 0;
    const bool live = (mask == nullptr) || (mask[tok] != 0);
    const int64_t vrow = (PART && live_idx) ? (int64_t)crow : tok;
    const uint16_t* kvt = kv + vrow * row;

    // KEEP: x and the value stay in registers from the loads to the output
    // pass; for wide geometries (HC * NCH > 8) they are re-read instead.
    constexpr bool KEEP = HS * NCH <= 8;
    constexpr int KC = KEEP ? NCH : 1;
    uint4 xr[HS][KC];
    if (!live) {
        // masked position: the gate is 0 and x passes through unchanged
        // (nothing to move when out is x)
#pragma unroll
        for (int i = 0; i < NCH && ot != xt; ++i) {
            const int c = tid + i * nthr;
            if (c < d8)
#pragma unroll
                for (int s = 0; s < HS; ++s) {
                    st_nt(ot + (int64_t)s * dim + c * 8,
                          *reinterpret_cast<const uint4*>(xt + (int64_t)s * dim + c * 8));
                }
        }
        if (gate && tid < HS) gate[tok * HC + s0 + tid] = 0.0f;
        return;
    }

    // PART: the token's HC * dim/128 partial pairs are fetched first, one per
    // thread, into LDS, so their latency overlaps the x loads; they are
    // summed in order after the block reduction
    __shared__ float2 psh[PART ? HS * 256 : 1];
    if constexpr (PART) {
        const int np = HS * (dim >> 7);  // dim <= 32768: at most HS * 256 pairs
        const float2* pt = part + (vrow * HC + s0) * (dim >> 7);
        for (int t = tid; t < np; t += nthr) psh[t] = pt[t];
    }

    float acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[j] = 0.0f;
    uint4 vr[KC];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * nthr;
        if (c < d8) {
            if (KEEP) vr[i < KC ? i : 0] = ld16<NT>(kvt + voff + c * 8);
#pragma unroll
            for (int s = 0; s < HS; ++s) {
                const uint4 h = ld16<NT>(xt + (int64_t)s * dim + c * 8);
                if (KEEP) xr[s][i < KC ? i : 0] = h;
                if constexpr (PART) {
                    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float h0 = lo_f(hw[e]), h1 = hi_f(hw[e]);
                        acc[s] += h0 * h0;
                        acc[s] += h1 * h1;
                    }
                } else {
                    const int64_t so = (int64_t)(s0 + s) * dim + c * 8;
                    const uint4 key = ld16<NT>(kvt + so);
                    const uint4 qq = *reinterpret_cast<const uint4*>(q + so);
                    const uint4 kk = *reinterpret_cast<const uint4*>(kw + so);
                    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
                    const uint32_t kyw[4] = {key.x, key.y, key.z, key.w};
                    const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
                    const uint32_t kw4[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float h0 = lo_f(hw[e]), h1 = hi_f(hw[e]);
                        const float k0 = lo_f(kyw[e]), k1 = hi_f(kyw[e]);
                        const float w0 = lo_f(qw[e]) * lo_f(kw4[e]);
                        const float w1 = hi_f(qw[e]) * hi_f(kw4[e]);
                        acc[s] += h0 * h0;
                        acc[s] += h1 * h1;
                        acc[HS + s] += k0 * k0;
                        acc[HS + s] += k1 * k1;
                        const float p0 = (h0 * w0) * k0;
                        const float p1 = (h1 * w1) * k1;
                        acc[2 * HS + s] += p0;
                        acc[2 * HS + s] += p1;
                    }
                }
            }
        }
    }

    // fixed-order block reduction
    const int lane = tid & 63, wave = tid >> 6, nwaves = (nthr + 63) >> 6;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const float v = wave_sum(acc[j]);
        if (lane == 0) red[wave][j] = v;
    }
    __syncthreads();
    if (tid < HS) {
        float shh = 0.f, skk = 0.f, shwk = 0.f;
        for (int w = 0; w < nwaves; ++w) {
            shh += red[w][tid];
            if constexpr (!PART) {
                skk += red[w][HS + tid];
                shwk += red[w][2 * HS + tid];
            }
        }
        if constexpr (PART) {
            const int nq = dim >> 7;
            for (int b = 0; b < nq; ++b) {
                const float2 p = psh[tid * nq + b];
                skk += p.x;
                shwk += p.y;
            }
        }
        const float fd = (float)dim;
        const float rstd = (1.0f / sqrtf(shh / fd + eps)) * (1.0f / sqrtf(skk / fd + eps));
        const float a = shwk * rstd * inv_sqrt_dim;
        // the clamp keeps a NaN (fmaxf would drop it): a NaN a gives a NaN
        // g, as the block's elementwise clamp on a tensor does
        const float mag = fabsf(a) < 1e-6f ? 1e-6f : fabsf(a);
        const float sg = copysignf(sqrtf(mag), a);
        const float g = 1.0f / (1.0f + expf(-sg));
        gsh[tid] = g;
        if (gate) gate[tok * HC + s0 + tid] = g;
    }
    __syncthreads();

    float g[HS];
#pragma unroll
    for (int s = 0; s < HS; ++s) g[s] = gsh[s];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * nthr;
        if (c < d8) {
            const uint4 vv = KEEP ? vr[i < KC ? i : 0]
                                  : *reinterpret_cast<const uint4*>(kvt + voff + c * 8);
            const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int s = 0; s < HS; ++s) {
                const uint4 hh = KEEP ? xr[s][i < KC ? i : 0]
                                      : *reinterpret_cast<const uint4*>(xt + (int64_t)s * dim + c * 8);
                const uint32_t hw[4] = {hh.x, hh.y, hh.z, hh.w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float r0 = __fmaf_rn(g[s], lo_f(vw[e]), lo_f(hw[e]));
                    const float r1 = __fmaf_rn(g[s], hi_f(vw[e]), hi_f(hw[e]));
                    o[e] = pack2_bf16(r0, r1);
                }
                st_nt(ot + (int64_t)s * dim + c * 8, make_uint4(o[0], o[1], o[2], o[3]));
            }
        }
    }
}

template <int HC, bool PART>
hipError_t run_hc(const Geom& g, const uint16_t* x, const uint16_t* kv, const uint16_t* q,
                  const uint16_t* k, const float2* part, const uint8_t* mask,
                  const int32_t* live_idx, int64_t n_tok, uint16_t* out, float* gate,
                  hipStream_t s) {
    const int d8 = g.dim / 8;
    // one 16-byte chunk per thread and stream up to 1024 threads (640 at
    // dim 5120): measured faster than fewer threads holding more chunks
    int nch = 1;
    while (nch < 4 && (d8 + nch - 1) / nch > 1024) nch *= 2;  // dim <= 32768
    int threads = (d8 + nch - 1) / nch;
    threads = (threads + 63) / 64 * 64;
    const float inv_sqrt_dim = (float)(1.0 / sqrt((double)g.dim));
    // fewer tokens than about four workgroups per compute unit: one
    // workgroup per (token, stream) instead of one per token
    const bool split = HC > 1 && n_tok < 4 * (int64_t)cu_count();
    const dim3 grid((unsigned)n_tok, split ? HC : 1), block(threads);
#define ENGRAM_GATE_CASE(N)                                                                  \
    case N:                                                                                  \
        if (split)                                                                           \
            gate_kernel<HC, N, PART, true><<<grid, block, 0, s>>>(                           \
                x, kv, q, k, part, mask, live_idx, g.dim, g.eps, inv_sqrt_dim, out, gate);   \
        else                                                                                 \
            gate_kernel<HC, N, PART, false><<<grid, block, 0, s>>>(                          \
                x, kv, q, k, part, mask, live_idx, g.dim, g.eps, inv_sqrt_dim, out, gate);   \
        break;
    switch (nch) {
        ENGRAM_GATE_CASE(1)
        ENGRAM_GATE_CASE(2)
        ENGRAM_GATE_CASE(4)
        default: return hipErrorInvalidValue;
    }
#undef ENGRAM_GATE_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_add(const Geom& g, const uint16_t* x, const uint16_t* kv,
                           const uint16_t* q, const uint16_t* k, const uint8_t* mask,
                           int64_t n_tok, uint16_t* out, float* gate, hipStream_t s) {
    if (n_tok == 0) return hipSuccess;
    switch (g.hc) {
        case 1: return run_hc<1, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 2: return run_hc<2, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 3: return run_hc<3, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 4: return run_hc<4, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 5: return run_hc<5, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 6: return run_hc<6, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 7: return run_hc<7, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        case 8: return run_hc<8, false>(g, x, kv, q, k, nullptr, mask, nullptr, n_tok, out, gate, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gate_from_partials(const Geom& g, const uint16_t* x, const uint16_t* v,
                                     const float2* part, const uint8_t* mask, int64_t n_tok,
                                     uint16_t* out, float* gate, hipStream_t s,
                                     const int32_t* live_idx) {
    if (n_tok == 0) return hipSuccess;
    if (g.dim % 128 != 0 || (live_idx && !mask)) return hipErrorInvalidValue;
    switch (g.hc) {
        case 1: return run_hc<1, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 2: return run_hc<2, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 3: return run_hc<3, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 4: return run_hc<4, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 5: return run_hc<5, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 6: return run_hc<6, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 7: return run_hc<7, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        case 8: return run_hc<8, true>(g, x, v, nullptr, nullptr, part, mask, live_idx, n_tok, out, gate, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace engram
