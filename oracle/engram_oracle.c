/*
 * Engram forward path -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct reference
 * that the HIP library is checked against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the library itself
 * never does, and the two share no code, headers or tables.
 *
 * Sources (the three pages this method is described on):
 *   [block]  "DeepSeek V4.1" model atlas, Engram block (value view, prefill):
 *            the `Engram` module listing, constructor and `forward`.
 *   [gate]   "DeepSeek V4.1 - Gate per stream" page: the equation for a_k,
 *            the equation for g, the in/out box and the parameter table.
 *   [docs]   "Module engram" API docs of the CPU reference
 *            (spark_model / layers / deepseek_v41_ref / engram): the
 *            four-stage list, the note on given tables, the structs
 *            EngramTables and NgramHashState, and the functions e4m3_to_f32,
 *            embed_rows, f32_to_e4m3_rne, f32_to_e8m0_rne, gate_and_add,
 *            linear_bf16.
 *
 * Precision: every floating-point step is evaluated in fp64 and rounded once
 * to the output format (bf16 for rows, kv and out; fp32 for the gate).  The
 * one place the definition itself rounds in between -- the dequantising
 * product, which the docs (regen_table) form in fp32 and only then round to
 * bf16 -- is rounded to fp32 first and then to bf16, in that order.
 *
 * Parity status: every function here is pinned by the CPU tests (closed
 * forms, special cases, library cross-checks, brute force); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EO_OK 0
#define EO_BAD_TOKEN 1
#define EO_BAD_HASH 2
#define EO_HISTORY_FULL 3
#define EO_BAD_ID 4

int eo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (timing only; results do not
 * depend on it: every output element is computed by one thread). */
void eo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ bf16 */

/* Value of a bf16 bit pattern: the top half of an IEEE binary32. */
double eo_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a real number (held exactly in a double) to bf16, nearest-even.
 * bf16 = 1 sign, 8 exponent, 7 fraction bits: normal numbers 1.f * 2^E with
 * E in [-126, 127], subnormals k * 2^-133.  The quantum at v is 2^(E-7)
 * (2^-133 below the normal range); v / quantum is an exact double, rint()
 * rounds it half-to-even, and the product is the rounded value.  Results at or
 * beyond 2^128 overflow to infinity.  NaN becomes the canonical quiet NaN
 * 0x7FC0. */
uint16_t eo_bf16_round(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;               /* a = (2m) * 2^E, 2m in [1, 2) */
    double q = (E < -126) ? ldexp(1.0, -133) : ldexp(1.0, E - 7);
    double r = rint(a / q) * q;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)r;          /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* ------------------------------------------------------------------ e4m3 */

/* OCP fp8 e4m3fn decode ([docs] e4m3_to_f32; stage 2 says e4m3 values are
 * exactly representable in bf16).  1 sign, 4 exponent (bias 7), 3 fraction
 * bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN and the
 * format has no infinities. */
double eo_e4m3_decode(unsigned code) {
    code &= 0xFF;
    unsigned s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* [docs] f32_to_e4m3_rne: round to nearest, ties to the even code, and
 * saturate: any magnitude above 448 (the largest finite value), infinities
 * included, encodes as +-448.  NaN encodes as S.1111.111.  The nearest finite
 * code is found by plain search over the 127 non-negative finite codes. */
unsigned eo_e4m3_encode(float f) {
    unsigned sign = signbit(f) ? 0x80 : 0;
    if (isnan(f)) return sign | 0x7F;
    double a = fabs((double)f);
    if (a > 448.0) return sign | 0x7E;
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 0x7F; ++c) {
        double d = fabs(a - eo_e4m3_decode(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | best;
}

/* ------------------------------------------------------------------ e8m0 */

/* e8m0 scale decode: 2^(code - 127); code 255 is NaN ([docs] stage 2 and
 * regen_table: per-block power-of-two scales). */
double eo_e8m0_decode(unsigned code) {
    code &= 0xFF;
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* [docs] f32_to_e8m0_rne: nearest power of two; a tie (exactly 1.5 * 2^e, the
 * midpoint of 2^e and 2^(e+1)) goes to whichever of e, e+1 is even.  Where
 * the docs are silent the cast it names is followed: the sign is dropped,
 * zero and values below 2^-127 give code 0, and NaN, infinity and anything
 * rounding above 2^127 give code 255. */
unsigned eo_e8m0_encode(float f) {
    if (isnan(f) || isinf(f)) return 0xFF;
    double a = fabs((double)f);
    if (a == 0.0) return 0;
    int e;
    double m = frexp(a, &e);     /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;
    double r = 2.0 * m;          /* a = r * 2^E, r in [1, 2) */
    int k;
    if (r < 1.5) k = E;
    else if (r > 1.5) k = E + 1;
    else k = ((E % 2) == 0) ? E : E + 1;
    int code = k + 127;
    if (code < 0) return 0;
    if (code > 254) return 0xFF;
    return (unsigned)code;
}

/* Array helpers (for the tests). */
void eo_e4m3_decode_n(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = eo_e4m3_decode(c[i]);
}
void eo_e4m3_encode_n(const float* f, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)eo_e4m3_encode(f[i]);
}
void eo_e8m0_encode_n(const float* f, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)eo_e8m0_encode(f[i]);
}
void eo_bf16_round_n(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = eo_bf16_round(v[i]);
}

/* ------------------------------------------------------------------ stage 1: hash */

/* [docs] stage 1 (Hash, NgramHashState); [block] `forward` takes the result as
 * hash_ids [B, L, n_hash_cols] with n_hash_cols = (max_ngram_size - 1) * n_heads.
 *
 * The state is the page's full cache: `hist[b]` holds the compressed id of
 * every position of sequence b seen so far (hist_len[b] of them, capacity
 * hist_cap).  For each new token id: compress it through token_map, append it,
 * then for every n-gram size n in 2..max_ngram and head h, column
 * col = (n-2)*n_heads + h:
 *     mix  = XOR over lookback k = 0..n-1 of  c[t-k] * mult[col][k]  (mod 2^64)
 *     hash = mix % prime[col] + offset[col]
 * where c[t-0] is the current token, c[t-k] for positions before the start of
 * the sequence is pad_id, compressed ids are taken as unsigned 32-bit numbers,
 * and all arithmetic is unsigned 64-bit.  Tables are used as given.
 * Returns EO_BAD_TOKEN for an id outside [0, vocab), EO_BAD_HASH if a hash
 * does not fit int32, EO_HISTORY_FULL if a history would overflow. */
int eo_hash(int max_ngram, int n_heads, int32_t pad_id, int64_t vocab,
            const int32_t* token_map, const uint64_t* mult, const uint64_t* prime,
            const uint64_t* offset, int B, int64_t T, const int32_t* ids,
            int32_t* hist, int64_t hist_cap, int64_t* hist_len, int32_t* hash_ids) {
    const int n_cols = (max_ngram - 1) * n_heads;
    for (int b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            int32_t tok = ids[(int64_t)b * T + t];
            if (tok < 0 || tok >= vocab) return EO_BAD_TOKEN;
            if (hist_len[b] >= hist_cap) return EO_HISTORY_FULL;
            int32_t* h = hist + (int64_t)b * hist_cap;
            h[hist_len[b]] = token_map[tok];
            hist_len[b] += 1;
            const int64_t now = hist_len[b] - 1;
            for (int col = 0; col < n_cols; ++col) {
                const int n = 2 + col / n_heads;
                uint64_t mix = 0;
                for (int k = 0; k < n; ++k) {
                    int64_t p = now - k;
                    int32_t c = (p >= 0) ? h[p] : pad_id;
                    mix ^= (uint64_t)(uint32_t)c * mult[(int64_t)col * max_ngram + k];
                }
                uint64_t v = mix % prime[col] + offset[col];
                if (v > (uint64_t)INT32_MAX) return EO_BAD_HASH;
                hash_ids[((int64_t)b * T + t) * n_cols + col] = (int32_t)v;
            }
        }
    }
    return EO_OK;
}

/* ------------------------------------------------------------------ stage 2: rows */

/* [docs] stage 2 (embed_rows) and regen_table; [block] `self.embed(hash_ids)`.
 * Row `id` of the fp8 e4m3 table [num_rows, head_dim], dequantised per block
 * of 32 by its e8m0 scale [num_rows, head_dim/32]: the fp32 product
 * value * scale, then bf16.  The exact product is formed in fp64, rounded to
 * fp32 (what a binary32 multiply returns) and then to bf16.
 * Returns EO_BAD_ID for an id outside [0, num_rows). */
int eo_embed_rows(int head_dim, int64_t num_rows, const uint8_t* table,
                  const uint8_t* scales, const int32_t* ids, int64_t n_ids,
                  uint16_t* out) {
    const int nb = head_dim / 32;
    for (int64_t i = 0; i < n_ids; ++i) {
        int64_t id = ids[i];
        if (id < 0 || id >= num_rows) return EO_BAD_ID;
        for (int j = 0; j < head_dim; ++j) {
            double v = eo_e4m3_decode(table[id * head_dim + j]);
            double s = eo_e8m0_decode(scales[id * nb + j / 32]);
            float p = (float)(v * s);
            out[i * head_dim + j] = eo_bf16_round((double)p);
        }
    }
    return EO_OK;
}

/* ------------------------------------------------------------------ stage 3: wkv */

/* [docs] stage 3 and linear_bf16; [block] `self.wkv(...)`.  F.linear without
 * bias on bf16: out[m][n] = bf16( sum_k a[m][k] * w[n][k] ), x [rows, in],
 * w [out, in].  Every bf16 x bf16 product is exact in fp64 and the sum is
 * accumulated in fp64, then rounded once to bf16. */
void eo_linear(int64_t M, int64_t N, int64_t K, const uint16_t* a, const uint16_t* w,
               uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += eo_bf16_value(a[m * K + k]) * eo_bf16_value(w[n * K + k]);
            out[m * N + n] = eo_bf16_round(acc);
        }
    }
}

/* ------------------------------------------------------------------ stage 4: gate */

/* [docs] gate_and_add; [block] `forward` after the projection; [gate] the
 * equations for a_k and g.  Per token t and stream s (hc streams of width dim):
 *   key   = kv[t][s*dim : (s+1)*dim],   value = kv[t][hc*dim : (hc+1)*dim]
 *   w     = q_weight[s] * k_weight[s]            (elementwise)
 *   rstd  = 1/sqrt(mean(h^2) + eps) * 1/sqrt(mean(key^2) + eps)
 *           -- per (token, stream), not across streams
 *   a     = sum(h * w * key) * rstd * dim^-0.5
 *   g     = sigmoid( copysign( sqrt(max(|a|, clamp)), a ) ),  clamp = fp32(1e-6),
 *           where the max keeps a NaN (as the block's elementwise clamp on a
 *           tensor does): a NaN a gives a NaN g and a NaN out
 *   g     = 0 where token_mask is False
 *   out   = bf16(h + g * value)
 * All in fp64.  A masked position returns x unchanged (the block's forward
 * docstring says a False mask leaves the position as it was; the gate page
 * gives image positions a zero gate).  gate_out [tokens, hc] gets g
 * rounded to fp32 and a_out [tokens, hc] the fp64 a (either may be NULL).
 * mask may be NULL (every position live). */
void eo_gate_and_add(int64_t n_tok, int hc, int dim, float eps, const uint16_t* x,
                     const uint16_t* kv, const uint16_t* q, const uint16_t* k,
                     const uint8_t* mask, uint16_t* out, float* gate_out, double* a_out) {
    const int64_t row = (int64_t)dim * (hc + 1);
    const double clamp = (double)(float)1e-6;
    const double e = (double)eps;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        const int live = (mask == NULL) || (mask[t] != 0);
        const uint16_t* value = kv + t * row + (int64_t)hc * dim;
        for (int s = 0; s < hc; ++s) {
            const uint16_t* h = x + (t * hc + s) * dim;
            const uint16_t* key = kv + t * row + (int64_t)s * dim;
            double shh = 0.0, skk = 0.0, dot = 0.0;
            for (int f = 0; f < dim; ++f) {
                double hv = eo_bf16_value(h[f]);
                double kv_ = eo_bf16_value(key[f]);
                double wv = eo_bf16_value(q[s * dim + f]) * eo_bf16_value(k[s * dim + f]);
                shh += hv * hv;
                skk += kv_ * kv_;
                dot += hv * wv * kv_;
            }
            double rstd = (1.0 / sqrt(shh / dim + e)) * (1.0 / sqrt(skk / dim + e));
            double a = dot * rstd / sqrt((double)dim);
            double mag = fabs(a) < clamp ? clamp : fabs(a);  /* NaN stays NaN */
            double sg = copysign(sqrt(mag), a);
            double g = 1.0 / (1.0 + exp(-sg));
            if (!live) g = 0.0;
            if (gate_out) gate_out[t * hc + s] = (float)g;
            if (a_out) a_out[t * hc + s] = a;
            uint16_t* o = out + (t * hc + s) * dim;
            for (int f = 0; f < dim; ++f) {
                if (!live) o[f] = h[f];
                else o[f] = eo_bf16_round(eo_bf16_value(h[f]) + g * eo_bf16_value(value[f]));
            }
        }
    }
}
