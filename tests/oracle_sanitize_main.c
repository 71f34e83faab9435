/*
 * Test driver: runs the CPU oracle (oracle/engram_oracle.c) through all four
 * stages on inputs read from raw files, so the oracle can be built and run
 * under AddressSanitizer and UndefinedBehaviorSanitizer.  Test
 * infrastructure only; tests/test_oracle_sanitized.py builds and runs it and
 * compares what it writes with the normal oracle build.
 *
 * usage: eo_sanitized DIR
 *   DIR/geom.txt     dim hc max_ngram n_heads head_dim vocab pad_id num_rows eps B T
 *   DIR/token_map.bin int32 [vocab]         DIR/mult.bin   uint64 [n_cols][max_ngram]
 *   DIR/prime.bin     uint64 [n_cols]        DIR/offset.bin uint64 [n_cols]
 *   DIR/ids.bin       int32 [B][T]           DIR/table.bin  uint8 [num_rows][head_dim]
 *   DIR/scales.bin    uint8 [num_rows][head_dim/32]
 *   DIR/w.bin, q.bin, k.bin, x.bin, mask.bin  (bf16 bits; mask uint8 [B*T])
 * writes DIR/out_{hash,rows,kv,out,gate}.bin.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int eo_hash(int max_ngram, int n_heads, int32_t pad_id, int64_t vocab, const int32_t* token_map,
            const uint64_t* mult, const uint64_t* prime, const uint64_t* offset, int B,
            int64_t T, const int32_t* ids, int32_t* hist, int64_t hist_cap, int64_t* hist_len,
            int32_t* hash_ids);
int eo_embed_rows(int head_dim, int64_t num_rows, const uint8_t* table, const uint8_t* scales,
                  const int32_t* ids, int64_t n_ids, uint16_t* out);
void eo_linear(int64_t M, int64_t N, int64_t K, const uint16_t* a, const uint16_t* w,
               uint16_t* out);
void eo_gate_and_add(int64_t n_tok, int hc, int dim, float eps, const uint16_t* x,
                     const uint16_t* kv, const uint16_t* q, const uint16_t* k,
                     const uint8_t* mask, uint16_t* out, float* gate_out, double* a_out);

static char g_dir[4096];

/* Reads exactly `bytes` bytes of DIR/name into a fresh exact-size buffer. */
static void* load(const char* name, size_t bytes) {
    char path[4200];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void* p = malloc(bytes ? bytes : 1);
    if (fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void save(const char* name, const void* p, size_t bytes) {
    char path[4200];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s DIR\n", argv[0]); return 2; }
    snprintf(g_dir, sizeof g_dir, "%s", argv[1]);
    char path[4200];
    snprintf(path, sizeof path, "%s/geom.txt", g_dir);
    FILE* f = fopen(path, "r");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); return 2; }
    int dim, hc, mx, nh, hd, pad, B;
    long long vocab, rows, T;
    float eps;
    if (fscanf(f, "%d %d %d %d %d %lld %d %lld %f %d %lld", &dim, &hc, &mx, &nh, &hd, &vocab,
               &pad, &rows, &eps, &B, &T) != 11) {
        fprintf(stderr, "bad geom.txt\n");
        return 2;
    }
    fclose(f);
    const int n_cols = (mx - 1) * nh;
    const int64_t n = (int64_t)B * T, K = (int64_t)n_cols * hd, N = (int64_t)dim * (hc + 1);

    int32_t* token_map = load("token_map.bin", (size_t)vocab * 4);
    uint64_t* mult = load("mult.bin", (size_t)n_cols * mx * 8);
    uint64_t* prime = load("prime.bin", (size_t)n_cols * 8);
    uint64_t* offset = load("offset.bin", (size_t)n_cols * 8);
    int32_t* ids = load("ids.bin", (size_t)n * 4);
    uint8_t* table = load("table.bin", (size_t)rows * hd);
    uint8_t* scales = load("scales.bin", (size_t)rows * (hd / 32));
    uint16_t* w = load("w.bin", (size_t)N * K * 2);
    uint16_t* q = load("q.bin", (size_t)hc * dim * 2);
    uint16_t* k = load("k.bin", (size_t)hc * dim * 2);
    uint16_t* x = load("x.bin", (size_t)n * hc * dim * 2);
    uint8_t* mask = load("mask.bin", (size_t)n);

    /* the hash state holds exactly the history the call needs */
    int32_t* hist = malloc((size_t)B * T * 4);
    int64_t* hist_len = calloc((size_t)B, sizeof(int64_t));
    int32_t* hash = malloc((size_t)n * n_cols * 4);
    int rc = eo_hash(mx, nh, pad, vocab, token_map, mult, prime, offset, B, T, ids, hist, T,
                     hist_len, hash);
    if (rc != 0) { fprintf(stderr, "eo_hash: %d\n", rc); return 3; }
    uint16_t* a = malloc((size_t)n * K * 2);
    rc = eo_embed_rows(hd, rows, table, scales, hash, n * n_cols, a);
    if (rc != 0) { fprintf(stderr, "eo_embed_rows: %d\n", rc); return 3; }
    uint16_t* kv = malloc((size_t)n * N * 2);
    eo_linear(n, N, K, a, w, kv);
    uint16_t* out = malloc((size_t)n * hc * dim * 2);
    float* gate = malloc((size_t)n * hc * 4);
    double* av = malloc((size_t)n * hc * 8);
    eo_gate_and_add(n, hc, dim, eps, x, kv, q, k, mask, out, gate, av);

    save("out_hash.bin", hash, (size_t)n * n_cols * 4);
    save("out_rows.bin", a, (size_t)n * K * 2);
    save("out_kv.bin", kv, (size_t)n * N * 2);
    save("out_out.bin", out, (size_t)n * hc * dim * 2);
    save("out_gate.bin", gate, (size_t)n * hc * 4);

    free(token_map); free(mult); free(prime); free(offset); free(ids); free(table); free(scales);
    free(w); free(q); free(k); free(x); free(mask); free(hist); free(hist_len); free(hash);
    free(a); free(kv); free(out); free(gate); free(av);
    return 0;
}
