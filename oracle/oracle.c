/*
 * CPU oracle for sparse MLA decode -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 implementation of what one decode step computes, written
 * from the definition of attention over a top-k set of gathered latent rows.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library; the GPU library never links or calls it and the two
 * share no code.
 *
 * Method (pages: "The Moment of Compilation", section "The Context: A Kernel
 * Optimization Campaign"; "The Power-of-Two Trap", sections "The Scene" and
 * "The Scale Indexing Complication"): for one query token per sequence, every
 * head attends over the rows that the sequence's top-k list selects.  A row is
 * the 512-wide latent vector: 448 "nope" columns stored as fp8 e4m3fn codes,
 * each 64-column group carrying one scale, and 64 "rope" columns stored as
 * bf16.  Keys and values are the same dequantised latent row.  The oracle
 *   1. keeps the list entries j with 0 <= idx[b,j] < seqlens[b], in list order
 *      (with a paged cache also requiring that the entry's page exists, see
 *      cache_layout below);
 *   2. dequantises each selected row in fp64: K[i] = e4m3(code[i]) * s[i/64]
 *      for i < 448 and K[448+k] = rope[k];
 *   3. z_j = scale * sum_{d<512} q[d] * K_j[d], summed in index order;
 *   4. M = max z_j, L = sum exp(z_j - M), lse = M + ln L,
 *      out[d] = sum_j exp(z_j - M) * K_j[d] / L.
 * With no selected entry the result is out = 0, lse = -inf.  It re-dequantises
 * every row for every head (the naive per-head loop), parallel over (b, h).
 *
 * Cache layouts (its own constants, read from the row format descriptions):
 *   format 0: row stride 640 bytes; nope codes at 0..447; fp32 scales at 448
 *             (7 used, the 8th slot is padding); bf16 rope at 480..607.
 *   format 1: row stride 584 bytes; nope codes at 0..447; UE8M0 scales at
 *             448 (one byte per group, 7 used, the 8th is padding); bf16 rope
 *             at 456..583.  The pages give the deployed model's scales as
 *             unsigned 8-bit exponent-only values, one per 64-column group
 *             ("The Power-of-Two Trap", section "Input Knowledge Required");
 *             the value of byte e is read as 2^(e - 127), with e = 255 NaN.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_ROW_STRIDE 640
#define OR_NOPE 448
#define OR_ROPE 64
#define OR_LATENT 512
#define OR_GROUP 64
#define OR_SCALE_AT 448
#define OR_ROPE_AT 480
#define OR_UE8M0_ROW_STRIDE 584
#define OR_UE8M0_SCALE_AT 448
#define OR_UE8M0_ROPE_AT 456

/* OCP fp8 e4m3fn: sign, 4 exponent bits with bias 7, 3 mantissa bits.
 * Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities. */
double oracle_e4m3fn_value(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bf16 is the top half of an fp32 bit pattern. */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double f32_at(const uint8_t* p) {
    float f;
    memcpy(&f, p, 4);
    return (double)f;
}

/* UE8M0 scale byte: 2^(e - 127); 255 is NaN. */
double oracle_ue8m0_value(uint8_t e) {
    if (e == 0xFF) return NAN;
    return ldexp(1.0, (int)e - 127);
}

int oracle_row_stride(int fmt) { return fmt == 1 ? OR_UE8M0_ROW_STRIDE : OR_ROW_STRIDE; }

/* Dequantise one cache row of format fmt into K[512] (fp64, exact). */
void oracle_dequant_row_fmt(const uint8_t* row, int fmt, double* K) {
    for (int i = 0; i < OR_NOPE; i++) {
        const int g = i / OR_GROUP;
        const double s = fmt == 1 ? oracle_ue8m0_value(row[OR_UE8M0_SCALE_AT + g])
                                  : f32_at(row + OR_SCALE_AT + 4 * g);
        K[i] = oracle_e4m3fn_value(row[i]) * s;
    }
    const int rope_at = fmt == 1 ? OR_UE8M0_ROPE_AT : OR_ROPE_AT;
    for (int k = 0; k < OR_ROPE; k++) {
        uint16_t b;
        memcpy(&b, row + rope_at + 2 * k, 2);
        K[OR_NOPE + k] = oracle_bf16_value(b);
    }
}

void oracle_dequant_row(const uint8_t* row, double* K) { oracle_dequant_row_fmt(row, 0, K); }

/*
 * Where the cache row of list entry t of sequence b lives.  Contiguous: row t
 * of sequence b at (b * kv_seq_stride + t) rows from the start.  Paged: the
 * pool holds pages of page_size rows; block_table[b * pages_per_seq + p] is the
 * pool page holding positions p * page_size .. (p + 1) * page_size - 1 of
 * sequence b.  The paged reading of the pages' "paged FP8 format" ("The
 * Power-of-Two Trap", section "Input Knowledge Required"), which gives no
 * block size or table: the usual block-table page pool.
 */
typedef struct {
    const uint8_t* base;
    int64_t row_stride;       /* bytes per row */
    int64_t kv_seq_stride;    /* contiguous: rows per sequence */
    const int32_t* block_table;   /* NULL: contiguous */
    int64_t pages_per_seq, num_pages;
    int32_t page_size;
} cache_layout;

/* Row of entry t of sequence b, or NULL when the entry is skipped: t < 0,
 * t >= seqlen, (contiguous) t at or past the sequence stride, so that a
 * sequence never reaches another's rows, and (paged) a position past the
 * sequence's block-table row or a page id outside the pool. */
static const uint8_t* row_of(const cache_layout* c, int b, int32_t t, int32_t seqlen) {
    if (t < 0 || t >= seqlen) return NULL;
    if (!c->block_table) {
        if (t >= c->kv_seq_stride) return NULL;
        return c->base + ((int64_t)b * c->kv_seq_stride + t) * c->row_stride;
    }
    int64_t p = t / c->page_size;
    if (p >= c->pages_per_seq) return NULL;
    int64_t page = c->block_table[(int64_t)b * c->pages_per_seq + p];
    if (page < 0 || page >= c->num_pages) return NULL;
    return c->base + (page * c->page_size + t % c->page_size) * c->row_stride;
}

static int decode_core(const uint16_t* q, const cache_layout* c, const int32_t* idx,
                       int64_t idx_row_stride, const int32_t* seqlens, int B, int H, int topk,
                       double scale, double* out, double* lse, int nthreads, int fmt) {
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#endif
    int64_t total = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < total; bh++) {
        int b = (int)(bh / H), h = (int)(bh % H);
        const uint16_t* qh = q + ((int64_t)b * H + h) * OR_LATENT;
        double qd[OR_LATENT];
        for (int d = 0; d < OR_LATENT; d++) qd[d] = oracle_bf16_value(qh[d]);
        double K[OR_LATENT];
        /* pass 1: logits of the selected entries, in list order */
        double M = -INFINITY;
        int nsel = 0;
        for (int j = 0; j < topk; j++) {
            const uint8_t* row = row_of(c, b, idx[(int64_t)b * idx_row_stride + j], seqlens[b]);
            if (!row) continue;
            oracle_dequant_row_fmt(row, fmt, K);
            double z = 0.0;
            for (int d = 0; d < OR_LATENT; d++) z += qd[d] * K[d];
            z *= scale;
            if (nsel == 0 || z > M) M = z;
            nsel++;
        }
        double* o = out + bh * OR_LATENT;
        for (int d = 0; d < OR_LATENT; d++) o[d] = 0.0;
        if (nsel == 0) {
            lse[bh] = -INFINITY;
            continue;
        }
        /* pass 2: exact softmax weights and the weighted sum of value rows */
        double L = 0.0;
        for (int j = 0; j < topk; j++) {
            const uint8_t* row = row_of(c, b, idx[(int64_t)b * idx_row_stride + j], seqlens[b]);
            if (!row) continue;
            oracle_dequant_row_fmt(row, fmt, K);
            double z = 0.0;
            for (int d = 0; d < OR_LATENT; d++) z += qd[d] * K[d];
            z *= scale;
            double w = exp(z - M);
            L += w;
            for (int d = 0; d < OR_LATENT; d++) o[d] += w * K[d];
        }
        for (int d = 0; d < OR_LATENT; d++) o[d] /= L;
        lse[bh] = M + log(L);
    }
    return used;
}

/*
 * q:        bf16 bits [B][H][512]
 * kv:       cache bytes [B][kv_seq_stride][row bytes of the format]
 * idx:      int32, entry (b, j) at idx[b * idx_row_stride + j], j < topk
 * seqlens:  int32 [B]
 * out:      fp64 [B][H][512];  lse: fp64 [B][H]
 * nthreads: OpenMP threads (<= 0: library default).  Returns the thread count used.
 */
int oracle_decode_fmt(const uint16_t* q, const uint8_t* kv, int64_t kv_seq_stride,
                      const int32_t* idx, int64_t idx_row_stride, const int32_t* seqlens,
                      int B, int H, int topk, double scale, double* out, double* lse,
                      int nthreads, int fmt) {
    cache_layout c = {kv, oracle_row_stride(fmt), kv_seq_stride, NULL, 0, 0, 1};
    return decode_core(q, &c, idx, idx_row_stride, seqlens, B, H, topk, scale, out, lse, nthreads, fmt);
}

/*
 * The same step over a paged pool: pool holds num_pages * page_size rows of
 * the format; block_table int32 [B][pages_per_seq] (see cache_layout).
 */
int oracle_decode_paged(const uint16_t* q, const uint8_t* pool, int64_t num_pages, int32_t page_size,
                        const int32_t* block_table, int64_t pages_per_seq, const int32_t* idx,
                        int64_t idx_row_stride, const int32_t* seqlens, int B, int H, int topk,
                        double scale, double* out, double* lse, int nthreads, int fmt) {
    cache_layout c = {pool, oracle_row_stride(fmt), 0, block_table, pages_per_seq, num_pages, page_size};
    return decode_core(q, &c, idx, idx_row_stride, seqlens, B, H, topk, scale, out, lse, nthreads, fmt);
}

int oracle_decode(const uint16_t* q, const uint8_t* kv, int64_t kv_seq_stride,
                  const int32_t* idx, int64_t idx_row_stride, const int32_t* seqlens,
                  int B, int H, int topk, double scale, double* out, double* lse,
                  int nthreads) {
    return oracle_decode_fmt(q, kv, kv_seq_stride, idx, idx_row_stride, seqlens, B, H, topk, scale, out,
                             lse, nthreads, 0);
}

/*
 * The padded formulation of the same computation, as the Triton kernel on the
 * pages arranges it ("The Power-of-Two Trap", sections "The Padding Strategy"
 * and "The Scale Indexing Complication"): q and k nope are widened to 512
 * columns; columns 448..511 are zero in both and belong to the pad scale slot
 * (group 7), which is excluded by selection (the column is set to zero, never
 * multiplied by that slot); rope follows at 512..575.  Summation runs over the
 * 576 padded columns in index order.  Adding exact zero products leaves every
 * partial sum unchanged, so the result must be bitwise equal to
 * oracle_decode.
 */
int oracle_decode_padded512(const uint16_t* q, const uint8_t* kv, int64_t kv_seq_stride,
                            const int32_t* idx, int64_t idx_row_stride,
                            const int32_t* seqlens, int B, int H, int topk,
                            double scale, double* out, double* lse) {
    enum { PAD = 512, WIDE = PAD + OR_ROPE };
    for (int64_t bh = 0; bh < (int64_t)B * H; bh++) {
        int b = (int)(bh / H), h = (int)(bh % H);
        const uint16_t* qh = q + ((int64_t)b * H + h) * OR_LATENT;
        double qw[WIDE], Kw[WIDE];
        for (int c = 0; c < PAD; c++) qw[c] = c < OR_NOPE ? oracle_bf16_value(qh[c]) : 0.0;
        for (int k = 0; k < OR_ROPE; k++) qw[PAD + k] = oracle_bf16_value(qh[OR_NOPE + k]);
        double* o = out + bh * OR_LATENT;
        for (int d = 0; d < OR_LATENT; d++) o[d] = 0.0;
        double M = -INFINITY, L = 0.0;
        int nsel = 0;
        for (int pass = 0; pass < 2; pass++) {
            for (int j = 0; j < topk; j++) {
                int32_t t = idx[(int64_t)b * idx_row_stride + j];
                if (t < 0 || t >= seqlens[b]) continue;
                const uint8_t* row = kv + ((int64_t)b * kv_seq_stride + t) * OR_ROW_STRIDE;
                for (int c = 0; c < PAD; c++) {
                    int g = c / OR_GROUP; /* 0..6 real groups; 7 is the pad slot */
                    /* selection, not multiplication: a pad column is zero whatever slot 7 holds */
                    Kw[c] = c < OR_NOPE ? oracle_e4m3fn_value(row[c]) * f32_at(row + OR_SCALE_AT + 4 * g) : 0.0;
                }
                for (int k = 0; k < OR_ROPE; k++) {
                    uint16_t bb;
                    memcpy(&bb, row + OR_ROPE_AT + 2 * k, 2);
                    Kw[PAD + k] = oracle_bf16_value(bb);
                }
                double z = 0.0;
                for (int c = 0; c < WIDE; c++) z += qw[c] * Kw[c];
                z *= scale;
                if (pass == 0) {
                    if (nsel == 0 || z > M) M = z;
                    nsel++;
                } else {
                    double w = exp(z - M);
                    L += w;
                    /* only the 448 real nope columns and the rope columns are stored */
                    for (int c = 0; c < OR_NOPE; c++) o[c] += w * Kw[c];
                    for (int k = 0; k < OR_ROPE; k++) o[OR_NOPE + k] += w * Kw[PAD + k];
                }
            }
            if (nsel == 0) break;
        }
        if (nsel == 0) {
            lse[bh] = -INFINITY;
            continue;
        }
        for (int d = 0; d < OR_LATENT; d++) o[d] /= L;
        lse[bh] = M + log(L);
    }
    return 1;
}
