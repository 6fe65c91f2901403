/*
 * q8kv CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, deliberately unoptimised C implementation of single-query
 * decode attention over a paged int8 ("q8") KV cache, computed in one
 * online-softmax pass.  It exists to check the GPU library and nothing else:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, constant or helper with the HIP
 * library; neither side includes or links the other.
 *
 * Source of every rule: the page "Day 9-2: flash_attn_single_q_q8_neon"
 * (trdm.cn news 511694), section 2 (segments 1-3).  The code is organised
 * around those rules -- a generic absmax quantiser, a score function and an
 * online-softmax state with init / raise / push -- and keeps the rounding
 * order the rules fix:
 *   - segment 1 (Q -> int8, one absmax scale per 32 elements, same shape as
 *     Q8_0): per block  a = max|q|,  a < 1e-6 -> a = 1,  qsc = a * (1/127),
 *     iq = 127 / a,  qi = (int8) clamp(q * iq, -128, 127);
 *   - segment 2 (online softmax state): M = -1e9, S = 0; per token t the K row
 *     sits in page t / kv_bs at row t % kv_bs; each 32-block gives one int32
 *     dot, the score is  s = sum_b dot_b * qsc[b],  then  s = s * ks * scale;
 *     a new maximum rescales S and the V accumulator by exp(M - s), otherwise
 *     the weight is exp(s - M); S += w; the accumulator gains V_int8 * (w * vs)
 *     with the weight kept in fp32;
 *   - segment 3 (tail): out[i] = acc[i] / S, one division at the end.
 * The K/V quantizer (per token, per kv head, one scale per row) applies the
 * same rule to a whole head-dim row; the page names this "per-token per-head"
 * in the comment on its kscale argument.
 *
 * Readings taken where the garbled page text is silent (each one is listed
 * with its reason in the design notes):
 *   - float -> int8 conversion truncates toward zero (C conversion; no
 *     rounding call survives in the page text);
 *   - the guard is  a < 1e-6f -> a = 1.0f;
 *   - the stored K/V scale is the dequantisation factor a * (1/127), i.e. the
 *     very value the page multiplies in at use;
 *   - the new-maximum test is  s > M  and that branch's own weight is 1;
 *   - seq_len <= 0 gives an all-zero output row;
 *   - rows past seq_len and block-table pads are never read.
 *
 * Paged layout (the HIP library documents the same contract in its header):
 *   pages   int8  [num_blocks][n_kv][kv_bs][hd]
 *   scales  fp32  [num_blocks][n_kv][kv_bs]
 *   table   int32 [batch][max_blocks]      physical block of logical block
 *   q, out  fp32  [batch][n_q][hd];  kv head of q head h is h / (n_q / n_kv).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math; x86-64 SSE math,
 * so every float operation is one IEEE single-precision rounding).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_QBLOCK 32

/* 1/127 rounded once to fp32 (0x3C010204). */
static const float ORC_INV127 = 1.0f / 127.0f;
/* Initial running maximum as printed on the page (0xCE6E6B28). */
static const float ORC_M_INIT = -1e9f;
static const float ORC_TINY = 1e-6f;

float orc_inv127(void) { return ORC_INV127; }
float orc_m_init(void) { return ORC_M_INIT; }

/* clamp(v, lo, hi) followed by C's float -> int conversion (truncation). */
static int8_t orc_to_int8(float v) {
    if (v < -128.0f) v = -128.0f;
    if (v > 127.0f) v = 127.0f;
    return (int8_t)(int)v;
}

/* Quantise n consecutive floats with one absmax scale (segment 1 rule). */
void orc_quantize(const float* x, int n, int8_t* qv, float* scale_out) {
    float a = 0.0f;
    for (int i = 0; i < n; ++i) a = fmaxf(a, fabsf(x[i]));
    if (a < ORC_TINY) a = 1.0f;
    *scale_out = a * ORC_INV127;
    float inv = 127.0f / a;
    for (int i = 0; i < n; ++i) qv[i] = orc_to_int8(x[i] * inv);
}

/* Q rows -> int8 [rows][hd] plus one scale per 32-block [rows][hd/32]. */
void orc_quantize_q(int8_t* qi, float* qsc, const float* q, int rows, int hd) {
    int nb = hd / ORC_QBLOCK;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b)
            orc_quantize(q + (size_t)r * hd + b * ORC_QBLOCK, ORC_QBLOCK,
                         qi + (size_t)r * hd + b * ORC_QBLOCK, qsc + (size_t)r * nb + b);
}

static float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Append: quantise n_tokens source rows per kv head into the pages at
 * slot_mapping[t] = block * kv_bs + row; negative slots are skipped.
 * src_dtype 0 = fp32, 1 = bf16 (widened exactly to fp32 first). */
void orc_append(int8_t* k_pages, int8_t* v_pages, float* k_scale, float* v_scale,
                const void* k_src, const void* v_src, int src_dtype,
                const int32_t* slot_mapping, int n_tokens, int n_kv, int hd, int kv_bs) {
    float* row = (float*)malloc(sizeof(float) * (size_t)hd);
    for (int t = 0; t < n_tokens; ++t) {
        int32_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t blk = slot / kv_bs, r = slot % kv_bs;
        for (int kh = 0; kh < n_kv; ++kh) {
            size_t src_off = ((size_t)t * n_kv + kh) * hd;
            size_t dst_row = ((size_t)blk * n_kv + kh) * kv_bs + r;
            for (int pass = 0; pass < 2; ++pass) {
                const void* src = pass == 0 ? k_src : v_src;
                for (int i = 0; i < hd; ++i)
                    row[i] = src_dtype == 1 ? orc_bf16_to_f32(((const uint16_t*)src)[src_off + i])
                                            : ((const float*)src)[src_off + i];
                int8_t* dst = (pass == 0 ? k_pages : v_pages) + dst_row * hd;
                float* sc = (pass == 0 ? k_scale : v_scale) + dst_row;
                orc_quantize(row, hd, dst, sc);
            }
        }
    }
    free(row);
}

/* Everything one decode call needs, passed around by pointer. */
typedef struct {
    const float* q;
    const int8_t* k_pages;
    const int8_t* v_pages;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int max_blocks, batch, n_q, n_kv, hd, kv_bs;
    float scale;
} orc_args;

/* Row index of logical token t of sequence b for kv head kh. */
static size_t orc_row(const orc_args* a, int b, int kh, int t) {
    int32_t blk = a->block_table[(size_t)b * a->max_blocks + t / a->kv_bs];
    return ((size_t)blk * a->n_kv + kh) * a->kv_bs + (size_t)(t % a->kv_bs);
}

/* int32 dot of one 32-block of quantised q with the K row. */
static int32_t orc_block_dot(const int8_t* qi, const int8_t* k, int blk) {
    int32_t d = 0;
    for (int i = 0; i < ORC_QBLOCK; ++i)
        d += (int32_t)qi[blk * ORC_QBLOCK + i] * (int32_t)k[blk * ORC_QBLOCK + i];
    return d;
}

/* Optional per-token trace of the recurrence (one (b, h) at a time). */
typedef struct {
    float* s;   /* score of token t */
    float* m;   /* running max after token t */
    float* sum; /* running exp-sum after token t */
    float* w;   /* weight given to token t when it arrived */
} orc_trace;

/* Score of one K row (section 2, segment 2): one int32 dot per 32-block,
 * each times its query block's scale, added in block order; the sum times
 * the row's K factor, then times the softmax scale. */
static float orc_score(const int8_t* qi, const float* qsc, const int8_t* k, int nb, float ks, float scale) {
    float s = 0.0f;
    for (int blk = 0; blk < nb; ++blk) s = s + (float)orc_block_dot(qi, k, blk) * qsc[blk];
    return (s * ks) * scale;
}

/* The online-softmax state of one query head (section 2, segment 2): the
 * largest score so far M, the sum S of exp(s_t - M) over the tokens so far,
 * and acc = sum_t exp(s_t - M) * vs_t * V_t over the int8 V codes.  It starts
 * at the page's M = -1e9, S = 0, acc = 0. */
typedef struct {
    float M, S;
    float* acc;
    int hd;
} orc_state;

static void orc_state_init(orc_state* st, float* acc, int hd) {
    st->M = ORC_M_INIT;
    st->S = 0.0f;
    st->acc = acc;
    st->hd = hd;
    for (int i = 0; i < hd; ++i) acc[i] = 0.0f;
}

/* A score s above M moves the normalisation point to s: S and acc are
 * multiplied by exp(M - s). */
static void orc_state_raise(orc_state* st, float s) {
    float m = expf(st->M - s);
    st->S = st->S * m;
    for (int i = 0; i < st->hd; ++i) st->acc[i] = st->acc[i] * m;
    st->M = s;
}

/* Fold in one token of score s whose V row has codes v and factor vs; the
 * token's weight is exp(s - M) after any raise (exactly 1 when it raised M).
 * Returns that weight. */
static float orc_state_push(orc_state* st, float s, const int8_t* v, float vs) {
    float w;
    if (s > st->M) {
        orc_state_raise(st, s);
        w = 1.0f;
    } else {
        w = expf(s - st->M);
    }
    st->S = st->S + w;
    float f = w * vs;
    for (int i = 0; i < st->hd; ++i) st->acc[i] = st->acc[i] + (float)v[i] * f;
    return w;
}

/* The recurrence over tokens [t0, t1) of (b, h), in fp32, token by token.
 * qi/qsc hold the already quantised query row. */
static void orc_run_f32(const orc_args* a, int b, int h, const int8_t* qi, const float* qsc,
                        int t0, int t1, orc_state* st, const orc_trace* tr) {
    int G = a->n_q / a->n_kv, kh = h / G, nb = a->hd / ORC_QBLOCK;
    for (int t = t0; t < t1; ++t) {
        size_t row = orc_row(a, b, kh, t);
        float s = orc_score(qi, qsc, a->k_pages + row * a->hd, nb, a->k_scale[row], a->scale);
        float w = orc_state_push(st, s, a->v_pages + row * a->hd, a->v_scale[row]);
        if (tr) {
            tr->s[t - t0] = s;
            tr->m[t - t0] = st->M;
            tr->sum[t - t0] = st->S;
            tr->w[t - t0] = w;
        }
    }
}

/* The same recurrence with every float quantity held in double; it reads the
 * same int8 values and fp32 scales.  Used to compare the single pass with the
 * three-pass softmax free of fp32 rounding. */
static void orc_run_f64(const orc_args* a, int b, int h, const int8_t* qi, const float* qsc,
                        int t0, int t1, double* M_out, double* S_out, double* acc) {
    int G = a->n_q / a->n_kv, kh = h / G, nb = a->hd / ORC_QBLOCK;
    double M = (double)ORC_M_INIT, S = 0.0;
    for (int i = 0; i < a->hd; ++i) acc[i] = 0.0;
    for (int t = t0; t < t1; ++t) {
        size_t row = orc_row(a, b, kh, t);
        const int8_t* k = a->k_pages + row * a->hd;
        const int8_t* v = a->v_pages + row * a->hd;
        double s = 0.0;
        for (int blk = 0; blk < nb; ++blk) s = s + (double)orc_block_dot(qi, k, blk) * (double)qsc[blk];
        s = (s * (double)a->k_scale[row]) * (double)a->scale;
        double w = 1.0;
        if (s > M) {
            double m = exp(M - s);
            S = S * m;
            for (int i = 0; i < a->hd; ++i) acc[i] = acc[i] * m;
            M = s;
        } else {
            w = exp(s - M);
        }
        S = S + w;
        double f = w * (double)a->v_scale[row];
        for (int i = 0; i < a->hd; ++i) acc[i] = acc[i] + (double)v[i] * f;
    }
    *M_out = M;
    *S_out = S;
}

/* One (b, h) output row.  part_tokens <= 0: one pass over all tokens.
 * part_tokens > 0: split the tokens into consecutive ranges of that length,
 * run the recurrence on each, then merge the range states in range order with
 * the same rescale rule (new max M* = max M_p, S* = sum S_p exp(M_p - M*),
 * acc* = sum acc_p exp(M_p - M*)).  The page applies this rule token by
 * token; applying it to whole ranges is the split-context form. */
static void orc_head(const orc_args* a, int b, int h, int part_tokens, int use_f64,
                     float* out, const orc_trace* tr) {
    int hd = a->hd, nb = hd / ORC_QBLOCK;
    int L = a->seq_lens[b];
    int8_t* qi = (int8_t*)malloc((size_t)hd);
    float* qsc = (float*)malloc(sizeof(float) * (size_t)nb);
    float* acc = (float*)malloc(sizeof(float) * (size_t)hd);
    double* accd = (double*)malloc(sizeof(double) * (size_t)hd);
    float* tot = (float*)malloc(sizeof(float) * (size_t)hd);
    if (L <= 0) {
        for (int i = 0; i < hd; ++i) out[i] = 0.0f;
        goto done;
    }
    orc_quantize_q(qi, qsc, a->q + ((size_t)b * a->n_q + h) * hd, 1, hd);
    if (use_f64) {
        double M, S;
        orc_run_f64(a, b, h, qi, qsc, 0, L, &M, &S, accd);
        for (int i = 0; i < hd; ++i) out[i] = (float)(accd[i] / S);
        goto done;
    }
    if (part_tokens <= 0 || part_tokens >= L) {
        orc_state st;
        orc_state_init(&st, acc, hd);
        orc_run_f32(a, b, h, qi, qsc, 0, L, &st, tr);
        for (int i = 0; i < hd; ++i) out[i] = acc[i] / st.S;
        goto done;
    }
    {
        int np = (L + part_tokens - 1) / part_tokens;
        float* Mp = (float*)malloc(sizeof(float) * (size_t)np);
        float* Sp = (float*)malloc(sizeof(float) * (size_t)np);
        float* accp = (float*)malloc(sizeof(float) * (size_t)np * hd);
        for (int p = 0; p < np; ++p) {
            int t0 = p * part_tokens, t1 = t0 + part_tokens < L ? t0 + part_tokens : L;
            orc_state st;
            orc_state_init(&st, accp + (size_t)p * hd, hd);
            orc_run_f32(a, b, h, qi, qsc, t0, t1, &st, NULL);
            Mp[p] = st.M;
            Sp[p] = st.S;
        }
        float Mx = ORC_M_INIT;
        for (int p = 0; p < np; ++p) Mx = fmaxf(Mx, Mp[p]);
        float St = 0.0f;
        for (int i = 0; i < hd; ++i) tot[i] = 0.0f;
        for (int p = 0; p < np; ++p) {
            float e = expf(Mp[p] - Mx);
            St = St + Sp[p] * e;
            for (int i = 0; i < hd; ++i) tot[i] = tot[i] + accp[(size_t)p * hd + i] * e;
        }
        for (int i = 0; i < hd; ++i) out[i] = tot[i] / St;
        free(Mp);
        free(Sp);
        free(accp);
    }
done:
    free(qi);
    free(qsc);
    free(acc);
    free(accd);
    free(tot);
}

/* Decode attention for every (b, h).  threads > 1 splits the (b, h) pairs
 * over OpenMP threads (each pair is still computed by the sequential code
 * above, so the result is bitwise the same as threads == 1).
 * part_tokens: see orc_head.  use_f64: run the double-precision twin. */
int orc_decode(float* out, const float* q, const int8_t* k_pages, const int8_t* v_pages,
               const float* k_scale, const float* v_scale, const int32_t* block_table,
               const int32_t* seq_lens, int max_blocks, int batch, int n_q, int n_kv, int hd,
               int kv_bs, float scale, int part_tokens, int use_f64, int threads) {
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || n_q % n_kv || hd <= 0 || hd % ORC_QBLOCK || kv_bs <= 0)
        return -1;
    orc_args a = {q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens,
                  max_blocks, batch, n_q, n_kv, hd, kv_bs, scale};
    long total = (long)batch * n_q;
    if (threads < 1) threads = 1;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) if (threads > 1)
#endif
    for (long bh = 0; bh < total; ++bh) {
        int b = (int)(bh / n_q), h = (int)(bh % n_q);
        orc_head(&a, b, h, part_tokens, use_f64, out + (size_t)bh * hd, NULL);
    }
    return 0;
}

/* One (b, h) with the per-token trace (arrays of seq_lens[b] floats each). */
int orc_decode_trace(float* out, float* tr_s, float* tr_m, float* tr_sum, float* tr_w,
                     const float* q, const int8_t* k_pages, const int8_t* v_pages,
                     const float* k_scale, const float* v_scale, const int32_t* block_table,
                     const int32_t* seq_lens, int max_blocks, int batch, int n_q, int n_kv,
                     int hd, int kv_bs, float scale, int b, int h) {
    if (b < 0 || b >= batch || h < 0 || h >= n_q || n_q % n_kv || hd % ORC_QBLOCK) return -1;
    orc_args a = {q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens,
                  max_blocks, batch, n_q, n_kv, hd, kv_bs, scale};
    orc_trace tr = {tr_s, tr_m, tr_sum, tr_w};
    orc_head(&a, b, h, 0, 0, out, &tr);
    return 0;
}

/* int32 block dots [batch][n_q][max_tok][hd/32] for t < seq_lens[b]; other
 * entries are left untouched. */
int orc_block_dots(int32_t* dots, int max_tok, const float* q, const int8_t* k_pages,
                   const int32_t* block_table, const int32_t* seq_lens, int max_blocks,
                   int batch, int n_q, int n_kv, int hd, int kv_bs) {
    if (n_q % n_kv || hd % ORC_QBLOCK) return -1;
    orc_args a = {q, k_pages, NULL, NULL, NULL, block_table, seq_lens,
                  max_blocks, batch, n_q, n_kv, hd, kv_bs, 0.0f};
    int nb = hd / ORC_QBLOCK, G = n_q / n_kv;
    int8_t* qi = (int8_t*)malloc((size_t)hd);
    float* qsc = (float*)malloc(sizeof(float) * (size_t)nb);
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < n_q; ++h) {
            orc_quantize_q(qi, qsc, q + ((size_t)b * n_q + h) * hd, 1, hd);
            int L = seq_lens[b] < max_tok ? seq_lens[b] : max_tok;
            for (int t = 0; t < L; ++t) {
                const int8_t* k = k_pages + orc_row(&a, b, h / G, t) * hd;
                for (int blk = 0; blk < nb; ++blk)
                    dots[(((size_t)b * n_q + h) * max_tok + t) * nb + blk] = orc_block_dot(qi, k, blk);
            }
        }
    free(qi);
    free(qsc);
    return 0;
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
