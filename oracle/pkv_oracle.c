/*
 * pkv_oracle.c -- float64 CPU oracle for paged-KV varlen attention.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the GPU
 * path is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code, header, table or
 * constant with the GPU library, and the GPU library never calls it.
 *
 * What it follows (page titles of the source material):
 *  - "How vLLM attention kernels handle multiple requests in parallel"
 *      §1  packed varlen batch; requests never see each other
 *      §4-§5  causal mask from request-local positions
 *      §7  online softmax (unnormalised form) -- or_attention_online
 *      §9  decode: a single query sees the whole context
 *      §10 multi-token verification: query t sees keys [0, ctx + t]
 *      §11 paged address translation -- or_slot
 *      §12 split-KV segments (m_s, l_s, O_s) and their reduction
 *  - "FlashAttention deep dive" (vLLM V1 FlashAttention backend)
 *      Memory-I/O section: online softmax in the normalised form -- or_attention_online_normalised
 *      Core implementation section: KV cache write by slot_mapping
 *      Cascade attention section: prefix/suffix merge by log-sum-exp -- or_merge
 *      FA3 FP8 section: float8_e4m3fn cache with per-tensor scales
 *
 * The attention result is computed from its definition: for each request,
 * query token and head, softmax(scale * q . k_j) over the visible keys j, then
 * the weighted sum of v_j, in float64, two passes, no tiling. Inputs are
 * decoded exactly to double (bf16 and fp32 are exact; e4m3fn through the OCP
 * definition) and multiplied by the per-tensor scale.
 *
 * Readings where the source is silent (all listed in the design notes):
 *  - lse is the natural log, laid out [H, T] (head-major);
 *  - q head h uses kv head h / (H / Hkv);
 *  - causal is bottom-right aligned: query t of a request with context ctx
 *    (= seq_len - q_len) sees keys 0 .. ctx + t;
 *  - masked keys are excluded (weight 0), so a row with no visible key has
 *    out = 0 and lse = -inf;
 *  - fp8 encode: q = fl32(x / scale), then nearest e4m3fn value with ties to
 *    the even code, finite overflow and +-inf saturate to +-448, NaN stays NaN
 *    (code 0x7F with the input's sign bit).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3FN = 2 };

/* ---------------------------------------------------------------- values */

/* OCP 8-bit float E4M3 ("fn" variant: no infinities, one NaN pattern per sign,
 * exponent bias 7, subnormals m * 2^-9). */
double or_decode_e4m3fn(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static double g_e4m3_pos[127]; /* values of codes 0x00..0x7E, increasing */
static int g_e4m3_ready = 0;

static void e4m3_table_init(void) {
    if (g_e4m3_ready) return;
    for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = or_decode_e4m3fn((uint8_t)c);
    g_e4m3_ready = 1;
}

/* Nearest representable e4m3fn value to y (a float), ties to the even code;
 * |y| >= 448 saturates; NaN -> 0x7F | sign. Defined by search over the value
 * table, not by bit manipulation. */
uint8_t or_encode_e4m3fn(float y) {
    e4m3_table_init();
    uint32_t bits;
    memcpy(&bits, &y, 4);
    uint8_t sign = (uint8_t)((bits >> 31) << 7);
    if (isnan(y)) return (uint8_t)(0x7F | sign);
    double a = fabs((double)y);
    if (a >= 448.0) return (uint8_t)(0x7E | sign);
    /* largest code lo with value <= a */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_e4m3_pos[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int best = lo;
    if (lo < 126 && g_e4m3_pos[lo] != a) {
        double dlo = a - g_e4m3_pos[lo], dhi = g_e4m3_pos[lo + 1] - a;
        if (dhi < dlo) best = lo + 1;
        else if (dhi == dlo) best = (lo % 2 == 0) ? lo : lo + 1;
    }
    return (uint8_t)(best | sign);
}

/* bf16 storage (upper 16 bits of an IEEE binary32) -> double, exact. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Nearest bf16 to a binary32, ties to even; NaN stays a quiet NaN. */
uint16_t or_encode_bf16(float x) {
    if (isnan(x)) {
        uint32_t u;
        memcpy(&u, &x, 4);
        return (uint16_t)((u >> 16) | 0x0040);
    }
    /* candidates: truncation toward zero, and the next bf16 away from zero */
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t t = (uint16_t)(u >> 16);
    uint32_t tu = (uint32_t)t << 16;
    float tf;
    memcpy(&tf, &tu, 4);
    if (tf == x) return t;
    uint16_t n = (uint16_t)(t + 1); /* same sign, larger magnitude */
    double tv = bf16_to_double(t);
    /* past the largest finite bf16 the next step would be 2^128 */
    double nv = ((n & 0x7FFF) == 0x7F80) ? copysign(ldexp(1.0, 128), (double)x) : bf16_to_double(n);
    double dt = fabs((double)x - tv);
    double dn = fabs(nv - (double)x);
    if (dn < dt) return n;
    if (dt < dn) return t;
    return (t & 1) ? n : t;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
        case OR_F32: return (double)((const float*)base)[idx];
        case OR_BF16: return bf16_to_double(((const uint16_t*)base)[idx]);
        case OR_E4M3FN: return or_decode_e4m3fn(((const uint8_t*)base)[idx]);
        default: return NAN;
    }
}

/* ---------------------------------------------------------- translation */

/* Paged address translation: logical position -> physical slot
 * (logical block = pos / bs, physical block from the request's row of the
 * block table, slot = physical * bs + pos % bs). */
int64_t or_slot(const int32_t* block_table, int64_t bt_stride, int r, int64_t pos, int bs) {
    int64_t logical_block = pos / bs;
    int64_t physical_block = block_table[(int64_t)r * bt_stride + logical_block];
    return physical_block * bs + pos % bs;
}

/* ----------------------------------------------------------- cache write */

/* Scatter each new token's K and V into the cache at slot_mapping[t]
 * (block = slot / bs, offset = slot % bs). slot < 0 marks padding and is
 * skipped. Encodings: same type -> bit copy; f32 -> bf16 nearest-even;
 * f32 or bf16 -> e4m3fn via fl32(x / scale) then or_encode_e4m3fn.
 * Returns 0, or -1 for an unsupported pair. */
int or_cache_write(const void* key, const void* value, int src_dtype,
                   void* k_cache, void* v_cache, int cache_dtype,
                   const int64_t* slot_mapping, int T, int Hkv, int hd, int bs,
                   float k_scale, float v_scale) {
    if (!(src_dtype == OR_F32 || src_dtype == OR_BF16)) return -1;
    if (cache_dtype == OR_F32 && src_dtype != OR_F32) return -1;
    if (!(cache_dtype == src_dtype || cache_dtype == OR_BF16 || cache_dtype == OR_E4M3FN)) return -1;
    if (cache_dtype == OR_E4M3FN) e4m3_table_init();
    int64_t row = (int64_t)Hkv * hd;
    /* Tokens are independent (their slots are distinct), so they may be
     * written in any order; each element is encoded exactly as below. */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t blk = slot / bs, off = slot % bs;
        int64_t dst0 = (blk * bs + off) * row;
        for (int kv = 0; kv < 2; ++kv) {
            const void* src = kv ? value : key;
            void* dst = kv ? v_cache : k_cache;
            float sc = kv ? v_scale : k_scale;
            for (int64_t i = 0; i < row; ++i) {
                int64_t si = (int64_t)t * row + i, di = dst0 + i;
                if (cache_dtype == src_dtype) {
                    if (src_dtype == OR_F32) ((float*)dst)[di] = ((const float*)src)[si];
                    else ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
                } else if (cache_dtype == OR_BF16) {
                    ((uint16_t*)dst)[di] = or_encode_bf16(((const float*)src)[si]);
                } else if (cache_dtype == OR_E4M3FN) {
                    float x = (float)load_elem(src, src_dtype, si); /* exact */
                    volatile float y = x / sc;                      /* binary32 division, round to nearest */
                    ((uint8_t*)dst)[di] = or_encode_e4m3fn(y);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------- attention */

typedef struct {
    const void* q; int q_dtype;                  /* [T, H, hd] */
    const void* k; const void* v; int kv_dtype;  /* paged: [num_blocks, bs, Hkv, hd]; contiguous: [T, Hkv, hd] */
    double k_scale, v_scale;                     /* multiply decoded K / V */
    const int32_t* qsl;                          /* [B+1] query_start_loc */
    const int32_t* seq_lens;                     /* [B] KV length incl. new tokens */
    const int32_t* block_table;                  /* [B, bt_stride], NULL => contiguous */
    int64_t bt_stride;
    int B, H, Hkv, hd, bs;
    double scale;
    int causal;
    /* attention variants (the deep-dive page lists sliding window, logits soft
     * cap and attention sinks among the supported variants; the readings are
     * stated at or_attention_ex) */
    int64_t window_left;  /* < 0: no window */
    double softcap;       /* <= 0: no cap */
    const double* sinks;  /* [H] or NULL */
    const double* alibi;  /* [H] ALiBi slopes or NULL */
} or_problem;

static int request_of(const or_problem* p, int64_t tok) {
    int lo = 0, hi = p->B - 1;
    while (lo < hi) { /* last r with qsl[r] <= tok */
        int mid = (lo + hi + 1) / 2;
        if (p->qsl[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* row offset (in elements) of key/value j of request r, kv head g */
static int64_t kv_offset(const or_problem* p, int r, int64_t j, int g) {
    int64_t row;
    if (p->block_table) row = or_slot(p->block_table, p->bt_stride, r, j, p->bs);
    else row = p->qsl[r] + j;
    return (row * p->Hkv + g) * p->hd;
}

/* number of keys query token (request r, local index t) may attend */
static int64_t visible(const or_problem* p, int r, int64_t t) {
    int64_t q_len = p->qsl[r + 1] - p->qsl[r];
    int64_t L = p->block_table ? p->seq_lens[r] : q_len;
    if (!p->causal) return L;
    int64_t ctx = L - q_len;
    int64_t n = ctx + t + 1;
    if (n < 0) n = 0;
    if (n > L) n = L;
    return n;
}

/* first key query token (request r, local index t) may attend: with a
 * window, key j is visible only if j >= i - window_left, where i = ctx + t is
 * the query's position in its sequence */
static int64_t first_visible(const or_problem* p, int r, int64_t t) {
    if (p->window_left < 0) return 0;
    int64_t q_len = p->qsl[r + 1] - p->qsl[r];
    int64_t L = p->block_table ? p->seq_lens[r] : q_len;
    int64_t lo = (L - q_len) + t - p->window_left;
    return lo > 0 ? lo : 0;
}

/* Definition: two passes over the visible keys of one (token, head). */
static void attend_one(const or_problem* p, int64_t tok, int h, double* s, double* qv,
                       double* out /* [hd] */, double* lse) {
    int r = request_of(p, tok);
    int64_t t = tok - p->qsl[r];
    int g = h / (p->H / p->Hkv);
    int64_t n = visible(p, r, t);
    int64_t lo = first_visible(p, r, t);
    int64_t q_len = p->qsl[r + 1] - p->qsl[r];
    int64_t i_pos = (p->block_table ? p->seq_lens[r] : q_len) - q_len + t;  /* the query's position */
    int hd = p->hd;
    double sink = p->sinks ? p->sinks[h] : -INFINITY;
    for (int d = 0; d < hd; ++d) qv[d] = load_elem(p->q, p->q_dtype, (tok * p->H + h) * hd + d);
    for (int d = 0; d < hd; ++d) out[d] = 0.0;
    if (n <= lo && sink == -INFINITY) { *lse = -INFINITY; return; }
    double m = sink;
    for (int64_t j = lo; j < n; ++j) {
        int64_t off = kv_offset(p, r, j, g);
        double dot = 0.0;
        for (int d = 0; d < hd; ++d) dot += qv[d] * (load_elem(p->k, p->kv_dtype, off + d) * p->k_scale);
        s[j] = p->scale * dot;
        if (p->softcap > 0) s[j] = p->softcap * tanh(s[j] / p->softcap);
        if (p->alibi) s[j] -= p->alibi[h] * fabs((double)(i_pos - j));
        if (s[j] > m) m = s[j];
    }
    /* the sink is one more logit in the normaliser; it adds no value row */
    double z = sink == -INFINITY ? 0.0 : exp(sink - m);
    for (int64_t j = lo; j < n; ++j) {
        double w = exp(s[j] - m);
        z += w;
        int64_t off = kv_offset(p, r, j, g);
        for (int d = 0; d < hd; ++d) out[d] += w * (load_elem(p->v, p->kv_dtype, off + d) * p->v_scale);
    }
    for (int d = 0; d < hd; ++d) out[d] /= z;
    *lse = m + log(z);
}

static int64_t max_len(const or_problem* p) {
    int64_t mx = 1;
    for (int r = 0; r < p->B; ++r) {
        int64_t L = p->block_table ? p->seq_lens[r] : (p->qsl[r + 1] - p->qsl[r]);
        if (L > mx) mx = L;
    }
    return mx;
}

/* rows: packed token indices to evaluate (NULL => all T tokens, n_rows = T).
 * out: [n_rows, H, hd]; lse: [H, n_rows]. nthreads <= 0 => OpenMP default. */
/* Attention variants, the plainest reading of the deep-dive page's table of
 * supported variants (it names them but gives no formulas):
 *  window_left >= 0: sliding window -- query position i (= ctx + t) sees keys
 *                    j >= i - window_left only (on top of the causal bound);
 *  softcap > 0:      logits soft cap -- each scaled score s becomes
 *                    softcap * tanh(s / softcap) before the softmax;
 *  sinks != NULL:    attention sinks -- one extra logit sinks[h] per head
 *                    joins the softmax normaliser and contributes no value:
 *                    out = sum_j e^{s_j} v_j / (e^{sink} + sum_j e^{s_j}),
 *                    lse = log(e^{sink} + sum_j e^{s_j}); a row with no
 *                    visible key then has out = 0 and lse = sink;
 *  alibi != NULL:    ALiBi -- the score of query position i and key j
 *                    (after the cap) gets -alibi[h] * |i - j| added. */
int or_attention_ex(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                    double k_scale, double v_scale, const int32_t* qsl, const int32_t* seq_lens,
                    const int32_t* block_table, int64_t bt_stride, int B, int H, int Hkv, int hd, int bs,
                    double scale, int causal, int64_t window_left, double softcap, const double* sinks,
                    const double* alibi, const int64_t* rows, int64_t n_rows, double* out, double* lse,
                    int nthreads) {
    if (H % Hkv != 0 || B <= 0) return -1;
    or_problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, qsl, seq_lens, block_table,
                    bt_stride, B, H, Hkv, hd, bs, scale, causal, window_left, softcap, sinks, alibi};
    int64_t L = max_len(&p);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int64_t total = n_rows * H;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * L);
        double* qv = (double*)malloc(sizeof(double) * hd);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < total; ++i) {
            int64_t ri = i / H;
            int h = (int)(i % H);
            int64_t tok = rows ? rows[ri] : ri;
            double l;
            attend_one(&p, tok, h, s, qv, out + (ri * H + h) * hd, &l);
            lse[(int64_t)h * n_rows + ri] = l;
        }
        free(s);
        free(qv);
    }
    return 0;
}

/* The plain definition (no variant). */
int or_attention(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                 double k_scale, double v_scale, const int32_t* qsl, const int32_t* seq_lens,
                 const int32_t* block_table, int64_t bt_stride, int B, int H, int Hkv, int hd, int bs,
                 double scale, int causal, const int64_t* rows, int64_t n_rows,
                 double* out, double* lse, int nthreads) {
    return or_attention_ex(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, qsl, seq_lens, block_table, bt_stride,
                           B, H, Hkv, hd, bs, scale, causal, -1, 0.0, NULL, NULL, rows, n_rows, out, lse,
                           nthreads);
}

/* Number of threads OpenMP would use (for reporting). */
int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------- procedural forms (pins) */

/* Online softmax in the unnormalised form, tile by tile over the visible keys
 * (multiple-requests page, §7): running max m, running sum l, accumulator acc;
 * per tile: m_new = max(m, rowmax), alpha = exp(m - m_new), p = exp(s - m_new),
 * l = alpha l + sum p, acc = alpha acc + p V; finally out = acc / l. */
int or_attention_online(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                        double k_scale, double v_scale, const int32_t* qsl, const int32_t* seq_lens,
                        const int32_t* block_table, int64_t bt_stride, int B, int H, int Hkv, int hd, int bs,
                        double scale, int causal, int tile, double* out, double* lse) {
    or_problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, qsl, seq_lens, block_table,
                    bt_stride, B, H, Hkv, hd, bs, scale, causal, -1, 0.0, NULL};
    int64_t T = qsl[B];
    double* qv = (double*)malloc(sizeof(double) * hd);
    double* sc = (double*)malloc(sizeof(double) * tile);
    for (int64_t tok = 0; tok < T; ++tok) {
        int r = request_of(&p, tok);
        int64_t t = tok - qsl[r];
        int64_t n = visible(&p, r, t);
        for (int h = 0; h < H; ++h) {
            int g = h / (H / Hkv);
            double* acc = out + (tok * H + h) * hd;
            for (int d = 0; d < hd; ++d) qv[d] = load_elem(q, q_dtype, (tok * H + h) * hd + d);
            for (int d = 0; d < hd; ++d) acc[d] = 0.0;
            double m = -INFINITY, l = 0.0;
            for (int64_t j0 = 0; j0 < n; j0 += tile) {
                int64_t j1 = j0 + tile < n ? j0 + tile : n;
                double rowmax = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    int64_t off = kv_offset(&p, r, j, g);
                    double dot = 0.0;
                    for (int d = 0; d < hd; ++d) dot += qv[d] * load_elem(k, kv_dtype, off + d) * k_scale;
                    sc[j - j0] = scale * dot;
                    if (sc[j - j0] > rowmax) rowmax = sc[j - j0];
                }
                double m_new = m > rowmax ? m : rowmax;
                double alpha = exp(m - m_new);
                double psum = 0.0;
                for (int d = 0; d < hd; ++d) acc[d] *= alpha;
                for (int64_t j = j0; j < j1; ++j) {
                    double pj = exp(sc[j - j0] - m_new);
                    psum += pj;
                    int64_t off = kv_offset(&p, r, j, g);
                    for (int d = 0; d < hd; ++d) acc[d] += pj * load_elem(v, kv_dtype, off + d) * v_scale;
                }
                l = alpha * l + psum;
                m = m_new;
            }
            if (n == 0) { lse[(int64_t)h * T + tok] = -INFINITY; continue; }
            for (int d = 0; d < hd; ++d) acc[d] /= l;
            lse[(int64_t)h * T + tok] = m + log(l);
        }
    }
    free(qv);
    free(sc);
    return 0;
}

/* Online softmax in the normalised form (deep-dive page, memory-I/O section):
 * the output is kept divided by the running sum; per tile
 * o = exp(m - m_new) * o * (l / l_new) + (exp(s - m_new) V) / l_new. */
int or_attention_online_normalised(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                                   double k_scale, double v_scale, const int32_t* qsl, const int32_t* seq_lens,
                                   const int32_t* block_table, int64_t bt_stride, int B, int H, int Hkv, int hd,
                                   int bs, double scale, int causal, int tile, double* out, double* lse) {
    or_problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, qsl, seq_lens, block_table,
                    bt_stride, B, H, Hkv, hd, bs, scale, causal, -1, 0.0, NULL};
    int64_t T = qsl[B];
    double* qv = (double*)malloc(sizeof(double) * hd);
    double* sc = (double*)malloc(sizeof(double) * tile);
    double* pv = (double*)malloc(sizeof(double) * hd);
    for (int64_t tok = 0; tok < T; ++tok) {
        int r = request_of(&p, tok);
        int64_t t = tok - qsl[r];
        int64_t n = visible(&p, r, t);
        for (int h = 0; h < H; ++h) {
            int g = h / (H / Hkv);
            double* o = out + (tok * H + h) * hd;
            for (int d = 0; d < hd; ++d) qv[d] = load_elem(q, q_dtype, (tok * H + h) * hd + d);
            for (int d = 0; d < hd; ++d) o[d] = 0.0;
            double m = -INFINITY, l = 0.0;
            for (int64_t j0 = 0; j0 < n; j0 += tile) {
                int64_t j1 = j0 + tile < n ? j0 + tile : n;
                double tmax = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    int64_t off = kv_offset(&p, r, j, g);
                    double dot = 0.0;
                    for (int d = 0; d < hd; ++d) dot += qv[d] * load_elem(k, kv_dtype, off + d) * k_scale;
                    sc[j - j0] = scale * dot;
                    if (sc[j - j0] > tmax) tmax = sc[j - j0];
                }
                double m_new = m > tmax ? m : tmax;
                double esum = 0.0;
                for (int d = 0; d < hd; ++d) pv[d] = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    double e = exp(sc[j - j0] - m_new);
                    esum += e;
                    int64_t off = kv_offset(&p, r, j, g);
                    for (int d = 0; d < hd; ++d) pv[d] += e * load_elem(v, kv_dtype, off + d) * v_scale;
                }
                double l_new = exp(m - m_new) * l + esum;
                for (int d = 0; d < hd; ++d) o[d] = exp(m - m_new) * o[d] * (l / l_new) + pv[d] / l_new;
                m = m_new;
                l = l_new;
            }
            lse[(int64_t)h * T + tok] = n ? m + log(l) : -INFINITY;
        }
    }
    free(qv);
    free(sc);
    free(pv);
    return 0;
}

/* Split-KV as segments (multiple-requests page, §12): the visible keys of each
 * (token, head) are cut into segments of seg_len keys; each segment yields its
 * local max m_s, local exponent sum l_s and unnormalised weighted output O_s;
 * a reduction then forms m = max m_s, l = sum exp(m_s - m) l_s,
 * O = sum exp(m_s - m) O_s / l. Segments with no key are skipped. */
int or_attention_split(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                       double k_scale, double v_scale, const int32_t* qsl, const int32_t* seq_lens,
                       const int32_t* block_table, int64_t bt_stride, int B, int H, int Hkv, int hd, int bs,
                       double scale, int causal, int64_t seg_len, double* out, double* lse) {
    or_problem p = {q, q_dtype, k, v, kv_dtype, k_scale, v_scale, qsl, seq_lens, block_table,
                    bt_stride, B, H, Hkv, hd, bs, scale, causal, -1, 0.0, NULL};
    int64_t T = qsl[B];
    int64_t L = max_len(&p);
    int64_t S = (L + seg_len - 1) / seg_len;
    double* qv = (double*)malloc(sizeof(double) * hd);
    double* ms = (double*)malloc(sizeof(double) * S);
    double* ls = (double*)malloc(sizeof(double) * S);
    double* Os = (double*)malloc(sizeof(double) * S * hd);
    for (int64_t tok = 0; tok < T; ++tok) {
        int r = request_of(&p, tok);
        int64_t t = tok - qsl[r];
        int64_t n = visible(&p, r, t);
        for (int h = 0; h < H; ++h) {
            int g = h / (H / Hkv);
            for (int d = 0; d < hd; ++d) qv[d] = load_elem(q, q_dtype, (tok * H + h) * hd + d);
            int64_t nseg = 0;
            for (int64_t j0 = 0; j0 < n; j0 += seg_len, ++nseg) {
                int64_t j1 = j0 + seg_len < n ? j0 + seg_len : n;
                double m_s = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    int64_t off = kv_offset(&p, r, j, g);
                    double dot = 0.0;
                    for (int d = 0; d < hd; ++d) dot += qv[d] * load_elem(k, kv_dtype, off + d) * k_scale;
                    double s = scale * dot;
                    if (s > m_s) m_s = s;
                }
                double l_s = 0.0;
                double* O = Os + nseg * hd;
                for (int d = 0; d < hd; ++d) O[d] = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    int64_t off = kv_offset(&p, r, j, g);
                    double dot = 0.0;
                    for (int d = 0; d < hd; ++d) dot += qv[d] * load_elem(k, kv_dtype, off + d) * k_scale;
                    double e = exp(scale * dot - m_s);
                    l_s += e;
                    for (int d = 0; d < hd; ++d) O[d] += e * load_elem(v, kv_dtype, off + d) * v_scale;
                }
                ms[nseg] = m_s;
                ls[nseg] = l_s;
            }
            double* o = out + (tok * H + h) * hd;
            if (nseg == 0) {
                for (int d = 0; d < hd; ++d) o[d] = 0.0;
                lse[(int64_t)h * T + tok] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t s = 0; s < nseg; ++s) if (ms[s] > m) m = ms[s];
            double l = 0.0;
            for (int64_t s = 0; s < nseg; ++s) l += exp(ms[s] - m) * ls[s];
            for (int d = 0; d < hd; ++d) {
                double acc = 0.0;
                for (int64_t s = 0; s < nseg; ++s) acc += exp(ms[s] - m) * Os[s * hd + d];
                o[d] = acc / l;
            }
            lse[(int64_t)h * T + tok] = m + log(l);
        }
    }
    free(qv); free(ms); free(ls); free(Os);
    return 0;
}

/* Merge two attention states of the same queries (cascade section of the
 * deep-dive page): lse = log(exp(lse1) + exp(lse2)),
 * out = exp(lse1 - lse) o1 + exp(lse2 - lse) o2. A state with lse = -inf
 * has weight 0; two such states give out = 0, lse = -inf.
 * o*: [T, H, hd]; lse*: [H, T]. */
void or_merge(const double* o1, const double* lse1, const double* o2, const double* lse2,
              int64_t T, int H, int hd, double* out, double* lse) {
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double a = lse1[(int64_t)h * T + t], b = lse2[(int64_t)h * T + t];
            double* o = out + (t * H + h) * hd;
            const double* x = o1 + (t * H + h) * hd;
            const double* y = o2 + (t * H + h) * hd;
            if (a == -INFINITY && b == -INFINITY) {
                for (int d = 0; d < hd; ++d) o[d] = 0.0;
                lse[(int64_t)h * T + t] = -INFINITY;
                continue;
            }
            double mx = a > b ? a : b;
            double l = mx + log(exp(a - mx) + exp(b - mx));
            double wa = exp(a - l), wb = exp(b - l);
            for (int d = 0; d < hd; ++d) o[d] = wa * x[d] + wb * y[d];
            lse[(int64_t)h * T + t] = l;
        }
    }
}

/* Encode n binary32 values: out[i] = or_encode_e4m3fn(fl32(x[i] / scale)).
 * Used to check an encoder exhaustively over all 2^32 inputs. */
void or_encode_e4m3fn_array(const float* x, int64_t n, float scale, uint8_t* out) {
    e4m3_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        volatile float y = x[i] / scale;
        out[i] = or_encode_e4m3fn(y);
    }
}
