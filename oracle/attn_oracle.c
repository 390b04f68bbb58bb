/*
 * Scaled-dot-product attention oracle: plain, slow, fp64, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library. The GPU product path
 * never calls it, and the two share no code, header or constant.
 *
 * Pages followed (cited by title and section):
 *   [Ch2]  "2. 自注意力机制算子：QKV投影、注意力分数计算、Softmax、加权求和，
 *          以及FlashAttention优化"
 *            §2.2  scores S = Q K^T / sqrt(D_k), one score per (query, key) pair
 *            §2.3  softmax along the key axis in three steps: the row maximum,
 *                  the sum of exponentials of the max-shifted scores, then the
 *                  division of each shifted exponential by that sum
 *            §2.4  weighted sum O = A V
 *            §2.6  the online (m, d) update and the rescale of earlier partial
 *                  results by exp(m_old - m)   (test aids below only)
 *   [OSM]  "[Performance] [WebGPU] Proposal: Add an option to use online
 *          softmax instead of naive softmax"
 *            §四   per-element running-max / running-sum recurrence (test aid)
 *   [Blog] "WebGPU 算子优化：QKV 内存合并与 FlashAttention 分块计算"
 *            section "FlashAttention 分块计算原理与浏览器适配": merging the
 *            (m, l) statistics of separate key blocks (test aid)
 *            section "QKV 矩阵的内存合并模式选择": Q, K, V of all heads, each
 *            in its own buffer of B x S x heads x d elements, heads outermost
 *            ("Contiguous"), interleaved per token ("Interleaved") or in
 *            groups of heads stored together ("Split")
 *   [OSM]  §三-§四 softmax of a row of scores on its own (three passes,
 *                or the one-pass online recurrence)
 *   [Ch2]  §2.1  the Q, K, V projections X W_Q, X W_K, X W_V, computed as one
 *                product with the three weight matrices side by side and
 *                then split
 *
 * The oracle is the plain definition, not the tiled method: for every query
 * row it materialises the whole score row over the valid keys, then runs the
 * three softmax steps, then the weighted sum. Readings where the pages are
 * silent (all stated again in the design notes):
 *   - masks: a key j is valid for query i of sequence b iff j < n_b and, when
 *     causal, j <= i ("key j > query i masked"); n_b = kv_len[b] clamped to
 *     [0, Sk], or Sk when no lengths are given. Masked keys are left out of
 *     the max, the sum and the weighted sum.
 *   - a row with no valid key gives O = 0 and LSE = -inf.
 *   - LSE = m + ln(sum), natural log of the scaled scores.
 *   - inputs are decoded exactly from their storage type (fp32, fp16, bf16).
 *
 * Build: gcc -O2 -fopenmp -fno-fast-math -ffp-contract=off -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* storage types, oracle-side codes (the Python wrapper maps names to these) */
#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* layouts, oracle-side codes */
#define ORC_BHSD 0 /* [B, H, S, d]: all rows of one head contiguous      */
#define ORC_BSHD 1 /* [B, S, H, d]: heads interleaved within each token  */
#define ORC_SPLIT 0x10000 /* | g: [B, H/g, S, g, d], groups of g heads    */

/* ---- exact decoding of one stored element to double -------------------- */

static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0) {
        mag = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        mag = f ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(f + 1024), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

static double decode_bf16(uint16_t h) {
    /* bf16 is the top half of an IEEE binary32 */
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double load(const void* base, int64_t idx, int dtype) {
    switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_F16: return decode_f16(((const uint16_t*)base)[idx]);
    default:      return decode_bf16(((const uint16_t*)base)[idx]);
    }
}

double oracle_decode(const void* base, int64_t idx, int dtype) {
    return load(base, idx, dtype);
}

/* element index of (b, h, s, c) in a tensor with S rows per head */
static int64_t at(int layout, int64_t H, int64_t S, int64_t d,
                  int64_t b, int64_t h, int64_t s, int64_t c) {
    if (layout == ORC_BHSD) return ((b * H + h) * S + s) * d + c;
    if (layout == ORC_BSHD) return ((b * S + s) * H + h) * d + c;
    /* [Blog] "Split": heads in groups of g, [B, H/g, S, g, d] */
    const int64_t g = layout & 0xffff;
    return (((b * (H / g) + h / g) * S + s) * g + h % g) * d + c;
}

/* a layout code the oracle knows: BHSD, BSHD, or ORC_SPLIT | g with g | H */
static int layout_valid(int layout, int64_t H) {
    if (layout == ORC_BHSD || layout == ORC_BSHD) return 1;
    if ((layout & ~0xffff) != ORC_SPLIT) return 0;
    const int64_t g = layout & 0xffff;
    return g >= 1 && H % g == 0;
}

typedef struct {
    const void *q, *k, *v;
    int dtype, layout;
    int64_t B, H, Sq, Sk, d;
    double scale;
    int causal;
    const int32_t* kv_len;
} problem;

static int64_t keys_of_batch(const problem* p, int64_t b) {
    if (!p->kv_len) return p->Sk;
    int64_t n = p->kv_len[b];
    if (n < 0) n = 0;
    if (n > p->Sk) n = p->Sk;
    return n;
}

static int key_valid(const problem* p, int64_t nb, int64_t i, int64_t j) {
    if (j >= nb) return 0;                 /* key padding */
    if (p->causal && j > i) return 0;      /* key j > query i is masked */
    return 1;
}

/* score of (query i, key j): [Ch2] §2.2, dot product then the scale */
static double score(const problem* p, int64_t b, int64_t h, int64_t i, int64_t j) {
    double acc = 0.0;
    for (int64_t c = 0; c < p->d; ++c) {
        double qc = load(p->q, at(p->layout, p->H, p->Sq, p->d, b, h, i, c), p->dtype);
        double kc = load(p->k, at(p->layout, p->H, p->Sk, p->d, b, h, j, c), p->dtype);
        acc += qc * kc;
    }
    return p->scale * acc;
}

/*
 * One query row, by definition. `s` and `a` are scratch rows of Sk doubles.
 * Writes d outputs to o and the log-sum-exp to *lse.
 */
static void attn_row(const problem* p, int64_t row, double* s, double* a,
                     double* o, double* lse) {
    int64_t i = row % p->Sq;
    int64_t h = (row / p->Sq) % p->H;
    int64_t b = row / (p->Sq * p->H);
    int64_t nb = keys_of_batch(p, b);

    /* materialise the score row over the valid keys */
    int64_t nvalid = 0;
    for (int64_t j = 0; j < p->Sk; ++j)
        if (key_valid(p, nb, i, j)) { s[j] = score(p, b, h, i, j); ++nvalid; }

    if (nvalid == 0) {
        for (int64_t c = 0; c < p->d; ++c) o[c] = 0.0;
        *lse = -INFINITY;
        return;
    }

    /* softmax step 1 ([Ch2] §2.3): m = max over the row */
    double m = -INFINITY;
    for (int64_t j = 0; j < p->Sk; ++j)
        if (key_valid(p, nb, i, j) && s[j] > m) m = s[j];

    /* softmax step 2: l = sum of exp(s - m) */
    double l = 0.0;
    for (int64_t j = 0; j < p->Sk; ++j)
        if (key_valid(p, nb, i, j)) { a[j] = exp(s[j] - m); l += a[j]; }

    /* softmax step 3: normalise */
    for (int64_t j = 0; j < p->Sk; ++j)
        if (key_valid(p, nb, i, j)) a[j] = a[j] / l;

    /* weighted sum ([Ch2] §2.4): O_i = sum_j A_ij V_j */
    for (int64_t c = 0; c < p->d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < p->Sk; ++j)
            if (key_valid(p, nb, i, j))
                acc += a[j] * load(p->v, at(p->layout, p->H, p->Sk, p->d, b, h, j, c), p->dtype);
        o[c] = acc;
    }
    *lse = m + log(l);
}

static int check(const problem* p) {
    if (!p->q || !p->k || !p->v) return 1;
    if (p->B < 1 || p->H < 1 || p->Sq < 1 || p->Sk < 1 || p->d < 1) return 2;
    if (p->dtype < ORC_F32 || p->dtype > ORC_BF16) return 3;
    if (!layout_valid(p->layout, p->H)) return 3;
    return 0;
}

/*
 * Rows given by linear index row = (b * H + h) * Sq + i. o_rows is
 * [n_rows, d], lse_rows is [n_rows]. Returns 0, or a nonzero code on bad
 * arguments (nothing written) or on allocation failure.
 */
int oracle_attn_rows(const void* q, const void* k, const void* v, int dtype, int layout,
                     int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t d,
                     double scale, int causal, const int32_t* kv_len,
                     const int64_t* rows, int64_t n_rows,
                     double* o_rows, double* lse_rows, int nthreads) {
    problem p = {q, k, v, dtype, layout, B, H, Sq, Sk, d, scale, causal, kv_len};
    int rc = check(&p);
    if (rc) return rc;
    if (!rows || !o_rows || !lse_rows) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * H * Sq) return 2;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
        double* a = (double*)malloc(sizeof(double) * (size_t)Sk);
        if (!s || !a) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; ++r)
                attn_row(&p, rows[r], s, a, o_rows + r * d, lse_rows + r);
        }
        free(s);
        free(a);
    }
    return failed ? 5 : 0;
}

/*
 * Every row. o is written in the layout of q (fp64), lse as [B, H, Sq].
 */
int oracle_attn(const void* q, const void* k, const void* v, int dtype, int layout,
                int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t d,
                double scale, int causal, const int32_t* kv_len,
                double* o, double* lse, int nthreads) {
    problem p = {q, k, v, dtype, layout, B, H, Sq, Sk, d, scale, causal, kv_len};
    int rc = check(&p);
    if (rc) return rc;
    if (!o || !lse) return 1;
    int failed = 0;
    int64_t n_rows = B * H * Sq;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
        double* a = (double*)malloc(sizeof(double) * (size_t)Sk);
        double* orow = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s || !a || !orow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t i = r % Sq, h = (r / Sq) % H, b = r / (Sq * H);
                attn_row(&p, r, s, a, orow, lse + r);
                for (int64_t c = 0; c < d; ++c) o[at(layout, H, Sq, d, b, h, i, c)] = orow[c];
            }
        }
        free(s);
        free(a);
        free(orow);
    }
    return failed ? 5 : 0;
}

/*
 * Test aid: the per-element online recurrence of [OSM] §四, read with its
 * lost operators restored: m = max(m_prev, s); d = d_prev*exp(m_prev - m) +
 * exp(s - m). Traces of m and d after each element go to m_trace, l_trace;
 * p gets exp(s_j - m_final) / d_final.
 */
void oracle_online_softmax(const double* s, int64_t n, double* m_trace, double* l_trace,
                           double* p) {
    double m_prev = -INFINITY, d_prev = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double m = s[j] > m_prev ? s[j] : m_prev;
        double carry = (d_prev == 0.0) ? 0.0 : d_prev * exp(m_prev - m);
        double d = carry + exp(s[j] - m);
        m_trace[j] = m;
        l_trace[j] = d;
        m_prev = m;
        d_prev = d;
    }
    for (int64_t j = 0; j < n; ++j) p[j] = exp(s[j] - m_prev) / d_prev;
}

/*
 * Test aid for the split-over-keys form: the unnormalised partial of one
 * query row over keys [j0, j1) (intersected with the valid set):
 * m = max score, l = sum exp(s - m), o = sum exp(s - m) V_j.
 * An empty range gives m = -inf, l = 0, o = 0.
 */
int oracle_partial(const void* q, const void* k, const void* v, int dtype, int layout,
                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t d,
                   double scale, int causal, const int32_t* kv_len,
                   int64_t row, int64_t j0, int64_t j1,
                   double* m_out, double* l_out, double* o_out) {
    problem p = {q, k, v, dtype, layout, B, H, Sq, Sk, d, scale, causal, kv_len};
    int rc = check(&p);
    if (rc) return rc;
    if (row < 0 || row >= B * H * Sq) return 2;
    int64_t i = row % Sq, h = (row / Sq) % H, b = row / (Sq * H);
    int64_t nb = keys_of_batch(&p, b);
    if (j0 < 0) j0 = 0;
    if (j1 > Sk) j1 = Sk;
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j)
        if (key_valid(&p, nb, i, j)) {
            double sj = score(&p, b, h, i, j);
            if (sj > m) m = sj;
        }
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c) o_out[c] = 0.0;
    if (m != -INFINITY) {
        for (int64_t j = j0; j < j1; ++j)
            if (key_valid(&p, nb, i, j)) {
                double e = exp(score(&p, b, h, i, j) - m);
                l += e;
                for (int64_t c = 0; c < d; ++c)
                    o_out[c] += e * load(v, at(layout, H, Sk, d, b, h, j, c), dtype);
            }
    }
    *m_out = m;
    *l_out = l;
    return 0;
}

/*
 * Test aid: merge n partials (m_s, l_s, o_s) of one row, the block-merge
 * rule of [Blog] "FlashAttention 分块计算原理与浏览器适配" and [Ch2] §2.6:
 * m = max_s m_s; each partial is weighted by exp(m_s - m) (0 if empty);
 * O = sum w_s o_s / sum w_s l_s; LSE = m + ln(sum w_s l_s).
 */
void oracle_merge(int64_t n, const double* m, const double* l, const double* o, int64_t d,
                  double* o_out, double* lse_out) {
    double mx = -INFINITY;
    for (int64_t s = 0; s < n; ++s) if (m[s] > mx) mx = m[s];
    for (int64_t c = 0; c < d; ++c) o_out[c] = 0.0;
    if (mx == -INFINITY) { *lse_out = -INFINITY; return; }
    double lt = 0.0;
    for (int64_t s = 0; s < n; ++s) {
        if (m[s] == -INFINITY) continue;
        double w = exp(m[s] - mx);
        lt += w * l[s];
        for (int64_t c = 0; c < d; ++c) o_out[c] += w * o[s * d + c];
    }
    for (int64_t c = 0; c < d; ++c) o_out[c] /= lt;
    *lse_out = mx + log(lt);
}

/*
 * QKV projection, [Ch2] §2.1 by definition: for t = 0, 1, 2 (Q, K, V),
 *   out_t[b, h, s, c] = sum_i x[b, s, i] * W[i, t*H*d + h*d + c]
 * where W = [W_Q | W_K | W_V] is the D x 3Hd concatenated weight. The weight
 * is passed out-major, w[n * D + i] = W[i, n] (n = t*H*d + h*d + c), the
 * usual storage of a linear layer's weight. x is [B, S, D] row-major; the
 * three outputs are written in `layout` ([B,H,S,d] or [B,S,H,d]) as fp64.
 * Returns 0, or 1 on bad sizes.
 */
int oracle_qkv_proj(const void* x, const void* w, int dtype, int layout, int64_t B, int64_t S,
                    int64_t D, int64_t H, int64_t d, double* q, double* k, double* v,
                    int nthreads) {
    if (B < 0 || S < 0 || D < 1 || H < 1 || d < 1) return 1;
    if (!layout_valid(layout, H)) return 1;
    double* outs[3] = {q, k, v};
    const int64_t HD = H * d;
    (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bs = 0; bs < B * S; ++bs) {
        const int64_t b = bs / S, s_ = bs % S;
        for (int t = 0; t < 3; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t c = 0; c < d; ++c) {
                    const int64_t n = t * HD + h * d + c;
                    double acc = 0.0;
                    for (int64_t i = 0; i < D; ++i)
                        acc += load(x, bs * D + i, dtype) * load(w, n * D + i, dtype);
                    outs[t][at(layout, H, S, d, b, h, s_, c)] = acc;
                }
    }
    return 0;
}

/*
 * Row softmax by definition ([Ch2] §2.3 three steps, the computation [OSM]
 * §三-§四 discusses on its own): for each row r of x [rows, n],
 *   y[r, j] = exp(scale*x[r, j] - m_r) / l_r,  m_r = max_j scale*x[r, j],
 *   l_r = sum_j exp(scale*x[r, j] - m_r),      lse[r] = m_r + ln l_r.
 * Entries equal to -inf take no part (probability 0); a row with no finite
 * entry gives y = 0 and lse = -inf. Outputs fp64. Returns 0, or 1 on bad
 * sizes.
 */
int oracle_softmax_rows(const void* x, int dtype, int64_t rows, int64_t n, double scale,
                        double* y, double* lse, int nthreads) {
    if (rows < 0 || n < 1) return 1;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {                 /* step 1: the maximum */
            const double v = load(x, r * n + j, dtype);
            if (v == -INFINITY) continue;
            if (scale * v > m) m = scale * v;
        }
        double* yr = y + r * n;
        if (m == -INFINITY) {
            for (int64_t j = 0; j < n; ++j) yr[j] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int64_t j = 0; j < n; ++j) {                 /* step 2: the sum */
            const double v = load(x, r * n + j, dtype);
            yr[j] = v == -INFINITY ? 0.0 : exp(scale * v - m);
            l += yr[j];
        }
        for (int64_t j = 0; j < n; ++j) yr[j] = yr[j] / l;   /* step 3: divide */
        lse[r] = m + log(l);
    }
    return 0;
}
