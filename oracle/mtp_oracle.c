/*
 * mtp_oracle.c -- scalar C99 reference of the quantized MTP draft-layer
 * forward.  TEST INFRASTRUCTURE ONLY (see mtp_oracle.h): only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may call it.
 *
 * Page titles used in the citations below:
 *   [mtp.rs]    hf2q 0.1.13, src/inference/models/qwen35/mtp.rs
 *   [mimo.rs]   cortiq-engine 0.8.49, src/mimo_mtp.rs
 *   [shared.rs] hf2q 0.1.1, src/serve/forward_mlx_shared.rs
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared (no -ffast-math: the ascending-order
 * double sums and the single-rounding fmaf below must stay as written).
 */
#include "mtp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 32

static void* xmalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) abort();
    return p;
}

/* ------------------------------------------------------------------------ */
/* Weight formats                                                            */
/* ------------------------------------------------------------------------ */

/* Code of element (row, col) of a 4-bit packed matrix.  [shared.rs]
 * `MlxQWeight::from_mlx_affine_linear` packs eight codes per u32 with code j
 * of the word at bit offset 4*j, so element col sits in word col/8 at nibble
 * col%8. */
static unsigned code4(const uint32_t* codes, int32_t k, int32_t row, int32_t col) {
    uint32_t word = codes[(size_t)row * (size_t)(k / 8) + (size_t)(col / 8)];
    return (unsigned)((word >> (4 * (col % 8))) & 0xFu);
}

void orc_unpack4(const uint32_t* codes, int32_t n, int32_t k, uint8_t* out) {
    for (int32_t r = 0; r < n; ++r)
        for (int32_t c = 0; c < k; ++c) out[(size_t)r * k + c] = (uint8_t)code4(codes, k, r, c);
}

/* f32 dequantized 4-bit weight: scale*code + bias for the element's group of
 * 32 ([shared.rs] `MlxAffineExtra`: per-group scales and biases [N, K/32]).
 * The exact value is rounded once to f32 (fmaf is correctly rounded). */
void orc_deq4(const orc_q4* w, float* out) {
    const int32_t gpr = w->k / GROUP;
    for (int32_t r = 0; r < w->n; ++r)
        for (int32_t c = 0; c < w->k; ++c) {
            size_t gi = (size_t)r * gpr + (size_t)(c / GROUP);
            out[(size_t)r * w->k + c] =
                fmaf(w->scales[gi], (float)code4(w->codes, w->k, r, c), w->biases[gi]);
        }
}

/* f32 dequantized 8-bit block weight: scale * code, one rounding. */
void orc_deq8(const orc_q8* w, float* out) {
    const int32_t gpr = w->k / GROUP;
    for (int32_t r = 0; r < w->n; ++r)
        for (int32_t c = 0; c < w->k; ++c) {
            size_t i = (size_t)r * w->k + c;
            out[i] = w->scales[(size_t)r * gpr + (size_t)(c / GROUP)] * (float)w->codes[i];
        }
}

/* The f32 a bf16 value stands for: its 16 bits are the upper half of that
 * f32's bits, the lower half zero (so the widening is exact). */
float orc_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* f32 dequantized 4-bit weight with bf16 group constants ([shared.rs]
 * `MlxAffineMoeStack`): scale*code + bias with scale and bias widened to f32,
 * the exact value rounded once (fmaf), as orc_deq4. */
void orc_deq4e(const orc_q4e* w, float* out) {
    const int32_t gpr = w->k / GROUP;
    for (int32_t r = 0; r < w->n; ++r)
        for (int32_t c = 0; c < w->k; ++c) {
            size_t gi = (size_t)r * gpr + (size_t)(c / GROUP);
            out[(size_t)r * w->k + c] =
                fmaf(orc_bf16(w->scales[gi]), (float)code4(w->codes, w->k, r, c), orc_bf16(w->biases[gi]));
        }
}

/* ------------------------------------------------------------------------ */
/* Primitives                                                                */
/* ------------------------------------------------------------------------ */

/* y[r][n] = sum_k x[r][k] * (q[n][k]*s + b), the weight kept exact in double
 * as in the CPU check of [shared.rs] test module
 * `ac5_iter_b_affine_qweight_roundtrip`; the weight is stored out x in, so
 * this is x times W transposed. */
void orc_gemv4(const orc_q4* w, const float* x, int32_t m, float* y) {
    const int32_t n = w->n, k = w->k, gpr = k / GROUP;
    /* output rows are independent: a build with OpenMP shares them out over
     * threads, each element keeping its own ascending sum (same bits) */
#pragma omp parallel
    {
        double* row = (double*)xmalloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int32_t o = 0; o < n; ++o) {
            for (int32_t c = 0; c < k; ++c) {
                size_t gi = (size_t)o * gpr + (size_t)(c / GROUP);
                row[c] = (double)w->scales[gi] * (double)code4(w->codes, k, o, c) + (double)w->biases[gi];
            }
            for (int32_t r = 0; r < m; ++r) {
                const float* xr = x + (size_t)r * k;
                double acc = 0.0;
                for (int32_t c = 0; c < k; ++c) acc += (double)xr[c] * row[c];
                y[(size_t)r * n + o] = (float)acc;
            }
        }
        free(row);
    }
}

void orc_gemv8(const orc_q8* w, const float* x, int32_t m, float* y) {
    const int32_t n = w->n, k = w->k, gpr = k / GROUP;
#pragma omp parallel
    {
        double* row = (double*)xmalloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int32_t o = 0; o < n; ++o) {
            for (int32_t c = 0; c < k; ++c)
                row[c] = (double)w->scales[(size_t)o * gpr + (size_t)(c / GROUP)] *
                         (double)w->codes[(size_t)o * k + c];
            for (int32_t r = 0; r < m; ++r) {
                const float* xr = x + (size_t)r * k;
                double acc = 0.0;
                for (int32_t c = 0; c < k; ++c) acc += (double)xr[c] * row[c];
                y[(size_t)r * n + o] = (float)acc;
            }
        }
        free(row);
    }
}

/* The 4-bit GEMV of orc_gemv4 over bf16 group constants: the weight
 * scale*code + bias exact in double with scale and bias widened. */
void orc_gemv4e(const orc_q4e* w, const float* x, int32_t m, float* y) {
    const int32_t n = w->n, k = w->k, gpr = k / GROUP;
#pragma omp parallel
    {
        double* row = (double*)xmalloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int32_t o = 0; o < n; ++o) {
            for (int32_t c = 0; c < k; ++c) {
                size_t gi = (size_t)o * gpr + (size_t)(c / GROUP);
                row[c] = (double)orc_bf16(w->scales[gi]) * (double)code4(w->codes, k, o, c) +
                         (double)orc_bf16(w->biases[gi]);
            }
            for (int32_t r = 0; r < m; ++r) {
                const float* xr = x + (size_t)r * k;
                double acc = 0.0;
                for (int32_t c = 0; c < k; ++c) acc += (double)xr[c] * row[c];
                y[(size_t)r * n + o] = (float)acc;
            }
        }
        free(row);
    }
}

/* Dense f32 projection (the MoE router). */
void orc_gemv_f32(const float* w, int32_t n, int32_t k, const float* x, int32_t m, float* y) {
    for (int32_t r = 0; r < m; ++r)
#pragma omp parallel for schedule(static)
        for (int32_t o = 0; o < n; ++o) {
            double acc = 0.0;
            for (int32_t c = 0; c < k; ++c)
                acc += (double)x[(size_t)r * k + c] * (double)w[(size_t)o * k + c];
            y[(size_t)r * n + o] = (float)acc;
        }
}

/* RMSNorm with a stored weight: y = x / sqrt(mean(x^2) + eps) * gamma
 * ([mtp.rs] `rms_norm_with_weight`, parameters [eps, hidden]). */
void orc_rmsnorm(const float* x, const float* gamma, int32_t m, int32_t h, float eps, float* y) {
    for (int32_t r = 0; r < m; ++r) {
        const float* xr = x + (size_t)r * h;
        double ss = 0.0;
        for (int32_t i = 0; i < h; ++i) ss += (double)xr[i] * (double)xr[i];
        double inv = 1.0 / sqrt(ss / (double)h + (double)eps);
        for (int32_t i = 0; i < h; ++i)
            y[(size_t)r * h + i] = (float)((double)xr[i] * inv * (double)gamma[i]);
    }
}

/* Rotary embedding of the first rotary_dim dims of every head with
 * half-split pairs (i, i + rotary_dim/2) and inverse frequency
 * theta^(-2i/rotary_dim); the dims from rotary_dim on pass unchanged; row r
 * sits at position pos0 + r.  [mtp.rs] `forward_full_attention` applies it
 * (`apply_imrope`, with `rotary_dim`) to q and k after the projections; with
 * text-only positions all rope sections share one id, so the sections do not
 * change the angles. */
void orc_rope_partial(float* x, int32_t m, int32_t n_heads, int32_t head_dim, int32_t rotary_dim, int32_t pos0,
                      double theta) {
    const int32_t half = rotary_dim / 2;
    for (int32_t r = 0; r < m; ++r) {
        double pos = (double)(pos0 + r);
        for (int32_t hh = 0; hh < n_heads; ++hh) {
            float* v = x + ((size_t)r * n_heads + hh) * head_dim;
            for (int32_t i = 0; i < half; ++i) {
                double inv_freq = pow(theta, -2.0 * (double)i / (double)rotary_dim);
                double ang = pos * inv_freq;
                double c = cos(ang), s = sin(ang);
                double a = v[i], b = v[i + half];
                v[i] = (float)(a * c - b * s);
                v[i + half] = (float)(a * s + b * c);
            }
        }
    }
}

/* The same over the full head dimension. */
void orc_rope(float* x, int32_t m, int32_t n_heads, int32_t head_dim, int32_t pos0, double theta) {
    orc_rope_partial(x, m, n_heads, head_dim, head_dim, pos0, theta);
}

/* Which of a token's four position ids turns rotary pair j under the
 * interleaved multi-section rotary of [mtp.rs] `apply_imrope` (sections
 * `mrope_section` = sizes s0, s1, s2 of the first three ids; reading: the
 * pairs cycle through ids 0, 1, 2 by j mod 3, each id keeping the pairs of
 * its residue while it has pairs left (id k owns the pairs j = k mod 3 with
 * j < 3 s_k), and every other pair takes the fourth id). */
int32_t orc_imrope_section(int32_t pair, const int32_t* sections) {
    const int32_t k = pair % 3;
    return pair < 3 * sections[k] ? k : 3;
}

/* orc_rope_partial with a position per (row, section): pair i of row r turns
 * by positions[4 r + orc_imrope_section(i)] * theta^(-2i/rotary_dim). */
void orc_rope_sections(float* x, int32_t m, int32_t n_heads, int32_t head_dim, int32_t rotary_dim,
                       const int32_t* positions, const int32_t* sections, double theta) {
    const int32_t half = rotary_dim / 2;
    for (int32_t r = 0; r < m; ++r)
        for (int32_t hh = 0; hh < n_heads; ++hh) {
            float* v = x + ((size_t)r * n_heads + hh) * head_dim;
            for (int32_t i = 0; i < half; ++i) {
                double pos = (double)positions[4 * (size_t)r + (size_t)orc_imrope_section(i, sections)];
                double inv_freq = pow(theta, -2.0 * (double)i / (double)rotary_dim);
                double ang = pos * inv_freq;
                double c = cos(ang), s = sin(ang);
                double a = v[i], b = v[i + half];
                v[i] = (float)(a * c - b * s);
                v[i + half] = (float)(a * s + b * c);
            }
        }
}

/* The rotary step of the layer for m rows of a call at cache_len. */
static void layer_rope(const orc_layer* L, float* x, int32_t m, int32_t n_heads, int32_t cache_len) {
    const int32_t d = L->head_dim, rot = L->rotary_dim > 0 ? L->rotary_dim : d;
    if (L->positions)
        orc_rope_sections(x, m, n_heads, d, rot, L->positions, L->mrope_section, L->rope_theta);
    else
        orc_rope_partial(x, m, n_heads, d, rot, cache_len, L->rope_theta);
}

/* Causal grouped-query attention over the cache ([mtp.rs]
 * `apply_sdpa_with_kv_cache` call in `forward_full_attention`; [mimo.rs]
 * `qwen_attention_batch` call in `mimo_mtp_block_with_probe`).  Query row r
 * sees cache rows 0 .. cache_len + r (its own freshly appended row included);
 * query head h reads KV head h / (n_heads / n_kv_heads); scores are scaled by
 * 1/sqrt(head_dim).  Caches are [n_kv_heads][capacity][head_dim]. */
void orc_sdpa(const float* q, const float* k_cache, const float* v_cache, int32_t m,
              int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t cache_len,
              int32_t capacity, float* out) {
    orc_sdpa_window(q, k_cache, v_cache, m, n_heads, n_kv_heads, head_dim, cache_len, capacity, 0, NULL, out);
}

/* The same with the sliding window and the sinks of the MiMo draft attention
 * ([mimo.rs] module doc "The draft forward": "window 128, sinks"): row r at
 * position p = cache_len + r scores positions max(0, p-W+1) .. p when W > 0
 * (all of 0 .. p when W = 0), and with sinks the softmax of head hh runs over
 * those scores and the extra logit sinks[hh], whose value row is zero:
 *   o = sum_j e^(s_j - M) v_j / (sum_j e^(s_j - M) + e^(sink - M)),
 *   M = max(sink, max_j s_j). */
void orc_sdpa_window(const float* q, const float* k_cache, const float* v_cache, int32_t m, int32_t n_heads,
                     int32_t n_kv_heads, int32_t head_dim, int32_t cache_len, int32_t capacity, int32_t window,
                     const float* sinks, float* out) {
    orc_sdpa_kv(q, k_cache, v_cache, m, n_heads, n_kv_heads, head_dim, head_dim, cache_len, capacity, window, sinks,
                out);
}

/* The same with V heads of their own width v_dim (MiMo's head 192 / V 128):
 * scores over head_dim, scale 1/sqrt(head_dim), outputs and V cache rows of
 * v_dim floats ([n_kv_heads][capacity][v_dim]). */
void orc_sdpa_kv(const float* q, const float* k_cache, const float* v_cache, int32_t m, int32_t n_heads,
                 int32_t n_kv_heads, int32_t head_dim, int32_t v_dim, int32_t cache_len, int32_t capacity,
                 int32_t window, const float* sinks, float* out) {
    const int32_t group = n_heads / n_kv_heads;
    const double scale = 1.0 / sqrt((double)head_dim);
    const int32_t max_len = cache_len + m;
    /* (row, head) pairs are independent (threads with OpenMP) */
#pragma omp parallel
    {
    double* p = (double*)xmalloc(sizeof(double) * (size_t)max_len);
    double* o = (double*)xmalloc(sizeof(double) * (size_t)v_dim);
#pragma omp for collapse(2) schedule(static)
    for (int32_t r = 0; r < m; ++r) {
        for (int32_t hh = 0; hh < n_heads; ++hh) {
            const int32_t pos = cache_len + r;
            const int32_t lo = (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
            const int32_t g = hh / group;
            const float* qv = q + ((size_t)r * n_heads + hh) * head_dim;
            const float* K = k_cache + (size_t)g * capacity * head_dim;
            const float* V = v_cache + (size_t)g * capacity * v_dim;
            double mx = sinks ? (double)sinks[hh] : -INFINITY;
            for (int32_t j = lo; j <= pos; ++j) {
                double s = 0.0;
                for (int32_t t = 0; t < head_dim; ++t)
                    s += (double)qv[t] * (double)K[(size_t)j * head_dim + t];
                p[j] = s * scale;
                if (p[j] > mx) mx = p[j];
            }
            double z = sinks ? exp((double)sinks[hh] - mx) : 0.0;
            for (int32_t j = lo; j <= pos; ++j) {
                p[j] = exp(p[j] - mx);
                z += p[j];
            }
            for (int32_t t = 0; t < v_dim; ++t) o[t] = 0.0;
            for (int32_t j = lo; j <= pos; ++j)
                for (int32_t t = 0; t < v_dim; ++t) o[t] += p[j] * (double)V[(size_t)j * v_dim + t];
            float* dst = out + ((size_t)r * n_heads + hh) * v_dim;
            for (int32_t t = 0; t < v_dim; ++t) dst[t] = (float)(o[t] / z);
        }
    }
    free(p);
    free(o);
    }
}

/* Greedy pick: first index of the largest value (ties go to the lowest index;
 * NaN never wins). */
int32_t orc_argmax(const float* v, int32_t n) {
    int32_t best = -1;
    for (int32_t i = 0; i < n; ++i)
        if (v[i] == v[i] && (best < 0 || v[i] > v[best])) best = i;
    return best < 0 ? 0 : best;
}

/* ------------------------------------------------------------------------ */
/* Layer steps                                                               */
/* ------------------------------------------------------------------------ */

/* u = eh_proj * [rms(e; gamma_e) ; rms(h; gamma_h)], the embedding half first
 * ([mimo.rs] module doc "The draft forward"; [mtp.rs]
 * `project_embedding_and_hidden`, both norms with eps 1e-6). */
void orc_norm_concat_proj(const float* e, const float* h, const float* gamma_e, const float* gamma_h,
                          float eps, const orc_q4* eh_proj, int32_t m, float* u) {
    const int32_t H = eh_proj->k / 2;
    float* en = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* hn = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* cat = (float*)xmalloc(sizeof(float) * (size_t)m * 2 * H);
    orc_rmsnorm(e, gamma_e, m, H, eps, en);
    orc_rmsnorm(h, gamma_h, m, H, eps, hn);
    for (int32_t r = 0; r < m; ++r) {
        memcpy(cat + (size_t)r * 2 * H, en + (size_t)r * H, sizeof(float) * (size_t)H);
        memcpy(cat + (size_t)r * 2 * H + H, hn + (size_t)r * H, sizeof(float) * (size_t)H);
    }
    orc_gemv4(eh_proj, cat, m, u);
    free(en);
    free(hn);
    free(cat);
}

/* r1 = u + Wo * attention(rope(Wq xa), rope(Wk xa), Wv xa) with
 * xa = rms(u; gamma_attn).  The m new K/V rows are written into the caches
 * at rows cache_len .. cache_len+m-1 before the attention reads them
 * ([mtp.rs] `forward_full_attention`; the residual add is the first half of
 * `forward_ffn_residual`'s fused residual norm).  The optional variant steps
 * (see orc_layer) follow that function's order: q (and gate) projection, k
 * and v projections, per-head q and k norms, rotary step, attention, sigmoid
 * gate, wo. */
void orc_attention(const orc_layer* L, const float* u, float* k_cache, float* v_cache,
                   int32_t cache_len, int32_t capacity, int32_t m, float* r1) {
    const int32_t H = L->hidden, d = L->head_dim, nh = L->n_heads, nkv = L->n_kv_heads;
    const int32_t dv = L->v_head_dim > 0 ? L->v_head_dim : d;
    const int32_t qrows = nh * (L->q_gated ? d + dv : d);
    float* xa = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* qg = (float*)xmalloc(sizeof(float) * (size_t)m * qrows);
    float* q = (float*)xmalloc(sizeof(float) * (size_t)m * nh * d);
    float* gate = (float*)xmalloc(sizeof(float) * (size_t)m * nh * dv);
    float* k = (float*)xmalloc(sizeof(float) * (size_t)m * nkv * d);
    float* v = (float*)xmalloc(sizeof(float) * (size_t)m * nkv * dv);
    float* o = (float*)xmalloc(sizeof(float) * (size_t)m * nh * dv);
    float* a = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    orc_rmsnorm(u, L->gamma_attn, m, H, L->eps, xa);
    orc_gemv4(&L->wq, xa, m, qg);
    for (int32_t r = 0; r < m; ++r)
        for (int32_t hh = 0; hh < nh; ++hh) {
            const float* src = qg + (size_t)r * qrows + (size_t)hh * (L->q_gated ? d + dv : d);
            memcpy(q + ((size_t)r * nh + hh) * d, src, sizeof(float) * (size_t)d);
            if (L->q_gated) memcpy(gate + ((size_t)r * nh + hh) * dv, src + d, sizeof(float) * (size_t)dv);
        }
    orc_gemv4(&L->wk, xa, m, k);
    orc_gemv4(&L->wv, xa, m, v);
    /* per-head norms: every head of every row is one RMSNorm row of head_dim */
    if (L->gamma_q_head) orc_rmsnorm(q, L->gamma_q_head, m * nh, d, L->eps, q);
    if (L->gamma_k_head) orc_rmsnorm(k, L->gamma_k_head, m * nkv, d, L->eps, k);
    layer_rope(L, q, m, nh, cache_len);
    layer_rope(L, k, m, nkv, cache_len);
    for (int32_t r = 0; r < m; ++r)
        for (int32_t g = 0; g < nkv; ++g) {
            const size_t row = (size_t)g * capacity + (size_t)(cache_len + r);
            memcpy(k_cache + row * d, k + ((size_t)r * nkv + g) * d, sizeof(float) * (size_t)d);
            memcpy(v_cache + row * dv, v + ((size_t)r * nkv + g) * dv, sizeof(float) * (size_t)dv);
        }
    orc_sdpa_kv(q, k_cache, v_cache, m, nh, nkv, d, dv, cache_len, capacity, L->window, L->sinks, o);
    if (L->q_gated)
        for (size_t i = 0; i < (size_t)m * nh * dv; ++i)
            o[i] = (float)((double)o[i] / (1.0 + exp(-(double)gate[i])));
    orc_gemv4(&L->wo, o, m, a);
    for (size_t i = 0; i < (size_t)m * H; ++i) r1[i] = (float)((double)u[i] + (double)a[i]);
    free(xa);
    free(qg);
    free(q);
    free(gate);
    free(k);
    free(v);
    free(o);
    free(a);
}

/* Catch-up of the draft layer's cache after a target batch ([mtp.rs]
 * `process_target_batch` and `append_attention_kv`): row r's hidden is the
 * target's post-norm hidden shifted one row right (row 0 = pending_h, or zero
 * when there is none; row r > 0 = target_h row r-1); u = eh_proj [rms(e_r);
 * rms(shifted_r)]; then only the attention's K/V side runs: xa = rms(u;
 * gamma_attn), k = Wk xa, v = Wv xa, the per-head k norm when present, the
 * rotary step at position cache_len + r (or at the row's position ids when
 * the layer carries them), and the rows are written at
 * cache_len + r.  Nothing else is computed (the FFN and the logits hold no
 * state). */
void orc_append_kv(const orc_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                   const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                   int32_t cache_len, int32_t capacity, int32_t m) {
    const int32_t H = L->hidden, d = L->head_dim, nkv = L->n_kv_heads;
    const int32_t dv = L->v_head_dim > 0 ? L->v_head_dim : d;
    float* er = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* sh = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* u = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* xa = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* k = (float*)xmalloc(sizeof(float) * (size_t)m * nkv * d);
    float* v = (float*)xmalloc(sizeof(float) * (size_t)m * nkv * dv);
    for (int32_t r = 0; r < m; ++r) {
        const float* src = (tokens && tokens[r] >= 0) ? embed_table + (size_t)tokens[r] * H : e + (size_t)r * H;
        memcpy(er + (size_t)r * H, src, sizeof(float) * (size_t)H);
        if (r == 0) {
            if (pending_h)
                memcpy(sh, pending_h, sizeof(float) * (size_t)H);
            else
                memset(sh, 0, sizeof(float) * (size_t)H);
        } else {
            memcpy(sh + (size_t)r * H, target_h + (size_t)(r - 1) * H, sizeof(float) * (size_t)H);
        }
    }
    orc_norm_concat_proj(er, sh, L->gamma_e, L->gamma_h, L->eps, &L->eh_proj, m, u);
    orc_rmsnorm(u, L->gamma_attn, m, H, L->eps, xa);
    orc_gemv4(&L->wk, xa, m, k);
    orc_gemv4(&L->wv, xa, m, v);
    if (L->gamma_k_head) orc_rmsnorm(k, L->gamma_k_head, m * nkv, d, L->eps, k);
    layer_rope(L, k, m, nkv, cache_len);
    for (int32_t r = 0; r < m; ++r)
        for (int32_t g = 0; g < nkv; ++g) {
            const size_t row = (size_t)g * capacity + (size_t)(cache_len + r);
            memcpy(k_cache + row * d, k + ((size_t)r * nkv + g) * d, sizeof(float) * (size_t)d);
            memcpy(v_cache + row * dv, v + ((size_t)r * nkv + g) * dv, sizeof(float) * (size_t)dv);
        }
    free(er);
    free(sh);
    free(u);
    free(xa);
    free(k);
    free(v);
}

static double silu(double a) { return a / (1.0 + exp(-a)); }

/* y = [residual +] down * (silu(gate * x) . (up * x)) with 4-bit weights
 * ([mtp.rs] `forward_ffn_residual` DenseQ arm; [mimo.rs] `dense_ffn_batch`
 * with the SiLU activation). */
void orc_ffn_dense(const float* x, const orc_q4* gate, const orc_q4* up, const orc_q4* down,
                   const float* residual, int32_t m, float* y) {
    const int32_t I = gate->n, H = down->n;
    float* a = (float*)xmalloc(sizeof(float) * (size_t)m * I);
    float* b = (float*)xmalloc(sizeof(float) * (size_t)m * I);
    float* dz = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    orc_gemv4(gate, x, m, a);
    orc_gemv4(up, x, m, b);
    for (size_t i = 0; i < (size_t)m * I; ++i) a[i] = (float)(silu((double)a[i]) * (double)b[i]);
    orc_gemv4(down, a, m, dz);
    for (size_t i = 0; i < (size_t)m * H; ++i)
        y[i] = residual ? (float)((double)residual[i] + (double)dz[i]) : dz[i];
    free(a);
    free(b);
    free(dz);
}

/* One SwiGLU expert applied to one row, out = down*(silu(gate x).(up x)),
 * over 8-bit (q8 set) or 4-bit bf16-constant matrices. */
typedef struct {
    const orc_q8 *g8, *u8, *d8;
    const orc_q4e *g4, *u4, *d4;
} expert_w;

static void expert(const expert_w* w, const float* x, float* out) {
    const int32_t I = w->g8 ? w->g8->n : w->g4->n;
    float* a = (float*)xmalloc(sizeof(float) * (size_t)I);
    float* b = (float*)xmalloc(sizeof(float) * (size_t)I);
    if (w->g8) {
        orc_gemv8(w->g8, x, 1, a);
        orc_gemv8(w->u8, x, 1, b);
    } else {
        orc_gemv4e(w->g4, x, 1, a);
        orc_gemv4e(w->u4, x, 1, b);
    }
    for (int32_t i = 0; i < I; ++i) a[i] = (float)(silu((double)a[i]) * (double)b[i]);
    if (w->d8)
        orc_gemv8(w->d8, a, 1, out);
    else
        orc_gemv4e(w->d4, a, 1, out);
    free(a);
    free(b);
}

/* Routing of one row: p = softmax(l) over all experts, the top_k experts by
 * (p descending, index ascending) into sel, their gates p_e / (sum of the
 * selected p) into gsel. */
static void route_row(const float* l, int32_t n_experts, int32_t top_k, int32_t* sel, double* gsel) {
    double* p = (double*)xmalloc(sizeof(double) * (size_t)n_experts);
    char* taken = (char*)xmalloc((size_t)n_experts);
    double mx = -INFINITY, z = 0.0;
    for (int32_t e = 0; e < n_experts; ++e)
        if ((double)l[e] > mx) mx = (double)l[e];
    for (int32_t e = 0; e < n_experts; ++e) {
        p[e] = exp((double)l[e] - mx);
        z += p[e];
    }
    for (int32_t e = 0; e < n_experts; ++e) p[e] /= z;
    memset(taken, 0, (size_t)n_experts);
    double psum = 0.0;
    for (int32_t s = 0; s < top_k; ++s) {
        int32_t best = -1;
        for (int32_t e = 0; e < n_experts; ++e)
            if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
        taken[best] = 1;
        sel[s] = best;
        psum += p[best];
    }
    for (int32_t s = 0; s < top_k; ++s) gsel[s] = p[sel[s]] / psum;
    free(p);
    free(taken);
}

/* The mixture over rows; ex(e) gives expert e's matrices, sh the shared
 * expert's (NULL: none). */
static int32_t moe_rows(const float* x, const float* router, int32_t n_experts, int32_t top_k, int32_t H,
                        const orc_q8* ge8, const orc_q8* ue8, const orc_q8* de8, const orc_q4e* ge4,
                        const orc_q4e* ue4, const orc_q4e* de4, const expert_w* sh, const float* residual,
                        int32_t m, float* y, int32_t* expert_ids, float* gates, float* router_logits) {
    if (top_k < 1 || top_k > n_experts) return -1;
    float* l = (float*)xmalloc(sizeof(float) * (size_t)n_experts);
    int32_t* sel = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)top_k);
    double* gsel = (double*)xmalloc(sizeof(double) * (size_t)top_k);
    float* eo = (float*)xmalloc(sizeof(float) * (size_t)H);
    double* acc = (double*)xmalloc(sizeof(double) * (size_t)H);
    for (int32_t r = 0; r < m; ++r) {
        const float* xr = x + (size_t)r * H;
        orc_gemv_f32(router, n_experts, H, xr, 1, l);
        if (router_logits) memcpy(router_logits + (size_t)r * n_experts, l, sizeof(float) * (size_t)n_experts);
        route_row(l, n_experts, top_k, sel, gsel);
        for (int32_t i = 0; i < H; ++i) acc[i] = residual ? (double)residual[(size_t)r * H + i] : 0.0;
        for (int32_t s = 0; s < top_k; ++s) {
            const int32_t e = sel[s];
            expert_w w = {NULL, NULL, NULL, NULL, NULL, NULL};
            if (ge8) {
                w.g8 = &ge8[e];
                w.u8 = &ue8[e];
                w.d8 = &de8[e];
            } else {
                w.g4 = &ge4[e];
                w.u4 = &ue4[e];
                w.d4 = &de4[e];
            }
            expert(&w, xr, eo);
            for (int32_t i = 0; i < H; ++i) acc[i] += gsel[s] * (double)eo[i];
            if (expert_ids) expert_ids[(size_t)r * top_k + s] = e;
            if (gates) gates[(size_t)r * top_k + s] = (float)gsel[s];
        }
        if (sh) {
            expert(sh, xr, eo);
            for (int32_t i = 0; i < H; ++i) acc[i] += (double)eo[i];
        }
        for (int32_t i = 0; i < H; ++i) y[(size_t)r * H + i] = (float)acc[i];
    }
    free(l);
    free(sel);
    free(gsel);
    free(eo);
    free(acc);
    return 0;
}

/* Routed mixture of 8-bit SwiGLU experts plus one always-on shared expert
 * ([mtp.rs] `MtpFfnWeightsGpu::Moe`: router `ffn_gate_inp`, stacked
 * gate/up/down experts and shared-expert tensors).  Per row: router logits
 * l = R x (f32 router), p = softmax(l), the top_k experts by (p descending,
 * index ascending), gates p_e / sum of the selected p, and
 * y = [residual] + sum_e gate_e * expert_e(x) + shared(x).
 * expert_ids/gates are [m][top_k] in selection order. Returns 0, or -1 on a
 * bad argument. */
int32_t orc_moe(const float* x, const float* router, int32_t n_experts, int32_t top_k,
                const orc_q8* gate_exps, const orc_q8* up_exps, const orc_q8* down_exps,
                const orc_q8* sh_gate, const orc_q8* sh_up, const orc_q8* sh_down,
                const float* residual, int32_t m, float* y, int32_t* expert_ids, float* gates,
                float* router_logits) {
    expert_w sh = {sh_gate, sh_up, sh_down, NULL, NULL, NULL};
    return moe_rows(x, router, n_experts, top_k, gate_exps[0].k, gate_exps, up_exps, down_exps, NULL, NULL, NULL,
                    sh_gate ? &sh : NULL, residual, m, y, expert_ids, gates, router_logits);
}

/* The same mixture over 4-bit experts with bf16 group constants ([shared.rs]
 * `MlxAffineMoeStack`), the shared expert in the same form. */
int32_t orc_moe4(const float* x, const float* router, int32_t n_experts, int32_t top_k,
                 const orc_q4e* gate_exps, const orc_q4e* up_exps, const orc_q4e* down_exps,
                 const orc_q4e* sh_gate, const orc_q4e* sh_up, const orc_q4e* sh_down,
                 const float* residual, int32_t m, float* y, int32_t* expert_ids, float* gates,
                 float* router_logits) {
    expert_w sh = {NULL, NULL, NULL, sh_gate, sh_up, sh_down};
    return moe_rows(x, router, n_experts, top_k, gate_exps[0].k, NULL, NULL, NULL, gate_exps, up_exps, down_exps,
                    sh_gate ? &sh : NULL, residual, m, y, expert_ids, gates, router_logits);
}

/* Shared head with greedy pick: yn = rms(hidden; gamma), logits = LM yn,
 * id = argmax(logits) per row ([mtp.rs] `forward_shared_head_greedy`; the
 * normed row is returned as the chain input, `forward_draft_with_hidden`). */
void orc_head(const float* hidden, const float* gamma, float eps, const orc_q4* lm_head, int32_t m,
              float* normed_out, float* logits_out, int32_t* ids_out) {
    const int32_t H = lm_head->k, V = lm_head->n;
    float* yn = normed_out ? normed_out : (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* lg = logits_out ? logits_out : (float*)xmalloc(sizeof(float) * (size_t)m * V);
    orc_rmsnorm(hidden, gamma, m, H, eps, yn);
    orc_gemv4(lm_head, yn, m, lg);
    for (int32_t r = 0; r < m; ++r) ids_out[r] = orc_argmax(lg + (size_t)r * V, V);
    if (!normed_out) free(yn);
    if (!logits_out) free(lg);
}

/* The same head over an 8-bit block lm_head ([mimo.rs]
 * `mimo_verify_head_rows`: the verify rows' final norm, then one head panel
 * over the q8 lm_head; the greedy pick of each row as in the 4-bit head). */
void orc_head8(const float* hidden, const float* gamma, float eps, const orc_q8* lm_head, int32_t m,
               float* normed_out, float* logits_out, int32_t* ids_out) {
    const int32_t H = lm_head->k, V = lm_head->n;
    float* yn = normed_out ? normed_out : (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* lg = logits_out ? logits_out : (float*)xmalloc(sizeof(float) * (size_t)m * V);
    orc_rmsnorm(hidden, gamma, m, H, eps, yn);
    orc_gemv8(lm_head, yn, m, lg);
    for (int32_t r = 0; r < m; ++r) ids_out[r] = orc_argmax(lg + (size_t)r * V, V);
    if (!normed_out) free(yn);
    if (!logits_out) free(lg);
}

/* The layer's FFN forms behind one wiring: the dense 4-bit SwiGLU of the
 * layer, or the routed mixture (8-bit or 4-bit experts) when moe is given. */
static int32_t ffn_residual(const orc_layer* L, const orc_moe_ffn* moe, const float* f, const float* r1, int32_t m,
                            float* r2) {
    if (!moe) {
        orc_ffn_dense(f, &L->gate, &L->up, &L->down, r1, m, r2);
        return 0;
    }
    if (moe->q4)
        return orc_moe4(f, moe->router, moe->n_experts, moe->top_k, moe->gate_exps4, moe->up_exps4,
                        moe->down_exps4, moe->sh_gate4, moe->sh_up4, moe->sh_down4, r1, m, r2, NULL, NULL, NULL);
    return orc_moe(f, moe->router, moe->n_experts, moe->top_k, moe->gate_exps, moe->up_exps, moe->down_exps,
                   moe->sh_gate, moe->sh_up, moe->sh_down, r1, m, r2, NULL, NULL, NULL);
}

/* One draft-layer forward over m rows at positions cache_len .. cache_len+m-1
 * ([mimo.rs] module doc "The draft forward" and `mimo_mtp_block_with_probe`;
 * [mtp.rs] `forward_draft_body`, whose FFN step `forward_ffn_residual` adds
 * the FFN output to its own input's residual, then `forward_shared_head_greedy`):
 *   u  = eh_proj [rms(e); rms(h)]
 *   r1 = u + attention(rms(u))            (appends K/V rows)
 *   r2 = r1 + ffn(rms(r1; gamma_post))    (dense SwiGLU, or the MoE of
 *                                          `MtpFfnWeightsGpu::Moe`)
 *   yn = rms(r2; gamma_final), logits = LM yn, id = argmax.
 * Row r's embedding is embed_table[tokens[r]] when tokens is given and
 * tokens[r] >= 0, else e[r].  hidden_out receives yn.  Returns 0, or -1 on a
 * bad argument (nothing is written then). */
static int32_t draft_step(const orc_layer* L, const orc_moe_ffn* moe, const float* e, const int32_t* tokens,
                          const float* embed_table, const float* h, float* k_cache, float* v_cache,
                          int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out, float* hidden_out,
                          float* logits_out) {
    const int32_t H = L->hidden;
    if (m < 1 || cache_len < 0 || cache_len + m > capacity) return -1;
    if (moe && (moe->top_k < 1 || moe->top_k > moe->n_experts ||
                (moe->q4 ? moe->gate_exps4[0].k : moe->gate_exps[0].k) != H))
        return -1;
    for (int32_t r = 0; r < m; ++r) {
        int use_table = tokens && tokens[r] >= 0;
        if (use_table && (!embed_table || tokens[r] >= L->vocab)) return -1;
        if (!use_table && !e) return -1;
    }
    float* ee = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* u = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* r1 = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* f = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    float* r2 = (float*)xmalloc(sizeof(float) * (size_t)m * H);
    for (int32_t r = 0; r < m; ++r) {
        const float* src = (tokens && tokens[r] >= 0) ? embed_table + (size_t)tokens[r] * H : e + (size_t)r * H;
        memcpy(ee + (size_t)r * H, src, sizeof(float) * (size_t)H);
    }
    orc_norm_concat_proj(ee, h, L->gamma_e, L->gamma_h, L->eps, &L->eh_proj, m, u);
    orc_attention(L, u, k_cache, v_cache, cache_len, capacity, m, r1);
    orc_rmsnorm(r1, L->gamma_post, m, H, L->eps, f);
    ffn_residual(L, moe, f, r1, m, r2);
    orc_head(r2, L->gamma_final, L->eps, &L->lm_head, m, hidden_out, logits_out, ids_out);
    free(ee);
    free(u);
    free(r1);
    free(f);
    free(r2);
    return 0;
}

int32_t orc_draft_step(const orc_layer* L, const float* e, const int32_t* tokens,
                       const float* embed_table, const float* h, float* k_cache, float* v_cache,
                       int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out,
                       float* hidden_out, float* logits_out) {
    return draft_step(L, NULL, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m, ids_out,
                      hidden_out, logits_out);
}

int32_t orc_draft_step_moe(const orc_layer* L, const orc_moe_ffn* moe, const float* e, const int32_t* tokens,
                           const float* embed_table, const float* h, float* k_cache, float* v_cache,
                           int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out, float* hidden_out,
                           float* logits_out) {
    if (!moe) return -1;
    return draft_step(L, moe, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m, ids_out,
                      hidden_out, logits_out);
}
