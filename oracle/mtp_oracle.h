/*
 * mtp_oracle.h -- plain, slow, scalar-C reference of the quantized MTP draft
 * layer forward.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check
 * and the benchmark's CPU-baseline leg call it; the product library never
 * links, loads or calls anything here, and nothing here is shared with it.
 *
 * Sources (public web pages, cited by title and Rust item):
 *   [mtp.rs]    hf2q 0.1.13, src/inference/models/qwen35/mtp.rs
 *   [mimo.rs]   cortiq-engine 0.8.49, src/mimo_mtp.rs
 *   [shared.rs] hf2q 0.1.1, src/serve/forward_mlx_shared.rs
 *
 * Arithmetic rules (the pages' own CPU checks accumulate in double; the
 * pages keep activations and logits in f32):
 *   - every sum is a double accumulator over ascending index;
 *   - every activation passed between steps is stored as f32;
 *   - the f32 dequantized weight is the exact affine value rounded once
 *     (fmaf), while the products inside a GEMV use the exact value in double.
 *
 * Pins: the pages print values for the 4-bit GEMV only; every other function
 * is pinned by closed forms written out in numpy (f64, from the raw codes),
 * special cases that reduce to a textbook routine, brute force on tiny
 * inputs and invariants (batched equals sequential, gates sum to one, ...).
 */
#ifndef MTP_ORACLE_H
#define MTP_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 4-bit affine weight, group size 32 ([shared.rs] `MlxAffineExtra`):
 * codes u32 [n][k/8], element k of a row is nibble (k%8) of word k/8, the low
 * nibble holding the lowest k; scales and biases f32 [n][k/32]. */
typedef struct {
    const uint32_t* codes;
    const float* scales;
    const float* biases;
    int32_t n, k;
} orc_q4;

/* 8-bit block weight, block 32: int8 codes [n][k], f32 scales [n][k/32],
 * value = scale * code.  One matrix; expert stacks are passed as arrays. */
typedef struct {
    const int8_t* codes;
    const float* scales;
    int32_t n, k;
} orc_q8;

/* 4-bit affine matrix with bf16 group constants, one matrix of an expert
 * stack ([shared.rs] `MlxAffineMoeStack`: packed-u32 codes [e][n][k/8] in the
 * nibble order of orc_q4, bf16 scales and biases [e][n][k/32]).  A bf16 value
 * is stored as its 16 bits, the upper half of the f32 it stands for; the
 * weight is scale*code + bias with scale and bias widened to f32.  Expert
 * stacks are passed as arrays of these. */
typedef struct {
    const uint32_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
    int32_t n, k;
} orc_q4e;

/* One dense MTP draft layer ([mimo.rs] module doc "The draft forward";
 * [mtp.rs] `MtpWeights`).  Attention variant of [mtp.rs]
 * `forward_full_attention` (all optional):
 *   q_gated       wq holds 2*n_heads*head_dim rows, per head h the head's q
 *                 rows then its gate rows (rows 2hd..2hd+d-1, 2hd+d..2hd+2d-1);
 *                 the attention output is multiplied by sigmoid(gate) before wo
 *                 (`MtpQGateWeightsGpu::Gated`, `apply_sigmoid_gate_multiply`);
 *   gamma_q_head, gamma_k_head  f32 [head_dim]: per-head RMSNorm of q and k
 *                 before the rotary step (`apply_q_or_k_per_head_rms_norm`);
 *   rotary_dim    0 or head_dim: rotary over all dims; else only the first
 *                 rotary_dim dims rotate (`apply_imrope`'s rotary_dim).
 * Sliding-window attention of the MiMo draft layer ([mimo.rs] module doc "The
 * draft forward": window 128, sinks), both optional:
 *   window        0: causal over the whole cache; W > 0: the row at position
 *                 p sees positions p-W+1 .. p only (W rows, itself included);
 *   sinks         f32 [n_heads] or NULL: one logit per query head that joins
 *                 the softmax denominator with no value row.
 * MiMo draft geometry ([mimo.rs] module doc "The draft forward": head 192 /
 * V 128):
 *   v_head_dim    0 = head_dim; else the width dv of the V heads (and of the
 *                 attention output per head): wv has n_kv_heads*dv rows, wo
 *                 n_heads*dv columns, the V cache rows are dv wide, and with
 *                 q_gated a head's gate rows (dv of them) follow its head_dim
 *                 q rows.
 * Multi-section rotary positions ([mtp.rs] `apply_imrope` with
 * `mrope_section` and four position ids per token):
 *   positions     NULL: row r of a call at cache_len sits at cache_len + r for
 *                 every rotary pair; else int32 [m][4], the four position ids
 *                 of each row of the call, and rotary pair j of row r turns by
 *                 positions[4r + orc_imrope_section(j, mrope_section)];
 *   mrope_section the four section sizes (see orc_imrope_section). */
typedef struct {
    int32_t hidden, n_heads, n_kv_heads, head_dim, vocab, ffn_inter;
    double rope_theta;
    float eps;
    const float *gamma_e, *gamma_h, *gamma_attn, *gamma_post, *gamma_final;
    orc_q4 eh_proj, wq, wk, wv, wo, gate, up, down, lm_head;
    const float *gamma_q_head, *gamma_k_head;
    int32_t q_gated, rotary_dim;
    const float* sinks;
    int32_t window;
    int32_t v_head_dim;
    int32_t mrope_section[4];
    const int32_t* positions;
} orc_layer;

/* The routed FFN of the MoE draft layer ([mtp.rs] `MtpFfnWeightsGpu::Moe`):
 * f32 router [n_experts][hidden], per-expert gate/up [inter][hidden] and down
 * [hidden][inter] (arrays of n_experts matrices), and an optional shared
 * expert (its gate NULL: none).  q4 = 0: the 8-bit matrices (gate_exps ...);
 * q4 != 0: the 4-bit bf16-constant matrices of [shared.rs]
 * `MlxAffineMoeStack` (gate_exps4 ...), the shared expert in the same form. */
typedef struct {
    const float* router;
    int32_t n_experts, top_k;
    const orc_q8 *gate_exps, *up_exps, *down_exps;
    const orc_q8 *sh_gate, *sh_up, *sh_down;
    int32_t q4;
    const orc_q4e *gate_exps4, *up_exps4, *down_exps4;
    const orc_q4e *sh_gate4, *sh_up4, *sh_down4;
} orc_moe_ffn;

/* ---- weight formats ---- */
void orc_unpack4(const uint32_t* codes, int32_t n, int32_t k, uint8_t* out);
void orc_deq4(const orc_q4* w, float* out);
void orc_deq8(const orc_q8* w, float* out);
float orc_bf16(uint16_t bits);
void orc_deq4e(const orc_q4e* w, float* out);

/* ---- primitives ---- */
void orc_gemv4(const orc_q4* w, const float* x, int32_t m, float* y);
void orc_gemv8(const orc_q8* w, const float* x, int32_t m, float* y);
void orc_gemv4e(const orc_q4e* w, const float* x, int32_t m, float* y);
void orc_gemv_f32(const float* w, int32_t n, int32_t k, const float* x, int32_t m, float* y);
void orc_rmsnorm(const float* x, const float* gamma, int32_t m, int32_t h, float eps, float* y);
void orc_rope(float* x, int32_t m, int32_t n_heads, int32_t head_dim, int32_t pos0, double theta);
int32_t orc_imrope_section(int32_t pair, const int32_t* sections);
void orc_rope_sections(float* x, int32_t m, int32_t n_heads, int32_t head_dim, int32_t rotary_dim,
                       const int32_t* positions, const int32_t* sections, double theta);
void orc_rope_partial(float* x, int32_t m, int32_t n_heads, int32_t head_dim, int32_t rotary_dim, int32_t pos0,
                      double theta);
void orc_sdpa(const float* q, const float* k_cache, const float* v_cache, int32_t m,
              int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t cache_len,
              int32_t capacity, float* out);
void orc_sdpa_window(const float* q, const float* k_cache, const float* v_cache, int32_t m, int32_t n_heads,
                     int32_t n_kv_heads, int32_t head_dim, int32_t cache_len, int32_t capacity, int32_t window,
                     const float* sinks, float* out);
void orc_sdpa_kv(const float* q, const float* k_cache, const float* v_cache, int32_t m, int32_t n_heads,
                 int32_t n_kv_heads, int32_t head_dim, int32_t v_dim, int32_t cache_len, int32_t capacity,
                 int32_t window, const float* sinks, float* out);
int32_t orc_argmax(const float* v, int32_t n);

/* ---- layer steps ---- */
void orc_norm_concat_proj(const float* e, const float* h, const float* gamma_e, const float* gamma_h,
                          float eps, const orc_q4* eh_proj, int32_t m, float* u);
void orc_attention(const orc_layer* L, const float* u, float* k_cache, float* v_cache,
                   int32_t cache_len, int32_t capacity, int32_t m, float* r1);
void orc_ffn_dense(const float* x, const orc_q4* gate, const orc_q4* up, const orc_q4* down,
                   const float* residual, int32_t m, float* y);
int32_t orc_moe(const float* x, const float* router, int32_t n_experts, int32_t top_k,
                const orc_q8* gate_exps, const orc_q8* up_exps, const orc_q8* down_exps,
                const orc_q8* sh_gate, const orc_q8* sh_up, const orc_q8* sh_down,
                const float* residual, int32_t m, float* y, int32_t* expert_ids, float* gates,
                float* router_logits);
int32_t orc_moe4(const float* x, const float* router, int32_t n_experts, int32_t top_k,
                 const orc_q4e* gate_exps, const orc_q4e* up_exps, const orc_q4e* down_exps,
                 const orc_q4e* sh_gate, const orc_q4e* sh_up, const orc_q4e* sh_down,
                 const float* residual, int32_t m, float* y, int32_t* expert_ids, float* gates,
                 float* router_logits);
void orc_head(const float* hidden, const float* gamma, float eps, const orc_q4* lm_head, int32_t m,
              float* normed_out, float* logits_out, int32_t* ids_out);
void orc_head8(const float* hidden, const float* gamma, float eps, const orc_q8* lm_head, int32_t m,
               float* normed_out, float* logits_out, int32_t* ids_out);
void orc_append_kv(const orc_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                   const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                   int32_t cache_len, int32_t capacity, int32_t m);
int32_t orc_draft_step(const orc_layer* L, const float* e, const int32_t* tokens,
                       const float* embed_table, const float* h, float* k_cache, float* v_cache,
                       int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out,
                       float* hidden_out, float* logits_out);
/* The same forward with the routed FFN (8-bit or 4-bit experts) in place of
 * the dense one (the layer's gate/up/down are not read). */
int32_t orc_draft_step_moe(const orc_layer* L, const orc_moe_ffn* moe, const float* e, const int32_t* tokens,
                           const float* embed_table, const float* h, float* k_cache, float* v_cache,
                           int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out, float* hidden_out,
                           float* logits_out);

#ifdef __cplusplus
}
#endif
#endif
