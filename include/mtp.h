/*
 * mtp.h -- C ABI of libmtp: the quantized-weight forward of one
 * Multi-Token-Prediction (MTP / NextN) draft layer on AMD Instinct MI355X
 * (gfx950), at m = 1 row for drafting and m = K+1 rows for a batched verify.
 *
 * Sources (public pages, cited by title and Rust item):
 *   [mtp.rs]    hf2q 0.1.13, src/inference/models/qwen35/mtp.rs
 *   [mimo.rs]   cortiq-engine 0.8.49, src/mimo_mtp.rs
 *   [shared.rs] hf2q 0.1.1, src/serve/forward_mlx_shared.rs
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is DEVICE memory owned by the caller, unless a
 *   comment says "host".  The library never allocates or frees device
 *   memory; scratch space is the caller's `ws` of at least the size the
 *   matching *_workspace_size() call returns (mtp_draft_step_noalloc alone
 *   uses a static device array of the library instead).
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work and return; outputs are valid once the stream has reached
 *   that point.  Calls that share an output or a workspace must be ordered on
 *   one stream.  Inputs and outputs must not alias unless stated.
 * - Activations, logits and norm weights are f32, row-major, rows contiguous.
 *   Row pointers (x, e, h, u, hidden, ...) must be 16-byte aligned and
 *   quantized code arrays 16-byte aligned.
 * - m (rows) is 1 .. MTP_MAX_ROWS.  Input features k are a multiple of 32 and
 *   at most MTP_MAX_K.
 * - All argument checks run on the host before anything is enqueued: a call
 *   that returns an error has launched nothing and written nothing (the KV
 *   cache included).  mtp_last_error() then describes the failure (a
 *   thread-local string).  A failed HIP launch returns MTP_ERR_HIP.
 * - Results are deterministic: the same inputs give bit-identical outputs.
 * - Workspaces: the first 1152 bytes of every workspace are reserved for the
 *   state of the lm_head's fused cross-block argmax.  They must be zero before
 *   a workspace's first use (zero-fill it once when it is allocated); no call
 *   writes anything else there and every call leaves them zero, so one
 *   workspace may serve any sequence of calls on one stream.
 * - Arithmetic: activations stay f32 throughout; weight codes enter the
 *   products exactly and every sum accumulates in f32.
 */
#ifndef MTP_H
#define MTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_MAX_ROWS 8
#define MTP_GROUP 32
#define MTP_MAX_K 8192
/* Size of the static device scratch array of mtp_draft_step_noalloc (32 MiB
 * per GPU, held from the library's first use of it on that GPU until the
 * process ends). */
#define MTP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum {
    MTP_OK = 0,
    MTP_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, cache overflow */
    MTP_ERR_UNSUPPORTED = 2, /* a shape this build does not implement */
    MTP_ERR_WORKSPACE = 3,   /* ws NULL or ws_bytes below the required size */
    MTP_ERR_HIP = 4          /* a HIP runtime error while enqueuing */
} mtp_status;

/* 4-bit affine weight, group 32 ([shared.rs] `MlxAffineExtra`,
 * `MlxQWeight::from_mlx_affine_linear`): a matrix of n output rows and k
 * input features, stored out x in.
 *   codes  u32 [n][k/8]: element k of a row is nibble k%8 of word k/8, the
 *          low nibble holding the lowest k;
 *   scales f32 [n][k/32], biases f32 [n][k/32]: value = scale*code + bias. */
typedef struct {
    const uint32_t* codes;
    const float* scales;
    const float* biases;
    int32_t n, k;
} mtp_q4;

/* 8-bit block weight, block 32, as a stack of n_experts matrices
 * (n_experts = 1 for a single matrix):
 *   codes  int8 [n_experts][n][k], scales f32 [n_experts][n][k/32];
 *   value = scale * code. */
typedef struct {
    const int8_t* codes;
    const float* scales;
    int32_t n, k, n_experts;
} mtp_q8;

/* 4-bit affine expert stack, group 32, with bf16 group constants
 * ([shared.rs] `MlxAffineMoeStack`; n_experts = 1 for a single matrix):
 *   codes  u32 [n_experts][n][k/8], nibble order as in mtp_q4;
 *   scales, biases bf16 [n_experts][n][k/32], each stored as its 16 bits (the
 *          upper half of the f32 it stands for);
 *   value = scale*code + bias with scale and bias widened to f32 (exactly),
 *   the f32 result rounded once. */
typedef struct {
    const uint32_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
    int32_t n, k, n_experts;
} mtp_q4e;

#define MTP_FFN_DENSE_Q4 0
#define MTP_FFN_MOE_Q8 1
#define MTP_FFN_MOE_Q4 2

/* One MTP draft layer ([mimo.rs] module doc "The draft forward"; [mtp.rs]
 * `MtpWeights`, `MtpFullAttnWeightsGpu`, `MtpFfnWeightsGpu`).
 * Shapes: eh_proj [hidden][2*hidden]; wq [n_heads*head_dim][hidden];
 * wk [n_kv_heads*head_dim][hidden], wv [n_kv_heads*dv][hidden]; wo [hidden][n_heads*dv]
 * (dv = v_head_dim, or head_dim when it is 0);
 * dense FFN: gate, up [ffn_inter][hidden], down [hidden][ffn_inter];
 * MoE FFN: router f32 [n_experts][hidden], gate_exps/up_exps
 * [n_experts][inter][hidden], down_exps [n_experts][hidden][inter], optional
 * shared expert sh_* (n_experts = 1); 8-bit experts in gate_exps ... sh_down
 * (ffn_kind MTP_FFN_MOE_Q8), 4-bit experts with bf16 constants in
 * gate_exps4 ... sh_down4 (MTP_FFN_MOE_Q4, the shared expert in the same
 * form); lm_head [vocab][hidden].
 * gamma_* are f32 [hidden] norm weights applied as x/rms(x)*gamma.
 * Attention variant ([mtp.rs] `forward_full_attention`, `MtpQGateWeightsGpu`;
 * zero / NULL fields give the plain attention):
 *   q_gated       wq is [2*n_heads*head_dim][hidden]: for head h its q rows
 *                 (2h*d .. 2h*d+d-1) then its gate rows (2h*d+d .. 2h*d+2d-1);
 *                 the attention output is multiplied by sigmoid(gate) before wo.
 *   gamma_q_head, gamma_k_head  f32 [head_dim] (both NULL or both set):
 *                 per-head RMSNorm of q and of k (eps = eps) before the rotary
 *                 step.
 *   rotary_dim    0 = head_dim; else a power of two <= head_dim: only the
 *                 first rotary_dim dims rotate, as pairs (i, i + rotary_dim/2)
 *                 with inverse frequency rope_theta^(-2i/rotary_dim).
 * Sliding-window attention of the MiMo draft layer ([mimo.rs] module doc "The
 * draft forward": "window 128, sinks"; zero / NULL give the plain causal
 * attention):
 *   window        0, or W > 0: the row at position p attends to positions
 *                 max(0, p-W+1) .. p only (W positions, itself included).
 *   sinks         f32 [n_heads] (4-byte aligned, finite) or NULL: per query
 *                 head h a logit sinks[h] that joins the softmax denominator
 *                 with no value row: o = sum_j e^(s_j-M) v_j /
 *                 (sum_j e^(s_j-M) + e^(sinks[h]-M)), M = max(sinks[h], max s_j),
 *                 s_j the scaled scores.
 * MiMo draft geometry ([mimo.rs] module doc "The draft forward": "head 192 /
 * V 128"):
 *   v_head_dim    0 = head_dim; else the V heads' width dv: wv is
 *                 [n_kv_heads*dv][hidden], wo [hidden][n_heads*dv], and the V
 *                 cache is [n_kv_heads][capacity][dv] (the K cache keeps
 *                 head_dim).  Built: head_dim 128 with V 128, and head_dim 192
 *                 with V 128 (no gated q or per-head norms there; rotary over
 *                 all 192 dims by default, pairs (i, i + 96)).
 * Multi-section rotary positions ([mtp.rs] `apply_imrope` with
 * `mrope_section` and four position ids per token; head_dim 128 only):
 *   positions     NULL: row r of a call at cache_len turns every rotary pair
 *                 by position cache_len + r.  Else device int32 [m][4] (4-byte
 *                 aligned), read by every call that takes this descriptor:
 *                 the four position ids of each of the call's m rows (for
 *                 mtp_append_kv, of all its rows), and rotary pair j of row r
 *                 turns by positions[4r + s(j)], where s(j) = j mod 3 when
 *                 j < 3 * mrope_section[j mod 3], else 3 (the three sections
 *                 interleave pair by pair, the fourth id takes the rest).  The
 *                 cache row of row r stays cache_len + r either way.
 *   mrope_section the section sizes (entries >= 0; only the first three are
 *                 read). */
typedef struct {
    int32_t hidden, n_heads, n_kv_heads, head_dim, vocab;
    int32_t ffn_kind; /* MTP_FFN_DENSE_Q4, MTP_FFN_MOE_Q8 or MTP_FFN_MOE_Q4 */
    int32_t ffn_inter;
    int32_t top_k;
    double rope_theta;
    float eps;
    const float *gamma_e, *gamma_h, *gamma_attn, *gamma_post, *gamma_final;
    mtp_q4 eh_proj, wq, wk, wv, wo, gate, up, down, lm_head;
    const float* router;
    mtp_q8 gate_exps, up_exps, down_exps, sh_gate, sh_up, sh_down;
    const float *gamma_q_head, *gamma_k_head;
    int32_t q_gated, rotary_dim;
    const float* sinks;
    int32_t window;
    int32_t v_head_dim;
    mtp_q4e gate_exps4, up_exps4, down_exps4, sh_gate4, sh_up4, sh_down4;
    int32_t mrope_section[4];
    const int32_t* positions;
} mtp_layer;

const char* mtp_status_string(mtp_status s);
const char* mtp_last_error(void);
const char* mtp_version(void);

/* ---------------------------------------------------------------------- */
/* Workspace sizes (bytes; 0 when the call needs none)                     */
/* ---------------------------------------------------------------------- */
size_t mtp_attn_decode_workspace_size(const mtp_layer* L, int32_t cache_len, int32_t m);
size_t mtp_ffn_dense_workspace_size(int32_t ffn_inter, int32_t m);
size_t mtp_ffn_moe_workspace_size(int32_t hidden, int32_t n_experts, int32_t top_k, int32_t inter,
                                  int32_t shared_inter, int32_t m);
size_t mtp_lmhead_workspace_size(int32_t vocab, int32_t m);
size_t mtp_draft_step_workspace_size(const mtp_layer* L, int32_t cache_len, int32_t m);

/* ---------------------------------------------------------------------- */
/* Test exports: dequantize through the same device routine the GEMVs use  */
/* ---------------------------------------------------------------------- */
/* out f32 [n][k] = scale*code + bias, rounded once to f32 ([shared.rs]
 * `MlxAffineExtra`). */
mtp_status mtp_dequant_q4(const mtp_q4* w, float* out, void* stream);
/* out f32 [n][k] = scale*code of matrix `expert` of the stack. */
mtp_status mtp_dequant_q8(const mtp_q8* w, int32_t expert, float* out, void* stream);
/* out f32 [n][k] = scale*code + bias of matrix `expert` of a 4-bit stack with
 * bf16 constants ([shared.rs] `MlxAffineMoeStack`), rounded once. */
mtp_status mtp_dequant_q4e(const mtp_q4e* w, int32_t expert, float* out, void* stream);

/* ---------------------------------------------------------------------- */
/* Hot-path calls                                                          */
/* ---------------------------------------------------------------------- */

/* y[m][w->n] = x[m][w->k] * W^T (+ residual[m][w->n] when not NULL): the
 * quantized linear of [shared.rs] `dispatch_qmatmul` (affine route) and
 * [mtp.rs] `apply_linear_projection_f32_with_ggml_type`.  y may alias
 * residual. */
mtp_status mtp_qgemv(const mtp_q4* w, const float* x, const float* residual, float* y, int32_t m,
                     void* stream);

/* The 8-bit counterpart of mtp_qgemv on matrix `expert` of a stack. */
mtp_status mtp_q8gemv(const mtp_q8* w, int32_t expert, const float* x, const float* residual, float* y,
                      int32_t m, void* stream);

/* u[m][H] = eh_proj * [rms(e; gamma_e) ; rms(h; gamma_h)] with the embedding
 * half first ([mtp.rs] `project_embedding_and_hidden`; [mimo.rs] module doc).
 * e, h [m][H]; eh_proj n = H, k = 2H.  The concatenation is never stored. */
mtp_status mtp_norm_concat_proj(const float* e, const float* h, const float* gamma_e, const float* gamma_h,
                                float eps, const mtp_q4* eh_proj, float* u, int32_t m, void* stream);

/* Attention block with its residual ([mtp.rs] `forward_full_attention`):
 *   xa = rms(u; gamma_attn); q = Wq xa, k = Wk xa, v = Wv xa;
 *   RoPE (half-split pairs, theta^(-2i/d)) on q and k at positions
 *   cache_len + r; the m new k (post-RoPE) and v rows are written to cache
 *   rows cache_len .. cache_len+m-1; causal GQA attention (query head h reads
 *   KV head h / (n_heads/n_kv_heads), scale 1/sqrt(head_dim)) over rows
 *   0 .. cache_len + r; out = u + Wo * attn.
 * k_cache f32 [n_kv_heads][capacity][head_dim], v_cache f32
 * [n_kv_heads][capacity][dv].  Requires cache_len + m <= capacity, and head_dim
 * 128 (dv 128) or 192 (dv 128). Uses only L's attention
 * fields. out [m][hidden] must not alias u. */
mtp_status mtp_attn_decode(const mtp_layer* L, const float* u, float* k_cache, float* v_cache,
                           int32_t cache_len, int32_t capacity, int32_t m, float* out, void* ws,
                           size_t ws_bytes, void* stream);

/* Dense SwiGLU with 4-bit weights ([mtp.rs] `forward_ffn_residual`, DenseQ):
 *   f = gamma ? rms(x; gamma) : x;  y = [residual +] down*(silu(gate f).(up f)).
 * x, residual, y [m][H]; y may alias residual but not x. */
mtp_status mtp_ffn_dense_q(const float* x, const float* gamma, float eps, const mtp_q4* gate,
                           const mtp_q4* up, const mtp_q4* down, const float* residual, float* y,
                           int32_t m, void* ws, size_t ws_bytes, void* stream);

/* Routed mixture of 8-bit SwiGLU experts plus an optional shared expert
 * ([mtp.rs] `MtpFfnWeightsGpu::Moe`).  Per row: f = gamma ? rms(x) : x;
 * router logits l = router f (router f32 [n_experts][H]); p = softmax(l);
 * the top_k experts by (p descending, index ascending); gates p_e / sum of
 * the selected p; y = [residual] + sum_e gate_e * expert_e(f) + shared(f).
 * expert_ids int32 [m][top_k] and gates f32 [m][top_k] (selection order) are
 * optional outputs.  sh_gate/sh_up/sh_down are all NULL or all set. */
mtp_status mtp_ffn_moe_q(const float* x, const float* gamma, float eps, const float* router, int32_t top_k,
                         const mtp_q8* gate_exps, const mtp_q8* up_exps, const mtp_q8* down_exps,
                         const mtp_q8* sh_gate, const mtp_q8* sh_up, const mtp_q8* sh_down,
                         const float* residual, float* y, int32_t* expert_ids, float* gates, int32_t m,
                         void* ws, size_t ws_bytes, void* stream);

/* The same routed mixture over 4-bit experts with bf16 group constants
 * ([shared.rs] `MlxAffineMoeStack`, consumed by the MoE-id path), the shared
 * expert in the same form.  Arguments as mtp_ffn_moe_q; the workspace is
 * mtp_ffn_moe_workspace_size's.  Built shapes (MTP_ERR_UNSUPPORTED
 * otherwise): hidden/32 and inter/32 each 2, 8, 16 or 64 groups, and a shared
 * expert of the routed experts' intermediate size. */
mtp_status mtp_ffn_moe_q4(const float* x, const float* gamma, float eps, const float* router, int32_t top_k,
                          const mtp_q4e* gate_exps, const mtp_q4e* up_exps, const mtp_q4e* down_exps,
                          const mtp_q4e* sh_gate, const mtp_q4e* sh_up, const mtp_q4e* sh_down,
                          const float* residual, float* y, int32_t* expert_ids, float* gates, int32_t m,
                          void* ws, size_t ws_bytes, void* stream);

/* Shared head with a greedy pick ([mtp.rs] `forward_shared_head_greedy`):
 *   yn = rms(hidden; gamma); logits = lm_head yn; ids[r] = argmax_v logits[r][v]
 * (ties to the lowest index).  normed_out [m][H] and logits_out [m][V] are
 * optional (NULL skips them); ids_out int32 [m] is required.  The fused
 * cross-block argmax keeps its state in the reserved first 1152 bytes of ws
 * (zero on entry; see the workspace convention above). */
mtp_status mtp_lmhead_argmax(const float* hidden, const float* gamma, float eps, const mtp_q4* lm_head,
                             float* normed_out, float* logits_out, int32_t* ids_out, int32_t m, void* ws,
                             size_t ws_bytes, void* stream);

/* The same over an 8-bit block lm_head (one matrix, n_experts = 1):
 * [mimo.rs] `mimo_verify_head_rows`, the verify rows' final norm and one head
 * panel over the q8 lm_head, here with the greedy pick fused.  Same
 * arguments, workspace (mtp_lmhead_workspace_size) and argmax-state rule as
 * mtp_lmhead_argmax. */
mtp_status mtp_lmhead_argmax_q8(const float* hidden, const float* gamma, float eps, const mtp_q8* lm_head,
                                float* normed_out, float* logits_out, int32_t* ids_out, int32_t m, void* ws,
                                size_t ws_bytes, void* stream);

/* One draft-layer forward over m rows at positions cache_len .. cache_len+m-1
 * ([mimo.rs] "The draft forward" and `mimo_mtp_block_with_probe`; [mtp.rs]
 * `forward_draft_body` and `forward_shared_head_greedy`):
 *   u  = eh_proj [rms(e_r; gamma_e) ; rms(h_r; gamma_h)]
 *   r1 = u + attention(rms(u; gamma_attn))   (appends K/V rows)
 *   r2 = r1 + ffn(rms(r1; gamma_post))        (dense 4-bit or MoE 8-bit)
 *   hidden_out = rms(r2; gamma_final), logits = lm_head hidden_out,
 *   ids_out = argmax.
 * Row r's embedding e_r is embed_table[tokens[r]] when tokens is not NULL and
 * tokens[r] >= 0 (device int32 [m]; embed_table f32 [vocab][H]), else row r
 * of e [m][H].  Token ids are read on the device, where the host cannot check
 * them: an id >= vocab is clamped to vocab-1 (the call rejects vocab < 1 when
 * tokens are given).  hidden_out [m][H] is the post-final-norm row, the input of a
 * chained next step ([mtp.rs] `forward_draft_with_hidden`); logits_out
 * [m][vocab] is optional.  The call never advances any cursor: the caller
 * owns cache_len and rolls back by passing a smaller one. */
mtp_status mtp_draft_step(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                          const float* h, float* k_cache, float* v_cache, int32_t cache_len,
                          int32_t capacity, int32_t m, int32_t* ids_out, float* hidden_out,
                          float* logits_out, void* ws, size_t ws_bytes, void* stream);

/* mtp_draft_step without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that keep
 * their memory fixed, harnesses that forbid hipMalloc).  Arguments and
 * results are those of mtp_draft_step minus ws / ws_bytes; the step's
 * scratch space is instead a static device array of the library,
 * MTP_NOALLOC_SCRATCH_BYTES on each GPU, whose device address is looked up
 * on the call's first use of a device.  The call allocates and frees
 * nothing.
 * - A step that needs more scratch than that
 *   (mtp_draft_step_workspace_size(L, cache_len, m) > MTP_NOALLOC_SCRATCH_BYTES)
 *   is rejected with MTP_ERR_WORKSPACE before anything is enqueued.
 * - The stream must belong to the current device (MTP_ERR_INVALID_ARG
 *   otherwise).
 * - Every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents (the step clears what must start at zero itself): calls
 *   that may overlap on one GPU (on different streams, or from several
 *   threads without ordering) race and give wrong results.  Order them on one
 *   stream, or use mtp_draft_step with a workspace per stream. */
mtp_status mtp_draft_step_noalloc(const mtp_layer* L, const float* e, const int32_t* tokens,
                                  const float* embed_table, const float* h, float* k_cache, float* v_cache,
                                  int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out,
                                  float* hidden_out, float* logits_out, void* stream);

/* Cache catch-up after a target batch ([mtp.rs] `process_target_batch` and
 * `append_attention_kv`): for rows r = 0 .. m-1 at positions cache_len + r,
 *   shifted_r = pending_h (zero when NULL) for r = 0, target_h row r-1 after;
 *   u_r = eh_proj [rms(e_r; gamma_e) ; rms(shifted_r; gamma_h)]
 * (e_r as in mtp_draft_step: embed_table[tokens[r]] or row r of e), and only
 * the attention's K/V side runs on u_r: rms(u_r; gamma_attn), the wk and wv
 * projections, the per-head k norm when set, the rotary step; the K and V
 * rows are written at cache_len + r.  No attention, FFN or logits.
 * target_h [m][H] is the target model's post-output-norm hidden of the same
 * m tokens; pending_h [H] the one left over from the previous batch.  m may
 * exceed MTP_MAX_ROWS (the call works in pieces of MTP_MAX_ROWS rows, so a
 * whole prompt can be caught up in one call); cache_len + m <= capacity.
 * ws needs mtp_append_kv_workspace_size(L) bytes. */
size_t mtp_append_kv_workspace_size(const mtp_layer* L);
mtp_status mtp_append_kv(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                         const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                         int32_t cache_len, int32_t capacity, int32_t m, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Multi-layer draft stack ([mimo.rs] module doc "How the three layers     */
/* chain"; `mimo_mtp_draft`)                                               */
/* ---------------------------------------------------------------------- */
/* One layer of the stack: its weights, its own K/V cache (row j holds
 * position j) and the first row this round recomputes (rows before it are
 * final from earlier rounds). */
typedef struct {
    const mtp_layer* layer;
    float* k_cache;
    float* v_cache;
    int32_t capacity;
    int32_t start;
} mtp_stack_layer;

/* Drafts n_layers tokens for the round that starts after the target
 * processed position t (token x_{t+1} pending).  Layer k drafts the token for
 * position t + k + 2: its rows j = start .. t pair the token x_{j+k+1} with
 * the target's hidden h_j (every layer reads the target's rows, never another
 * layer's output) at position j of its own cache, and its draft is the greedy
 * pick of row t.  Tokens past x_{t+1} are this round's earlier drafts.
 * tokens: device int32 [t + 2 + n_layers]: x_0 .. x_{t+1} on entry; the call
 * writes draft k at tokens[t + 2 + k].  target_h: device f32 [t + 1][H],
 * h_0 .. h_t.  Rows start .. t-1 go through the cache catch-up path (no
 * logits), row t through mtp_draft_step.  All layers share hidden and vocab.
 * Every layer's calls are checked before the first launch, so an error in
 * any layer leaves every cache and the token buffer untouched.
 * ws needs mtp_stack_draft_workspace_size(layers, n_layers, t) bytes. */
size_t mtp_stack_draft_workspace_size(const mtp_stack_layer* layers, int32_t n_layers, int32_t t);
mtp_status mtp_stack_draft(const mtp_stack_layer* layers, int32_t n_layers, int32_t* tokens, const float* embed_table,
                           const float* target_h, int32_t t, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Speculative round bookkeeping (host only; [mimo.rs] `mimo_spec_round`)  */
/* ---------------------------------------------------------------------- */
#define MTP_MAX_DRAFT 16
typedef struct {
    uint64_t rounds, drafted, accepted;
    uint64_t accept_hist[MTP_MAX_DRAFT + 1];  /* rounds that accepted exactly a drafts */
    uint64_t depth_drafted[MTP_MAX_DRAFT];    /* rounds that drafted at depth d */
    uint64_t depth_accepted[MTP_MAX_DRAFT];   /* rounds whose draft at depth d was accepted */
} mtp_stats;

/* The verify step's greedy acceptance: drafts[0..k-1] are the round's drafts,
 * target_ids[0..k] the target's greedy tokens after [pending, drafts[0..i-1]]
 * (host int32 arrays).  Returns a, the number of leading drafts equal to the
 * target's tokens (0..k); target_ids[a] is the round's bonus token, the
 * target's KV keeps a + 1 new rows and the draft layer's cache is caught up
 * over them with mtp_append_kv.  When stats is not NULL the round is added
 * to it.  Returns -1 (and records nothing) for k outside 1..MTP_MAX_DRAFT
 * or a NULL array. */
int32_t mtp_accept(const int32_t* drafts, const int32_t* target_ids, int32_t k, mtp_stats* stats);

#ifdef __cplusplus
}
#endif
#endif /* MTP_H */
