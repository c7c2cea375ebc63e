// api.cpp -- the C ABI of libmtp (declared in include/mtp.h): argument checks,
// workspace carving and the launch sequence of each call.  Every check runs
// before the first enqueue, so a rejected call has no effect on the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <string>

#include "../../include/mtp.h"
#include "api_internal.hpp"
#include "launch.hpp"

using namespace mtp;

namespace {
thread_local std::string g_err;
}  // namespace

namespace mtp {

mtp_status fail(mtp_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

mtp_status hip_fail(hipError_t e, const char* what) {
    return fail(MTP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace mtp

namespace {

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool a4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }


mtp_status check_rows(int32_t m) {
    if (m < 1 || m > MTP_MAX_ROWS) return fail(MTP_ERR_INVALID_ARG, "m=%d outside 1..%d", m, MTP_MAX_ROWS);
    return MTP_OK;
}

mtp_status check_q4(const mtp_q4* w, const char* name) {
    if (!w) return fail(MTP_ERR_INVALID_ARG, "%s: descriptor is NULL", name);
    if (!w->codes || !w->scales || !w->biases) return fail(MTP_ERR_INVALID_ARG, "%s: NULL codes/scales/biases", name);
    if (w->n < 1) return fail(MTP_ERR_INVALID_ARG, "%s: n=%d must be >= 1", name, w->n);
    if (w->k < MTP_GROUP || w->k % MTP_GROUP) return fail(MTP_ERR_INVALID_ARG, "%s: k=%d must be a positive multiple of 32", name, w->k);
    if (w->k > MTP_MAX_K) return fail(MTP_ERR_UNSUPPORTED, "%s: k=%d above %d", name, w->k, MTP_MAX_K);
    if (!a16(w->codes) || !a4(w->scales) || !a4(w->biases)) return fail(MTP_ERR_INVALID_ARG, "%s: misaligned pointer", name);
    return MTP_OK;
}

mtp_status check_q8(const mtp_q8* w, const char* name) {
    if (!w) return fail(MTP_ERR_INVALID_ARG, "%s: descriptor is NULL", name);
    if (!w->codes || !w->scales) return fail(MTP_ERR_INVALID_ARG, "%s: NULL codes/scales", name);
    if (w->n < 1 || w->n_experts < 1) return fail(MTP_ERR_INVALID_ARG, "%s: n=%d n_experts=%d", name, w->n, w->n_experts);
    if (w->k < MTP_GROUP || w->k % MTP_GROUP) return fail(MTP_ERR_INVALID_ARG, "%s: k=%d must be a positive multiple of 32", name, w->k);
    if (w->k > MTP_MAX_K) return fail(MTP_ERR_UNSUPPORTED, "%s: k=%d above %d", name, w->k, MTP_MAX_K);
    if (!a16(w->codes) || !a4(w->scales)) return fail(MTP_ERR_INVALID_ARG, "%s: misaligned pointer", name);
    return MTP_OK;
}

mtp_status check_vec(const void* p, const char* name) {
    if (!p) return fail(MTP_ERR_INVALID_ARG, "%s is NULL", name);
    if (!a16(p)) return fail(MTP_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return MTP_OK;
}

// An expert stack of either format as the MoE code takes it: 8-bit block
// (f32 scales) or 4-bit with bf16 scales and biases (q4).
struct ExpMat {
    const void* codes;
    const void* scales;
    const void* biases;
    int n, k, n_experts, q4;
};
ExpMat emat(const mtp_q8& w) { return ExpMat{w.codes, w.scales, nullptr, w.n, w.k, w.n_experts, 0}; }
ExpMat emat(const mtp_q4e& w) { return ExpMat{w.codes, w.scales, w.biases, w.n, w.k, w.n_experts, 1}; }

bool a2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

mtp_status check_emat(const ExpMat* w, const char* name) {
    if (!w) return fail(MTP_ERR_INVALID_ARG, "%s: descriptor is NULL", name);
    if (!w->codes || !w->scales || (w->q4 && !w->biases))
        return fail(MTP_ERR_INVALID_ARG, "%s: NULL codes/scales%s", name, w->q4 ? "/biases" : "");
    if (w->n < 1 || w->n_experts < 1) return fail(MTP_ERR_INVALID_ARG, "%s: n=%d n_experts=%d", name, w->n, w->n_experts);
    if (w->k < MTP_GROUP || w->k % MTP_GROUP) return fail(MTP_ERR_INVALID_ARG, "%s: k=%d must be a positive multiple of 32", name, w->k);
    if (w->k > MTP_MAX_K) return fail(MTP_ERR_UNSUPPORTED, "%s: k=%d above %d", name, w->k, MTP_MAX_K);
    if (!a16(w->codes) || !(w->q4 ? a2(w->scales) && a2(w->biases) : a4(w->scales)))
        return fail(MTP_ERR_INVALID_ARG, "%s: misaligned pointer", name);
    return MTP_OK;
}

QMat qmat(const mtp_q4& w) { return QMat{w.codes, w.scales, w.biases, w.n}; }
QMat qmat8(const mtp_q8& w, int expert) {
    const int64_t gpr = w.k / MTP_GROUP;
    return QMat{static_cast<const int8_t*>(w.codes) + (int64_t)expert * w.n * w.k,
                w.scales + (int64_t)expert * w.n * gpr, nullptr, w.n};
}

constexpr size_t kHeadStateBytesZ = (size_t)kHeadStateBytes;

// Bump allocator over the caller's workspace (256-byte aligned pieces).  With
// base == nullptr it only measures.  The first kHeadStateBytes of every
// workspace are reserved for the fused argmax state of the lm_head (see
// carve_head): no other buffer is carved there, so a workspace shared by any
// sequence of calls keeps those bytes at zero between calls.
struct Carve {
    char* base;
    size_t off = kHeadStateBytesZ;
    template <class T>
    T* take(size_t count) {
        off = (off + 255) & ~size_t(255);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

int chunks_for(int32_t cache_len, int32_t m) { return (cache_len + m + kAttnChunk - 1) / kAttnChunk; }

// ---- per-call workspace layouts ----
struct AttnWs {
    float *qkv, *part, *o;
};
int v_dim(const mtp_layer* L) { return L->v_head_dim > 0 ? L->v_head_dim : L->head_dim; }

AttnWs carve_attn(Carve& c, const mtp_layer* L, int32_t cache_len, int32_t m) {
    AttnWs w;
    const int d = L->head_dim, dv = v_dim(L), nh = L->n_heads, nkv = L->n_kv_heads;
    w.qkv = c.take<float>((size_t)m * (nh * (L->q_gated ? d + dv : d) + nkv * (d + dv)));
    w.part = c.take<float>((size_t)chunks_for(cache_len, m) * nkv * (nh / (nkv ? nkv : 1)) * m * (dv + 2));
    w.o = c.take<float>((size_t)m * nh * dv);
    return w;
}

// State of the fused lm_head argmax, the reserved start of the workspace:
// MTP_MAX_ROWS 64-bit keys on their own 128-byte lines, then the arrival
// counter on one more line.  Every head launch leaves it zero, and the draft
// step also clears it in its first kernel.
struct HeadWs {
    unsigned long long* keys;
    unsigned* counter;
};
static_assert(kHeadRows == MTP_MAX_ROWS, "argmax state sized for the ABI's row limit");
constexpr int kHeadStateWords = kHeadStateBytes / 4;
HeadWs carve_head(Carve& c, int32_t m) {
    (void)m;
    HeadWs w;
    w.keys = reinterpret_cast<unsigned long long*>(c.base);
    w.counter = reinterpret_cast<unsigned*>(w.keys + kHeadRows * kKeyStride);
    return w;
}

struct MoeWs {
    float *f, *logits, *gates, *slot_gate, *z, *ypart;
    int *ids, *slot_expert, *n_slots;
    int max_slots;
};
MoeWs carve_moe(Carve& c, int H, int E, int top_k, int inter, int sh_inter, int m) {
    MoeWs w;
    const int routed = (m * top_k < E) ? m * top_k : E;
    w.max_slots = routed + (sh_inter > 0 ? 1 : 0);
    const int imax = inter > sh_inter ? inter : sh_inter;
    w.f = c.take<float>((size_t)m * H);
    w.logits = c.take<float>((size_t)m * E);
    w.ids = c.take<int>((size_t)m * top_k);
    w.gates = c.take<float>((size_t)m * top_k);
    w.slot_expert = c.take<int>((size_t)w.max_slots);
    w.slot_gate = c.take<float>((size_t)w.max_slots * m);
    w.n_slots = c.take<int>(1);
    w.z = c.take<float>((size_t)w.max_slots * m * imax);
    w.ypart = c.take<float>((size_t)w.max_slots * m * H);
    return w;
}

mtp_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MTP_OK;
    if (!ws) return fail(MTP_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (ws_bytes < need) return fail(MTP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MTP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return MTP_OK;
}

// ---- shared launch helpers ----
hipError_t run_gemv(int fmt, int pro, int epi, int m, GemvParams& p, int max_blocks, hipStream_t st) {
    p.m = m;
    p.G = p.K / MTP_GROUP;
    p.S = (p.G + 63) / 64;
    return launch_gemv(fmt, pro, epi, m, p, max_blocks, st);
}

int default_blocks() { return 4 * device_cu_count(); }

hipError_t run_head_fmt(int fmt, const QMat& lm, int k, const float* hidden, const float* gamma, float eps,
                        float* normed_out, float* logits_out, int* ids, int m, const HeadWs& w, hipStream_t st) {
    GemvParams p{};
    p.w[0] = lm;
    p.nmat = 1;
    p.N = lm.n;
    p.K = k;
    p.x0 = hidden;
    p.g0 = gamma;
    p.eps = eps;
    p.normed_out = normed_out;
    p.logits = logits_out;
    p.head_keys = w.keys;
    p.counter = w.counter;
    p.ids = ids;
    p.m = m;
    p.G = p.K / MTP_GROUP;
    p.S = (p.G + 63) / 64;
    // persistent: a compute unit's worth of waves per block, its waves sharing
    // the block's rows at run time
    p.balance = 1;
    return launch_gemv(fmt, PRO_RMS, EPI_ARGMAX, m, p, 0, st);
}

hipError_t run_head(const float* hidden, const float* gamma, float eps, const mtp_q4& lm, float* normed_out,
                    float* logits_out, int* ids, int m, const HeadWs& w, hipStream_t st) {
    return run_head_fmt(FMT_Q4, qmat(lm), lm.k, hidden, gamma, eps, normed_out, logits_out, ids, m, w, st);
}

// The rotary position ids of rows row0 .. of a call (NULL: the cache rows).
void set_positions(AttnParams& a, const mtp_layer* L, int row0) {
    a.positions = L->positions ? L->positions + 4 * (int64_t)row0 : nullptr;
    for (int k = 0; k < 4; ++k) a.sec[k] = L->mrope_section[k];
}

hipError_t run_attention(const mtp_layer* L, const float* u, float* kc, float* vc, int cache_len, int capacity,
                         int m, float* out, const AttnWs& w, hipStream_t st) {
    GemvParams p{};
    p.w[0] = qmat(L->wq);
    p.w[1] = qmat(L->wk);
    p.w[2] = qmat(L->wv);
    p.nmat = 3;
    p.N = L->wq.n + L->wk.n + L->wv.n;
    p.K = L->hidden;
    p.x0 = u;
    p.g0 = L->gamma_attn;
    p.eps = L->eps;
    p.y = w.qkv;
    hipError_t e = run_gemv(FMT_Q4, PRO_RMS, EPI_STORE, m, p, default_blocks(), st);
    if (e != hipSuccess) return e;
    AttnParams a{};
    a.qkv = w.qkv;
    a.k_cache = kc;
    a.v_cache = vc;
    a.cache_len = cache_len;
    a.capacity = capacity;
    a.m = m;
    a.nh = L->n_heads;
    a.nkv = L->n_kv_heads;
    a.d = L->head_dim;
    a.vd = v_dim(L);
    a.log2_theta = log2(L->rope_theta);
    a.part = w.part;
    a.o = w.o;
    a.chunks = chunks_for(cache_len, m);
    a.qg = L->q_gated ? 2 : 1;
    a.gq = L->gamma_q_head;
    a.gk = L->gamma_k_head;
    a.eps = L->eps;
    a.rot = L->rotary_dim > 0 ? L->rotary_dim : L->head_dim;
    a.window = L->window;
    a.sinks = L->sinks;
    // the first row (position cache_len) sees nothing before cache_len - W + 1
    a.c0 = (L->window > 0 && cache_len - L->window + 1 > 0) ? (cache_len - L->window + 1) / kAttnChunk : 0;
    set_positions(a, L, 0);
    if ((e = launch_attention(a, st)) != hipSuccess) return e;
    GemvParams o{};
    o.w[0] = qmat(L->wo);
    o.nmat = 1;
    o.N = L->wo.n;
    o.K = L->wo.k;
    o.x0 = w.o;
    o.residual = u;
    o.y = out;
    return run_gemv(FMT_Q4, PRO_PLAIN, EPI_STORE, m, o, default_blocks(), st);
}

hipError_t run_ffn_dense(const float* x, const float* gamma, float eps, const mtp_q4& gate, const mtp_q4& up,
                         const mtp_q4& down, const float* residual, float* y, int m, float* z, hipStream_t st) {
    GemvParams g{};
    g.w[0] = qmat(gate);
    g.w[1] = qmat(up);
    g.nmat = 2;
    g.N = gate.n;
    g.K = gate.k;
    g.x0 = x;
    g.g0 = gamma;
    g.eps = eps;
    g.y = z;
    hipError_t e = run_gemv(FMT_Q4, gamma ? PRO_RMS : PRO_PLAIN, EPI_SWIGLU, m, g, default_blocks(), st);
    if (e != hipSuccess) return e;
    GemvParams d{};
    d.w[0] = qmat(down);
    d.nmat = 1;
    d.N = down.n;
    d.K = down.k;
    d.x0 = z;
    d.residual = residual;
    d.y = y;
    return run_gemv(FMT_Q4, PRO_PLAIN, EPI_STORE, m, d, default_blocks(), st);
}

// The first matrix of an expert stack as the MoE launch takes it (for 4-bit
// stacks the QMat's scale and bias fields carry the bf16 arrays).
QMat qmat_e(const ExpMat& w) {
    return QMat{w.codes, static_cast<const float*>(w.scales), static_cast<const float*>(w.biases), w.n};
}

hipError_t run_moe(const float* x, const float* gamma, float eps, const float* router, int top_k, const ExpMat& ge,
                   const ExpMat& ue, const ExpMat& de, const ExpMat* sg, const ExpMat* su, const ExpMat* sd,
                   const float* residual, float* y, int* ids_out, float* gates_out, int m, const MoeWs& w,
                   hipStream_t st) {
    MoeParams p{};
    p.x = x;
    p.gamma = gamma;
    p.eps = eps;
    p.f = w.f;
    p.router = router;
    p.logits = w.logits;
    p.E = ge.n_experts;
    p.H = ge.k;
    p.top_k = top_k;
    p.m = m;
    p.expert_ids = ids_out ? ids_out : w.ids;
    p.gates = gates_out ? gates_out : w.gates;
    p.slot_expert = w.slot_expert;
    p.slot_gate = w.slot_gate;
    p.n_slots = w.n_slots;
    p.max_slots = w.max_slots;
    p.ge = qmat_e(ge);
    p.ue = qmat_e(ue);
    p.de = qmat_e(de);
    if (sg) {
        p.sg = qmat_e(*sg);
        p.su = qmat_e(*su);
        p.sd = qmat_e(*sd);
        p.sh_inter = sg->n;
    }
    p.q4 = ge.q4;
    p.inter = ge.n;
    p.z = w.z;
    p.ypart = w.ypart;
    p.residual = residual;
    p.y = y;
    return launch_moe(p, st);
}

mtp_status check_layer_attn(const mtp_layer* L) {
    if (!L) return fail(MTP_ERR_INVALID_ARG, "layer is NULL");
    const int H = L->hidden;
    if (H < MTP_GROUP || H % MTP_GROUP || H > MTP_MAX_K) return fail(MTP_ERR_INVALID_ARG, "hidden=%d", H);
    if (L->head_dim != 128 && L->head_dim != 192)
        return fail(MTP_ERR_UNSUPPORTED, "head_dim=%d (128, or 192 with v_head_dim 128)", L->head_dim);
    if (L->v_head_dim < 0) return fail(MTP_ERR_INVALID_ARG, "v_head_dim=%d", L->v_head_dim);
    const int dv = v_dim(L);
    if (dv != 128)
        return fail(MTP_ERR_UNSUPPORTED, "v_head_dim=%d (V heads of 128 are built)", L->v_head_dim);
    if (L->head_dim != 128 && (L->q_gated || L->gamma_q_head || L->gamma_k_head))
        return fail(MTP_ERR_UNSUPPORTED, "head_dim=%d: no gated q or per-head norms", L->head_dim);
    if (L->n_heads < 1 || L->n_kv_heads < 1 || L->n_heads % L->n_kv_heads)
        return fail(MTP_ERR_INVALID_ARG, "n_heads=%d n_kv_heads=%d", L->n_heads, L->n_kv_heads);
    if (!(L->eps >= 0.0f)) return fail(MTP_ERR_INVALID_ARG, "eps must be >= 0");
    if (!(L->rope_theta > 0.0)) return fail(MTP_ERR_INVALID_ARG, "rope_theta must be > 0");
    mtp_status s;
    if ((s = check_vec(L->gamma_attn, "gamma_attn")) != MTP_OK) return s;
    if ((s = check_q4(&L->wq, "wq")) || (s = check_q4(&L->wk, "wk")) || (s = check_q4(&L->wv, "wv")) ||
        (s = check_q4(&L->wo, "wo")))
        return s;
    const int qn = L->n_heads * L->head_dim, kvn = L->n_kv_heads * L->head_dim;
    const int on = L->n_heads * dv, vn = L->n_kv_heads * dv;
    if (L->q_gated != 0 && L->q_gated != 1) return fail(MTP_ERR_INVALID_ARG, "q_gated=%d (0 or 1)", L->q_gated);
    if (L->wq.n != qn + (L->q_gated ? on : 0) || L->wq.k != H || L->wk.n != kvn || L->wk.k != H || L->wv.n != vn ||
        L->wv.k != H || L->wo.n != H || L->wo.k != on)
        return fail(MTP_ERR_INVALID_ARG, "attention weight shapes do not match hidden/heads/head_dim");
    if ((L->gamma_q_head == nullptr) != (L->gamma_k_head == nullptr))
        return fail(MTP_ERR_INVALID_ARG, "gamma_q_head and gamma_k_head: give both or neither");
    if (L->gamma_q_head && (!a16(L->gamma_q_head) || !a16(L->gamma_k_head)))
        return fail(MTP_ERR_INVALID_ARG, "gamma_q_head/gamma_k_head must be 16-byte aligned");
    const int rot = L->rotary_dim;
    if (rot != 0 && (rot < 2 || rot > L->head_dim || (rot & (rot - 1)) != 0))
        return fail(MTP_ERR_UNSUPPORTED, "rotary_dim=%d (0 or a power of two <= head_dim)", rot);
    if (on > MTP_MAX_K) return fail(MTP_ERR_UNSUPPORTED, "n_heads*v_head_dim=%d above %d", on, MTP_MAX_K);
    if (L->window < 0) return fail(MTP_ERR_INVALID_ARG, "window=%d (0 or positive)", L->window);
    if (L->sinks && !a4(L->sinks))
        return fail(MTP_ERR_INVALID_ARG, "sinks must be 4-byte aligned");
    for (int k = 0; k < 4; ++k)
        if (L->mrope_section[k] < 0) return fail(MTP_ERR_INVALID_ARG, "mrope_section[%d]=%d", k, L->mrope_section[k]);
    if (L->positions) {
        if (!a4(L->positions)) return fail(MTP_ERR_INVALID_ARG, "positions must be 4-byte aligned");
        if (L->head_dim != 128)
            return fail(MTP_ERR_UNSUPPORTED, "positions (multi-section rotary) with head_dim=%d (128 is built)",
                        L->head_dim);
    }
    return MTP_OK;
}


mtp_status check_cache(const float* kc, const float* vc, int32_t cache_len, int32_t capacity, int32_t m,
                       const mtp_layer* L) {
    if (!kc || !vc) return fail(MTP_ERR_INVALID_ARG, "k_cache/v_cache is NULL");
    if (!a16(kc) || !a16(vc)) return fail(MTP_ERR_INVALID_ARG, "caches must be 16-byte aligned");
    if (kc == vc) return fail(MTP_ERR_INVALID_ARG, "k_cache and v_cache alias");
    if (cache_len < 0 || capacity < 1) return fail(MTP_ERR_INVALID_ARG, "cache_len=%d capacity=%d", cache_len, capacity);
    if ((int64_t)cache_len + m > capacity)
        return fail(MTP_ERR_INVALID_ARG, "cache overflow: cache_len %d + m %d > capacity %d", cache_len, m, capacity);
    if ((L->n_heads / L->n_kv_heads) * m > 64)
        return fail(MTP_ERR_UNSUPPORTED, "(n_heads/n_kv_heads)*m=%d above 64", (L->n_heads / L->n_kv_heads) * m);
    return MTP_OK;
}

// The slot kernel's feature counts: 2, 8, 16 or 64 groups of 32.
bool slot_groups(int k) { return k == 64 || k == 256 || k == 512 || k == 2048; }

mtp_status check_moe_weights(const float* router, int top_k, const ExpMat* ge, const ExpMat* ue, const ExpMat* de,
                             const ExpMat* sg, const ExpMat* su, const ExpMat* sd, int H) {
    mtp_status s;
    if ((s = check_emat(ge, "gate_exps")) || (s = check_emat(ue, "up_exps")) || (s = check_emat(de, "down_exps")))
        return s;
    if (ue->q4 != ge->q4 || de->q4 != ge->q4) return fail(MTP_ERR_INVALID_ARG, "expert stacks differ in format");
    if (!router || !a4(router)) return fail(MTP_ERR_INVALID_ARG, "router is NULL or misaligned");
    const int E = ge->n_experts, I = ge->n;
    if (ue->n_experts != E || de->n_experts != E) return fail(MTP_ERR_INVALID_ARG, "expert stacks differ in n_experts");
    if (E > 1024) return fail(MTP_ERR_UNSUPPORTED, "n_experts=%d above 1024", E);
    if (top_k < 1 || top_k > E || top_k > 64) return fail(MTP_ERR_INVALID_ARG, "top_k=%d (1..min(n_experts, 64))", top_k);
    if (ge->k != H || ue->k != H || ue->n != I || de->n != H || de->k != I)
        return fail(MTP_ERR_INVALID_ARG, "expert shapes: gate/up [E][I][H], down [E][H][I] expected");
    const bool any = sg || su || sd, all = sg && su && sd;
    if (any && !all) return fail(MTP_ERR_INVALID_ARG, "shared expert: give all of sh_gate/sh_up/sh_down or none");
    if (all) {
        if ((s = check_emat(sg, "sh_gate")) || (s = check_emat(su, "sh_up")) || (s = check_emat(sd, "sh_down"))) return s;
        if (sg->q4 != ge->q4 || su->q4 != ge->q4 || sd->q4 != ge->q4)
            return fail(MTP_ERR_INVALID_ARG, "the shared expert must have the routed experts' format");
        const int Is = sg->n;
        if (sg->k != H || su->k != H || su->n != Is || sd->n != H || sd->k != Is)
            return fail(MTP_ERR_INVALID_ARG, "shared expert shapes do not match");
        if ((I + 2047) / 2048 != (Is + 2047) / 2048)
            return fail(MTP_ERR_UNSUPPORTED, "expert and shared intermediate sizes need the same 2048-wide chunk count");
        if (ge->q4 && Is != I)
            return fail(MTP_ERR_UNSUPPORTED, "4-bit experts: the shared expert needs the routed intermediate size %d (got %d)",
                        I, Is);
    }
    if (ge->q4 && (!slot_groups(H) || !slot_groups(I)))
        return fail(MTP_ERR_UNSUPPORTED, "4-bit experts: hidden %d and intermediate %d must each be 64, 256, 512 or 2048",
                    H, I);
    return MTP_OK;
}

// The expert stacks of a MoE layer (ffn_kind MTP_FFN_MOE_Q8 or _Q4); shared
// ones are left zero (codes NULL) when the layer has none.
struct LayerExperts {
    ExpMat ge, ue, de, sg, su, sd;
    bool shared;
};
LayerExperts layer_experts(const mtp_layer* L) {
    LayerExperts x{};
    if (L->ffn_kind == MTP_FFN_MOE_Q4) {
        x.ge = emat(L->gate_exps4);
        x.ue = emat(L->up_exps4);
        x.de = emat(L->down_exps4);
        x.shared = L->sh_gate4.codes != nullptr;
        if (x.shared) {
            x.sg = emat(L->sh_gate4);
            x.su = emat(L->sh_up4);
            x.sd = emat(L->sh_down4);
        }
    } else {
        x.ge = emat(L->gate_exps);
        x.ue = emat(L->up_exps);
        x.de = emat(L->down_exps);
        x.shared = L->sh_gate.codes != nullptr;
        if (x.shared) {
            x.sg = emat(L->sh_gate);
            x.su = emat(L->sh_up);
            x.sd = emat(L->sh_down);
        }
    }
    return x;
}

// Checks and launches of the draft step and the cache catch-up, apart, so
// that a call made of several of them checks everything before launching
// (the draft step's pair is declared in api_internal.hpp).
mtp_status check_draft_step(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                            const float* h, float* k_cache, float* v_cache, int32_t cache_len, int32_t capacity,
                            int32_t m, int32_t* ids_out, float* hidden_out, float* logits_out, void* ws,
                            size_t ws_bytes);
mtp_status check_append_kv(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                           const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                           int32_t cache_len, int32_t capacity, int32_t m, void* ws, size_t ws_bytes);
mtp_status enqueue_append_kv(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                             const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                             int32_t cache_len, int32_t capacity, int32_t m, void* ws, void* stream);

}  // namespace

extern "C" {

const char* mtp_status_string(mtp_status s) {
    switch (s) {
        case MTP_OK: return "ok";
        case MTP_ERR_INVALID_ARG: return "invalid argument";
        case MTP_ERR_UNSUPPORTED: return "unsupported shape";
        case MTP_ERR_WORKSPACE: return "workspace too small";
        case MTP_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* mtp_last_error(void) { return g_err.c_str(); }

const char* mtp_version(void) { return "libmtp 0.1 gfx950"; }

size_t mtp_attn_decode_workspace_size(const mtp_layer* L, int32_t cache_len, int32_t m) {
    if (!L || m < 1 || cache_len < 0 || L->n_kv_heads < 1) return 0;
    Carve c{nullptr};
    carve_attn(c, L, cache_len, m);
    return c.off;
}

size_t mtp_ffn_dense_workspace_size(int32_t ffn_inter, int32_t m) {
    if (ffn_inter < 1 || m < 1) return 0;
    Carve c{nullptr};
    c.take<float>((size_t)m * ffn_inter);
    return c.off;
}

size_t mtp_ffn_moe_workspace_size(int32_t hidden, int32_t n_experts, int32_t top_k, int32_t inter,
                                  int32_t shared_inter, int32_t m) {
    if (hidden < 1 || n_experts < 1 || top_k < 1 || inter < 1 || m < 1 || shared_inter < 0) return 0;
    Carve c{nullptr};
    carve_moe(c, hidden, n_experts, top_k, inter, shared_inter, m);
    return c.off;
}

size_t mtp_lmhead_workspace_size(int32_t vocab, int32_t m) {
    (void)vocab;
    if (m < 1) return 0;
    Carve c{nullptr};
    carve_head(c, m);
    return c.off;
}

size_t mtp_draft_step_workspace_size(const mtp_layer* L, int32_t cache_len, int32_t m) {
    if (!L || m < 1 || cache_len < 0 || L->n_kv_heads < 1) return 0;
    Carve c{nullptr};
    c.take<float>((size_t)m * L->hidden);  // u
    c.take<float>((size_t)m * L->hidden);  // r1
    c.take<float>((size_t)m * L->hidden);  // r2
    carve_attn(c, L, cache_len, m);
    if (L->ffn_kind == MTP_FFN_MOE_Q8 || L->ffn_kind == MTP_FFN_MOE_Q4) {
        const LayerExperts x = layer_experts(L);
        carve_moe(c, L->hidden, x.ge.n_experts, L->top_k, x.ge.n, x.shared ? x.sg.n : 0, m);
    }
    else
        c.take<float>((size_t)m * L->ffn_inter);
    carve_head(c, m);
    return c.off;
}

size_t mtp_append_kv_workspace_size(const mtp_layer* L) {
    if (!L || L->hidden < 1 || L->n_kv_heads < 1 || L->head_dim < 1) return 0;
    Carve c{nullptr};
    c.take<float>((size_t)MTP_MAX_ROWS * L->hidden);                           // shifted hidden
    c.take<float>((size_t)MTP_MAX_ROWS * L->hidden);                           // u
    c.take<float>((size_t)MTP_MAX_ROWS * L->n_kv_heads * (L->head_dim + v_dim(L)));  // k, v
    return c.off;
}

}  // extern "C"

namespace {

// Every check of mtp_append_kv; launches nothing.
mtp_status check_append_kv(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                           const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                           int32_t cache_len, int32_t capacity, int32_t m, void* ws, size_t ws_bytes) {
    mtp_status s;
    if (m < 1) return fail(MTP_ERR_INVALID_ARG, "m=%d (at least 1)", m);
    if ((s = check_layer_attn(L))) return s;
    const int H = L->hidden;
    if (!k_cache || !v_cache) return fail(MTP_ERR_INVALID_ARG, "k_cache/v_cache is NULL");
    if (!a16(k_cache) || !a16(v_cache)) return fail(MTP_ERR_INVALID_ARG, "caches must be 16-byte aligned");
    if (k_cache == v_cache) return fail(MTP_ERR_INVALID_ARG, "k_cache and v_cache alias");
    if (cache_len < 0 || capacity < 1) return fail(MTP_ERR_INVALID_ARG, "cache_len=%d capacity=%d", cache_len, capacity);
    if ((int64_t)cache_len + m > capacity)
        return fail(MTP_ERR_INVALID_ARG, "cache overflow: cache_len %d + m %d > capacity %d", cache_len, m, capacity);
    if ((s = check_vec(target_h, "target_h")) || (s = check_vec(L->gamma_e, "gamma_e")) ||
        (s = check_vec(L->gamma_h, "gamma_h")) || (s = check_q4(&L->eh_proj, "eh_proj")))
        return s;
    if (pending_h && (s = check_vec(pending_h, "pending_h"))) return s;
    if (L->eh_proj.n != H || L->eh_proj.k != 2 * H) return fail(MTP_ERR_INVALID_ARG, "eh_proj must be [hidden][2*hidden]");
    if (!tokens && !e) return fail(MTP_ERR_INVALID_ARG, "give e or tokens");
    if (e && (s = check_vec(e, "e"))) return s;
    if (tokens && (!a4(tokens) || !embed_table)) return fail(MTP_ERR_INVALID_ARG, "tokens needs an aligned pointer and embed_table");
    if (tokens && L->vocab < 1) return fail(MTP_ERR_INVALID_ARG, "vocab=%d: tokens need a table of at least one row", L->vocab);
    if (embed_table && !a16(embed_table)) return fail(MTP_ERR_INVALID_ARG, "embed_table misaligned");
    return check_ws(ws, ws_bytes, mtp_append_kv_workspace_size(L));
}

// The launches of mtp_append_kv (arguments already checked).
mtp_status enqueue_append_kv(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                             const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                             int32_t cache_len, int32_t capacity, int32_t m, void* ws, void* stream) {
    const int H = L->hidden;
    hipStream_t st = (hipStream_t)stream;
    Carve c{static_cast<char*>(ws)};
    float* shifted = c.take<float>((size_t)MTP_MAX_ROWS * H);
    float* u = c.take<float>((size_t)MTP_MAX_ROWS * H);
    float* kv = c.take<float>((size_t)MTP_MAX_ROWS * L->n_kv_heads * (L->head_dim + v_dim(L)));
    AttnParams a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.capacity = capacity;
    a.nkv = L->n_kv_heads;
    a.d = L->head_dim;
    a.vd = v_dim(L);
    a.log2_theta = log2(L->rope_theta);
    a.gk = L->gamma_k_head;
    a.eps = L->eps;
    a.rot = L->rotary_dim > 0 ? L->rotary_dim : L->head_dim;
    hipError_t err = hipSuccess;
    // pieces of MTP_MAX_ROWS rows; after the first piece the shifted hidden
    // of row c0 + r is the target's row c0 + r - 1, a contiguous run
    for (int c0 = 0; c0 < m && err == hipSuccess; c0 += MTP_MAX_ROWS) {
        const int mc = m - c0 < MTP_MAX_ROWS ? m - c0 : MTP_MAX_ROWS;
        const float* hrows = target_h + (int64_t)(c0 - 1) * H;
        if (c0 == 0) {
            if ((err = launch_shift_rows(pending_h, target_h, shifted, mc, H, st)) != hipSuccess) break;
            hrows = shifted;
        }
        GemvParams p{};
        p.w[0] = qmat(L->eh_proj);
        p.nmat = 1;
        p.N = H;
        p.K = 2 * H;
        p.H = H;
        p.x0 = e ? e + (int64_t)c0 * H : nullptr;
        p.x1 = hrows;
        p.tokens = tokens ? tokens + c0 : nullptr;
        p.table = embed_table;
        p.vocab = L->vocab;
        p.g0 = L->gamma_e;
        p.g1 = L->gamma_h;
        p.eps = L->eps;
        p.y = u;
        if ((err = run_gemv(FMT_Q4, PRO_CONCAT, EPI_STORE, mc, p, default_blocks(), st)) != hipSuccess) break;
        GemvParams q{};
        q.w[0] = qmat(L->wk);
        q.w[1] = qmat(L->wv);
        q.nmat = 2;
        q.N = L->wk.n + L->wv.n;
        q.K = H;
        q.x0 = u;
        q.g0 = L->gamma_attn;
        q.eps = L->eps;
        q.y = kv;
        if ((err = run_gemv(FMT_Q4, PRO_RMS, EPI_STORE, mc, q, default_blocks(), st)) != hipSuccess) break;
        set_positions(a, L, c0);
        err = launch_append_kv(a, kv, mc, cache_len + c0, st);
    }
    return err == hipSuccess ? MTP_OK : hip_fail(err, "mtp_append_kv");
}

}  // namespace

extern "C" {

mtp_status mtp_append_kv(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                         const float* pending_h, const float* target_h, float* k_cache, float* v_cache,
                         int32_t cache_len, int32_t capacity, int32_t m, void* ws, size_t ws_bytes, void* stream) {
    mtp_status s;
    if ((s = check_append_kv(L, e, tokens, embed_table, pending_h, target_h, k_cache, v_cache, cache_len, capacity, m,
                             ws, ws_bytes)))
        return s;
    return enqueue_append_kv(L, e, tokens, embed_table, pending_h, target_h, k_cache, v_cache, cache_len, capacity, m,
                             ws, stream);
}

size_t mtp_stack_draft_workspace_size(const mtp_stack_layer* layers, int32_t n_layers, int32_t t) {
    if (!layers || n_layers < 1 || t < 0) return 0;
    size_t need = 0;
    for (int32_t k = 0; k < n_layers; ++k) {
        const mtp_layer* L = layers[k].layer;
        if (!L) return 0;
        Carve c{nullptr};
        c.take<float>((size_t)L->hidden);  // the draft row's normed hidden (unused after the call)
        c.off = (c.off + 255) & ~size_t(255);
        const size_t a = mtp_draft_step_workspace_size(L, t, 1), b = mtp_append_kv_workspace_size(L);
        c.off += a > b ? a : b;
        need = c.off > need ? c.off : need;
    }
    return need;
}

mtp_status mtp_stack_draft(const mtp_stack_layer* layers, int32_t n_layers, int32_t* tokens, const float* embed_table,
                           const float* target_h, int32_t t, void* ws, size_t ws_bytes, void* stream) {
    if (!layers || n_layers < 1 || n_layers > MTP_MAX_DRAFT)
        return fail(MTP_ERR_INVALID_ARG, "n_layers=%d (1..%d)", n_layers, MTP_MAX_DRAFT);
    if (!tokens || !a4(tokens) || !embed_table || !target_h || t < 0)
        return fail(MTP_ERR_INVALID_ARG, "tokens, embed_table and target_h are required; t=%d", t);
    for (int32_t k = 0; k < n_layers; ++k) {
        const mtp_stack_layer& S = layers[k];
        if (!S.layer) return fail(MTP_ERR_INVALID_ARG, "layer %d is NULL", k);
        if (S.layer->hidden != layers[0].layer->hidden || S.layer->vocab != layers[0].layer->vocab)
            return fail(MTP_ERR_INVALID_ARG, "layer %d: hidden/vocab differ from layer 0", k);
        if (S.start < 0 || S.start > t) return fail(MTP_ERR_INVALID_ARG, "layer %d: start=%d outside 0..t=%d", k, S.start, t);
        if (t >= S.capacity) return fail(MTP_ERR_INVALID_ARG, "layer %d: row t=%d beyond capacity %d", k, t, S.capacity);
    }
    const size_t need = mtp_stack_draft_workspace_size(layers, n_layers, t);
    mtp_status s;
    if ((s = check_ws(ws, ws_bytes, need))) return s;
    const int H = layers[0].layer->hidden;
    Carve c{static_cast<char*>(ws)};
    float* hid = c.take<float>((size_t)H);
    c.off = (c.off + 255) & ~size_t(255);
    void* rest = static_cast<char*>(ws) + c.off;
    const size_t rest_bytes = ws_bytes - c.off;
    // row start + r of layer k pairs x_{start+r+k+1} with h_{start+r}: the
    // catch-up's pending hidden is h_start and its target rows h_{start+1} ..;
    // every layer's calls are checked before the first launch
    for (int pass = 0; pass < 2; ++pass) {
        for (int32_t k = 0; k < n_layers; ++k) {
            const mtp_stack_layer& S = layers[k];
            const int n = t - S.start;  // catch-up rows start .. t-1
            const int32_t* ctok = tokens + S.start + k + 1;
            const float* pend = target_h + (int64_t)S.start * H;
            const float* tgt = target_h + (int64_t)(S.start + 1) * H;
            const int32_t* dtok = tokens + t + k + 1;
            const float* dh = target_h + (int64_t)t * H;
            if (pass == 0) {
                if (n > 0 && (s = check_append_kv(S.layer, nullptr, ctok, embed_table, pend, tgt, S.k_cache, S.v_cache,
                                                  S.start, S.capacity, n, rest, rest_bytes)))
                    return fail(s, "layer %d catch-up: %s", k, mtp_last_error());
                if ((s = check_draft_step(S.layer, nullptr, dtok, embed_table, dh, S.k_cache, S.v_cache, t, S.capacity, 1,
                                          tokens + t + k + 2, hid, nullptr, rest, rest_bytes)))
                    return fail(s, "layer %d draft: %s", k, mtp_last_error());
            } else {
                if (n > 0 && (s = enqueue_append_kv(S.layer, nullptr, ctok, embed_table, pend, tgt, S.k_cache,
                                                    S.v_cache, S.start, S.capacity, n, rest, stream)))
                    return s;
                if ((s = enqueue_draft_step(S.layer, nullptr, dtok, embed_table, dh, S.k_cache, S.v_cache, t,
                                            S.capacity, 1, tokens + t + k + 2, hid, nullptr, rest, stream)))
                    return s;
            }
        }
    }
    return MTP_OK;
}

int32_t mtp_accept(const int32_t* drafts, const int32_t* target_ids, int32_t k, mtp_stats* stats) {
    if (!drafts || !target_ids || k < 1 || k > MTP_MAX_DRAFT) {
        fail(MTP_ERR_INVALID_ARG, "mtp_accept: k=%d (1..%d) and both arrays are required", k, MTP_MAX_DRAFT);
        return -1;
    }
    int32_t a = 0;
    while (a < k && drafts[a] == target_ids[a]) ++a;
    if (stats) {
        stats->rounds += 1;
        stats->drafted += (uint64_t)k;
        stats->accepted += (uint64_t)a;
        stats->accept_hist[a] += 1;
        for (int32_t d = 0; d < k; ++d) {
            stats->depth_drafted[d] += 1;
            if (d < a) stats->depth_accepted[d] += 1;
        }
    }
    return a;
}

mtp_status mtp_dequant_q4(const mtp_q4* w, float* out, void* stream) {
    mtp_status s = check_q4(w, "w");
    if (s) return s;
    if (!out || !a4(out)) return fail(MTP_ERR_INVALID_ARG, "out is NULL or misaligned");
    hipError_t e = launch_dequant(FMT_Q4, qmat(*w), w->k, out, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_dequant_q4");
}

mtp_status mtp_dequant_q8(const mtp_q8* w, int32_t expert, float* out, void* stream) {
    mtp_status s = check_q8(w, "w");
    if (s) return s;
    if (expert < 0 || expert >= w->n_experts) return fail(MTP_ERR_INVALID_ARG, "expert=%d outside 0..%d", expert, w->n_experts - 1);
    if (!out || !a4(out)) return fail(MTP_ERR_INVALID_ARG, "out is NULL or misaligned");
    hipError_t e = launch_dequant(FMT_Q8, qmat8(*w, expert), w->k, out, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_dequant_q8");
}

mtp_status mtp_dequant_q4e(const mtp_q4e* w, int32_t expert, float* out, void* stream) {
    if (!w) return fail(MTP_ERR_INVALID_ARG, "w: descriptor is NULL");
    const ExpMat e = emat(*w);
    mtp_status s = check_emat(&e, "w");
    if (s) return s;
    if (expert < 0 || expert >= w->n_experts) return fail(MTP_ERR_INVALID_ARG, "expert=%d outside 0..%d", expert, w->n_experts - 1);
    if (!out || !a4(out)) return fail(MTP_ERR_INVALID_ARG, "out is NULL or misaligned");
    const int64_t gpe = (int64_t)w->n * (w->k / MTP_GROUP);
    hipError_t err = launch_dequant_q4e(reinterpret_cast<const char*>(w->codes) + expert * (int64_t)w->n * (w->k / 2),
                                        w->scales + expert * gpe, w->biases + expert * gpe, w->n, w->k, out,
                                        (hipStream_t)stream);
    return err == hipSuccess ? MTP_OK : hip_fail(err, "mtp_dequant_q4e");
}

mtp_status mtp_qgemv(const mtp_q4* w, const float* x, const float* residual, float* y, int32_t m, void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_q4(w, "w")) || (s = check_vec(x, "x"))) return s;
    if (!y || !a4(y)) return fail(MTP_ERR_INVALID_ARG, "y is NULL or misaligned");
    if (residual && !a4(residual)) return fail(MTP_ERR_INVALID_ARG, "residual misaligned");
    if ((const void*)y == (const void*)x) return fail(MTP_ERR_INVALID_ARG, "y aliases x");
    GemvParams p{};
    p.w[0] = qmat(*w);
    p.nmat = 1;
    p.N = w->n;
    p.K = w->k;
    p.x0 = x;
    p.residual = residual;
    p.y = y;
    hipError_t e = run_gemv(FMT_Q4, PRO_PLAIN, EPI_STORE, m, p, default_blocks(), (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_qgemv");
}

mtp_status mtp_q8gemv(const mtp_q8* w, int32_t expert, const float* x, const float* residual, float* y, int32_t m,
                      void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_q8(w, "w")) || (s = check_vec(x, "x"))) return s;
    if (expert < 0 || expert >= w->n_experts) return fail(MTP_ERR_INVALID_ARG, "expert=%d outside 0..%d", expert, w->n_experts - 1);
    if (!y || !a4(y)) return fail(MTP_ERR_INVALID_ARG, "y is NULL or misaligned");
    if (residual && !a4(residual)) return fail(MTP_ERR_INVALID_ARG, "residual misaligned");
    if ((const void*)y == (const void*)x) return fail(MTP_ERR_INVALID_ARG, "y aliases x");
    GemvParams p{};
    p.w[0] = qmat8(*w, expert);
    p.nmat = 1;
    p.N = w->n;
    p.K = w->k;
    p.x0 = x;
    p.residual = residual;
    p.y = y;
    hipError_t e = run_gemv(FMT_Q8, PRO_PLAIN, EPI_STORE, m, p, default_blocks(), (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_q8gemv");
}

mtp_status mtp_norm_concat_proj(const float* e, const float* h, const float* gamma_e, const float* gamma_h, float eps,
                                const mtp_q4* eh_proj, float* u, int32_t m, void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_q4(eh_proj, "eh_proj")) || (s = check_vec(e, "e")) ||
        (s = check_vec(h, "h")) || (s = check_vec(gamma_e, "gamma_e")) || (s = check_vec(gamma_h, "gamma_h")))
        return s;
    if (eh_proj->k % 64) return fail(MTP_ERR_INVALID_ARG, "eh_proj k=%d must be 2*hidden with hidden %% 32 == 0", eh_proj->k);
    if (!u || !a4(u)) return fail(MTP_ERR_INVALID_ARG, "u is NULL or misaligned");
    if (!(eps >= 0.0f)) return fail(MTP_ERR_INVALID_ARG, "eps must be >= 0");
    const int H = eh_proj->k / 2;
    if ((const float*)u == e || (const float*)u == h) return fail(MTP_ERR_INVALID_ARG, "u aliases an input");
    GemvParams p{};
    p.w[0] = qmat(*eh_proj);
    p.nmat = 1;
    p.N = eh_proj->n;
    p.K = 2 * H;
    p.H = H;
    p.x0 = e;
    p.x1 = h;
    p.g0 = gamma_e;
    p.g1 = gamma_h;
    p.eps = eps;
    p.y = u;
    hipError_t err = run_gemv(FMT_Q4, PRO_CONCAT, EPI_STORE, m, p, default_blocks(), (hipStream_t)stream);
    return err == hipSuccess ? MTP_OK : hip_fail(err, "mtp_norm_concat_proj");
}

mtp_status mtp_attn_decode(const mtp_layer* L, const float* u, float* k_cache, float* v_cache, int32_t cache_len,
                           int32_t capacity, int32_t m, float* out, void* ws, size_t ws_bytes, void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_layer_attn(L)) || (s = check_vec(u, "u")) ||
        (s = check_cache(k_cache, v_cache, cache_len, capacity, m, L)))
        return s;
    if (!out || !a16(out)) return fail(MTP_ERR_INVALID_ARG, "out is NULL or misaligned");
    if ((const float*)out == u) return fail(MTP_ERR_INVALID_ARG, "out aliases u");
    Carve c{static_cast<char*>(ws)};
    Carve probe{nullptr};
    carve_attn(probe, L, cache_len, m);
    if ((s = check_ws(ws, ws_bytes, probe.off))) return s;
    const AttnWs w = carve_attn(c, L, cache_len, m);
    hipError_t e = run_attention(L, u, k_cache, v_cache, cache_len, capacity, m, out, w, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_attn_decode");
}

mtp_status mtp_ffn_dense_q(const float* x, const float* gamma, float eps, const mtp_q4* gate, const mtp_q4* up,
                           const mtp_q4* down, const float* residual, float* y, int32_t m, void* ws, size_t ws_bytes,
                           void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_vec(x, "x")) || (s = check_q4(gate, "gate")) || (s = check_q4(up, "up")) ||
        (s = check_q4(down, "down")))
        return s;
    if (gamma && (s = check_vec(gamma, "gamma"))) return s;
    if (gate->n != up->n || gate->k != up->k || down->k != gate->n || down->n != gate->k)
        return fail(MTP_ERR_INVALID_ARG, "FFN shapes: gate/up [I][H], down [H][I] expected");
    if (!y || !a16(y)) return fail(MTP_ERR_INVALID_ARG, "y is NULL or misaligned");
    if (residual && !a4(residual)) return fail(MTP_ERR_INVALID_ARG, "residual misaligned");
    if ((const float*)y == x) return fail(MTP_ERR_INVALID_ARG, "y aliases x");
    if (!(eps >= 0.0f)) return fail(MTP_ERR_INVALID_ARG, "eps must be >= 0");
    const size_t need = mtp_ffn_dense_workspace_size(gate->n, m);
    if ((s = check_ws(ws, ws_bytes, need))) return s;
    Carve c{static_cast<char*>(ws)};
    float* z = c.take<float>((size_t)m * gate->n);
    hipError_t e = run_ffn_dense(x, gamma, eps, *gate, *up, *down, residual, y, m, z, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_ffn_dense_q");
}

}  // extern "C"

namespace {

// mtp_ffn_moe_q and mtp_ffn_moe_q4 over either expert format.
mtp_status ffn_moe(const char* what, const float* x, const float* gamma, float eps, const float* router, int32_t top_k,
                   const ExpMat* ge, const ExpMat* ue, const ExpMat* de, const ExpMat* sg, const ExpMat* su,
                   const ExpMat* sd, const float* residual, float* y, int32_t* expert_ids, float* gates, int32_t m,
                   void* ws, size_t ws_bytes, void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_vec(x, "x"))) return s;
    if (!ge) return fail(MTP_ERR_INVALID_ARG, "gate_exps is NULL");
    const int H = ge->k;
    if ((s = check_moe_weights(router, top_k, ge, ue, de, sg, su, sd, H))) return s;
    if (gamma && (s = check_vec(gamma, "gamma"))) return s;
    if (!y || !a4(y)) return fail(MTP_ERR_INVALID_ARG, "y is NULL or misaligned");
    if (residual && !a4(residual)) return fail(MTP_ERR_INVALID_ARG, "residual misaligned");
    if ((const float*)y == x) return fail(MTP_ERR_INVALID_ARG, "y aliases x");
    if (!(eps >= 0.0f)) return fail(MTP_ERR_INVALID_ARG, "eps must be >= 0");
    const int sh_inter = sg ? sg->n : 0;
    const size_t need = mtp_ffn_moe_workspace_size(H, ge->n_experts, top_k, ge->n, sh_inter, m);
    if ((s = check_ws(ws, ws_bytes, need))) return s;
    Carve c{static_cast<char*>(ws)};
    const MoeWs w = carve_moe(c, H, ge->n_experts, top_k, ge->n, sh_inter, m);
    hipError_t e = run_moe(x, gamma, eps, router, top_k, *ge, *ue, *de, sg, su, sd, residual, y, expert_ids, gates, m,
                           w, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, what);
}

}  // namespace

extern "C" {

mtp_status mtp_ffn_moe_q(const float* x, const float* gamma, float eps, const float* router, int32_t top_k,
                         const mtp_q8* gate_exps, const mtp_q8* up_exps, const mtp_q8* down_exps, const mtp_q8* sh_gate,
                         const mtp_q8* sh_up, const mtp_q8* sh_down, const float* residual, float* y,
                         int32_t* expert_ids, float* gates, int32_t m, void* ws, size_t ws_bytes, void* stream) {
    if (!gate_exps || !up_exps || !down_exps) return fail(MTP_ERR_INVALID_ARG, "expert stack descriptor is NULL");
    const ExpMat ge = emat(*gate_exps), ue = emat(*up_exps), de = emat(*down_exps);
    ExpMat sg{}, su{}, sd{};
    if (sh_gate) sg = emat(*sh_gate);
    if (sh_up) su = emat(*sh_up);
    if (sh_down) sd = emat(*sh_down);
    return ffn_moe("mtp_ffn_moe_q", x, gamma, eps, router, top_k, &ge, &ue, &de, sh_gate ? &sg : nullptr,
                   sh_up ? &su : nullptr, sh_down ? &sd : nullptr, residual, y, expert_ids, gates, m, ws, ws_bytes,
                   stream);
}

mtp_status mtp_ffn_moe_q4(const float* x, const float* gamma, float eps, const float* router, int32_t top_k,
                          const mtp_q4e* gate_exps, const mtp_q4e* up_exps, const mtp_q4e* down_exps,
                          const mtp_q4e* sh_gate, const mtp_q4e* sh_up, const mtp_q4e* sh_down,
                          const float* residual, float* y, int32_t* expert_ids, float* gates, int32_t m, void* ws,
                          size_t ws_bytes, void* stream) {
    if (!gate_exps || !up_exps || !down_exps) return fail(MTP_ERR_INVALID_ARG, "expert stack descriptor is NULL");
    const ExpMat ge = emat(*gate_exps), ue = emat(*up_exps), de = emat(*down_exps);
    ExpMat sg{}, su{}, sd{};
    if (sh_gate) sg = emat(*sh_gate);
    if (sh_up) su = emat(*sh_up);
    if (sh_down) sd = emat(*sh_down);
    return ffn_moe("mtp_ffn_moe_q4", x, gamma, eps, router, top_k, &ge, &ue, &de, sh_gate ? &sg : nullptr,
                   sh_up ? &su : nullptr, sh_down ? &sd : nullptr, residual, y, expert_ids, gates, m, ws, ws_bytes,
                   stream);
}

mtp_status mtp_lmhead_argmax(const float* hidden, const float* gamma, float eps, const mtp_q4* lm_head,
                             float* normed_out, float* logits_out, int32_t* ids_out, int32_t m, void* ws,
                             size_t ws_bytes, void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_vec(hidden, "hidden")) || (s = check_vec(gamma, "gamma")) ||
        (s = check_q4(lm_head, "lm_head")))
        return s;
    if (!ids_out || !a4(ids_out)) return fail(MTP_ERR_INVALID_ARG, "ids_out is NULL or misaligned");
    if (normed_out && !a16(normed_out)) return fail(MTP_ERR_INVALID_ARG, "normed_out misaligned");
    if (logits_out && !a4(logits_out)) return fail(MTP_ERR_INVALID_ARG, "logits_out misaligned");
    if (normed_out == hidden && normed_out) return fail(MTP_ERR_INVALID_ARG, "normed_out aliases hidden");
    if (!(eps >= 0.0f)) return fail(MTP_ERR_INVALID_ARG, "eps must be >= 0");
    const size_t need = mtp_lmhead_workspace_size(lm_head->n, m);
    if ((s = check_ws(ws, ws_bytes, need))) return s;
    Carve c{static_cast<char*>(ws)};
    const HeadWs w = carve_head(c, m);
    hipError_t e = run_head(hidden, gamma, eps, *lm_head, normed_out, logits_out, ids_out, m, w, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_lmhead_argmax");
}

mtp_status mtp_lmhead_argmax_q8(const float* hidden, const float* gamma, float eps, const mtp_q8* lm_head,
                                float* normed_out, float* logits_out, int32_t* ids_out, int32_t m, void* ws,
                                size_t ws_bytes, void* stream) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_vec(hidden, "hidden")) || (s = check_vec(gamma, "gamma")) ||
        (s = check_q8(lm_head, "lm_head")))
        return s;
    if (lm_head->n_experts != 1) return fail(MTP_ERR_INVALID_ARG, "lm_head: one matrix (n_experts = 1) expected");
    if (lm_head->k > MTP_MAX_K) return fail(MTP_ERR_UNSUPPORTED, "lm_head k=%d above %d", lm_head->k, MTP_MAX_K);
    if (!ids_out || !a4(ids_out)) return fail(MTP_ERR_INVALID_ARG, "ids_out is NULL or misaligned");
    if (normed_out && !a16(normed_out)) return fail(MTP_ERR_INVALID_ARG, "normed_out misaligned");
    if (logits_out && !a4(logits_out)) return fail(MTP_ERR_INVALID_ARG, "logits_out misaligned");
    if (normed_out == hidden && normed_out) return fail(MTP_ERR_INVALID_ARG, "normed_out aliases hidden");
    if (!(eps >= 0.0f)) return fail(MTP_ERR_INVALID_ARG, "eps must be >= 0");
    const size_t need = mtp_lmhead_workspace_size(lm_head->n, m);
    if ((s = check_ws(ws, ws_bytes, need))) return s;
    Carve c{static_cast<char*>(ws)};
    const HeadWs w = carve_head(c, m);
    hipError_t e = run_head_fmt(FMT_Q8, qmat8(*lm_head, 0), lm_head->k, hidden, gamma, eps, normed_out, logits_out,
                                ids_out, m, w, (hipStream_t)stream);
    return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_lmhead_argmax_q8");
}

}  // extern "C"

namespace mtp {

// Every check of mtp_draft_step but the workspace's; launches nothing and
// makes no HIP call.
mtp_status check_draft_step_args(const mtp_layer* L, const float* e, const int32_t* tokens,
                                 const float* embed_table, const float* h, float* k_cache, float* v_cache,
                                 int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out,
                                 float* hidden_out, float* logits_out) {
    mtp_status s;
    if ((s = check_rows(m)) || (s = check_layer_attn(L)) || (s = check_cache(k_cache, v_cache, cache_len, capacity, m, L)))
        return s;
    const int H = L->hidden;
    if ((s = check_vec(h, "h")) || (s = check_vec(L->gamma_e, "gamma_e")) || (s = check_vec(L->gamma_h, "gamma_h")) ||
        (s = check_vec(L->gamma_post, "gamma_post")) || (s = check_vec(L->gamma_final, "gamma_final")) ||
        (s = check_q4(&L->eh_proj, "eh_proj")) || (s = check_q4(&L->lm_head, "lm_head")))
        return s;
    if (L->eh_proj.n != H || L->eh_proj.k != 2 * H) return fail(MTP_ERR_INVALID_ARG, "eh_proj must be [hidden][2*hidden]");
    if (L->lm_head.k != H || L->lm_head.n != L->vocab) return fail(MTP_ERR_INVALID_ARG, "lm_head must be [vocab][hidden]");
    if (!tokens && !e) return fail(MTP_ERR_INVALID_ARG, "give e or tokens");
    if (e && (s = check_vec(e, "e"))) return s;
    if (tokens && (!a4(tokens) || !embed_table)) return fail(MTP_ERR_INVALID_ARG, "tokens needs an aligned pointer and embed_table");
    if (tokens && L->vocab < 1) return fail(MTP_ERR_INVALID_ARG, "vocab=%d: tokens need a table of at least one row", L->vocab);
    if (embed_table && !a16(embed_table)) return fail(MTP_ERR_INVALID_ARG, "embed_table misaligned");
    if (!ids_out || !a4(ids_out)) return fail(MTP_ERR_INVALID_ARG, "ids_out is NULL or misaligned");
    if (!hidden_out || !a16(hidden_out)) return fail(MTP_ERR_INVALID_ARG, "hidden_out is NULL or misaligned");
    if (logits_out && !a4(logits_out)) return fail(MTP_ERR_INVALID_ARG, "logits_out misaligned");
    if (hidden_out == h || hidden_out == e) return fail(MTP_ERR_INVALID_ARG, "hidden_out aliases an input");
    if (L->ffn_kind == MTP_FFN_DENSE_Q4) {
        if ((s = check_q4(&L->gate, "gate")) || (s = check_q4(&L->up, "up")) || (s = check_q4(&L->down, "down"))) return s;
        if (L->gate.n != L->ffn_inter || L->up.n != L->ffn_inter || L->gate.k != H || L->up.k != H ||
            L->down.n != H || L->down.k != L->ffn_inter)
            return fail(MTP_ERR_INVALID_ARG, "dense FFN shapes do not match hidden/ffn_inter");
    } else if (L->ffn_kind == MTP_FFN_MOE_Q8 || L->ffn_kind == MTP_FFN_MOE_Q4) {
        const LayerExperts x = layer_experts(L);
        if ((s = check_moe_weights(L->router, L->top_k, &x.ge, &x.ue, &x.de, x.shared ? &x.sg : nullptr,
                                   x.shared ? &x.su : nullptr, x.shared ? &x.sd : nullptr, H)))
            return s;
    } else {
        return fail(MTP_ERR_INVALID_ARG, "ffn_kind=%d", L->ffn_kind);
    }
    return MTP_OK;
}

}  // namespace mtp

namespace {

// Every check of mtp_draft_step; launches nothing.
mtp_status check_draft_step(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                            const float* h, float* k_cache, float* v_cache, int32_t cache_len, int32_t capacity,
                            int32_t m, int32_t* ids_out, float* hidden_out, float* logits_out, void* ws,
                            size_t ws_bytes) {
    mtp_status s = check_draft_step_args(L, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m,
                                         ids_out, hidden_out, logits_out);
    if (s) return s;
    return check_ws(ws, ws_bytes, mtp_draft_step_workspace_size(L, cache_len, m));
}

}  // namespace

namespace mtp {

// The launches of mtp_draft_step (arguments already checked).
mtp_status enqueue_draft_step(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                              const float* h, float* k_cache, float* v_cache, int32_t cache_len, int32_t capacity,
                              int32_t m, int32_t* ids_out, float* hidden_out, float* logits_out, void* ws,
                              void* stream) {
    const int H = L->hidden;
    hipStream_t st = (hipStream_t)stream;
    // carve in the order mtp_draft_step_workspace_size measures
    Carve c{static_cast<char*>(ws)};
    float* u = c.take<float>((size_t)m * H);
    float* r1 = c.take<float>((size_t)m * H);
    float* r2 = c.take<float>((size_t)m * H);
    const AttnWs aw = carve_attn(c, L, cache_len, m);
    const bool moe = L->ffn_kind == MTP_FFN_MOE_Q8 || L->ffn_kind == MTP_FFN_MOE_Q4;
    const LayerExperts xe = moe ? layer_experts(L) : LayerExperts{};
    const bool sh = xe.shared;
    float* z = nullptr;
    MoeWs mw{};
    if (moe)
        mw = carve_moe(c, H, xe.ge.n_experts, L->top_k, xe.ge.n, sh ? xe.sg.n : 0, m);
    else
        z = c.take<float>((size_t)m * L->ffn_inter);
    const HeadWs hw = carve_head(c, m);

    // u = eh_proj [rms(e); rms(h)]
    GemvParams p{};
    p.w[0] = qmat(L->eh_proj);
    p.nmat = 1;
    p.N = H;
    p.K = 2 * H;
    p.H = H;
    p.x0 = e;
    p.x1 = h;
    p.tokens = tokens;
    p.table = embed_table;
    p.vocab = L->vocab;
    p.g0 = L->gamma_e;
    p.g1 = L->gamma_h;
    p.eps = L->eps;
    p.y = u;
    p.zero_words = reinterpret_cast<unsigned*>(hw.keys);  // the head's argmax state starts from zero
    p.zero_n = kHeadStateWords;
    hipError_t err = run_gemv(FMT_Q4, PRO_CONCAT, EPI_STORE, m, p, default_blocks(), st);
    if (err != hipSuccess) return hip_fail(err, "mtp_draft_step eh_proj");
    if ((err = run_attention(L, u, k_cache, v_cache, cache_len, capacity, m, r1, aw, st)) != hipSuccess)
        return hip_fail(err, "mtp_draft_step attention");
    if (!moe) {
        err = run_ffn_dense(r1, L->gamma_post, L->eps, L->gate, L->up, L->down, r1, r2, m, z, st);
    } else {
        err = run_moe(r1, L->gamma_post, L->eps, L->router, L->top_k, xe.ge, xe.ue, xe.de, sh ? &xe.sg : nullptr,
                      sh ? &xe.su : nullptr, sh ? &xe.sd : nullptr, r1, r2, nullptr, nullptr, m, mw, st);
    }
    if (err != hipSuccess) return hip_fail(err, "mtp_draft_step ffn");
    if ((err = run_head(r2, L->gamma_final, L->eps, L->lm_head, hidden_out, logits_out, ids_out, m, hw, st)) != hipSuccess)
        return hip_fail(err, "mtp_draft_step head");
    return MTP_OK;
}

}  // namespace mtp

extern "C" {

mtp_status mtp_draft_step(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                          const float* h, float* k_cache, float* v_cache, int32_t cache_len, int32_t capacity,
                          int32_t m, int32_t* ids_out, float* hidden_out, float* logits_out, void* ws,
                          size_t ws_bytes, void* stream) {
    mtp_status s;
    if ((s = check_draft_step(L, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m, ids_out,
                              hidden_out, logits_out, ws, ws_bytes)))
        return s;
    return enqueue_draft_step(L, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m, ids_out,
                              hidden_out, logits_out, ws, stream);
}

}  // extern "C"
