// moe.hip -- routed mixture of SwiGLU experts (hf2q 0.1.13,
// src/inference/models/qwen35/mtp.rs, `MtpFfnWeightsGpu::Moe`: router
// `ffn_gate_inp`, stacked gate/up/down experts, shared-expert tensors), over
// 8-bit block experts or 4-bit affine experts with bf16 group constants
// (hf2q 0.1.1, src/serve/forward_mlx_shared.rs, `MlxAffineMoeStack`).
//
// Launch sequence (one stream, no host round trip):
//   k_moe_router   one block per expert row: optional input RMSNorm, f32
//                  router dot products for the m <= 4 rows of a pass (block 0
//                  stores the normalised rows for the expert GEMVs).
//   k_moe_topk     one block: per row softmax, top-k by (p desc, index asc),
//                  renormalised gates; then the union of selected experts over
//                  the m rows is compacted (ascending expert id) into slots,
//                  each with its per-row gate (0 where a row did not pick it);
//                  the shared expert becomes the last slot with gate 1.
//   gate/up        quantized SwiGLU GEMV per slot (grid.y = slot), scaled by
//                  the slot's row gates.
//   down           quantized GEMV per slot into a per-slot partial.
//   k_moe_combine  y = residual + sum over slots in slot order.
// The two slot GEMVs take k_moe_slot (below) when both feature counts are a
// power-of-two number of groups up to 64 and the shared expert has the
// routed experts' size; other shapes take the generic GEMV kernel (8-bit
// experts only: the host rejects other shapes for 4-bit experts).
#include <climits>
#include <cmath>
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace mtp {

constexpr int kMaxE = 1024;

// One block per router row e, m <= 4 rows: every global value the block
// needs (its router row, the rows' features and the norm weights) is
// requested in one round, and the rows' sums of squares and their dot
// products with the row are formed together, so the norm costs no second
// memory round trip: logit = rsqrt(mean(x^2) + eps) * sum_k w_k x_k gamma_k.
constexpr int kRouterU = 8;  // features per thread and round (2048 per block round)
constexpr int kCombThreads = 64;  // threads of a combine block
constexpr int kRouterThreads = 256;  // threads of a router block
// The launch parameters the first requests of a kernel depend on, named in
// empty asm statements as scalar operands: the compiler issues their loads
// together and waits for them once, where it would otherwise load each group
// where it is first used and wait there, one round trip after another.
__device__ __forceinline__ void gather_router(const MoeParams& p) {
    asm volatile("" ::"s"(p.x), "s"(p.gamma), "s"(p.eps), "s"(p.f), "s"(p.router), "s"(p.logits), "s"(p.E), "s"(p.H),
                 "s"(p.m));
}

__global__ void __launch_bounds__(kRouterThreads) k_moe_router(const MoeParams p) {
    __shared__ float red[4][2][4];  // [wave][sum of squares | dot][row]
    __shared__ float inv_s[4];
    gather_router(p);
    const int e = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
    const float* w = p.router + (int64_t)e * p.H;
    const bool norm = p.gamma != nullptr;
    float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < p.H; k0 += 256 * kRouterU) {
        float wv[kRouterU], gv[kRouterU], xv[4][kRouterU];
#pragma unroll
        for (int u = 0; u < kRouterU; ++u) {
            const int k = k0 + t + 256 * u;
            const bool in = k < p.H;
            wv[u] = in ? w[k] : 0.0f;
            gv[u] = (in && norm) ? p.gamma[k] : 1.0f;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) xv[mi][u] = (in && mi < p.m) ? p.x[(int64_t)mi * p.H + k] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kRouterU; ++u)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                ss[mi] = fmaf(xv[mi][u], xv[mi][u], ss[mi]);
                dot[mi] = fmaf(wv[u], xv[mi][u] * gv[u], dot[mi]);
            }
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const float a = wave_sum(ss[mi]), d = wave_sum(dot[mi]);
        if (lane == 0) {
            red[wid][0][mi] = a;
            red[wid][1][mi] = d;
        }
    }
    __syncthreads();
    if (t < p.m) {
        float a = 0.0f, d = 0.0f;
        for (int j = 0; j < 4; ++j) {
            a += red[j][0][t];
            d += red[j][1][t];
        }
        const float inv = norm ? rsqrtf(a / (float)p.H + p.eps) : 1.0f;
        inv_s[t] = inv;
        p.logits[(int64_t)t * p.E + e] = d * inv;
    }
    if (norm && e == 0) {  // the normalised rows for the expert GEMVs
        __syncthreads();
        for (int mi = 0; mi < p.m; ++mi)
            for (int k = t; k < p.H; k += kRouterThreads)
                p.f[(int64_t)mi * p.H + k] = p.x[(int64_t)mi * p.H + k] * inv_s[mi] * p.gamma[k];
    }
}

// Top-k of one row of router logits by one wave.  Each lane keeps its share
// of the row (experts lane + 64 j, j < NJ) in registers, so the selection
// makes no memory round trip.  Selection runs on the logits (softmax is
// monotonic, so the order of p is the order of the logits).  Lane s < top_k
// returns selection s: its expert and its renormalised gate p_e / sum of the
// selected p; row_mask (when given) receives the row's selected experts as
// NJ 64-bit words.
constexpr int kTopkPerLane = kMaxE / kWave;
// A step finds the largest remaining logit with a 32-bit wave maximum, then
// the lowest expert index holding it with one ballot per register (index
// lane + 64 j grows with j first).  Equal values (and -0, +0) go to the lower
// index; NaN is never selected.  Lane s < top_k returns selection s.
template <int NJ>
__device__ __forceinline__ void row_topk_n(const float* l, int E, int top_k, int lane, int& my_id, float& my_gate,
                                           unsigned long long* row_mask) {
    float lv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + kWave * j;
        lv[j] = e < E ? l[e] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) mx = fmaxf(mx, lv[j]);
    mx = wave_max(mx);
    unsigned taken = 0;  // bit j: expert lane + 64 j chosen
    float psum = 0.0f, my_pe = 0.0f;
    my_id = 0;
    for (int s = 0; s < top_k; ++s) {
        float lm = -INFINITY;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (!((taken >> j) & 1u) && lane + kWave * j < E) lm = fmaxf(lm, lv[j]);
        const float vmax = wave_max(lm);
        int bi = -1;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const unsigned long long hit =
                __ballot(!((taken >> j) & 1u) && lane + kWave * j < E && lv[j] == vmax);
            if (bi < 0 && hit) bi = kWave * j + __ffsll((long long)hit) - 1;
        }
        float bv = vmax;
        if (bi < 0) {  // only NaN logits left
            bi = 0;
            bv = __shfl(lv[0], 0);
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        const float pe = __expf(bv - mx);
        psum += pe;
        my_id = (lane == s) ? bi : my_id;
        my_pe = (lane == s) ? pe : my_pe;
    }
    my_gate = my_pe / psum;
    if (row_mask) {  // word j: experts 64 j .. 64 j + 63
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const unsigned long long w = __ballot((taken >> j) & 1u);
            if (lane == 0) row_mask[j] = w;
        }
    }
}

__device__ __forceinline__ void row_topk(const float* l, int E, int top_k, int lane, int& my_id, float& my_gate,
                                         unsigned long long* row_mask = nullptr) {
    if (E <= 4 * kWave)
        row_topk_n<4>(l, E, top_k, lane, my_id, my_gate, row_mask);
    else
        row_topk_n<kTopkPerLane>(l, E, top_k, lane, my_id, my_gate, row_mask);
}

// One block of 512 threads; wave mi handles row mi (top_k <= 64: lane s
// holds selection s).
__global__ void __launch_bounds__(512) k_moe_topk(const MoeParams p) {
    __shared__ int sel[kMaxE];
    __shared__ float gsel[kMaxE][8];
    const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
    for (int e = t; e < p.E; e += blockDim.x) {
        sel[e] = 0;
        for (int mi = 0; mi < 8; ++mi) gsel[e][mi] = 0.0f;
    }
    __syncthreads();
    if (wid < p.m) {
        const int mi = wid;
        int my_id;
        float gate;
        row_topk(p.logits + (int64_t)mi * p.E, p.E, p.top_k, lane, my_id, gate);
        if (lane < p.top_k) {
            p.expert_ids[mi * p.top_k + lane] = my_id;
            p.gates[mi * p.top_k + lane] = gate;
            gsel[my_id][mi] = gate;
            sel[my_id] = 1;
        }
    }
    __syncthreads();
    if (wid == 0) {
        int count = 0;
        for (int base = 0; base < p.E; base += kWave) {
            const int e = base + lane;
            const int f = (e < p.E) ? sel[e] : 0;
            const unsigned long long mask = __ballot(f);
            const int prefix = __popcll(mask & ((1ull << lane) - 1ull));
            if (f) {
                const int slot = count + prefix;
                p.slot_expert[slot] = e;
                for (int mi = 0; mi < p.m; ++mi) p.slot_gate[(int64_t)slot * p.m + mi] = gsel[e][mi];
            }
            count += __popcll(mask);
        }
        if (p.sg.codes) {
            if (lane == 0) p.slot_expert[count] = -1;
            if (lane < p.m) p.slot_gate[(int64_t)count * p.m + lane] = 1.0f;
            count += 1;
        }
        if (lane == 0) *p.n_slots = count;
    }
}

// y = residual + the slots' partials added one after another in slot order;
// the partials are requested eight at a time.
// The first kCombFirst slots' partials (rows of the max_slots the buffer
// holds) are requested with the residual before the slot count arrives; the
// sum runs in slot order either way.
constexpr int kCombFirst = 12;

__global__ void __launch_bounds__(kCombThreads) k_moe_combine(const MoeParams p) {
    asm volatile("" ::"s"(p.m), "s"(p.H), "s"(p.n_slots), "s"(p.max_slots), "s"(p.ypart), "s"(p.residual),
                 "s"(p.y));
    const int64_t idx = (int64_t)blockIdx.x * kCombThreads + threadIdx.x;
    if (idx >= (int64_t)p.m * p.H) return;
    const int64_t step = (int64_t)p.m * p.H;
    const float* src = p.ypart + idx;
    float t0[kCombFirst];
#pragma unroll
    for (int i = 0; i < kCombFirst; ++i) t0[i] = i < p.max_slots ? src[i * step] : 0.0f;
    float acc = p.residual ? p.residual[idx] : 0.0f;
    const int ns = *p.n_slots;
#pragma unroll
    for (int i = 0; i < kCombFirst; ++i)
        if (i < ns) acc += t0[i];
    for (int s = kCombFirst; s < ns; s += 8) {  // the rest in batches of 8 (one round trip each)
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = s + i < ns ? src[(s + i) * step] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s + i < ns) acc += t[i];
    }
    p.y[idx] = acc;
}

// ---------------------------------------------------------------------------
// k_moe_slot: one expert GEMV per slot (grid.y = slot), for K = 32*G
// features with G a power of two up to 64; FMT_Q8 (8-bit block experts) or
// FMT_Q4 (4-bit experts with bf16 scale and bias per group).
//
// Lane mapping: a row's G groups take LG = G consecutive lanes, so one wave
// load covers RPL = 64/LG rows (lane = rs*LG + g reads the codes and group
// constants of row rs, group g: 32 bytes and a scale for 8-bit, 16 bytes and
// two bf16 for 4-bit); at K = 512 that is four rows per load instead of one
// row on a quarter of the lanes.  A "load-set" is those RPL rows (for SwiGLU,
// the same RPL rows of gate and of up).
//
// Activations: the block stages its slot's m activation rows once in LDS,
// per (row, group of 32) the 32 f32 values and their sum; each lane reads the
// fragments of its group into registers, in the order of its format's code
// halves.  A row's group term is s * (2^24 sum((c + 128) 2^-24 x) - 128 sum(x))
// for 8-bit codes and (s 2^24) sum(c 2^-24 x) + b sum(x) for 4-bit codes,
// with the exact code subnormals of q8_halves / q4_halves (see device.hpp).
//
// Work: a slot's load-sets are spread evenly over the waves of its
// gridDim.x blocks and taken UB at a time (a batch); two batches are in
// flight per wave, the
// next one requested before the current one is reduced (a transposed
// butterfly over the LG lanes of each row) and stored.  The first two are
// requested before the activation setup.
// ---------------------------------------------------------------------------
struct SlotGemv {
    const void* codes[2];      // expert stacks (codes[1]: up, SwiGLU only): int8 [E][N][K] or u32 [E][N][K/8]
    const void* scales[2];     // [E][N][K/32]: f32 (8-bit) or bf16 bits (4-bit)
    const void* biases[2];     // [E][N][K/32] bf16 bits (4-bit only)
    const void* sh_codes[2];   // shared expert, one matrix of the same format (NULL when absent)
    const void* sh_scales[2];
    const void* sh_biases[2];
    int64_t ex_codes, ex_scales;  // per-expert strides: code bytes, group constants
    int N, K, m;
    const float* act;     // [slot][m][K] activations (slot stride act_slot; 0 = shared by all slots)
    int64_t act_slot;
    float* out;           // [slot][m][N]
    int64_t out_slot;
    const float* slot_gate;  // [slot][m]: SwiGLU output scale (the row's gate of that expert)
    const int* slot_expert;
    const int* n_slots;
    // Routing in the gate/up launch: when logits ([m][E] router logits) is
    // set, every block selects the experts itself, so no launch sits between
    // the router and the experts.  With a shared expert it takes slot 0 (its
    // blocks skip the routing and stream at once) and slot 1 + j is the j-th
    // selected expert in ascending order; without one slot j is.  Block 0 of
    // the first routed slot publishes the slot table and count (read by
    // the down and combine launches) and the per-row selections.
    const float* logits;
    int E, top_k, has_shared;
    int* slot_expert_out;
    int* n_slots_out;
    int* expert_ids_out;
    float* gates_out;
};

constexpr int kFragWords = 36;  // 32 values, their sum, pad (16-byte multiple)

template <int LG>
__host__ __device__ constexpr int seg_step0() {
    return LG >= 64 ? 0 : (LG == 32 ? 1 : (LG == 16 ? 2 : (LG == 8 ? 3 : (LG == 4 ? 4 : (LG == 2 ? 5 : 6)))));
}

// Position of this lane's first value after Butterfly<V, FIN, seg_step0<LG>>.
template <int V, int FIN, int LG>
__device__ __forceinline__ int seg_base(int lane) {
    int base = 0, cur = V;
#pragma unroll
    for (int d = LG / 2; d >= 1; d >>= 1) {
        if (cur > FIN) {
            cur >>= 1;
            if (lane & d) base += cur;
        }
    }
    return base;
}

// The block's routing (see SlotGemv): returns in *s_e the slot's expert (-1
// the shared expert, -2 no such slot) and in s_gate[mi] row mi's gate for it.
template <int W>
__device__ __forceinline__ void route_slot(const SlotGemv& p, int slot, int lane, int wid,
                                           unsigned long long (*rmask)[kMaxE / kWave], int (*rid)[kWave],
                                           float (*rgate)[kWave], int* s_e, float* s_gate) {
    const int words = (p.E + kWave - 1) / kWave;
    const bool publish = blockIdx.x == 0 && slot == p.has_shared;
    const int rslot = slot - p.has_shared;  // routed slot index (the shared expert holds slot 0)
    for (int mi = wid; mi < p.m; mi += W) {
        int id;
        float gate;
        row_topk(p.logits + (int64_t)mi * p.E, p.E, p.top_k, lane, id, gate, rmask[mi]);
        if (lane < p.top_k) {
            rid[mi][lane] = id;
            rgate[mi][lane] = gate;
            if (publish) {
                p.expert_ids_out[mi * p.top_k + lane] = id;
                p.gates_out[mi * p.top_k + lane] = gate;
            }
        }
    }
    __syncthreads();
    if (wid != 0) return;
    // lane w < words owns mask word w; its experts take the slots after those
    // of the words before it
    unsigned long long mw = 0ull;  // the union of the rows' masks
    if (lane < words)
        for (int mi = 0; mi < p.m; ++mi) mw |= rmask[mi][lane];
    const int c = __popcll(mw);
    int incl = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    const int excl = incl - c;
    const int n_routed = __shfl(incl, kWave - 1);
    const int n_slots = n_routed + p.has_shared;
    if (publish) {
        int idx = p.has_shared + excl;
        for (unsigned long long b = mw; b; b &= b - 1ull) p.slot_expert_out[idx++] = lane * kWave + __ffsll((long long)b) - 1;
        if (lane == 0) {
            if (p.has_shared) p.slot_expert_out[0] = -1;
            *p.n_slots_out = n_slots;
        }
    }
    int e;
    if (rslot < n_routed) {
        const bool mine = lane < words && rslot >= excl && rslot < incl;
        int cand = 0;
        if (mine) {
            unsigned long long b = mw;
            for (int k = rslot - excl; k > 0; --k) b &= b - 1ull;
            cand = lane * kWave + __ffsll((long long)b) - 1;
        }
        const unsigned long long who = __ballot(mine);
        e = __shfl(cand, __ffsll((long long)who) - 1);
    } else {
        e = -2;  // past the selected experts: no such slot
    }
    for (int mi = 0; mi < p.m; ++mi) {
        float gate = 1.0f;
        if (e >= 0) {
            const bool hit = lane < p.top_k && rid[mi][lane] == e;
            const unsigned long long hm = __ballot(hit);
            const float g = lane < p.top_k ? rgate[mi][lane] : 0.0f;
            gate = hm ? __shfl(g, __ffsll((long long)hm) - 1) : 0.0f;
        }
        if (lane == 0) s_gate[mi] = gate;
    }
    if (lane == 0) *s_e = e;
}

// Load-sets per batch; two batches are in flight per wave.
template <int M>
__host__ __device__ constexpr int slot_batch() { return M >= 4 ? 1 : 2; }


// The lane's fragment of a row of format FMT from a stored (row, group)
// fragment (the order of make_frag<FMT>).
template <int FMT>
__device__ __forceinline__ void read_frag(const unsigned* f, XFrag& xf) {
    const float4* f4 = reinterpret_cast<const float4*>(f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float4 t = f4[k];
        const float xv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (FMT == FMT_Q4) {
                const int f8 = 4 * (k & 1) + q;  // feature within the 4-bit word k/2
                xf.v[8 * (k >> 1) + q4_slot(f8)] = xv[q] * q4_factor(f8);
            } else {
                xf.v[4 * k + q8_slot(q)] = xv[q];
            }
        }
    }
    xf.sum = (FMT == FMT_Q4 ? 1.0f : -128.0f) * f4[8].x;
}

__device__ __forceinline__ void zero_frag(WFrag<FMT_Q8>& w) {
    w.c0 = (u32x4){0u, 0u, 0u, 0u};
    w.c1 = (u32x4){0u, 0u, 0u, 0u};
    w.s = 0.0f;
}
__device__ __forceinline__ void zero_frag(WFrag<FMT_Q4>& w) {
    w.c = (u32x4){0u, 0u, 0u, 0u};
    w.s = 0.0f;
    w.b = 0.0f;
}
__device__ __forceinline__ float dot_frag(const WFrag<FMT_Q8>& w, const XFrag& x) { return dot_q8(w, x); }
__device__ __forceinline__ float dot_frag(const WFrag<FMT_Q4>& w, const XFrag& x) { return dot_q4(w.c, w.s, w.b, x); }

template <int FMT, int M, int EPI, int LG, int W>
__global__ void __launch_bounds__(W * 64) k_moe_slot(const SlotGemv p) {
    constexpr int P = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int RPL = kWave / LG;
    constexpr int UB = slot_batch<M>();
    constexpr int V = UB * M * P;
    constexpr int FIN = (V / LG > P) ? V / LG : P;  // values a lane holds after the reduction
    constexpr int DUP = LG * FIN / V;               // lanes holding each of them
    constexpr int RT = (EPI == EPI_SWIGLU) ? 8 : 1;  // routing state rows (gate/up launch only)
    __shared__ __align__(16) unsigned frag[M * LG * kFragWords];
    __shared__ unsigned long long rmask[RT][kMaxE / kWave];
    __shared__ int rid[RT][kWave];
    __shared__ float rgate[RT][kWave];
    __shared__ int s_e;
    __shared__ float s_gate[8];

    asm volatile("" ::"s"(p.act), "s"(p.act_slot), "s"(p.K), "s"(p.m), "s"(p.N), "s"(p.logits), "s"(p.E),
                 "s"(p.top_k), "s"(p.has_shared), "s"(p.n_slots), "s"(p.slot_expert), "s"(p.codes[0]),
                 "s"(p.codes[1]), "s"(p.scales[0]), "s"(p.scales[1]), "s"(p.sh_codes[0]), "s"(p.sh_codes[1]),
                 "s"(p.sh_scales[0]), "s"(p.sh_scales[1]), "s"(p.ex_codes), "s"(p.ex_scales));
    if constexpr (FMT == FMT_Q4)
        asm volatile("" ::"s"(p.biases[0]), "s"(p.biases[1]), "s"(p.sh_biases[0]), "s"(p.sh_biases[1]));
    const int slot = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool route = EPI == EPI_SWIGLU && p.logits != nullptr;
    const int G = LG;  // groups per row

    // the activations are requested before the routing / slot lookup, whose
    // memory latency they then share: the m rows (K = 32 G features each,
    // contiguous) in 16-byte pieces, thread t taking pieces t, t + 64 W, ...,
    // so that a load instruction reads one contiguous kilobyte (eight lines);
    // the eight pieces of a group sit in eight consecutive lanes
    const float* act = p.act + (int64_t)slot * p.act_slot;
    constexpr int kRowF4 = LG * kGroup / 4;  // 16-byte pieces per row (K = 32 LG)
    constexpr int kActF4 = (M * kRowF4 + W * kWave - 1) / (W * kWave);
    float4 xa[kActF4];
#pragma unroll
    for (int i = 0; i < kActF4; ++i) {
        const int f4 = threadIdx.x + W * kWave * i;
        const bool ok = f4 < M * kRowF4 && f4 / kRowF4 < p.m;
        const float4 x = reinterpret_cast<const float4*>(act)[ok ? f4 : 0];  // rows past m: any valid address
        xa[i] = ok ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }

    int e;
    if (route && p.has_shared && slot == 0) {
        // the shared expert: no routing to wait for, a gate of 1 for every row
        e = -1;
        if (threadIdx.x < 8) s_gate[threadIdx.x] = 1.0f;
    } else if (route) {
        if constexpr (EPI == EPI_SWIGLU) route_slot<W>(p, slot, lane, wid, rmask, rid, rgate, &s_e, s_gate);
        __syncthreads();
        e = s_e;
        if (e == -2) return;
    } else {
        if (slot >= *p.n_slots) return;
        e = p.slot_expert[slot];
    }
    // this slot's matrices (typed by format; the 4-bit constants are bf16)
    using SC = typename std::conditional<FMT == FMT_Q4, unsigned short, float>::type;
    const char* cw[2];
    const SC* sw[2];
    const unsigned short* bw[2];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        cw[i] = e >= 0 ? static_cast<const char*>(p.codes[i]) + (int64_t)e * p.ex_codes
                       : static_cast<const char*>(p.sh_codes[i]);
        sw[i] = e >= 0 ? static_cast<const SC*>(p.scales[i]) + (int64_t)e * p.ex_scales
                       : static_cast<const SC*>(p.sh_scales[i]);
        bw[i] = nullptr;
        if constexpr (FMT == FMT_Q4)
            bw[i] = e >= 0 ? static_cast<const unsigned short*>(p.biases[i]) + (int64_t)e * p.ex_scales
                           : static_cast<const unsigned short*>(p.sh_biases[i]);
    }
    const int g = lane % LG, rs = lane / LG;
    const int L = (p.N + RPL - 1) / RPL;  // load-sets of the slot
    // the slot's load-sets are spread evenly over its gridDim.x * W waves (a
    // wave's last batch may be partly past its range: those loads are skipped)
    const int NW = gridDim.x * W, wv = blockIdx.x * W + wid;
    const int j_begin = (int)((int64_t)wv * L / NW);
    const int j_end = (int)((int64_t)(wv + 1) * L / NW);

    WFrag<FMT> wa[UB][P], wb[UB][P];
    auto load_batch = [&](WFrag<FMT> (&wf)[UB][P], int j0) {
#pragma unroll
        for (int b = 0; b < UB; ++b) {
            if (j0 + b >= j_end) {  // wave-uniform: past the range, a zero fragment
#pragma unroll
                for (int i = 0; i < P; ++i) zero_frag(wf[b][i]);
                continue;
            }
            int n = (j0 + b) * RPL + rs;
            n = n < p.N ? n : p.N - 1;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                if constexpr (FMT == FMT_Q4)
                    load_frag_b16(wf[b][i], cw[i], sw[i], bw[i], n, G, g);
                else
                    load_frag(wf[b][i], cw[i], sw[i], nullptr, n, G, g);
            }
        }
    };
    // two batches in flight from the start
    if (j_begin < j_end) load_batch(wa, j_begin);
    if (j_begin + UB < j_end) load_batch(wb, j_begin + UB);

    // activation setup: each (row, group) fragment is the group's 32 values
    // and their sum, which its eight lanes form together
#pragma unroll
    for (int i = 0; i < kActF4; ++i) {
        const int f4 = threadIdx.x + W * kWave * i;
        const float4 x = xa[i];
        float sum = (x.x + x.y) + (x.z + x.w);
        sum += dpp_partner<1>(sum);
        sum += dpp_partner<2>(sum);
        sum += dpp_partner<4>(sum);
        if (f4 < M * kRowF4) {
            const int mi = f4 / kRowF4, k4 = f4 % kRowF4;
            float4* fr = reinterpret_cast<float4*>(frag + (mi * LG + k4 / 8) * kFragWords);
            fr[k4 % 8] = x;
            if (k4 % 8 == 0) fr[8] = make_float4(sum, 0.0f, 0.0f, 0.0f);
        }
    }
    __syncthreads();
    if (j_begin >= j_end) return;
    XFrag xf[M];
#pragma unroll
    for (int mi = 0; mi < M; ++mi) read_frag<FMT>(frag + (mi * LG + g) * kFragWords, xf[mi]);

    const int base = seg_base<V, FIN, LG>(lane);
    const bool writer = (lane & (DUP - 1)) == 0;
    float* out = p.out + (int64_t)slot * p.out_slot;
    // dot products of one batch, then (after the caller's next request) the
    // reduction over the row's lanes and the epilogue
    auto dots = [&](const WFrag<FMT> (&wf)[UB][P], float (&v)[V]) {
#pragma unroll
        for (int b = 0; b < UB; ++b)
#pragma unroll
            for (int i = 0; i < P; ++i)
#pragma unroll
                for (int mi = 0; mi < M; ++mi) v[(b * M + mi) * P + i] = dot_frag(wf[b][i], xf[mi]);
    };
    auto finish = [&](float (&v)[V], int j0) {
        Butterfly<V, FIN, seg_step0<LG>()>::run(v, lane);
        if (writer) {
#pragma unroll
            for (int f = 0; f < FIN; f += P) {
                const int pos = (base + f) / P;  // = b*M + mi
                const int b = pos / M, mi = pos % M;
                const int j = j0 + b;
                const int n = j * RPL + rs;
                if (j < j_end && n < p.N && mi < p.m) {
                    const int64_t o = (int64_t)mi * p.N + n;
                    if constexpr (EPI == EPI_SWIGLU)
                        out[o] = silu(v[f]) * v[f + 1] * (route ? s_gate[mi] : p.slot_gate[(int64_t)slot * p.m + mi]);
                    else
                        out[o] = v[f];
                }
            }
        }
    };
    for (int j0 = j_begin; j0 < j_end; j0 += 2 * UB) {
        {
            float v[V];
            dots(wa, v);
            if (j0 + 2 * UB < j_end) load_batch(wa, j0 + 2 * UB);
            finish(v, j0);
        }
        if (j0 + UB >= j_end) break;
        {
            float v[V];
            dots(wb, v);
            if (j0 + 3 * UB < j_end) load_batch(wb, j0 + 3 * UB);
            finish(v, j0 + UB);
        }
    }
}

// Resident blocks per compute unit of one kernel (from its registers and
// LDS), asked once.
template <int FMT, int M, int EPI, int LG, int W>
static int slot_blocks_per_cu() {
    static int cached = 0;
    if (!cached) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_moe_slot<FMT, M, EPI, LG, W>, W * kWave, 0) != hipSuccess ||
            n < 1)
            n = 1;
        cached = n;
    }
    return cached;
}

// Blocks per slot: as many as fill the resident capacity over the launch's
// slots (so no block waits for a second round and compute units carry equal
// shares), at most one per wave's batch.
template <int FMT, int M, int EPI, int LG>
static hipError_t launch_slot_g(const SlotGemv& p, int max_slots, hipStream_t st) {
    constexpr int W = 4;
    constexpr int RPL = kWave / LG;
    constexpr int UB = slot_batch<M>();
    const int L = (p.N + RPL - 1) / RPL;
    const int U = (L + UB - 1) / UB;
    const int cap = device_cu_count() * slot_blocks_per_cu<FMT, M, EPI, LG, W>();
    int per_slot = cap / max_slots;
    per_slot = per_slot < 1 ? 1 : per_slot;
    const int most = (U + W - 1) / W;
    per_slot = per_slot > most ? most : per_slot;
    const dim3 grid((unsigned)per_slot, (unsigned)max_slots);
    hipLaunchKernelGGL((k_moe_slot<FMT, M, EPI, LG, W>), grid, dim3(W * kWave), 0, st, p);
    return hipGetLastError();
}

template <int FMT, int M, int EPI>
static hipError_t launch_slot_m(const SlotGemv& p, int max_slots, hipStream_t st) {
    switch (p.K / kGroup) {
        case 64: return launch_slot_g<FMT, M, EPI, 64>(p, max_slots, st);
        case 16: return launch_slot_g<FMT, M, EPI, 16>(p, max_slots, st);
        case 8: return launch_slot_g<FMT, M, EPI, 8>(p, max_slots, st);
        case 2: return launch_slot_g<FMT, M, EPI, 2>(p, max_slots, st);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT>
static hipError_t launch_slot_f(int epi, const SlotGemv& p, int max_slots, hipStream_t st) {
    switch (inst_m(p.m)) {
        case 1: return epi == EPI_SWIGLU ? launch_slot_m<FMT, 1, EPI_SWIGLU>(p, max_slots, st)
                                         : launch_slot_m<FMT, 1, EPI_STORE>(p, max_slots, st);
        case 2: return epi == EPI_SWIGLU ? launch_slot_m<FMT, 2, EPI_SWIGLU>(p, max_slots, st)
                                         : launch_slot_m<FMT, 2, EPI_STORE>(p, max_slots, st);
        case 4: return epi == EPI_SWIGLU ? launch_slot_m<FMT, 4, EPI_SWIGLU>(p, max_slots, st)
                                         : launch_slot_m<FMT, 4, EPI_STORE>(p, max_slots, st);
        default: return hipErrorInvalidValue;  // launch_moe runs at most four rows per pass
    }
}

static bool slot_groups_ok(int K) {
    const int G = K / kGroup;
    return K % kGroup == 0 && (G == 64 || G == 16 || G == 8 || G == 2);
}

static hipError_t launch_slot(int fmt, int epi, const SlotGemv& p, int max_slots, hipStream_t st) {
    return fmt == FMT_Q4 ? launch_slot_f<FMT_Q4>(epi, p, max_slots, st) : launch_slot_f<FMT_Q8>(epi, p, max_slots, st);
}

static bool moe_slot_path(const MoeParams& p);

// One pass of the MoE over p.m rows (at most four on the slot kernel, two on
// the generic path).
static hipError_t moe_pass(const MoeParams& p, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_router, dim3(p.E), dim3(kRouterThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool slot_path = moe_slot_path(p);
    if (!slot_path) {
        hipLaunchKernelGGL(k_moe_topk, dim3(1), dim3(512), 0, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    const float* fin = p.gamma ? p.f : p.x;
    const int imax = p.inter > p.sh_inter ? p.inter : p.sh_inter;
    const int fmt = p.q4 ? FMT_Q4 : FMT_Q8;
    const int64_t cdiv = p.q4 ? 2 : 1;                                   // code bytes per weight: 1/2 or 1
    const int64_t ex_codes_gu = (int64_t)p.inter * p.H / cdiv;          // code bytes per gate/up expert
    const int64_t ex_sc_gu = (int64_t)p.inter * (p.H / kGroup);
    const int64_t ex_codes_d = (int64_t)p.H * p.inter / cdiv;
    const int64_t ex_sc_d = (int64_t)p.H * (p.inter / kGroup);
    if (p.q4 && !slot_path) return hipErrorInvalidValue;  // the host admits only slot-kernel shapes

    if (slot_path) {
        SlotGemv g{};
        g.codes[0] = p.ge.codes;
        g.codes[1] = p.ue.codes;
        g.scales[0] = p.ge.scales;
        g.scales[1] = p.ue.scales;
        g.biases[0] = p.ge.biases;
        g.biases[1] = p.ue.biases;
        g.sh_codes[0] = p.sg.codes;
        g.sh_codes[1] = p.su.codes;
        g.sh_scales[0] = p.sg.scales;
        g.sh_scales[1] = p.su.scales;
        g.sh_biases[0] = p.sg.biases;
        g.sh_biases[1] = p.su.biases;
        g.ex_codes = ex_codes_gu;
        g.ex_scales = ex_sc_gu;
        g.N = p.inter;
        g.K = p.H;
        g.m = p.m;
        g.act = fin;
        g.act_slot = 0;
        g.out = p.z;
        g.out_slot = (int64_t)p.m * imax;
        g.logits = p.logits;
        g.E = p.E;
        g.top_k = p.top_k;
        g.has_shared = p.sg.codes ? 1 : 0;
        g.slot_expert_out = p.slot_expert;
        g.n_slots_out = p.n_slots;
        g.expert_ids_out = p.expert_ids;
        g.gates_out = p.gates;
        if ((e = launch_slot(fmt, EPI_SWIGLU, g, p.max_slots, st)) != hipSuccess) return e;

        SlotGemv d{};
        d.codes[0] = p.de.codes;
        d.scales[0] = p.de.scales;
        d.biases[0] = p.de.biases;
        d.sh_codes[0] = p.sd.codes;
        d.sh_scales[0] = p.sd.scales;
        d.sh_biases[0] = p.sd.biases;
        d.ex_codes = ex_codes_d;
        d.ex_scales = ex_sc_d;
        d.N = p.H;
        d.K = p.inter;
        d.m = p.m;
        d.act = p.z;
        d.act_slot = (int64_t)p.m * imax;
        d.out = p.ypart;
        d.out_slot = (int64_t)p.m * p.H;
        d.slot_expert = p.slot_expert;
        d.n_slots = p.n_slots;
        if ((e = launch_slot(fmt, EPI_STORE, d, p.max_slots, st)) != hipSuccess) return e;
        const int64_t n = (int64_t)p.m * p.H;
        hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n + kCombThreads - 1) / kCombThreads)), dim3(kCombThreads), 0, st,
                           p);
        return hipGetLastError();
    }

    GemvParams g{};
    g.w[0] = p.ge;
    g.w[1] = p.ue;
    g.nmat = 2;
    g.m = p.m;
    g.N = p.inter;
    g.K = p.H;
    g.G = p.H / kGroup;
    g.S = (g.G + kWave - 1) / kWave;
    g.x0 = fin;
    g.y = p.z;
    g.rowscale = p.slot_gate;
    g.slot_expert = p.slot_expert;
    g.n_slots = p.n_slots;
    g.ex_codes = ex_codes_gu;
    g.ex_scales = ex_sc_gu;
    g.shw[0] = p.sg;
    g.shw[1] = p.su;
    g.N_sh = p.sh_inter;
    g.K_sh = p.H;
    g.x_slot = 0;
    g.y_slot = (int64_t)p.m * imax;
    g.rs_slot = p.m;
    if ((e = launch_gemv_slots(FMT_Q8, EPI_SWIGLU, p.m, g, 1 << 20, p.max_slots, st)) != hipSuccess) return e;

    GemvParams d{};
    d.w[0] = p.de;
    d.nmat = 1;
    d.m = p.m;
    d.N = p.H;
    d.K = p.inter;
    d.G = p.inter / kGroup;
    d.S = (d.G + kWave - 1) / kWave;
    d.x0 = p.z;
    d.y = p.ypart;
    d.slot_expert = p.slot_expert;
    d.n_slots = p.n_slots;
    d.ex_codes = ex_codes_d;
    d.ex_scales = ex_sc_d;
    d.shw[0] = p.sd;
    d.N_sh = p.H;
    d.K_sh = p.sh_inter;
    d.x_slot = (int64_t)p.m * imax;
    d.y_slot = (int64_t)p.m * p.H;
    if ((e = launch_gemv_slots(FMT_Q8, EPI_STORE, p.m, d, 1 << 20, p.max_slots, st)) != hipSuccess) return e;

    const int64_t n = (int64_t)p.m * p.H;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n + kCombThreads - 1) / kCombThreads)), dim3(kCombThreads), 0, st,
                           p);
    return hipGetLastError();
}

// out [n][K] = the f32 weights of one 4-bit matrix with bf16 constants (the
// rounding of the 4-bit GEMVs' dequantization, device.hpp).
__global__ void __launch_bounds__(256) k_dequant_q4e(const void* codes, const unsigned short* scales,
                                                     const unsigned short* biases, int n, int K, float* out) {
    const int G = K / kGroup;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)n * G) return;
    const int64_t row = gid / G;
    const int g = (int)(gid % G);
    WFrag<FMT_Q4> f;
    load_frag_b16(f, codes, scales, biases, row, G, g);
    dequant_q4_group(f, out + row * K + (int64_t)g * kGroup);
}

hipError_t launch_dequant_q4e(const void* codes, const unsigned short* scales, const unsigned short* biases, int n,
                              int k, float* out, hipStream_t st) {
    const int64_t groups = (int64_t)n * (k / kGroup);
    const int64_t blocks = (groups + 255) / 256;
    hipLaunchKernelGGL(k_dequant_q4e, dim3((unsigned)blocks), dim3(256), 0, st, codes, scales, biases, n, k, out);
    return hipGetLastError();
}

static bool moe_slot_path(const MoeParams& p) {
    return slot_groups_ok(p.H) && slot_groups_ok(p.inter) && (!p.sg.codes || p.sh_inter == p.inter);
}

// Rows in passes (each a whole MoE over its rows, sharing the workspace's
// slot tables, which every pass rebuilds): four rows per pass on the slot
// kernel, two on the generic path.
hipError_t launch_moe(const MoeParams& p, hipStream_t st) {
    const int per = moe_slot_path(p) ? 4 : 2;
    for (int r0 = 0; r0 < p.m; r0 += per) {
        MoeParams q = p;
        q.m = p.m - r0 < per ? p.m - r0 : per;
        q.x += (int64_t)r0 * p.H;
        q.f += (int64_t)r0 * p.H;
        q.logits += (int64_t)r0 * p.E;
        q.expert_ids += (int64_t)r0 * p.top_k;
        q.gates += (int64_t)r0 * p.top_k;
        if (q.residual) q.residual += (int64_t)r0 * p.H;
        q.y += (int64_t)r0 * p.H;
        const hipError_t e = moe_pass(q, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mtp
