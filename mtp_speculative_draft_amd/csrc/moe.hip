// moe.hip -- routed mixture of 8-bit SwiGLU experts (hf2q 0.1.13,
// src/inference/models/qwen35/mtp.rs, `MtpFfnWeightsGpu::Moe`: router
// `ffn_gate_inp`, stacked gate/up/down experts, shared-expert tensors).
//
// Launch sequence (one stream, no host round trip):
//   k_moe_router   one block per expert row: optional input RMSNorm, f32
//                  router dot products for all m rows (block 0 stores the
//                  normalised rows for the expert GEMVs).
//   k_moe_topk     one block: per row softmax, top-k by (p desc, index asc),
//                  renormalised gates; then the union of selected experts over
//                  the m rows is compacted (ascending expert id) into slots,
//                  each with its per-row gate (0 where a row did not pick it);
//                  the shared expert becomes the last slot with gate 1.
//   gate/up        quantized SwiGLU GEMV per slot (grid.y = slot), scaled by
//                  the slot's row gates.
//   down           quantized GEMV per slot into a per-slot partial.
//   k_moe_combine  y = residual + sum over slots in slot order.
#include <climits>
#include <cmath>

#include "device.hpp"
#include "launch.hpp"

namespace mtp {

constexpr int kMaxE = 1024;

__global__ void __launch_bounds__(256) k_moe_router(const MoeParams p) {
    __shared__ float red[4][8];
    __shared__ float inv_s[8];
    const int e = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
    const float* w = p.router + (int64_t)e * p.H;
    float inv[8];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) inv[mi] = 1.0f;
    if (p.gamma) {
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            if (mi < p.m) {
                float ss = 0.0f;
                for (int k = t; k < p.H; k += blockDim.x) {
                    const float v = p.x[(int64_t)mi * p.H + k];
                    ss = fmaf(v, v, ss);
                }
                ss = wave_sum(ss);
                if (lane == 0) red[wid][mi] = ss;
            }
        }
        __syncthreads();
        if (t < p.m) {
            float ss = 0.0f;
            for (int j = 0; j < (int)(blockDim.x / kWave); ++j) ss += red[j][t];
            inv_s[t] = rsqrtf(ss / (float)p.H + p.eps);
        }
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) inv[mi] = (mi < p.m) ? inv_s[mi] : 1.0f;
        if (e == 0) {
            for (int mi = 0; mi < p.m; ++mi)
                for (int k = t; k < p.H; k += blockDim.x)
                    p.f[(int64_t)mi * p.H + k] = p.x[(int64_t)mi * p.H + k] * inv_s[mi] * p.gamma[k];
        }
        __syncthreads();
    }
    float acc[8];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) acc[mi] = 0.0f;
    for (int k = t; k < p.H; k += blockDim.x) {
        const float wv = w[k];
        const float gk = p.gamma ? p.gamma[k] : 1.0f;
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            if (mi < p.m) {
                float xv = p.x[(int64_t)mi * p.H + k];
                if (p.gamma) xv = xv * inv[mi] * gk;
                acc[mi] = fmaf(wv, xv, acc[mi]);
            }
        }
    }
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        if (mi < p.m) {
            const float s = wave_sum(acc[mi]);
            if (lane == 0) red[wid][mi] = s;
        }
    }
    __syncthreads();
    if (t < p.m) {
        float s = 0.0f;
        for (int j = 0; j < (int)(blockDim.x / kWave); ++j) s += red[j][t];
        p.logits[(int64_t)t * p.E + e] = s;
    }
}

// One block of 512 threads; wave mi handles row mi.
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
        const float* l = p.logits + (int64_t)mi * p.E;
        float mx = -INFINITY;
        for (int e = lane; e < p.E; e += kWave) mx = fmaxf(mx, l[e]);
        mx = wave_max(mx);
        // selection on the logits: softmax is monotonic, so the order of p is
        // the order of the logits; ties go to the lower expert index
        unsigned long long taken = 0;  // bit j: expert lane + 64*j already chosen
        float psum = 0.0f;
        for (int s = 0; s < p.top_k; ++s) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int j = 0, e = lane; e < p.E; ++j, e += kWave)
                if (!((taken >> j) & 1ull)) argmax_merge(bv, bi, l[e], e);
            wave_argmax(bv, bi);
            if (bi == INT_MAX) bi = 0;  // only for non-finite logits
            if ((bi & (kWave - 1)) == lane) taken |= 1ull << (bi / kWave);
            const float pe = __expf(l[bi] - mx);
            psum += pe;
            if (lane == 0) {
                p.expert_ids[mi * p.top_k + s] = bi;
                gsel[bi][mi] = pe;
                sel[bi] = 1;
            }
        }
        __syncwarp();
        if (lane == 0) {
            for (int s = 0; s < p.top_k; ++s) {
                const int e = p.expert_ids[mi * p.top_k + s];
                const float gate = gsel[e][mi] / psum;
                gsel[e][mi] = gate;
                p.gates[mi * p.top_k + s] = gate;
            }
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

__global__ void __launch_bounds__(256) k_moe_combine(const MoeParams p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)p.m * p.H) return;
    const int ns = *p.n_slots;
    float acc = p.residual ? p.residual[idx] : 0.0f;
    for (int s = 0; s < ns; ++s) acc += p.ypart[(int64_t)s * p.m * p.H + idx];
    p.y[idx] = acc;
}

hipError_t launch_moe(const MoeParams& p, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_router, dim3(p.E), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_moe_topk, dim3(1), dim3(512), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const float* fin = p.gamma ? p.f : p.x;
    const int imax = p.inter > p.sh_inter ? p.inter : p.sh_inter;
    const int64_t ex_codes_gu = (int64_t)p.inter * p.H;          // int8 bytes per gate/up expert
    const int64_t ex_sc_gu = (int64_t)p.inter * (p.H / kGroup);
    const int64_t ex_codes_d = (int64_t)p.H * p.inter;
    const int64_t ex_sc_d = (int64_t)p.H * (p.inter / kGroup);

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
    GemvShape sh = gemv_shape(FMT_Q8, EPI_SWIGLU, p.m, imax, p.H, 1 << 20);
    if ((e = launch_gemv_slots(FMT_Q8, EPI_SWIGLU, p.m, g, sh, p.max_slots, st)) != hipSuccess) return e;

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
    GemvShape shd = gemv_shape(FMT_Q8, EPI_STORE, p.m, p.H, imax, 1 << 20);
    if ((e = launch_gemv_slots(FMT_Q8, EPI_STORE, p.m, d, shd, p.max_slots, st)) != hipSuccess) return e;

    const int64_t n = (int64_t)p.m * p.H;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace mtp
