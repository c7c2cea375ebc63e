// attn.hip -- decode attention over the f32 KV cache for m <= 8 query rows.
//
// Semantics (hf2q 0.1.13, src/inference/models/qwen35/mtp.rs,
// `forward_full_attention` and its `apply_sdpa_with_kv_cache` call):
// rotary embedding on q and k at positions cache_len + r (half-split pairs
// (i, i + d/2), inverse frequency theta^(-2i/d)), the m new k/v rows appended
// to the cache before attention, causal grouped-query attention with scale
// 1/sqrt(d), query head h reading KV head h / (n_heads / n_kv_heads).
//
// Kernel 1 (grid: position chunks x KV heads): each block takes kAttnChunk
// cache positions of one KV head and every query head of its group for all m
// rows, so a K/V row is read from HBM once for the whole group.  The block
// that owns a new position rotates its k, writes k and v into the cache and
// uses them from LDS.  It emits per (chunk, query row-head) the chunk maximum,
// the exp-sum and the unnormalised sum of p*V.
// Kernel 2 (grid: KV heads x query row-heads) merges the chunks with the
// log-sum-exp rule.
#include <cmath>

#include "device.hpp"
#include "launch.hpp"

namespace mtp {

constexpr int kD = 128;            // head_dim handled here
constexpr int kC = kAttnChunk;     // positions per block
constexpr int kKStride = kD + 4;   // padded LDS row (floats)
constexpr int kMaxHM = 64;         // query row-heads per KV head (group * m)

__global__ void __launch_bounds__(256) k_attn_partial(const AttnParams p) {
    __shared__ float qs[kMaxHM][kD];
    __shared__ float ks[kC][kKStride];
    __shared__ float vs[kC][kD];
    __shared__ float sc[kMaxHM][kC + 1];
    __shared__ float rc[8][kD / 2], rs[8][kD / 2];  // rotary cos/sin per new row
    __shared__ float stat_m[kMaxHM], stat_l[kMaxHM];

    const int c = blockIdx.x, g = blockIdx.y;
    const int t = threadIdx.x;
    const int GQ = p.nh / p.nkv;
    const int HM = GQ * p.m;
    const int ld = (p.nh + 2 * p.nkv) * kD;  // qkv row stride
    const int p0 = c * kC;
    const float scale = 1.0f / sqrtf((float)kD);

    // rotary table for positions cache_len + mi (double precision angles)
    for (int idx = t; idx < p.m * (kD / 2); idx += blockDim.x) {
        const int mi = idx / (kD / 2), i = idx % (kD / 2);
        const double inv_freq = pow(p.theta, -2.0 * (double)i / (double)kD);
        const double ang = (double)(p.cache_len + mi) * inv_freq;
        rc[mi][i] = (float)cos(ang);
        rs[mi][i] = (float)sin(ang);
    }
    __syncthreads();

    // rotated queries of this group: hm = mi * GQ + local head
    for (int idx = t; idx < HM * (kD / 2); idx += blockDim.x) {
        const int hm = idx / (kD / 2), i = idx % (kD / 2);
        const int mi = hm / GQ, hq = g * GQ + hm % GQ;
        const float* q = p.qkv + (int64_t)mi * ld + hq * kD;
        const float a = q[i], b = q[i + kD / 2];
        const float cs = rc[mi][i], sn = rs[mi][i];
        qs[hm][i] = a * cs - b * sn;
        qs[hm][i + kD / 2] = a * sn + b * cs;
    }
    // cached K/V rows of the chunk (float4); new and out-of-range rows later
    const int64_t cbase = (int64_t)g * p.capacity * kD;
    for (int idx = t; idx < kC * (kD / 4); idx += blockDim.x) {
        const int j = idx / (kD / 4), u = idx % (kD / 4);
        const int pos = p0 + j;
        float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
        if (pos < p.cache_len) {
            kv4 = reinterpret_cast<const float4*>(p.k_cache + cbase + (int64_t)pos * kD)[u];
            vv4 = reinterpret_cast<const float4*>(p.v_cache + cbase + (int64_t)pos * kD)[u];
        }
        *reinterpret_cast<float4*>(&ks[j][4 * u]) = kv4;
        *reinterpret_cast<float4*>(&vs[j][4 * u]) = vv4;
    }
    __syncthreads();
    // new rows owned by this chunk: rotate k, keep in LDS, append to the cache
    for (int idx = t; idx < p.m * (kD / 2); idx += blockDim.x) {
        const int mi = idx / (kD / 2), i = idx % (kD / 2);
        const int pos = p.cache_len + mi;
        if (pos < p0 || pos >= p0 + kC) continue;
        const int j = pos - p0;
        const float* kr = p.qkv + (int64_t)mi * ld + p.nh * kD + g * kD;
        const float* vr = p.qkv + (int64_t)mi * ld + (p.nh + p.nkv) * kD + g * kD;
        const float a = kr[i], b = kr[i + kD / 2];
        const float cs = rc[mi][i], sn = rs[mi][i];
        const float k0 = a * cs - b * sn, k1 = a * sn + b * cs;
        ks[j][i] = k0;
        ks[j][i + kD / 2] = k1;
        vs[j][i] = vr[i];
        vs[j][i + kD / 2] = vr[i + kD / 2];
        float* kd = p.k_cache + cbase + (int64_t)pos * kD;
        float* vd = p.v_cache + cbase + (int64_t)pos * kD;
        kd[i] = k0;
        kd[i + kD / 2] = k1;
        vd[i] = vr[i];
        vd[i + kD / 2] = vr[i + kD / 2];
    }
    __syncthreads();

    // scores (masked: query row mi sees positions <= cache_len + mi)
    for (int idx = t; idx < HM * kC; idx += blockDim.x) {
        const int hm = idx / kC, j = idx % kC;
        const int mi = hm / GQ;
        const int pos = p0 + j;
        float s = -INFINITY;
        if (pos <= p.cache_len + mi) {
            const float4* qa = reinterpret_cast<const float4*>(&qs[hm][0]);
            const float4* ka = reinterpret_cast<const float4*>(&ks[j][0]);
            float acc = 0.0f;
#pragma unroll 8
            for (int u = 0; u < kD / 4; ++u) {
                const float4 a = qa[u], b = ka[u];
                acc = fmaf(a.x, b.x, acc);
                acc = fmaf(a.y, b.y, acc);
                acc = fmaf(a.z, b.z, acc);
                acc = fmaf(a.w, b.w, acc);
            }
            s = acc * scale;
        }
        sc[hm][j] = s;
    }
    __syncthreads();

    // chunk softmax statistics, one thread per query row-head
    for (int hm = t; hm < HM; hm += blockDim.x) {
        float mx = -INFINITY;
        for (int j = 0; j < kC; ++j) mx = fmaxf(mx, sc[hm][j]);
        float l = 0.0f;
        if (mx != -INFINITY) {
            for (int j = 0; j < kC; ++j) {
                const float e = __expf(sc[hm][j] - mx);
                sc[hm][j] = e;
                l += e;
            }
        } else {
            for (int j = 0; j < kC; ++j) sc[hm][j] = 0.0f;
        }
        stat_m[hm] = mx;
        stat_l[hm] = l;
    }
    __syncthreads();

    // unnormalised p*V per (hm, dim)
    float* out = p.part + ((int64_t)c * p.nkv + g) * HM * (kD + 2);
    for (int idx = t; idx < HM * kD; idx += blockDim.x) {
        const int hm = idx / kD, dd = idx % kD;
        float acc = 0.0f;
#pragma unroll 8
        for (int j = 0; j < kC; ++j) acc = fmaf(sc[hm][j], vs[j][dd], acc);
        out[hm * (kD + 2) + dd] = acc;
        if (dd == 0) {
            out[hm * (kD + 2) + kD] = stat_m[hm];
            out[hm * (kD + 2) + kD + 1] = stat_l[hm];
        }
    }
}

// One block per (KV head, query row-head, half of the head dims): 8 chunk
// lanes x 64 dims.  Each lane requests a batch of chunks' (max, exp-sum, p*V)
// at once, merges them with the online log-sum-exp rule, and the 8 lanes are
// merged through LDS.
constexpr int kCombDims = 64;
constexpr int kCombLanes = 8;
constexpr int kCombBatch = 16;

__device__ __forceinline__ void lse_merge(float& M, float& L, float& A, float m2, float l2, float a2) {
    if (!(l2 > 0.0f)) return;
    if (m2 > M) {
        const float r = __expf(M - m2);  // M = -inf gives 0
        A *= r;
        L *= r;
        M = m2;
    }
    const float w = __expf(m2 - M);
    A = fmaf(w, a2, A);
    L = fmaf(w, l2, L);
}

__global__ void __launch_bounds__(kCombLanes * kCombDims) k_attn_combine(const AttnParams p) {
    __shared__ float sm[kCombLanes][kCombDims], sl[kCombLanes][kCombDims], sa[kCombLanes][kCombDims];
    const int g = blockIdx.x, hm = blockIdx.y;
    const int t = threadIdx.x, dl = t % kCombDims, cs = t / kCombDims;
    const int dd = blockIdx.z * kCombDims + dl;
    const int GQ = p.nh / p.nkv;
    const int HM = GQ * p.m;
    const int mi = hm / GQ, hq = g * GQ + hm % GQ;
    const int64_t stride = (int64_t)p.nkv * HM * (kD + 2);  // between chunks
    const float* base = p.part + ((int64_t)g * HM + hm) * (kD + 2);

    float M = -INFINITY, L = 0.0f, A = 0.0f;
    for (int c0 = cs; c0 < p.chunks; c0 += kCombLanes * kCombBatch) {
        float lv[kCombBatch], mv[kCombBatch], av[kCombBatch];
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const int c = c0 + u * kCombLanes;
            const float* pr = base + (int64_t)(c < p.chunks ? c : 0) * stride;
            lv[u] = pr[kD + 1];
            mv[u] = pr[kD];
            av[u] = pr[dd];
            if (c >= p.chunks) lv[u] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) lse_merge(M, L, A, mv[u], lv[u], av[u]);
    }
    sm[cs][dl] = M;
    sl[cs][dl] = L;
    sa[cs][dl] = A;
    __syncthreads();
    if (cs == 0) {
        for (int j = 1; j < kCombLanes; ++j) lse_merge(M, L, A, sm[j][dl], sl[j][dl], sa[j][dl]);
        p.o[(int64_t)mi * p.nh * kD + hq * kD + dd] = L > 0.0f ? A / L : 0.0f;
    }
}

hipError_t launch_attention(const AttnParams& p, hipStream_t st) {
    hipLaunchKernelGGL(k_attn_partial, dim3(p.chunks, p.nkv), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int HM = (p.nh / p.nkv) * p.m;
    hipLaunchKernelGGL(k_attn_combine, dim3(p.nkv, HM, kD / kCombDims), dim3(kCombLanes * kCombDims), 0, st, p);
    return hipGetLastError();
}

}  // namespace mtp
