// attn.hip -- decode attention over the f32 KV cache for m <= 8 query rows.
//
// Semantics (hf2q 0.1.13, src/inference/models/qwen35/mtp.rs,
// `forward_full_attention` and its `apply_sdpa_with_kv_cache` call):
// rotary embedding on q and k at positions cache_len + r (half-split pairs
// (i, i + d/2), inverse frequency theta^(-2i/d)), the m new k/v rows appended
// to the cache before attention, causal grouped-query attention with scale
// 1/sqrt(d), query head h reading KV head h / (n_heads / n_kv_heads).
//
// Kernel 1 (one block per position chunk x KV head x slice of at most
// kSliceHM query row-heads): each block takes kAttnChunk cache positions of
// one KV head for up to kSliceHM (query head, row) pairs of its group, so a
// K/V row is read from HBM once per slice.  The slices of one chunk are given
// consecutive block slots on one XCD so they share its L2.  Every row-head's
// arithmetic is the same whatever the slicing, so m rows at once give
// bitwise the results of m single-row calls.  The block that owns a new
// position rotates its k and uses it from LDS; the first slice also writes k
// and v into the cache.  It emits per (chunk, query row-head) the chunk
// maximum, the exp-sum and the unnormalised sum of p*V.
// Kernel 2 (grid: KV heads x query row-heads) merges the chunks with the
// log-sum-exp rule.
#include <cmath>

#include "device.hpp"
#include "launch.hpp"

namespace mtp {

constexpr int kD = 128;           // head_dim handled here
constexpr int kC = kAttnChunk;    // positions per block
constexpr int kKStride = kD + 4;  // padded LDS row (floats)
constexpr int kSliceHM = 16;      // query row-heads per partial block, at most
constexpr int kSStride = kC + 4;  // score row stride (16-byte aligned)

// cos/sin of pos * inv_freq: the angle and its reduction to [-pi, pi] in
// double, the sine and cosine of the reduced angle in single precision.
__device__ __forceinline__ void rotary(double pos, double inv_freq, float& c, float& s) {
    const double two_pi = 6.283185307179586476925286766559;
    const double ang = pos * inv_freq;
    const double red = ang - two_pi * rint(ang * (1.0 / two_pi));
    __sincosf((float)red, &s, &c);
}

// Block slot -> (chunk, KV head, slice): slots are dealt to the XCDs in turn
// (slot % 8), so the Z slices of a (chunk, head) pair take Z consecutive
// slots of one XCD.  Returns false for the padding slots of the last round.
__device__ __forceinline__ bool attn_block(const AttnParams& p, int Z, int& c, int& g, int& z) {
    const int L = blockIdx.x, x = L % 8, r = L / 8;
    z = r % Z;
    const int pair = (r / Z) * 8 + x;
    if (pair >= p.chunks * p.nkv) return false;
    c = pair / p.nkv;
    g = pair % p.nkv;
    return true;
}

// HMT: the block's row-head count rounded up to 8 or 16; the register-blocked
// loops below are sized by it.  Local row-head hl of slice z is the group's
// row-head z * kSliceHM + hl (= mi * GQ + local query head).
template <int HMT>
__global__ void __launch_bounds__(256) k_attn_partial(const AttnParams p) {
    __shared__ float qs[HMT][kD];
    __shared__ float ks[kC][kKStride];
    __shared__ float vs[kC][kD];
    __shared__ float sc[HMT][kSStride];
    __shared__ float rc[8][kD / 2], rs[8][kD / 2];  // rotary cos/sin per new row
    __shared__ float stat_m[HMT], stat_l[HMT];

    const int GQ = p.nh / p.nkv;
    const int HMall = GQ * p.m;
    const int Z = (HMall + kSliceHM - 1) / kSliceHM;
    int c, g, z;
    if (!attn_block(p, Z, c, g, z)) return;
    const int hm0 = z * kSliceHM;
    const int HM = HMall - hm0 < kSliceHM ? HMall - hm0 : kSliceHM;  // row-heads of this block
    const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
    const int ld = (p.nh + 2 * p.nkv) * kD;  // qkv row stride
    const int p0 = c * kC;
    const int64_t cbase = (int64_t)g * p.capacity * kD;
    constexpr int kQuads = kC * (kD / 4) / 256;  // float4 slots of K (and of V) per thread

    // 1. the chunk's cached K/V rows are requested first ...
    float4 kr[kQuads], vr[kQuads];
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
        const int idx = t + 256 * u, j = idx / (kD / 4), w = idx % (kD / 4);
        const int pos = p0 + j;
        kr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        vr[u] = kr[u];
        if (pos < p.cache_len) {
            kr[u] = reinterpret_cast<const float4*>(p.k_cache + cbase + (int64_t)pos * kD)[w];
            vr[u] = reinterpret_cast<const float4*>(p.v_cache + cbase + (int64_t)pos * kD)[w];
        }
    }
    // ... and the rotary table for positions cache_len + mi is built meanwhile
    for (int idx = t; idx < p.m * (kD / 2); idx += blockDim.x) {
        const int mi = idx / (kD / 2), i = idx % (kD / 2);
        const double inv_freq = exp2(-(2.0 * (double)i / (double)kD) * p.log2_theta);
        rotary((double)(p.cache_len + mi), inv_freq, rc[mi][i], rs[mi][i]);
    }
    __syncthreads();

    // 2. rotated queries of this group (hm = mi * GQ + local head), cached
    //    rows into LDS, rows past the new ones zeroed, the new rows rotated and
    //    appended to the cache (only by the chunk that owns them)
    for (int idx = t; idx < HM * (kD / 2); idx += blockDim.x) {
        const int hm = idx / (kD / 2), i = idx % (kD / 2);
        const int mi = (hm0 + hm) / GQ, hq = g * GQ + (hm0 + hm) % GQ;
        const float* q = p.qkv + (int64_t)mi * ld + hq * kD;
        const float a = q[i], b = q[i + kD / 2];
        const float cs = rc[mi][i], sn = rs[mi][i];
        qs[hm][i] = a * cs - b * sn;
        qs[hm][i + kD / 2] = a * sn + b * cs;
    }
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
        const int idx = t + 256 * u, j = idx / (kD / 4), w = idx % (kD / 4);
        const int pos = p0 + j;
        if (pos < p.cache_len || pos >= p.cache_len + p.m) {
            *reinterpret_cast<float4*>(&ks[j][4 * w]) = kr[u];
            *reinterpret_cast<float4*>(&vs[j][4 * w]) = vr[u];
        }
    }
    for (int idx = t; idx < p.m * (kD / 2); idx += blockDim.x) {
        const int mi = idx / (kD / 2), i = idx % (kD / 2);
        const int pos = p.cache_len + mi;
        if (pos < p0 || pos >= p0 + kC) continue;
        const int j = pos - p0;
        const float* kn = p.qkv + (int64_t)mi * ld + p.nh * kD + g * kD;
        const float* vn = p.qkv + (int64_t)mi * ld + (p.nh + p.nkv) * kD + g * kD;
        const float a = kn[i], b = kn[i + kD / 2];
        const float cs = rc[mi][i], sn = rs[mi][i];
        const float k0 = a * cs - b * sn, k1 = a * sn + b * cs;
        ks[j][i] = k0;
        ks[j][i + kD / 2] = k1;
        vs[j][i] = vn[i];
        vs[j][i + kD / 2] = vn[i + kD / 2];
        if (z != 0) continue;  // one slice writes the cache
        float* kd = p.k_cache + cbase + (int64_t)pos * kD;
        float* vd = p.v_cache + cbase + (int64_t)pos * kD;
        kd[i] = k0;
        kd[i + kD / 2] = k1;
        vd[i] = vn[i];
        vd[i + kD / 2] = vn[i + kD / 2];
    }
    __syncthreads();

    // 3. scores: thread = (position j, row-head block hb); one K row read
    //    serves every row-head hm = hb + 8r of the thread (masked: query row
    //    mi sees positions <= cache_len + mi)
    {
        const int j = t % kC, hb = t / kC;  // 8 blocks of row-heads
        const int pos = p0 + j;
        const float scale = 1.0f / sqrtf((float)kD);
        float acc[HMT / 8];
#pragma unroll
        for (int r = 0; r < HMT / 8; ++r) acc[r] = 0.0f;
        const float4* ka = reinterpret_cast<const float4*>(&ks[j][0]);
#pragma unroll 4
        for (int u = 0; u < kD / 4; ++u) {
            const float4 kv = ka[u];
#pragma unroll
            for (int r = 0; r < HMT / 8; ++r) {
                const int hm = hb + 8 * r;
                if (hm < HM) {
                    const float4 qv = reinterpret_cast<const float4*>(&qs[hm][0])[u];
                    acc[r] = fmaf(qv.x, kv.x, fmaf(qv.y, kv.y, fmaf(qv.z, kv.z, fmaf(qv.w, kv.w, acc[r]))));
                }
            }
        }
#pragma unroll
        for (int r = 0; r < HMT / 8; ++r) {
            const int hm = hb + 8 * r;
            if (hm < HM) sc[hm][j] = (pos <= p.cache_len + (hm0 + hm) / GQ) ? acc[r] * scale : -INFINITY;
        }
    }
    __syncthreads();

    // 4. chunk softmax statistics: a wave takes two row-heads at a time, one
    //    per 32-lane half, one position per lane
    for (int hp = 2 * wid; hp < HM; hp += 2 * (int)(blockDim.x / kWave)) {
        const int hm = hp + (lane >> 5);
        const bool ok = hm < HM;
        const float sv = ok ? sc[hm][lane & 31] : -INFINITY;
        float mx = sv;
        mx = half_max(mx);
        const float e = (mx == -INFINITY) ? 0.0f : __expf(sv - mx);
        float l = e;
        l = half_sum(l);
        if (ok) {
            sc[hm][lane & 31] = e;
            if ((lane & 31) == 0) {
                stat_m[hm] = mx;
                stat_l[hm] = l;
            }
        }
    }
    __syncthreads();

    // 5. unnormalised p*V: thread = (dim, half of the row-heads)
    float* out = p.part + (((int64_t)c * p.nkv + g) * HMall + hm0) * (kD + 2);
    {
        const int dd = t % kD, hh = t / kD;
        float acc[HMT / 2];
#pragma unroll
        for (int r = 0; r < HMT / 2; ++r) acc[r] = 0.0f;
        for (int j0 = 0; j0 < kC; j0 += 4) {
            const float v0 = vs[j0][dd], v1 = vs[j0 + 1][dd], v2 = vs[j0 + 2][dd], v3 = vs[j0 + 3][dd];
#pragma unroll
            for (int r = 0; r < HMT / 2; ++r) {
                const int hm = hh + 2 * r;
                if (hm < HM) {
                    const float4 pv = *reinterpret_cast<const float4*>(&sc[hm][j0]);
                    acc[r] = fmaf(pv.x, v0, fmaf(pv.y, v1, fmaf(pv.z, v2, fmaf(pv.w, v3, acc[r]))));
                }
            }
        }
#pragma unroll
        for (int r = 0; r < HMT / 2; ++r) {
            const int hm = hh + 2 * r;
            if (hm < HM) {
                out[hm * (kD + 2) + dd] = acc[r];
                if (dd == 0) {
                    out[hm * (kD + 2) + kD] = stat_m[hm];
                    out[hm * (kD + 2) + kD + 1] = stat_l[hm];
                }
            }
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
    const int hm = (p.nh / p.nkv) * p.m;
    const int Z = (hm + kSliceHM - 1) / kSliceHM;
    const int pairs = p.chunks * p.nkv;
    const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * Z)), block(256);
    if (hm <= 8)
        hipLaunchKernelGGL(k_attn_partial<8>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(k_attn_partial<kSliceHM>, grid, block, 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int HM = (p.nh / p.nkv) * p.m;
    hipLaunchKernelGGL(k_attn_combine, dim3(p.nkv, HM, kD / kCombDims), dim3(kCombLanes * kCombDims), 0, st, p);
    return hipGetLastError();
}

}  // namespace mtp
