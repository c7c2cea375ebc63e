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
// and v into the cache.  The scores and the p*V sums are f32 matrix-core
// products over 16-row tiles of row-heads.  It emits per (chunk, query
// row-head) the chunk maximum, the exp-sum and the unnormalised sum of p*V.
// Kernel 2 (grid: KV heads x query row-heads) merges the chunks with the
// log-sum-exp rule.
// Variant steps of the same function (when set): per-head RMSNorm of q and
// of the new k before the rotary step, a rotary step over the first rot
// dims only, and the output multiplied by sigmoid(gate) in kernel 2, the
// gate values of a head following its q values in the projection output.
// Sliding window and sinks (cortiq-engine mimo_mtp.rs, module doc "The draft
// forward": window 128, sinks): with a window W the row at position p sees
// positions p-W+1 .. p (a score mask in kernel 1, and the chunks before the
// first row's window are not launched: partials are stored from chunk c0
// on); a head's sink logit starts kernel 2's merge as a (max = sink,
// exp-sum = 1, p*V = 0) term.  With a window the m-row call and m single-row
// calls may merge the same chunk terms in another order (c0 follows the
// first row), so they agree to rounding rather than bitwise.
#include <cmath>

#include "device.hpp"
#include "launch.hpp"

namespace mtp {

constexpr int kD = 128;           // head_dim handled here
constexpr int kC = kAttnChunk;    // positions per block
constexpr int kKStride = kD + 4;  // padded LDS row (floats)
constexpr int kSliceHM = 16;      // query row-heads per partial block, at most
constexpr int kAttnThreads = 256;  // threads of a partial block (the launch's block size)
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
    if (pair >= (p.chunks - p.c0) * p.nkv) return false;
    c = p.c0 + pair / p.nkv;
    g = pair % p.nkv;
    return true;
}

// The launch parameters the first requests of a block depend on, named in one
// empty asm statement as scalar operands, so that their loads are issued
// together and waited for once (loaded where first used, the block mapping's
// fields, then the cache pointers, take one round trip after another).
__device__ __forceinline__ void gather_attn(const AttnParams& p) {
    asm volatile("" ::"s"(p.qkv), "s"(p.k_cache), "s"(p.v_cache), "s"(p.cache_len), "s"(p.capacity), "s"(p.m),
                 "s"(p.nh), "s"(p.nkv), "s"(p.part), "s"(p.o), "s"(p.chunks), "s"(p.qg), "s"(p.sinks), "s"(p.c0));
}

// Local row-head hl of slice z is the group's row-head z * kSliceHM + hl
// (= mi * GQ + local query head).
typedef float v4f_t __attribute__((ext_vector_type(4)));
// VAR: the per-head norm and partial rotary steps are compiled in (the
// plain attention runs without them).
template <bool VAR>
__global__ void __launch_bounds__(kAttnThreads) k_attn_partial(const AttnParams p) {
    __shared__ float qs[kSliceHM][kKStride];  // padded rows: the score reads of 16 rows spread over the banks
    __shared__ float ks[kC][kKStride];
    __shared__ float vs[kC][kD];
    __shared__ float sc[kSliceHM][kSStride];
    __shared__ float spart[2][kSliceHM][kSStride];  // score halves (dims 0-63, 64-127)
    __shared__ float rc[8][kD / 2], rs[8][kD / 2];  // rotary cos/sin per new row

    gather_attn(p);
    const int GQ = p.nh / p.nkv;
    const int HMall = GQ * p.m;
    const int Z = (HMall + kSliceHM - 1) / kSliceHM;
    int c, g, z;
    if (!attn_block(p, Z, c, g, z)) return;
    const int hm0 = z * kSliceHM;
    const int HM = HMall - hm0 < kSliceHM ? HMall - hm0 : kSliceHM;  // row-heads of this block
    const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
    const int ld = (p.qg * p.nh + 2 * p.nkv) * kD;  // qkv row stride
    const int p0 = c * kC;
    const int64_t cbase = (int64_t)g * p.capacity * kD;
    constexpr int kQuads = kC * (kD / 4) / 256;  // float4 slots of K (and of V) per thread

    // 1. every global read of the block is requested up front, so that the
    //    block waits for memory once: the chunk's cached K/V rows, the query
    //    pairs (i, i + d/2) of its row-heads and the new k/v rows it owns
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
    constexpr int kQPairs = kSliceHM * (kD / 2) / 256;  // query pairs per thread
    float qa[kQPairs], qb[kQPairs];
#pragma unroll
    for (int u = 0; u < kQPairs; ++u) {
        const int idx = t + 256 * u, hm = idx / (kD / 2), i = idx % (kD / 2);
        qa[u] = 0.0f;
        qb[u] = 0.0f;
        if (hm < HM) {
            const int mi = (hm0 + hm) / GQ, hq = g * GQ + (hm0 + hm) % GQ;
            const float* q = p.qkv + (int64_t)mi * ld + hq * p.qg * kD;
            qa[u] = q[i];
            qb[u] = q[i + kD / 2];
        }
    }
    constexpr int kNPairs = 8 * (kD / 2) / 256;  // new-row pairs per thread (m <= 8)
    float ka[kNPairs], kb[kNPairs], va[kNPairs], vb[kNPairs];
#pragma unroll
    for (int u = 0; u < kNPairs; ++u) {
        const int idx = t + 256 * u, mi = idx / (kD / 2), i = idx % (kD / 2);
        const int pos = p.cache_len + mi;
        ka[u] = kb[u] = va[u] = vb[u] = 0.0f;
        if (mi < p.m && pos >= p0 && pos < p0 + kC) {
            const float* kn = p.qkv + (int64_t)mi * ld + p.qg * p.nh * kD + g * kD;
            const float* vn = p.qkv + (int64_t)mi * ld + (p.qg * p.nh + p.nkv) * kD + g * kD;
            ka[u] = kn[i];
            kb[u] = kn[i + kD / 2];
            va[u] = vn[i];
            vb[u] = vn[i + kD / 2];
        }
    }
    // per-head norm weights of this lane's pair (i, i + d/2), i = lane
    float gqa = 1.0f, gqb = 1.0f, gka = 1.0f, gkb = 1.0f;
    if (VAR && p.gq) {
        gqa = p.gq[lane];
        gqb = p.gq[lane + kD / 2];
        gka = p.gk[lane];
        gkb = p.gk[lane + kD / 2];
    }
    // ... and the rotary table for positions cache_len + mi is built meanwhile
    const int rot = VAR ? p.rot : kD;
    const int rh = rot / 2;  // rotated pairs (i, i + rot/2), i < rh
    for (int idx = t; idx < p.m * rh; idx += kAttnThreads) {
        const int mi = idx / rh, i = idx % rh;
        const double inv_freq = exp2(-(2.0 * (double)i / (double)rot) * p.log2_theta);
        const int pos = (VAR && p.positions) ? p.positions[4 * mi + imrope_sec(i, p.sec)] : p.cache_len + mi;
        rotary((double)pos, inv_freq, rc[mi][i], rs[mi][i]);
    }
    __syncthreads();

    // per-head RMSNorm of q and of the new k: a wave holds one row-head (or
    // one new k row) per load slot, lane i its dims i and i + d/2
    if (VAR && p.gq) {
#pragma unroll
        for (int u = 0; u < kQPairs; ++u) {
            const float inv = rsqrtf(wave_sum(qa[u] * qa[u] + qb[u] * qb[u]) * (1.0f / kD) + p.eps);
            qa[u] = qa[u] * inv * gqa;
            qb[u] = qb[u] * inv * gqb;
        }
#pragma unroll
        for (int u = 0; u < kNPairs; ++u) {
            const float inv = rsqrtf(wave_sum(ka[u] * ka[u] + kb[u] * kb[u]) * (1.0f / kD) + p.eps);
            ka[u] = ka[u] * inv * gka;
            kb[u] = kb[u] * inv * gkb;
        }
    }
    // Rotation of a pair-loaded row (lane i holds dims i and i + d/2): over
    // all dims the pair is the lane's own; over rot < d dims, dim i < rot
    // pairs with dim i ^ (rot/2) in the neighbouring lane, and dims from rot
    // on pass unchanged.
    auto rotate = [&](float a, float b, int mi, float& ra, float& rb) {
        if (rot == kD) {
            const float cs = rc[mi][lane], sn = rs[mi][lane];
            ra = a * cs - b * sn;
            rb = a * sn + b * cs;
        } else {
            const float o = __shfl_xor(a, rh);
            const int j = lane & (rh - 1);
            const float cs = rc[mi][j], sn = rs[mi][j];
            ra = lane >= rot ? a : (lane < rh ? a * cs - o * sn : o * sn + a * cs);
            rb = b;
        }
    };

    // 2. rotated queries of this group (hm = mi * GQ + local head), cached
    //    rows into LDS, rows past the new ones zeroed, the new rows rotated and
    //    appended to the cache (only by the chunk that owns them)
#pragma unroll
    for (int u = 0; u < kQPairs; ++u) {
        const int idx = t + 256 * u, hm = idx / (kD / 2), i = idx % (kD / 2);
        const int mi = hm < HM ? (hm0 + hm) / GQ : 0;
        float ra, rb;
        rotate(qa[u], qb[u], mi, ra, rb);
        if (hm < HM) {
            qs[hm][i] = ra;
            qs[hm][i + kD / 2] = rb;
        }
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
#pragma unroll
    for (int u = 0; u < kNPairs; ++u) {
        const int idx = t + 256 * u, mi = idx / (kD / 2), i = idx % (kD / 2);
        const int pos = p.cache_len + mi;
        float k0, k1;
        rotate(ka[u], kb[u], mi < p.m ? mi : 0, k0, k1);
        if (mi < p.m && pos >= p0 && pos < p0 + kC) {
            const int j = pos - p0;
            ks[j][i] = k0;
            ks[j][i + kD / 2] = k1;
            vs[j][i] = va[u];
            vs[j][i + kD / 2] = vb[u];
            if (z == 0) {  // one slice writes the cache
                float* kd = p.k_cache + cbase + (int64_t)pos * kD;
                float* vd = p.v_cache + cbase + (int64_t)pos * kD;
                kd[i] = k0;
                kd[i + kD / 2] = k1;
                vd[i] = va[u];
                vd[i + kD / 2] = vb[u];
            }
        }
    }
    __syncthreads();

    // 3. scores on the matrix cores (16x16x4 f32): a 16 x 16 tile of
    //    (row-head, position) per wave and half of the dims (wave w: positions
    //    16 (w & 1) .., dims 64 (w >> 1) ..); row-heads past HM read as zero.
    //    Lane l supplies row l % 16 of each operand and, over four products,
    //    the four dims 4 (l / 16) .. of every 16.
    const int r16 = lane & 15, kq = lane >> 4;
    const float4 zero4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    {
        const int jt = wid & 1, dh = wid >> 1;
        v4f_t acc[4];  // four independent product chains
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int d = 64 * dh + 16 * s2 + 4 * kq;
            const float4 a = r16 < HM ? *reinterpret_cast<const float4*>(&qs[r16][d]) : zero4;
            const float4 b = *reinterpret_cast<const float4*>(&ks[16 * jt + r16][d]);
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc[1], 0, 0, 0);
            acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc[2], 0, 0, 0);
            acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc[3], 0, 0, 0);
        }
        const v4f_t sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        // result lane l, register r: row-head 4 (l / 16) + r, position l % 16
#pragma unroll
        for (int r = 0; r < 4; ++r) spart[dh][4 * kq + r][16 * jt + r16] = sum[r];
    }
    __syncthreads();

    // 4. chunk softmax statistics: a wave takes two row-heads at a time, one
    //    per 32-lane half, one position per lane (masked: query row mi sees
    //    positions <= cache_len + mi)
    float* out = p.part + (((int64_t)(c - p.c0) * p.nkv + g) * HMall + hm0) * (kD + 2);
    const float scale = 1.0f / sqrtf((float)kD);
    for (int hp = 2 * wid; hp < HM; hp += 2 * (kAttnThreads / kWave)) {
        const int hm = hp + (lane >> 5), j = lane & 31;
        const int qpos = p.cache_len + (hm0 + hm) / GQ;  // the row's position
        const bool ok = hm < HM && p0 + j <= qpos && (p.window == 0 || p0 + j > qpos - p.window);
        const float sv = ok ? (spart[0][hm][j] + spart[1][hm][j]) * scale : -INFINITY;
        float mx = sv;
        mx = half_max(mx);
        const float e = (mx == -INFINITY) ? 0.0f : __expf(sv - mx);
        float l = e;
        l = half_sum(l);
        if (hm < HM) {
            sc[hm][j] = e;
            if (j == 0) {
                out[hm * (kD + 2) + kD] = mx;
                out[hm * (kD + 2) + kD + 1] = l;
            }
        }
    }
    __syncthreads();

    // 5. unnormalised p*V on the matrix cores: wave w takes the dims
    //    32 w .. 32 w + 31 as two 16-dim tiles, the positions as the product
    //    dimension (lane l supplies positions 4 (l / 16) .. of every 16)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
        const int d0 = 16 * (2 * wid + t2);
        v4f_t acc[2];  // two independent product chains
#pragma unroll
        for (int e = 0; e < 2; ++e) acc[e] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int j = 16 * s2 + 4 * kq;
            const float4 a = r16 < HM ? *reinterpret_cast<const float4*>(&sc[r16][j]) : zero4;
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, vs[j][d0 + r16], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, vs[j + 1][d0 + r16], acc[1], 0, 0, 0);
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, vs[j + 2][d0 + r16], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, vs[j + 3][d0 + r16], acc[1], 0, 0, 0);
        }
        const v4f_t sum = acc[0] + acc[1];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hm = 4 * kq + r;
            if (hm < HM) out[hm * (kD + 2) + d0 + r16] = sum[r];
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
    gather_attn(p);
    const int g = blockIdx.x, hm = blockIdx.y;
    const int t = threadIdx.x, dl = t % kCombDims, cs = t / kCombDims;
    const int dd = blockIdx.z * kCombDims + dl;
    const int GQ = p.nh / p.nkv;
    const int HM = GQ * p.m;
    const int mi = hm / GQ, hq = g * GQ + hm % GQ;
    const int64_t stride = (int64_t)p.nkv * HM * (kD + 2);  // between chunks
    const float* base = p.part + ((int64_t)g * HM + hm) * (kD + 2);

    // the first batch of partials is requested before anything else: the
    // head's sink and gate values go out behind it (the sink is a scalar
    // load, and waiting for it would also wait for the parameters)
    const int nch = p.chunks - p.c0;  // partials stored from chunk c0 on
    // The 64 lanes of a wave take one dim each of the same chunks, so a
    // chunk's (max, exp-sum) pair is the same for all of them: lane u of the
    // wave requests the pair of the batch's chunk u (one load for the batch
    // instead of two per chunk, each a request of its own), and the merge
    // reads the pairs back with readlane.
    static_assert(kCombDims == kWave && kCombBatch <= kWave, "one wave per chunk lane");
    float2 ml;
    float av[kCombBatch];
    auto request = [&](int c0) {
        const int cl = c0 + (dl < kCombBatch ? dl : 0) * kCombLanes;
        ml = *reinterpret_cast<const float2*>(base + (int64_t)(cl < nch ? cl : 0) * stride + kD);
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const int c = c0 + u * kCombLanes;
            av[u] = base[(int64_t)(c < nch ? c : 0) * stride + dd];
        }
    };
    request(cs);
    float gv = 0.0f;
    if (p.qg == 2 && cs == 0) gv = p.qkv[(int64_t)mi * (2 * p.nh + 2 * p.nkv) * kD + (2 * hq + 1) * kD + dd];
    // the head's sink is a logit with no value row: lane 0 starts from it
    float M = -INFINITY, L = 0.0f, A = 0.0f;
    if (p.sinks && cs == 0) {
        M = p.sinks[hq];
        L = 1.0f;
    }
    for (int c0 = cs;;) {
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const float m2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.x), u));
            float l2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.y), u));
            if (c0 + u * kCombLanes >= nch) l2 = 0.0f;
            lse_merge(M, L, A, m2, l2, av[u]);
        }
        c0 += kCombLanes * kCombBatch;
        if (c0 >= nch) break;
        request(c0);
    }
    sm[cs][dl] = M;
    sl[cs][dl] = L;
    sa[cs][dl] = A;
    __syncthreads();
    if (cs == 0) {
        for (int j = 1; j < kCombLanes; ++j) lse_merge(M, L, A, sm[j][dl], sl[j][dl], sa[j][dl]);
        float o = L > 0.0f ? A / L : 0.0f;
        if (p.qg == 2) o = o / (1.0f + __expf(-gv));  // sigmoid gate (the head's gate values follow its q values)
        p.o[(int64_t)mi * p.nh * kD + hq * kD + dd] = o;
    }
}

// ---------------------------------------------------------------------------
// Cache catch-up after a target batch ([mtp.rs] `process_target_batch`,
// `append_attention_kv`): the K/V side of the attention alone.
// ---------------------------------------------------------------------------
// The hidden rows of a batch's first piece, shifted one row right: row 0 is
// the pending hidden (zero when there is none), row r the target's row r-1.
__global__ void __launch_bounds__(256) k_shift_rows(const float* pending, const float* target, float* out, int m,
                                                    int H) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)m * H) return;
    const int r = (int)(idx / H), c = (int)(idx % H);
    out[idx] = r == 0 ? (pending ? pending[c] : 0.0f) : target[(int64_t)(r - 1) * H + c];
}

// One wave per (row, KV head): lane i holds dims i and i + d/2 of the row's k
// (kv [m][2 nkv d]: k heads, then v heads), applies the per-head norm and the
// rotary step at position pos0 + row exactly as k_attn_partial does for a new
// row, and writes k and v into the cache.
template <bool VAR>
__global__ void __launch_bounds__(64) k_append_kv(const AttnParams p, const float* kv, int pos0) {
    const int r = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const float* kr = kv + (int64_t)r * 2 * p.nkv * kD + g * kD;
    const float* vr = kr + p.nkv * kD;
    float a = kr[lane], b = kr[lane + kD / 2];
    const float va = vr[lane], vb = vr[lane + kD / 2];
    if (VAR && p.gk) {
        const float inv = rsqrtf(wave_sum(a * a + b * b) * (1.0f / kD) + p.eps);
        a = a * inv * p.gk[lane];
        b = b * inv * p.gk[lane + kD / 2];
    }
    const int pos = pos0 + r;
    const int rot = VAR ? p.rot : kD, rh = rot / 2;
    // rotary position of pair j (the row's ids, offset by the piece's first row)
    auto rpos = [&](int j) { return (VAR && p.positions) ? p.positions[4 * r + imrope_sec(j, p.sec)] : pos; };
    float ra, rb;
    if (rot == kD) {
        float cs, sn;
        rotary((double)rpos(lane), exp2(-(2.0 * (double)lane / (double)kD) * p.log2_theta), cs, sn);
        ra = a * cs - b * sn;
        rb = a * sn + b * cs;
    } else {
        const float o = __shfl_xor(a, rh);
        const int j = lane & (rh - 1);
        float cs, sn;
        rotary((double)rpos(j), exp2(-(2.0 * (double)j / (double)rot) * p.log2_theta), cs, sn);
        ra = lane >= rot ? a : (lane < rh ? a * cs - o * sn : o * sn + a * cs);
        rb = b;
    }
    float* kd = p.k_cache + ((int64_t)g * p.capacity + pos) * kD;
    float* vd = p.v_cache + ((int64_t)g * p.capacity + pos) * kD;
    kd[lane] = ra;
    kd[lane + kD / 2] = rb;
    vd[lane] = va;
    vd[lane + kD / 2] = vb;
}

// ---------------------------------------------------------------------------
// Wide geometry (cortiq-engine mimo_mtp.rs, module doc "The draft forward":
// q/k heads of 192 with V heads of 128): q/k rows of p.d floats, V rows of
// p.vd.  Plain f32 arithmetic, one block per (chunk, KV head, slice of up to
// kSliceHM row-heads) as in k_attn_partial, emitting the same records (p*V
// sums over the V dims, then the chunk maximum and exp-sum), so the same
// combine merges them.  Rotary pairs (i, i + rot/2) over the first rot dims;
// window and sinks as in k_attn_partial; no per-head norms or gate (the caller
// rejects them for this geometry).
// ---------------------------------------------------------------------------
constexpr int kWideKD = 192;  // q/k head dims at most
constexpr int kWideVD = 128;  // V head dims at most

__global__ void __launch_bounds__(kAttnThreads) k_attn_partial_wide(const AttnParams p) {
    __shared__ __align__(16) float qs[kSliceHM][kWideKD];
    __shared__ float ks[kC][kWideKD + 1];  // odd row stride: the score loop reads a column per lane
    __shared__ __align__(16) float vs[kC][kWideVD];
    __shared__ float sc[kSliceHM][kC + 1];
    __shared__ float rc[8][kWideKD / 2], rs[8][kWideKD / 2];

    const int KD = p.d, VD = p.vd;
    const int GQ = p.nh / p.nkv;
    const int HMall = GQ * p.m;
    const int Z = (HMall + kSliceHM - 1) / kSliceHM;
    int c, g, z;
    if (!attn_block(p, Z, c, g, z)) return;
    const int hm0 = z * kSliceHM;
    const int HM = HMall - hm0 < kSliceHM ? HMall - hm0 : kSliceHM;
    const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
    const int ld = (p.nh + p.nkv) * KD + p.nkv * VD;  // qkv row stride
    const int p0 = c * kC;
    const int rot = p.rot, rh = rot / 2;

    // 1. every global read of the block is requested up front (the chunk's
    //    cached K/V rows and the raw query rows, as float4), so the block
    //    waits for memory once; rows at or past cache_len are filled below
    constexpr int kKQ = kC * kWideKD / 4 / 256;  // float4 of K per thread at most
    constexpr int kVQ = kC * kWideVD / 4 / 256;
    constexpr int kQQ = kSliceHM * kWideKD / 4 / 256;
    const int KD4 = KD / 4, VD4 = VD / 4;
    const float4 zero4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float4 kq[kKQ], vq[kVQ], qq[kQQ];
#pragma unroll
    for (int u = 0; u < kKQ; ++u) {
        const int idx = t + 256 * u, j = idx / KD4, w = idx % KD4, pos = p0 + j;
        kq[u] = zero4;
        if (idx < kC * KD4 && pos < p.cache_len)
            kq[u] = reinterpret_cast<const float4*>(p.k_cache + ((int64_t)g * p.capacity + pos) * KD)[w];
    }
#pragma unroll
    for (int u = 0; u < kVQ; ++u) {
        const int idx = t + 256 * u, j = idx / VD4, w = idx % VD4, pos = p0 + j;
        vq[u] = zero4;
        if (idx < kC * VD4 && pos < p.cache_len)
            vq[u] = reinterpret_cast<const float4*>(p.v_cache + ((int64_t)g * p.capacity + pos) * VD)[w];
    }
#pragma unroll
    for (int u = 0; u < kQQ; ++u) {
        const int idx = t + 256 * u, hm = idx / KD4, w = idx % KD4;
        qq[u] = zero4;
        if (hm < HM) {
            const int mi = (hm0 + hm) / GQ, hq = g * GQ + (hm0 + hm) % GQ;
            qq[u] = reinterpret_cast<const float4*>(p.qkv + (int64_t)mi * ld + hq * KD)[w];
        }
    }
    // ... the rotary table of the new rows' positions meanwhile
    for (int idx = t; idx < p.m * rh; idx += kAttnThreads) {
        const int mi = idx / rh, i = idx % rh;
        const double inv_freq = exp2(-(2.0 * (double)i / (double)rot) * p.log2_theta);
        rotary((double)(p.cache_len + mi), inv_freq, rc[mi][i], rs[mi][i]);
    }
    // 2. raw rows into LDS (the new rows this chunk owns from the projection
    //    output), then the rotation of q and the new k rows in place, pair by
    //    pair; slice 0 writes the new rows to the cache
#pragma unroll
    for (int u = 0; u < kKQ; ++u) {
        const int idx = t + 256 * u, j = idx / KD4, w = idx % KD4;
        if (idx < kC * KD4) {
            ks[j][4 * w] = kq[u].x;
            ks[j][4 * w + 1] = kq[u].y;
            ks[j][4 * w + 2] = kq[u].z;
            ks[j][4 * w + 3] = kq[u].w;
        }
    }
#pragma unroll
    for (int u = 0; u < kVQ; ++u) {
        const int idx = t + 256 * u, j = idx / VD4, w = idx % VD4;
        if (idx < kC * VD4) *reinterpret_cast<float4*>(&vs[j][4 * w]) = vq[u];
    }
#pragma unroll
    for (int u = 0; u < kQQ; ++u) {
        const int idx = t + 256 * u, hm = idx / KD4, w = idx % KD4;
        if (hm < HM) *reinterpret_cast<float4*>(&qs[hm][4 * w]) = qq[u];
    }
    __syncthreads();
    for (int idx = t; idx < p.m * KD; idx += kAttnThreads) {
        const int mi = idx / KD, d = idx % KD, pos = p.cache_len + mi;
        if (pos >= p0 && pos < p0 + kC) ks[pos - p0][d] = p.qkv[(int64_t)mi * ld + p.nh * KD + g * KD + d];
    }
    for (int idx = t; idx < p.m * VD; idx += kAttnThreads) {
        const int mi = idx / VD, d = idx % VD, pos = p.cache_len + mi;
        if (pos >= p0 && pos < p0 + kC) {
            const float vval = p.qkv[(int64_t)mi * ld + (p.nh + p.nkv) * KD + g * VD + d];
            vs[pos - p0][d] = vval;
            if (z == 0) p.v_cache[((int64_t)g * p.capacity + pos) * VD + d] = vval;
        }
    }
    __syncthreads();
    auto rotate_pair = [&](float* x, int i, int mi) {  // dims i and i + rh, i < rh
        const float a = x[i], b = x[i + rh], cs = rc[mi][i], sn = rs[mi][i];
        x[i] = a * cs - b * sn;
        x[i + rh] = a * sn + b * cs;
    };
    for (int idx = t; idx < HM * rh; idx += kAttnThreads) {
        const int hm = idx / rh, i = idx % rh;
        rotate_pair(qs[hm], i, (hm0 + hm) / GQ);
    }
    for (int idx = t; idx < p.m * rh; idx += kAttnThreads) {
        const int mi = idx / rh, i = idx % rh, pos = p.cache_len + mi;
        if (pos >= p0 && pos < p0 + kC) rotate_pair(ks[pos - p0], i, mi);
    }
    __syncthreads();
    if (z == 0)
        for (int idx = t; idx < p.m * KD; idx += kAttnThreads) {
            const int mi = idx / KD, d = idx % KD, pos = p.cache_len + mi;
            if (pos >= p0 && pos < p0 + kC) p.k_cache[((int64_t)g * p.capacity + pos) * KD + d] = ks[pos - p0][d];
        }

    // scores
    const float scale = 1.0f / sqrtf((float)KD);
    for (int idx = t; idx < HM * kC; idx += kAttnThreads) {
        const int hm = idx / kC, j = idx % kC;
        float sv = 0.0f;
        for (int d = 0; d < KD; ++d) sv = fmaf(qs[hm][d], ks[j][d], sv);
        sc[hm][j] = sv * scale;
    }
    __syncthreads();

    // chunk softmax statistics (causal, window), as in k_attn_partial
    float* out = p.part + (((int64_t)(c - p.c0) * p.nkv + g) * HMall + hm0) * (VD + 2);
    for (int hp = 2 * wid; hp < HM; hp += 2 * (kAttnThreads / kWave)) {
        const int hm = hp + (lane >> 5), j = lane & 31;
        const int qpos = p.cache_len + (hm0 + hm) / GQ;
        const bool ok = hm < HM && p0 + j <= qpos && (p.window == 0 || p0 + j > qpos - p.window);
        const float sv = ok ? sc[hm][j] : -INFINITY;
        float mx = sv;
        mx = half_max(mx);
        const float e = (mx == -INFINITY) ? 0.0f : __expf(sv - mx);
        float l = e;
        l = half_sum(l);
        if (hm < HM) {
            sc[hm][j] = e;
            if (j == 0) {
                out[hm * (VD + 2) + VD] = mx;
                out[hm * (VD + 2) + VD + 1] = l;
            }
        }
    }
    __syncthreads();

    // unnormalised p*V
    for (int idx = t; idx < HM * VD; idx += kAttnThreads) {
        const int hm = idx / VD, d = idx % VD;
        float acc = 0.0f;
        for (int j = 0; j < kC; ++j) acc = fmaf(sc[hm][j], vs[j][d], acc);
        out[hm * (VD + 2) + d] = acc;
    }
}

// Catch-up of the wide geometry: one wave per (row, KV head); kv rows are
// [m][n_kv*d k values | n_kv*vd v values].
__global__ void __launch_bounds__(64) k_append_kv_wide(const AttnParams p, const float* kv, int pos0) {
    const int r = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const int KD = p.d, VD = p.vd, rot = p.rot, rh = rot / 2;
    const float* kr = kv + (int64_t)r * p.nkv * (KD + VD) + g * KD;
    const float* vr = kv + (int64_t)r * p.nkv * (KD + VD) + p.nkv * KD + g * VD;
    const int pos = pos0 + r;
    float* kd = p.k_cache + ((int64_t)g * p.capacity + pos) * KD;
    float* vd = p.v_cache + ((int64_t)g * p.capacity + pos) * VD;
    for (int d = lane; d < KD; d += kWave) {
        float val = kr[d];
        if (d < rot) {
            const int i = d < rh ? d : d - rh;
            float cs, sn;
            rotary((double)pos, exp2(-(2.0 * (double)i / (double)rot) * p.log2_theta), cs, sn);
            val = d < rh ? kr[d] * cs - kr[d + rh] * sn : kr[i] * sn + kr[d] * cs;
        }
        kd[d] = val;
    }
    for (int d = lane; d < VD; d += kWave) vd[d] = vr[d];
}

hipError_t launch_shift_rows(const float* pending, const float* target, float* out, int m, int H, hipStream_t st) {
    const int64_t n = (int64_t)m * H;
    hipLaunchKernelGGL(k_shift_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pending, target, out, m, H);
    return hipGetLastError();
}

hipError_t launch_append_kv(const AttnParams& p, const float* kv, int m, int pos0, hipStream_t st) {
    const dim3 grid((unsigned)m, (unsigned)p.nkv), block(kWave);
    if (p.d != kD || p.vd != kD) {
        if (p.d > kWideKD || p.vd > kWideVD || p.rot > p.d || p.gk || p.positions) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_append_kv_wide, grid, block, 0, st, p, kv, pos0);
        return hipGetLastError();
    }
    if (p.gk || p.rot != kD || p.positions)
        hipLaunchKernelGGL(k_append_kv<true>, grid, block, 0, st, p, kv, pos0);
    else
        hipLaunchKernelGGL(k_append_kv<false>, grid, block, 0, st, p, kv, pos0);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, hipStream_t st) {
    const int hm = (p.nh / p.nkv) * p.m;
    const int Z = (hm + kSliceHM - 1) / kSliceHM;
    const int pairs = (p.chunks - p.c0) * p.nkv;
    const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * Z)), block(kAttnThreads);
    if (p.d != kD || p.vd != kD) {
        // the combine below reads records of kD + 2 floats: V heads of kD
        if (p.d > kWideKD || p.vd != kD || p.rot > p.d || p.gq || p.qg != 1 || p.m > 8 || p.positions)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_attn_partial_wide, grid, block, 0, st, p);
    } else if (p.gq || p.rot != kD || p.positions)
        hipLaunchKernelGGL(k_attn_partial<true>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(k_attn_partial<false>, grid, block, 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int HM = (p.nh / p.nkv) * p.m;
    hipLaunchKernelGGL(k_attn_combine, dim3(p.nkv, HM, kD / kCombDims), dim3(kCombLanes * kCombDims), 0, st, p);
    return hipGetLastError();
}

}  // namespace mtp
