// gemv.hip -- quantized GEMV kernels for m <= 8 activation rows (gfx950).
//
// One kernel template covers every weight-streaming op of the draft layer:
// the plain linear, the eh_proj with its two fused RMSNorms and virtual
// concat, the fused attention-norm + q/k/v projection, the SwiGLU gate/up
// pair, the MoE expert slots and the lm_head with its fused final norm and
// first argmax pass.  See device.hpp for the lane/group scheme.
#include <climits>
#include <cmath>

#include "device.hpp"
#include "launch.hpp"

namespace mtp {

// The matrices, sizes and row pointers one block works on (scalars only, so
// the whole view stays in registers).
struct View {
    const void *c0, *c1;
    const float *s0, *s1;
    const float *b0, *b1;
    int64_t dc1, dc2, ds1, ds2, db1, db2;  // byte distances matrix 0->1 and 1->2
    int n0, n1;
    int N, K, G;
    const float* x0;
    float* y;
    const float* rowscale;
};

__device__ __forceinline__ bool resolve_view(const GemvParams& p, View& v) {
    v.c0 = p.w[0].codes;
    v.s0 = p.w[0].scales;
    v.b0 = p.w[0].biases;
    v.c1 = p.w[1].codes;
    v.s1 = p.w[1].scales;
    v.b1 = p.w[1].biases;
    auto dist = [](const void* a, const void* b) -> int64_t {
        return (int64_t)(reinterpret_cast<uintptr_t>(b) - reinterpret_cast<uintptr_t>(a));
    };
    v.dc1 = dist(p.w[0].codes, p.w[1].codes);
    v.dc2 = dist(p.w[1].codes, p.w[2].codes);
    v.ds1 = dist(p.w[0].scales, p.w[1].scales);
    v.ds2 = dist(p.w[1].scales, p.w[2].scales);
    v.db1 = dist(p.w[0].biases, p.w[1].biases);
    v.db2 = dist(p.w[1].biases, p.w[2].biases);
    v.n0 = p.w[0].n;
    v.n1 = p.w[1].n;
    v.N = p.N;
    v.K = p.K;
    v.G = p.G;
    v.x0 = p.x0;
    v.y = p.y;
    v.rowscale = p.rowscale;
    if (p.slot_expert) {
        const int slot = blockIdx.y;
        if (slot >= *p.n_slots) return false;
        const int e = p.slot_expert[slot];
        if (e >= 0) {
            v.c0 = static_cast<const char*>(p.w[0].codes) + p.ex_codes * e;
            v.s0 = p.w[0].scales + p.ex_scales * e;
            v.c1 = static_cast<const char*>(p.w[1].codes) + p.ex_codes * e;
            v.s1 = p.w[1].scales + p.ex_scales * e;
        } else {
            v.c0 = p.shw[0].codes;
            v.s0 = p.shw[0].scales;
            v.c1 = p.shw[1].codes;
            v.s1 = p.shw[1].scales;
            v.N = p.N_sh;
            v.K = p.K_sh;
            v.G = p.K_sh / kGroup;
        }
        v.x0 = p.x0 + p.x_slot * slot;
        v.y = p.y + p.y_slot * slot;
        if (p.rowscale) v.rowscale = p.rowscale + p.rs_slot * slot;
    }
    return true;
}

// Requests the lane's 32 activation features of row mi (for PRO_CONCAT: from
// the embedding rows, the token table or the hidden rows, by the lane's
// half of the virtual concat) and, when want_g, the matching gamma.
template <int PRO>
__device__ __forceinline__ void load_x_row(const GemvParams& p, const View& v, int mi, int kk, bool active,
                                           float (&xv)[32], float (&gv)[32], bool want_g) {
    int seg = 0, kl = kk;
    const float* src;
    const float* gam = p.g0;
    if constexpr (PRO == PRO_CONCAT) {
        seg = kk >= p.H ? 1 : 0;
        kl = seg ? kk - p.H : kk;
        if (seg) {
            src = p.x1 + (int64_t)mi * p.H;
            gam = p.g1;
        } else {
            src = v.x0 + (int64_t)mi * p.H;
            if (p.tokens && mi < p.m) {
                int tok = p.tokens[mi];
                if (tok >= 0 || v.x0 == nullptr) {  // no e rows given: every row is a token
                    tok = tok < 0 ? 0 : (tok < p.vocab ? tok : p.vocab - 1);
                    src = p.table + (int64_t)tok * p.H;
                }
            }
        }
    } else {
        src = v.x0 + (int64_t)mi * v.K;
    }
    if (active && mi < p.m) {
        load32(xv, src + kl);
        if constexpr (PRO != PRO_PLAIN)
            if (want_g) load32(gv, gam + kl);  // both requests in flight together
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            xv[i] = 0.0f;
            if (PRO != PRO_PLAIN && want_g) gv[i] = 0.0f;
        }
    }
}

// 16-bit activation quantization without a float-to-int conversion: adding
// 1.5 * 2^23 + 128 to the product x * inv (rounded first, as in split16)
// leaves q + 128 + 0x400000 in the low mantissa bits, rounded to nearest
// even exactly as split16 rounds, for |q| < 2^22.  Byte 1 of the result is
// then hi = (q + 128) >> 8 and byte 0 is lo = q - 256 hi with its sign bit
// flipped, and the bits of several values sum to sum(q) plus a known
// multiple of kQBiasBits.
constexpr float kQBias = 12583040.0f;  // 1.5 * 2^23 + 128
constexpr unsigned kQBiasBits = 0x4B400080u;
__device__ __forceinline__ unsigned q_bits(float x, float inv) {
#pragma clang fp contract(off)
    const float y = x * inv;
    return __float_as_uint(y + kQBias);
}

// Row mi's input for the features of segment seg (PRO_CONCAT: 0 = the
// embedding row, or the token's table row, 1 = the hidden row; otherwise the
// one input row) and the matching gamma.
template <int PRO>
__device__ __forceinline__ const float* x_segment(const GemvParams& p, const View& v, int mi, int seg,
                                                  const float*& gam) {
    if constexpr (PRO == PRO_CONCAT) {
        if (seg) {
            gam = p.g1;
            return p.x1 + (int64_t)mi * p.H;
        }
        gam = p.g0;
        if (p.tokens) {
            int tok = p.tokens[mi];
            if (tok >= 0 || v.x0 == nullptr) {
                tok = tok < 0 ? 0 : (tok < p.vocab ? tok : p.vocab - 1);
                return p.table + (int64_t)tok * p.H;
            }
        }
        return v.x0 + (int64_t)mi * p.H;
    } else {
        gam = p.g0;
        return v.x0 + (int64_t)mi * v.K;
    }
}

// Norm (for PRO_RMS / PRO_CONCAT) and 16-bit split of the lane's features of
// row mi.  Every thread of the block calls it; it holds block barriers when
// several waves share one weight row (S > 1).
template <int FMT, int PRO>
__device__ __forceinline__ void norm_quant_row(const GemvParams& p, const View& v, int wid, int lane, int S, int mi,
                                               int kk, bool active, float (&xv)[32], const float (&gv)[32],
                                               XFrag& xf, float& xs, float (*nred)[2]) {
    const int q = wid / S;
    if constexpr (PRO != PRO_PLAIN) {
        const int seg = (PRO == PRO_CONCAT && kk >= p.H) ? 1 : 0;
        const int nfeat = PRO == PRO_CONCAT ? p.H : v.K;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) ss = fmaf(xv[i], xv[i], ss);
        float s0 = wave_sum(seg == 0 ? ss : 0.0f);
        float s1 = (PRO == PRO_CONCAT) ? wave_sum(seg == 1 ? ss : 0.0f) : 0.0f;
        if (S > 1) {
            __syncthreads();
            if (lane == 0) {
                nred[wid][0] = s0;
                nred[wid][1] = s1;
            }
            __syncthreads();
            s0 = 0.0f;
            s1 = 0.0f;
            for (int j = 0; j < S; ++j) {
                s0 += nred[q * S + j][0];
                s1 += nred[q * S + j][1];
            }
        }
        const float tot = seg ? s1 : s0;
        const float inv = rsqrtf(tot / (float)nfeat + p.eps);
        if (active && mi < p.m) {
#pragma unroll
            for (int i = 0; i < 32; ++i) xv[i] = xv[i] * inv * gv[i];
            if (PRO == PRO_RMS && p.normed_out && blockIdx.x == 0 && blockIdx.y == 0 && q == 0)
                store32(p.normed_out + (int64_t)mi * v.K + kk, xv);
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(xv[i]));
    am = wave_max(am);
    const float inv_q = am > 0.0f ? kQMax / am : 0.0f;
    xs = am / kQMax;
    quantize_group<FMT>(xv, inv_q, xs, xf);
}

// Block-shared setup for two or more activation rows.  The (row, chunk)
// fragments are computed once per block instead of once per wave: wave
// (s, q) takes rows q, q + Q, ... of its chunk s (two rows' loads in flight
// at a time), norms combine the chunks' sums of squares through LDS, and
// each fragment goes to LDS, from where every wave of chunk s reads all M.
// Rows are independent work, so M rows cost about one row's latency when
// Q >= M.  Used for two and four rows (eight would not fit the registers
// beside the kernel's other state).
template <int M>
__host__ __device__ constexpr int xq_slots() { return M == 2 ? 8 : 12; }
constexpr int kXqWords = 18;  // hi[8], lo[8], sxd, one spare word

template <int PRO>
__device__ __forceinline__ const float* gamma_src(const GemvParams& p, int kk) {
    if constexpr (PRO == PRO_CONCAT) return kk >= p.H ? p.g1 + (kk - p.H) : p.g0 + kk;
    return p.g0 + kk;
}

template <int FMT, int M, int PRO>
__device__ __forceinline__ void shared_rows(const GemvParams& p, const View& v, int lane, int S, int Q, int s,
                                            int q, int kk, bool active, unsigned* xq, float* xsq, float (*nq)[2],
                                            XFrag (&xf)[M], float (&xs)[M]) {
    constexpr int JB = M >= 4 ? 4 : 2;  // rows whose loads are in flight together
    const int per = (M + Q - 1) / Q;  // rows per wave, the same in every wave
    float gv[32];
    if constexpr (PRO != PRO_PLAIN) {
        if (active) {
            load32(gv, gamma_src<PRO>(p, kk));
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) gv[i] = 0.0f;
        }
    }
    const int seg = (PRO == PRO_CONCAT && kk >= p.H) ? 1 : 0;
    for (int j0 = 0; j0 < per; j0 += JB) {
        float xv[JB][32];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int mi = q + Q * (j0 + jj);
            if (mi < M) load_x_row<PRO>(p, v, mi, kk, active, xv[jj], gv, false);
        }
        float inv[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) inv[jj] = 1.0f;
        if constexpr (PRO != PRO_PLAIN) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const int mi = q + Q * (j0 + jj);
                if (mi < M) {
                    float ss = 0.0f;
#pragma unroll
                    for (int i = 0; i < 32; ++i) ss = fmaf(xv[jj][i], xv[jj][i], ss);
                    const float s0 = wave_sum(seg == 0 ? ss : 0.0f);
                    const float s1 = (PRO == PRO_CONCAT) ? wave_sum(seg == 1 ? ss : 0.0f) : 0.0f;
                    if (lane == 0) {
                        nq[mi * S + s][0] = s0;
                        nq[mi * S + s][1] = s1;
                    }
                }
            }
            __syncthreads();
            const int nfeat = PRO == PRO_CONCAT ? p.H : v.K;
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const int mi = q + Q * (j0 + jj);
                if (mi < M) {
                    float tot = 0.0f;
                    for (int j = 0; j < S; ++j) tot += nq[mi * S + j][seg];
                    inv[jj] = rsqrtf(tot / (float)nfeat + p.eps);
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int mi = q + Q * (j0 + jj);
            if (mi < M) {
                if constexpr (PRO != PRO_PLAIN) {
                    if (active && mi < p.m) {
#pragma unroll
                        for (int i = 0; i < 32; ++i) xv[jj][i] = xv[jj][i] * inv[jj] * gv[i];
                        if (PRO == PRO_RMS && p.normed_out && blockIdx.x == 0 && blockIdx.y == 0)
                            store32(p.normed_out + (int64_t)mi * v.K + kk, xv[jj]);
                    }
                }
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(xv[jj][i]));
                am = wave_max(am);
                const float inv_q = am > 0.0f ? kQMax / am : 0.0f;
                const float x_s = am / kQMax;
                XFrag f;
                quantize_group<FMT>(xv[jj], inv_q, x_s, f);
                unsigned* dst = xq + (mi * S + s) * kXqWords * kWave + lane;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    dst[w * kWave] = (unsigned)f.hi[w];
                    dst[(8 + w) * kWave] = (unsigned)f.lo[w];
                }
                dst[16 * kWave] = __float_as_uint(f.sxd);
                if (lane == 0) xsq[mi * S + s] = x_s;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
        const unsigned* src = xq + (mi * S + s) * kXqWords * kWave + lane;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            xf[mi].hi[w] = (int)src[w * kWave];
            xf[mi].lo[w] = (int)src[(8 + w) * kWave];
        }
        xf[mi].sxd = __uint_as_float(src[16 * kWave]);
        xs[mi] = xsq[mi * S + s];
    }
}

// One activation row, 4-bit weights.  Each wave loads its whole chunk s of
// the row in 1 KB pieces (lane l holds features 256 i + 4 l .. +3 of piece
// i), so every load instruction reads a contiguous kilobyte; the loads are
// requested before the first weight tiles (row1_load), with no branches, so
// that the setup waits for them alone, and consumed after (row1_finish): the
// norm (over the block's chunk waves through LDS when S > 1), the chunk
// maximum, quantization with q_bits, and each group's fragment (hi[8],
// lo[8], sxd; the layout of quantize_group) passed through a wave-private
// LDS region to the lane that owns the group.
struct Row1Pieces {
    float4 x[8], g[8];
};
constexpr int kRow1Chunks = 4;  // K <= 8192
constexpr int kRow1Words = 17;  // hi[8], lo[8], sxd per group

template <int PRO>
__device__ __forceinline__ void row1_load(const GemvParams& p, const View& v, int lane, int s, Row1Pieces& rp) {
    const float *gam0 = nullptr, *gam1 = nullptr;
    const float* src0 = x_segment<PRO>(p, v, 0, 0, gam0);
    const float* src1 = PRO == PRO_CONCAT ? x_segment<PRO>(p, v, 0, 1, gam1) : src0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int f = kChunk * s + 256 * i + 4 * lane;
        f = f < v.K ? f : 0;  // past the end: any valid address, zeroed in row1_finish
        const bool sg = PRO == PRO_CONCAT && f >= p.H;
        const int kl = sg ? f - p.H : f;
        rp.x[i] = *reinterpret_cast<const float4*>((sg ? src1 : src0) + kl);
        if constexpr (PRO != PRO_PLAIN) rp.g[i] = *reinterpret_cast<const float4*>((sg ? gam1 : gam0) + kl);
    }
}

template <int PRO>
__device__ __forceinline__ void row1_finish(const GemvParams& p, const View& v, int lane, int S, int s, int q,
                                            Row1Pieces& rp, unsigned* xq, float (*part)[2], XFrag& xf,
                                            float& xs) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (kChunk * s + 256 * i + 4 * lane >= v.K) rp.x[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (PRO != PRO_PLAIN) {
        float ss0 = 0.0f, ss1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 x = rp.x[i];
            const float ss = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, x.w * x.w)));
            if (PRO == PRO_CONCAT && kChunk * s + 256 * i + 4 * lane >= p.H)
                ss1 += ss;
            else
                ss0 += ss;
        }
        ss0 = wave_sum(ss0);
        if constexpr (PRO == PRO_CONCAT) ss1 = wave_sum(ss1);
        if (S > 1) {  // the other chunks' sums
            if (lane == 0 && q == 0) {
                part[s][0] = ss0;
                part[s][1] = ss1;
            }
            __syncthreads();
            ss0 = 0.0f;
            ss1 = 0.0f;
            for (int k = 0; k < S; ++k) {
                ss0 += part[k][0];
                ss1 += part[k][1];
            }
        }
        const int nfeat = PRO == PRO_CONCAT ? p.H : v.K;
        const float inv0 = rsqrtf(ss0 / (float)nfeat + p.eps);
        const float inv1 = PRO == PRO_CONCAT ? rsqrtf(ss1 / (float)nfeat + p.eps) : inv0;
        const bool store = PRO == PRO_RMS && p.normed_out && blockIdx.x == 0 && blockIdx.y == 0 && q == 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int f = kChunk * s + 256 * i + 4 * lane;
            const float iv = (PRO == PRO_CONCAT && f >= p.H) ? inv1 : inv0;
            float4& x = rp.x[i];
            const float4 g = rp.g[i];
            x = make_float4(x.x * iv * g.x, x.y * iv * g.y, x.z * iv * g.z, x.w * iv * g.w);
            if (store && f < v.K) *reinterpret_cast<float4*>(p.normed_out + f) = x;
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 x = rp.x[i];
        am = fmaxf(am, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
    am = wave_max(am);
    const float inv_q = am > 0.0f ? kQMax / am : 0.0f;
    xs = am / kQMax;
    // lanes 2k and 2k+1 hold the first and last four features of a code
    // word, and one quad exchange forms the word's hi and lo operand words
    // (even features, then odd)
    const bool odd = lane & 1;
    const unsigned sel_h = odd ? 0x01000504u : 0x05040100u;
    const unsigned sel_l = odd ? 0x03020706u : 0x07060302u;
    const int k8 = lane & 7;  // word of the group
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 x = rp.x[i];
        const unsigned b0 = q_bits(x.x, inv_q), b1 = q_bits(x.y, inv_q), b2 = q_bits(x.z, inv_q),
                       b3 = q_bits(x.w, inv_q);
        unsigned qsum = (b0 + b1) + (b2 + b3);
        const unsigned p02 = __builtin_amdgcn_perm(b2, b0, 0x04000501u);
        const unsigned p13 = __builtin_amdgcn_perm(b3, b1, 0x04000501u);
        const unsigned keep = odd ? p13 : p02;
        const unsigned got = (unsigned)dpp_partner<1>((int)(odd ? p02 : p13));
        const int gl = 8 * i + (lane >> 3);  // group within the chunk
        xq[k8 * kWave + gl] = __builtin_amdgcn_perm(got, keep, sel_h);
        xq[(8 + k8) * kWave + gl] = __builtin_amdgcn_perm(got, keep, sel_l) ^ 0x80808080u;
        qsum += (unsigned)dpp_partner<1>((int)qsum);
        qsum += (unsigned)dpp_partner<2>((int)qsum);
        qsum += (unsigned)dpp_partner<4>((int)qsum);
        if (k8 == 0) xq[16 * kWave + gl] = __float_as_uint((float)(int)(qsum - 32u * kQBiasBits));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        xf.hi[k] = (int)xq[k * kWave + lane];
        xf.lo[k] = (int)xq[(8 + k) * kWave + lane];
    }
    xf.sxd = __uint_as_float(xq[16 * kWave + lane]);
}

// Weight fragments of one tile (R rows x P matrices) for this lane's group.
template <int FMT, int R, int P>
struct TileFrags {
    WFrag<FMT> f[R][P];
};

template <int FMT, int R, int P>
__device__ __forceinline__ void load_tile(TileFrags<FMT, R, P>& tf, const View& v, int row0, int gc) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int row = row0 + r;
        row = row < v.N ? row : v.N - 1;  // tail rows are computed and dropped
        if constexpr (P == 2) {
            load_frag(tf.f[r][0], v.c0, v.s0, v.b0, row, v.G, gc);
            load_frag(tf.f[r][1], v.c1, v.s1, v.b1, row, v.G, gc);
        } else {
            // rows of up to three matrices concatenated along n (row is
            // wave-uniform); the matrix is picked with 0/1 multiples of the
            // byte distances between the arrays, which keeps it in registers
            const int64_t in1 = row >= v.n0, in2 = row >= v.n0 + v.n1;
            const int lr = row - (int)in1 * v.n0 - (int)in2 * v.n1;
            const void* codes = static_cast<const char*>(v.c0) + in1 * v.dc1 + in2 * v.dc2;
            const float* scales = reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.s0) + in1 * v.ds1 +
                                                                 in2 * v.ds2);
            const float* biases = reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.b0) + in1 * v.db1 +
                                                                 in2 * v.db2);
            load_frag(tf.f[r][0], codes, scales, biases, lr, v.G, gc);
        }
    }
}

// acc[(r*M + mi)*P + pp] = partial of row r, activation row mi, matrix pp.
template <int FMT, int M, int R, int P>
__device__ __forceinline__ void compute_tile(const TileFrags<FMT, R, P>& tf, const XFrag (&xf)[M],
                                             float (&acc)[R * M * P]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
            const WFrag<FMT>& f = tf.f[r][pp];
            if constexpr (FMT == FMT_Q4) {
                const Nib n = unpack_nibbles(f.c);
#pragma unroll
                for (int mi = 0; mi < M; ++mi) acc[(r * M + mi) * P + pp] = dot_q4(n, f.s, f.b, xf[mi]);
            } else {
#pragma unroll
                for (int mi = 0; mi < M; ++mi) acc[(r * M + mi) * P + pp] = dot_q8(f, xf[mi]);
            }
        }
}

// Cross-block argmax, run by wave 0 of every block once the block's per-row
// bests (value, index) of its nw waves are in LDS (rows 0 .. MR-1 filled;
// MR >= m).  Lane r < MR offers the block's best key of row r to the row's
// key with a returning atomicMax, all rows in one instruction (rows >= m
// offer key 0, which changes nothing); the returns are consumed (stored to
// sink) before lane 0 counts the block on the arrival counter, so the updates
// have been performed by then.  The last block to arrive turns the keys into
// ids[m] and leaves keys and counter at zero.  A block thus spends two round
// trips and the last one three.  Only workgroup-scope fences are used: the
// device-scope atomics are performed at the memory side, and an agent-scope
// fence would write back and invalidate the L2 in every block.
template <int MR>
__device__ __forceinline__ void grid_argmax(const GemvParams& p, int nw, const float (*bv_s)[8],
                                            const int (*bi_s)[8], unsigned long long* sink, int lane) {
    static_assert(MR <= kHeadRows, "rows");
    if (lane < MR) {
        float bv = bv_s[0][lane];
        int bi = bi_s[0][lane];
        for (int w = 1; w < nw; ++w) argmax_merge(bv, bi, bv_s[w][lane], bi_s[w][lane]);
        const unsigned long long key = (lane < p.m && bi != INT_MAX) ? argmax_key(bv, bi) : 0ull;
        sink[lane] = atomicMax(p.head_keys + lane * kKeyStride, key);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    unsigned ticket = 0;
    if (lane == 0) ticket = atomicAdd(p.counter, 1u);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket == gridDim.x - 1) {
        unsigned long long k = 0ull;
        if (lane < MR) k = atomicExch(p.head_keys + lane * kKeyStride, 0ull);
        if (lane < MR && lane < p.m) p.ids[lane] = argmax_key_index(k);
        if (lane == 0) atomicExch(p.counter, 0u);
    }
}

// The work units one worker (a wave, or a whole block when S > 1) goes
// through.  Fixed shares: worker gid of W takes units gid, gid + W, ...  (for
// a grid of one unit per worker, unit gid).  Balanced (S == 1): the waves of
// a block share the units blockIdx.x + gridDim.x * k and claim k one at a
// time from a counter in LDS, so a wave that is served faster takes more
// units; one claim is kept in flight.
struct TileSeq {
    int base, step, NU, i;
    bool shared;
    int pend;  // claim in flight (valid in lane 0)

    template <class Claim>
    __device__ void init(int b, int st, int nu, bool sh, Claim claim) {
        base = b;
        step = st;
        NU = nu;
        i = 0;
        shared = sh;
        if (shared) pend = claim();
    }
    template <class Claim>
    __device__ int next(Claim claim) {
        int k;
        if (!shared) {
            k = i++;
        } else {
            k = __builtin_amdgcn_readfirstlane(pend);
            pend = claim();
        }
        const int u = base + step * k;
        return u < NU ? u : -1;
    }
};

template <int FMT, int M, int PRO, int EPI>
__global__ void __launch_bounds__(block_waves(FMT, EPI, M) * 64) k_gemv(const GemvParams p) {
    constexpr int P = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int R = gemv_rows(M, P, EPI);
    constexpr int V = R * M * P;
    constexpr int kWaves = block_waves(FMT, EPI, M);  // waves per block, at most
    __shared__ float red[kWaves][kWave * 2];
    __shared__ float nred[kWaves][2];
    __shared__ int claim_ctr;

    if (p.zero_words && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < p.zero_n; i += blockDim.x) p.zero_words[i] = 0u;
    View v;
    if (!resolve_view(p, v)) return;

    // the wave index is wave-uniform; saying so lets every row, pointer and
    // branch derived from it live in scalar registers
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int S = p.S;
    const int Q = (blockDim.x / kWave) / S;
    const int s = wid % S, q = wid / S;
    const int g = s * kWave + lane;
    const int gc = g < v.G ? g : v.G - 1;
    // Work units: with S == 1 every wave is its own row-group and works on
    // units of R rows; with S > 1 the row-groups of a block hold barriers
    // together, so the block moves as one over units of Q*R rows (wave q
    // taking the q-th R rows of each).
    const int per = S == 1 ? 1 : Q;
    const int qo = S == 1 ? 0 : q;
    const int NU = (v.N + per * R - 1) / (per * R);

    // the first tiles' weights are requested before the activation setup so
    // their latency overlaps it (two tiles where the loop double-buffers)
    constexpr bool kDouble = (M <= 2 && P == 1);
    const bool active = g < v.G;
    const int kk = g * kGroup;
    const bool balanced = S == 1 && p.balance;
    auto claim = [&]() {
        int r = 0;
        if (lane == 0) r = atomicAdd(&claim_ctr, 1);
        return r;
    };
    if (balanced) {
        if (threadIdx.x == 0) claim_ctr = 0;
        __syncthreads();
    }
    TileSeq ts;
    if (balanced)
        ts.init(blockIdx.x, gridDim.x, NU, true, claim);
    else if (S == 1)
        ts.init(blockIdx.x * Q + q, gridDim.x * Q, NU, false, claim);
    else
        ts.init(blockIdx.x, gridDim.x, NU, false, claim);
    auto row0 = [&](int u) { return (u * per + qo) * R; };
    TileFrags<FMT, R, P> tf, tf2;
    XFrag xf[M];
    float xs[M];
    bool shared_done = false;
    // one 4-bit activation row: its pieces are requested before the first
    // tiles, which are then requested unconditionally (tile 0 stands in for
    // none), so that the setup waits for the activations only
    constexpr bool kRow1 = M == 1 && FMT == FMT_Q4;  // S <= kRow1Chunks (checked at launch)
    Row1Pieces rp;
    if constexpr (kRow1) row1_load<PRO>(p, v, lane, s, rp);
    int wa = ts.next(claim), wb = -1;
    if constexpr (kRow1) {
        load_tile<FMT, R, P>(tf, v, row0(wa >= 0 ? wa : 0), gc);
        if constexpr (kDouble) {
            if (wa >= 0) wb = ts.next(claim);
            load_tile<FMT, R, P>(tf2, v, row0(wb >= 0 ? wb : 0), gc);
        }
    } else {
        if (wa >= 0) load_tile<FMT, R, P>(tf, v, row0(wa), gc);
        if constexpr (kDouble) {
            if (wa >= 0) wb = ts.next(claim);
            if (wb >= 0) load_tile<FMT, R, P>(tf2, v, row0(wb), gc);
        }
    }
    if constexpr (kRow1) {
        __shared__ unsigned xq1[kWaves][kRow1Words * kWave];
        __shared__ float part1[kRow1Chunks][2];
        row1_finish<PRO>(p, v, lane, S, s, q, rp, xq1[wid], part1, xf[0], xs[0]);
        shared_done = true;
    }
    if constexpr (M == 2 || M == 4) {
        __shared__ unsigned xq[xq_slots<M>() * kXqWords * kWave];
        __shared__ float xsq[xq_slots<M>()];
        __shared__ float nq[xq_slots<M>()][2];
        if (M * S <= xq_slots<M>()) {
            shared_rows<FMT, M, PRO>(p, v, lane, S, Q, s, q, kk, active, xq, xsq, nq, xf, xs);
            shared_done = true;
        }
    }
    if (!shared_done) {
        float gv[32];  // gamma is the same for every row: loaded with row 0
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
            float xv[32];
            load_x_row<PRO>(p, v, mi, kk, active, xv, gv, mi == 0);
            norm_quant_row<FMT, PRO>(p, v, wid, lane, S, mi, kk, active, xv, gv, xf[mi], xs[mi], nred);
        }
    }

    const int pos = reduce_base<V, P>(lane) / P;  // = r * M + mi of this lane's result
    const int r_l = pos / M, mi_l = pos % M;
    const bool writer = reduce_writer<V, P>(lane);
    const float xs_l = select_m<M>(xs, mi_l);
    float best = -INFINITY;
    int best_i = INT_MAX;

    // reduce one tile's partials across the lanes (and the S chunk waves) and
    // apply the epilogue
    auto finish = [&](float (&acc)[V], int row0) {
        reduce_transpose<V, P>(acc, lane);
        float v0 = acc[0] * xs_l;
        float v1 = (P == 2) ? acc[P - 1] * xs_l : 0.0f;
        if (S > 1) {
            red[wid][2 * lane] = v0;
            red[wid][2 * lane + 1] = v1;
            __syncthreads();
            if (s == 0) {
                v0 = 0.0f;
                v1 = 0.0f;
                for (int j = 0; j < S; ++j) {
                    v0 += red[q * S + j][2 * lane];
                    v1 += red[q * S + j][2 * lane + 1];
                }
            }
            __syncthreads();
        }
        if (s == 0) {
            const int row = row0 + r_l;
            if (row < v.N && mi_l < p.m) {
                const int64_t o = (int64_t)mi_l * v.N + row;
                if constexpr (EPI == EPI_STORE) {
                    if (writer) v.y[o] = p.residual ? v0 + p.residual[o] : v0;
                } else if constexpr (EPI == EPI_SWIGLU) {
                    if (writer) {
                        float z = silu(v0) * v1;
                        if (v.rowscale) z *= v.rowscale[mi_l];
                        v.y[o] = z;
                    }
                } else {
                    if (p.logits && writer) p.logits[o] = v0;
                    if (v0 > best || (v0 == best && row < best_i)) {  // ties keep the lower row
                        best = v0;
                        best_i = row;
                    }
                }
            }
        }
    };

    if constexpr (kDouble) {
        // double buffering where the registers allow it: a tile's weights are
        // requested two tiles ahead of their dot products
        while (wa >= 0) {
            {
                float acc[V];
                compute_tile<FMT, M, R, P>(tf, xf, acc);
                finish(acc, row0(wa));
            }
            if (wb < 0) break;
            wa = ts.next(claim);
            if (wa >= 0) load_tile<FMT, R, P>(tf, v, row0(wa), gc);
            {
                float acc[V];
                compute_tile<FMT, M, R, P>(tf2, xf, acc);
                finish(acc, row0(wb));
            }
            wb = wa >= 0 ? ts.next(claim) : -1;
            if (wb >= 0) load_tile<FMT, R, P>(tf2, v, row0(wb), gc);
        }
    } else {
        while (wa >= 0) {
            float acc[V];
            compute_tile<FMT, M, R, P>(tf, xf, acc);
            // next tile's loads fly while this one is reduced and stored
            const int nx = ts.next(claim);
            if (nx >= 0) load_tile<FMT, R, P>(tf, v, row0(nx), gc);
            finish(acc, row0(wa));
            wa = nx;
        }
    }
    if constexpr (EPI == EPI_ARGMAX) {
        // block best per activation row: waves -> LDS -> thread 0
        __shared__ float bv_s[kWaves][8];
        __shared__ int bi_s[kWaves][8];
        if (s == 0) {
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                float bv = (mi_l == mi) ? best : -INFINITY;
                int bi = (mi_l == mi) ? best_i : INT_MAX;
                wave_argmax(bv, bi);
                if (lane == 0) {
                    bv_s[q][mi] = bv;
                    bi_s[q][mi] = bi;
                }
            }
        }
        __syncthreads();
        __shared__ unsigned long long sink[kHeadRows];
        if (wid == 0) grid_argmax<M>(p, Q, bv_s, bi_s, sink, lane);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core GEMV: 4-bit weights, K = 2048, up to four activation rows.
//
// Work unit: 16 weight rows, one wave.  Lane l loads row l%16 and, per load
// t, the 16 bytes of group 4t + l/16, so a load covers 16 rows x 64 bytes.
// One v_permlane32_swap per word pair turns the lane quarters' groups into
// the A operands of two v_mfma_i32_16x16x64_i8 per load, each over a group
// pair: quarters 0 and 2 then hold the pair's first group (words 0-1 and
// 2-3), quarters 1 and 3 the second.  The B operand (the activations' int8
// halves, built once per block in LDS) pairs columns 0..7 with the first
// group and 8..15 with the second and is zero elsewhere; column c of a group
// is (activation row c/2, hi half if c is even, lo half if odd).  Each
// group's int32 result is scaled by its row's scale and accumulated in f32;
// the bias sums (b times the group's sum of quantized activations) are f32
// MFMAs (16x16x4) fed with the biases as loaded.  Two DPP adds then fold the
// group halves and the hi/lo columns, and the result is
// xs * (256 hi + lo + bias sums), the same quantity as in the vector path.
//
// 8-bit weights (int8 codes, one scale per group, no bias) use the same unit,
// B columns and scaling.  A row is 2048 bytes, so a unit is 32 loads, and
// load t of lane l is row l%16's bytes 64 t + 16 (l/16) .. +15, which is
// already the A operand of one MFMA over the group pair 2t, 2t + 1 (quarters
// 0-1 hold the first group, 2-3 the second).  The B operand holds the
// activations in natural order: feature f is byte f%16 of quarter (f/16)%4 of
// MFMA f/64, in the columns of group parity (f/32)%2.  With no bias there is
// no f32 MFMA, and the result is xs * (256 hi + lo).
// ---------------------------------------------------------------------------
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
constexpr int kMmaRows = 16;
constexpr int kMmaCols = 16;
constexpr int kStage = 20;  // floats per group in a wave's scale stage (16 rows, 16-byte aligned)

__device__ __forceinline__ void perm32_swap(unsigned& a, unsigned& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// Activation setup of the matrix-core kernels, shared by a block's waves:
// wave w takes activation row w % 4 and, of each of the S chunks, the 1 KB
// pieces NI (w / 4) .. NI (w / 4) + NI - 1 (lane l holds features
// 256 i + 4 l .. +3 of piece i), so that every load instruction reads one
// contiguous kilobyte.  The loads are issued first (mma_load_x), so that
// they overlap the weight requests that follow, and consumed by mma_quant_x.
template <int S, int NI>
struct XPieces {
    float4 x[S][NI], g[S][NI];
};

template <int PRO, int S, int NI>
__device__ __forceinline__ void mma_load_x(const GemvParams& p, const View& v, int mi, int sub, int lane,
                                           XPieces<S, NI>& xp) {
    const float *gam0 = nullptr, *gam1 = nullptr, *src0 = nullptr, *src1 = nullptr;
    const bool live = mi < p.m;
    if (live) {
        src0 = x_segment<PRO>(p, v, mi, 0, gam0);
        if constexpr (PRO == PRO_CONCAT) src1 = x_segment<PRO>(p, v, mi, 1, gam1);
    }
#pragma unroll
    for (int c = 0; c < S; ++c)
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
            const int f = kChunk * c + 256 * (sub * NI + ii) + 4 * lane;
            if (live) {
                const bool sg = PRO == PRO_CONCAT && f >= p.H;
                const int kl = sg ? f - p.H : f;
                xp.x[c][ii] = *reinterpret_cast<const float4*>((sg ? src1 : src0) + kl);
                if constexpr (PRO != PRO_PLAIN)
                    xp.g[c][ii] = *reinterpret_cast<const float4*>((sg ? gam1 : gam0) + kl);
            } else {
                xp.x[c][ii] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
}

// The rest of the setup: the norms (PRO_RMS, PRO_CONCAT) and the chunk
// maxima, each combined over the R waves of a row through part, then the
// 16-bit quantization into the B operands (bq), the bias factors (tx, which
// carry the chunk's activation scale) and the scales (xs_lds).  The codes'
// word of 8 features unpacks to the even features, then the odd ones, and
// lanes 2k and 2k+1 hold that word's first and last four features, so one
// quad exchange forms each operand word.  Ends with a block barrier.
template <int PRO, int S, int R, int FMT = FMT_Q4>
__device__ __forceinline__ void mma_quant_x(const GemvParams& p, const View& v, int mi, int sub, int lane,
                                            XPieces<S, 8 / R>& xp, u32x4 (*bq)[2][kWave],
                                            float (*tx)[kMmaCols], float (*xs_lds)[4], float (*part)[4][R]) {
    constexpr int NI = 8 / R;
    static_assert(FMT == FMT_Q4 || S == 1, "8-bit operands cover one chunk");
    const bool live = mi < p.m;
    if constexpr (PRO != PRO_PLAIN) {
        float ss0 = 0.0f, ss1 = 0.0f;
#pragma unroll
        for (int c = 0; c < S; ++c)
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) {
                const float4 x = xp.x[c][ii];
                const float ss = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, x.w * x.w)));
                if (PRO == PRO_CONCAT && kChunk * c + 256 * (sub * NI + ii) + 4 * lane >= p.H)
                    ss1 += ss;
                else
                    ss0 += ss;
            }
        ss0 = wave_sum(ss0);
        if constexpr (PRO == PRO_CONCAT) ss1 = wave_sum(ss1);
        if constexpr (R > 1) {
            if (lane == 0) {
                part[S][mi][sub] = ss0;
                part[S + 1][mi][sub] = ss1;
            }
            __syncthreads();
            ss0 = 0.0f;
            ss1 = 0.0f;
#pragma unroll
            for (int q = 0; q < R; ++q) {
                ss0 += part[S][mi][q];
                ss1 += part[S + 1][mi][q];
            }
        }
        const int nfeat = PRO == PRO_CONCAT ? p.H : v.K;
        const float inv0 = rsqrtf(ss0 / (float)nfeat + p.eps);
        const float inv1 = PRO == PRO_CONCAT ? rsqrtf(ss1 / (float)nfeat + p.eps) : inv0;
        if (live) {
#pragma unroll
            for (int c = 0; c < S; ++c)
#pragma unroll
                for (int ii = 0; ii < NI; ++ii) {
                    const int f = kChunk * c + 256 * (sub * NI + ii) + 4 * lane;
                    const float iv = (PRO == PRO_CONCAT && f >= p.H) ? inv1 : inv0;
                    float4& x = xp.x[c][ii];
                    const float4 g = xp.g[c][ii];
                    x = make_float4(x.x * iv * g.x, x.y * iv * g.y, x.z * iv * g.z, x.w * iv * g.w);
                    if (PRO == PRO_RMS && p.normed_out && blockIdx.x == 0)
                        *reinterpret_cast<float4*>(p.normed_out + (int64_t)mi * v.K + f) = x;
                }
        }
    }
    float am[S];
#pragma unroll
    for (int c = 0; c < S; ++c) {
        float a = 0.0f;
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
            const float4 x = xp.x[c][ii];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
        }
        am[c] = wave_max(a);
        if constexpr (R > 1)
            if (lane == 0) part[c][mi][sub] = am[c];
    }
    if constexpr (R > 1) {
        __syncthreads();
#pragma unroll
        for (int c = 0; c < S; ++c) {
            float a = part[c][mi][0];
#pragma unroll
            for (int q = 1; q < R; ++q) a = fmaxf(a, part[c][mi][q]);
            am[c] = a;
        }
    }
    const bool odd = lane & 1;
    const int wp = (lane >> 2) & 1, word = lane & 3;
    const unsigned sel_h = odd ? 0x01000504u : 0x05040100u;
    const unsigned sel_l = odd ? 0x03020706u : 0x07060302u;
#pragma unroll
    for (int c = 0; c < S; ++c) {
        const float inv_q = am[c] > 0.0f ? kQMax / am[c] : 0.0f;
        const float x_s = am[c] / kQMax;
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
            const float4 x = xp.x[c][ii];
            const unsigned b0 = q_bits(x.x, inv_q), b1 = q_bits(x.y, inv_q), b2 = q_bits(x.z, inv_q),
                           b3 = q_bits(x.w, inv_q);
            if constexpr (FMT == FMT_Q8) {
                // (hi 0, hi 1, lo 0, lo 1) and the same of 2, 3, then the hi
                // word and the lo word of the lane's four features
                const unsigned p01 = __builtin_amdgcn_perm(b1, b0, 0x04000501u);
                const unsigned p23 = __builtin_amdgcn_perm(b3, b2, 0x04000501u);
                const unsigned hw = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
                const unsigned lw = __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u;
                const int tq = 4 * (sub * NI + ii) + (lane >> 4);  // MFMA of features 256 i + 4 lane ..
                const int hq = (lane >> 2) & 3, par = hq >> 1;     // quarter, group parity
                unsigned* slot = reinterpret_cast<unsigned*>(&bq[tq >> 1][tq & 1][0]) + (lane & 3);
                slot[4 * (2 * mi + 8 * par + 16 * hq)] = hw;
                slot[4 * (2 * mi + 1 + 8 * par + 16 * hq)] = lw;
                slot[4 * (2 * mi + 8 * (1 - par) + 16 * hq)] = 0u;
                slot[4 * (2 * mi + 1 + 8 * (1 - par) + 16 * hq)] = 0u;
                continue;
            }
            unsigned qsum = (b0 + b1) + (b2 + b3);
            // bytes (hi of 0, hi of 2, lo of 0, lo of 2) and the same of 1, 3;
            // the even lane keeps the first and gives the second, the odd the reverse
            const unsigned p02 = __builtin_amdgcn_perm(b2, b0, 0x04000501u);
            const unsigned p13 = __builtin_amdgcn_perm(b3, b1, 0x04000501u);
            const unsigned keep = odd ? p13 : p02;
            const unsigned got = (unsigned)dpp_partner<1>((int)(odd ? p02 : p13));
            const unsigned hw = __builtin_amdgcn_perm(got, keep, sel_h);
            const unsigned lw = __builtin_amdgcn_perm(got, keep, sel_l) ^ 0x80808080u;
            const int gl = 8 * (sub * NI + ii) + (lane >> 3);  // group within the chunk
            const int t = 16 * c + (gl >> 2), pp = (gl >> 1) & 1, par = gl & 1, hq = 2 * wp + par;
            unsigned* slot = reinterpret_cast<unsigned*>(&bq[t][pp][0]) + word;
            slot[4 * (2 * mi + 8 * par + 16 * hq)] = hw;
            slot[4 * (2 * mi + 1 + 8 * par + 16 * hq)] = lw;
            slot[4 * (2 * mi + 8 * (1 - par) + 16 * hq)] = 0u;
            slot[4 * (2 * mi + 1 + 8 * (1 - par) + 16 * hq)] = 0u;
            qsum += (unsigned)dpp_partner<1>((int)qsum);
            qsum += (unsigned)dpp_partner<2>((int)qsum);
            qsum += (unsigned)dpp_partner<4>((int)qsum);  // the group's eight lanes
            const int qs = (int)(qsum - 32u * kQBiasBits);
            const int k8 = lane & 7;
            if (k8 < 4) {
                // the bias factor carries the chunk's activation scale (the sum is exact)
                const int col = k8 == 0 ? 2 * mi : (k8 == 1 ? 2 * mi + 1 : 8 + 2 * mi + (k8 - 2));
                tx[64 * c + gl][col] = k8 == 0 ? (float)qs * x_s : 0.0f;
            }
        }
        if (sub == 0 && lane == 0) xs_lds[c][mi] = x_s;
    }
    __syncthreads();
}

template <int FMT, int PRO>
__global__ void __launch_bounds__(64 * kMaxWaves) k_gemv_mma(const GemvParams p) {
    constexpr int R = kMaxWaves / 4;  // waves per activation row in the setup
    constexpr int NT = FMT == FMT_Q4 ? 16 : 32;  // 16-byte code loads per lane and unit
    __shared__ u32x4 bq[16][2][kWave];              // 32 KB: B operands (load t, group pair)
    __shared__ float tx[64][kMmaCols];              // 4 KB: sum of x^ per (group, column 2*row), else 0
    __shared__ float stage[kMaxWaves][64 * kStage];  // 40 KB: each wave's scales, [group][row]
    __shared__ float part[3][4][R];
    __shared__ float xs_lds[1][4];
    __shared__ int claim_ctr;

    if (p.zero_words && blockIdx.x == 0)
        for (int i = threadIdx.x; i < p.zero_n; i += blockDim.x) p.zero_words[i] = 0u;
    View v;
    resolve_view(p, v);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int NU = (v.N + kMmaRows - 1) / kMmaRows;

    auto claim = [&]() {
        int r = 0;
        if (lane == 0) r = atomicAdd(&claim_ctr, 1);
        return r;
    };
    if (threadIdx.x == 0) claim_ctr = 0;
    __syncthreads();
    TileSeq ts;
    ts.init(blockIdx.x, gridDim.x, NU, true, claim);

    const int j = lane & 15, h = lane >> 4;
    const int mi_l = (j & 7) >> 1;
    const bool lo_col = (j & 1) != 0;
    const float colf = lo_col ? 1.0f : 256.0f;
    const bool writer = j < 8 && !lo_col && mi_l < p.m;
    float* st = stage[wid];
    float best = -INFINITY;
    int best_i = INT_MAX;


    // unit u: rows 16 u .. 16 u + 15 of the one matrix
    auto row_ptrs = [&](int u, const char*& crow, const float*& srow, const float*& brow) {
        int row = u * kMmaRows + j;
        row = row < v.N ? row : v.N - 1;
        crow = static_cast<const char*>(v.c0) + (int64_t)row * (FMT == FMT_Q4 ? v.K / 2 : v.K) + 16 * h;
        srow = v.s0 + (int64_t)row * v.G + 4 * h;
        brow = FMT == FMT_Q4 ? v.b0 + (int64_t)row * v.G + 4 * h : nullptr;
    };
    u32x4 cw[NT];
    v4f_t sv[4], bv[4];
    // Plain loads: a load reads one half of a 128-byte line of each of 16
    // rows and the next load the other half, so the line is better kept in
    // L2 than streamed past it (nontemporal loads measured 5-9% slower here).
    auto load_codes = [&](const char* crow, int t) {
        cw[t] = *reinterpret_cast<const u32x4*>(crow + 64 * t);
    };
    auto load_sb = [&](const float* srow, const float* brow) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sv[t] = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(srow + 16 * t));
            if constexpr (FMT == FMT_Q4)
                bv[t] = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(brow + 16 * t));
        }
    };

    // Software pipeline: the activations are requested first, then the first
    // unit's weights, which arrive during the activation setup; the next
    // unit's weights go out register by register as soon as the current unit
    // has consumed them.
    XPieces<1, 8 / R> xp;
    mma_load_x<PRO, 1, 8 / R>(p, v, wid & 3, wid >> 2, lane, xp);
    int u = ts.next(claim);
    {
        // unconditional (unit 0 stands in for none), so that the setup waits
        // for the activations only and not for these requests as well
        const char* crow;
        const float *srow, *brow;
        row_ptrs(u >= 0 ? u : 0, crow, srow, brow);
#pragma unroll
        for (int t = 0; t < NT; ++t) load_codes(crow, t);
        load_sb(srow, brow);
    }
    mma_quant_x<PRO, 1, R, FMT>(p, v, wid & 3, wid >> 2, lane, xp, bq, tx, xs_lds, part);
    const float colx = colf * xs_lds[0][mi_l];  // integer sums carry the activation scale here
    while (u >= 0) {
        // the next unit's rows; past the last unit the requests still go out,
        // to unit 0 (one small region every wave shares, so they hit in L2),
        // which keeps the loads unconditional and the registers simple
        const int nu = ts.next(claim);
        const char* ncrow;
        const float *nsrow, *nbrow;
        row_ptrs(nu >= 0 ? nu : 0, ncrow, nsrow, nbrow);

        // bias sums on the f32 matrix core (two independent accumulators);
        // the scales go to this wave's stage
        v4f_t cb4[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) cb4[e] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gg = 16 * t + 4 * h + e;
                st[gg * kStage + j] = sv[t][e];
                if constexpr (FMT == FMT_Q4) {
                    const float tv = tx[gg][j];
                    cb4[e & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[t][e], tv, cb4[e & 1], 0, 0, 0);
                }
            }
        }
        load_sb(nsrow, nbrow);
        __builtin_amdgcn_wave_barrier();

        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (FMT == FMT_Q8) {
            // one MFMA per load, kTB8 at a time
            constexpr int kTB8 = 4;
#pragma unroll
            for (int t0 = 0; t0 < NT; t0 += kTB8) {
                v4i_t D[kTB8];
#pragma unroll
                for (int dt = 0; dt < kTB8; ++dt) {
                    const int t = t0 + dt;
                    const u32x4 bb = bq[t >> 1][t & 1][lane];
                    const v4i_t A = {(int)cw[t].x, (int)cw[t].y, (int)cw[t].z, (int)cw[t].w};
                    const v4i_t B = {(int)bb.x, (int)bb.y, (int)bb.z, (int)bb.w};
                    const v4i_t zero = {0, 0, 0, 0};
                    D[dt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, zero, 0, 0, 0);
                }
#pragma unroll
                for (int dt = 0; dt < kTB8; ++dt) {
                    const int gg = 2 * (t0 + dt) + (j >> 3);
                    const float4 s4 = *reinterpret_cast<const float4*>(&st[gg * kStage + 4 * h]);
                    acc[0] = fmaf(s4.x, (float)D[dt][0], acc[0]);
                    acc[1] = fmaf(s4.y, (float)D[dt][1], acc[1]);
                    acc[2] = fmaf(s4.z, (float)D[dt][2], acc[2]);
                    acc[3] = fmaf(s4.w, (float)D[dt][3], acc[3]);
                }
#pragma unroll
                for (int dt = 0; dt < kTB8; ++dt) load_codes(ncrow, t0 + dt);
            }
        } else {
            // integer products, kTB loads (2 kTB MFMAs) at a time
            constexpr int kTB = 2;
#pragma unroll
            for (int t0 = 0; t0 < 16; t0 += kTB) {
                v4i_t A[kTB][2];
#pragma unroll
                for (int dt = 0; dt < kTB; ++dt) {
                    const int t = t0 + dt;
                    unsigned w0 = cw[t].x, w1 = cw[t].y, w2 = cw[t].z, w3 = cw[t].w;
                    perm32_swap(w0, w2);
                    perm32_swap(w1, w3);
                    const unsigned M4 = 0x0F0F0F0Fu;
                    A[dt][0] = (v4i_t){(int)(w0 & M4), (int)((w0 >> 4) & M4), (int)(w1 & M4), (int)((w1 >> 4) & M4)};
                    A[dt][1] = (v4i_t){(int)(w2 & M4), (int)((w2 >> 4) & M4), (int)(w3 & M4), (int)((w3 >> 4) & M4)};
                }
                v4i_t D[kTB][2];
#pragma unroll
                for (int dt = 0; dt < kTB; ++dt)
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const u32x4 bb = bq[t0 + dt][pp][lane];
                        const v4i_t B = {(int)bb.x, (int)bb.y, (int)bb.z, (int)bb.w};
                        const v4i_t zero = {0, 0, 0, 0};
                        D[dt][pp] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[dt][pp], B, zero, 0, 0, 0);
                    }
#pragma unroll
                for (int dt = 0; dt < kTB; ++dt)
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const int gg = 4 * (t0 + dt) + 2 * pp + (j >> 3);
                        const float4 s4 = *reinterpret_cast<const float4*>(&st[gg * kStage + 4 * h]);
                        acc[0] = fmaf(s4.x, (float)D[dt][pp][0], acc[0]);
                        acc[1] = fmaf(s4.y, (float)D[dt][pp][1], acc[1]);
                        acc[2] = fmaf(s4.z, (float)D[dt][pp][2], acc[2]);
                        acc[3] = fmaf(s4.w, (float)D[dt][pp][3], acc[3]);
                    }
                // the registers of loads t0 .. t0+kTB-1 are free: request the
                // next unit's
#pragma unroll
                for (int dt = 0; dt < kTB; ++dt) load_codes(ncrow, t0 + dt);
            }
        }
        __builtin_amdgcn_wave_barrier();
        v4f_t cb = cb4[0] + cb4[1];
        // fold: group halves (lanes j, j^8), then hi and lo (lanes 2i, 2i+1)
        float res[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x = fmaf(acc[r], colx, cb[r]);
            x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x128, 0xF, 0xF, false));
            x += dpp_partner<1>(x);
            res[r] = x;
        }
        if (writer) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int orow = u * kMmaRows + 4 * h + r;
                if (orow < v.N) {
                    if (p.logits) p.logits[(int64_t)mi_l * v.N + orow] = res[r];
                    if (res[r] > best || (res[r] == best && orow < best_i)) {
                        best = res[r];
                        best_i = orow;
                    }
                }
            }
        }
        u = nu;
    }
    {
        __shared__ float bv_s[kMaxWaves][8];
        __shared__ int bi_s[kMaxWaves][8];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            float bvv = (writer && mi_l == mi) ? best : -INFINITY;
            int bii = (writer && mi_l == mi) ? best_i : INT_MAX;
            wave_argmax(bvv, bii);
            if (lane == 0) {
                bv_s[wid][mi] = bvv;
                bi_s[wid][mi] = bii;
            }
        }
        __syncthreads();
        __shared__ unsigned long long sink[kHeadRows];
        if (wid == 0) grid_argmax<4>(p, kMaxWaves, bv_s, bi_s, sink, lane);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core GEMV with the K range split over a block's W waves, for the
// projections that are not persistent: one block per unit (16 weight rows,
// or 8 output rows of the SwiGLU pair), K = 2048 S with S <= 3.  A block per
// unit puts many more compute units to work than a wave per unit, and each
// wave's share (16 S / W loads) is short; with W = 16 every SIMD holds four
// waves, which hides the latency of both the activation setup and the loop.
// In the setup, the W / 4 waves of activation row w % 4 split each chunk's
// features; the norms and chunk maxima meet in LDS.  The waves' partial sums
// meet in LDS at the end, and wave r < 4 folds and stores register r.
// Operand layout and arithmetic are those of k_gemv_mma; the activation
// scale of each chunk is applied when a wave's loads cross into the next
// chunk (and folded into the bias factors in LDS).
// ---------------------------------------------------------------------------
template <int PRO, int EPI, int S, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_mma_sk(const GemvParams p) {
    constexpr int R = W / 4;   // waves per activation row in the setup
    constexpr int NI = 8 / R;  // 1 KB pieces of each chunk per wave in the setup
    constexpr int T = 16 * S;  // loads (4 groups x 16 rows each) over K
    constexpr int TW = T / W;  // loads per wave
    constexpr int GW = 4 * TW;  // groups per wave
    constexpr int NE = GW / 4;  // groups per lane quarter
    static_assert(T % W == 0 && 8 % R == 0, "wave split");
    __shared__ u32x4 bq[T][2][kWave];        // B operands, 32 KB per chunk
    __shared__ float tx[64 * S][kMmaCols];   // bias factors x xs, 4 KB per chunk
    __shared__ float stage[W][GW * kStage];  // each wave's scales, [group][row]
    __shared__ float red[W][4][kWave];       // the waves' partial sums
    __shared__ float part[S + 2][4][R];      // setup partials: chunk maxima, then squares per segment
    __shared__ float xs_lds[S][4];

    if (p.zero_words && blockIdx.x == 0)
        for (int i = threadIdx.x; i < p.zero_n; i += blockDim.x) p.zero_words[i] = 0u;
    View v;
    resolve_view(p, v);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int u = blockIdx.x;

    // ---- activations first (they come from L2 and are needed first)
    const int mi = wid & 3, sub = wid >> 2;
    XPieces<S, NI> xp;
    mma_load_x<PRO, S, NI>(p, v, mi, sub, lane, xp);

    // ---- this wave's weights
    const int j = lane & 15, h = lane >> 4;
    const int mi_l = (j & 7) >> 1;
    const bool lo_col = (j & 1) != 0;
    const float colf = lo_col ? 1.0f : 256.0f;
    constexpr int kOutRows = EPI == EPI_SWIGLU ? kMmaRows / 2 : kMmaRows;
    int row = u * kOutRows + (EPI == EPI_SWIGLU ? (j & 7) : j);
    row = row < v.N ? row : v.N - 1;
    int64_t in1, in2;
    int lr;
    if constexpr (EPI == EPI_SWIGLU) {
        in1 = j >> 3;
        in2 = 0;
        lr = row;
    } else {
        in1 = row >= v.n0;
        in2 = row >= v.n0 + v.n1;
        lr = row - (int)in1 * v.n0 - (int)in2 * v.n1;
    }
    const int t0 = wid * TW, g0 = wid * GW;
    const char* crow = static_cast<const char*>(v.c0) + in1 * v.dc1 + in2 * v.dc2 + (int64_t)lr * (v.K / 2) + 16 * h;
    const float* srow = reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.s0) + in1 * v.ds1 +
                                                       in2 * v.ds2) + (int64_t)lr * v.G + g0 + NE * h;
    const float* brow = reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.b0) + in1 * v.db1 +
                                                       in2 * v.db2) + (int64_t)lr * v.G + g0 + NE * h;
    u32x4 cw[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i)
        cw[i] = *reinterpret_cast<const u32x4*>(crow + 64 * (t0 + i));  // plain, as in k_gemv_mma
    float sv[NE], bv[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        sv[e] = __builtin_nontemporal_load(srow + e);
        bv[e] = __builtin_nontemporal_load(brow + e);
    }

    mma_quant_x<PRO, S, R>(p, v, mi, sub, lane, xp, bq, tx, xs_lds, part);

    // ---- bias sums and this wave's scale stage
    float* st = stage[wid];
    v4f_t cb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int gl = NE * h + e;  // group within the wave's share
        st[gl * kStage + j] = sv[e];
        cb = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[e], tx[g0 + gl][j], cb, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();

    // ---- integer products
    float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f}, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int t = t0 + i;
        unsigned w0 = cw[i].x, w1 = cw[i].y, w2 = cw[i].z, w3 = cw[i].w;
        perm32_swap(w0, w2);
        perm32_swap(w1, w3);
        const unsigned M4 = 0x0F0F0F0Fu;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const unsigned a = pp ? w2 : w0, b = pp ? w3 : w1;
            const v4i_t A = {(int)(a & M4), (int)((a >> 4) & M4), (int)(b & M4), (int)((b >> 4) & M4)};
            const u32x4 bb = bq[t][pp][lane];
            const v4i_t B = {(int)bb.x, (int)bb.y, (int)bb.z, (int)bb.w};
            const v4i_t zero = {0, 0, 0, 0};
            const v4i_t D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, zero, 0, 0, 0);
            const float4 s4 = *reinterpret_cast<const float4*>(&st[(4 * i + 2 * pp + (j >> 3)) * kStage + 4 * h]);
            acc[0] = fmaf(s4.x, (float)D[0], acc[0]);
            acc[1] = fmaf(s4.y, (float)D[1], acc[1]);
            acc[2] = fmaf(s4.z, (float)D[2], acc[2]);
            acc[3] = fmaf(s4.w, (float)D[3], acc[3]);
        }
        if (((t + 1) & 15) == 0 || i == TW - 1) {  // end of a chunk or of the share: apply its scale
            const float xs_c = xs_lds[t >> 4][mi_l];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                tot[r] = fmaf(acc[r], xs_c, tot[r]);
                acc[r] = 0.0f;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wid][r][lane] = fmaf(tot[r], colf, cb[r]);
    __syncthreads();

    // ---- wave r < 4 sums, folds and stores register r
    if (wid >= 4) return;
    const int r = wid;
    float x = 0.0f;
#pragma unroll
    for (int q = 0; q < W; ++q) x += red[q][r][lane];
    x += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x128, 0xF, 0xF, false));
    x += dpp_partner<1>(x);
    const bool writer = j < 8 && !lo_col && mi_l < p.m;
    if constexpr (EPI == EPI_SWIGLU) {
        float lo, hi;
        swap_halves<32>(x, x, lo, hi);
        const int orow = u * kOutRows + 4 * h + r;
        if (writer && h < 2 && orow < v.N) {
            float z = silu(x) * hi;
            if (v.rowscale) z *= v.rowscale[mi_l];
            v.y[(int64_t)mi_l * v.N + orow] = z;
        }
    } else {
        const int orow = u * kMmaRows + 4 * h + r;
        if (writer && orow < v.N) {
            const int64_t o = (int64_t)mi_l * v.N + orow;
            v.y[o] = p.residual ? x + p.residual[o] : x;
        }
    }
}

// Dequantize through the GEMV fragment path (load_frag + nibble unpack): one
// thread per (row, group).
template <int FMT>
__global__ void __launch_bounds__(256) k_dequant(const QMat w, int n, int K, float* out) {
    const int G = K / kGroup;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)n * G) return;
    const int64_t row = gid / G;
    const int g = (int)(gid % G);
    float* dst = out + row * K + (int64_t)g * kGroup;
    WFrag<FMT> f;
    load_frag(f, w.codes, w.scales, w.biases, row, G, g);
    if constexpr (FMT == FMT_Q4) {
        const Nib nb = unpack_nibbles(f.c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                dst[8 * j + 2 * t] = fmaf(f.s, (float)((nb.e[j] >> (8 * t)) & 0xFF), f.b);
                dst[8 * j + 2 * t + 1] = fmaf(f.s, (float)((nb.o[j] >> (8 * t)) & 0xFF), f.b);
            }
    } else {
        const int c[8] = {(int)f.c0.x, (int)f.c0.y, (int)f.c0.z, (int)f.c0.w,
                          (int)f.c1.x, (int)f.c1.y, (int)f.c1.z, (int)f.c1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) dst[4 * j + t] = f.s * (float)(signed char)((c[j] >> (8 * t)) & 0xFF);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
        cached[dev] = cu;
    }
    return cached[dev];
}

GemvShape gemv_shape(int fmt, int epi, int m, int N, int K, int max_blocks, int waves) {
    (void)fmt;
    const int G = K / kGroup;
    const int S = (G + kWave - 1) / kWave;
    const int Q = waves / S > 1 ? waves / S : 1;
    const int Mi = inst_m(m);
    const int P = (epi == EPI_SWIGLU) ? 2 : 1;
    const int R = gemv_rows(Mi, P, epi);
    const int ntiles = (N + Q * R - 1) / (Q * R);
    GemvShape sh;
    sh.Q = Q;
    sh.R = R;
    sh.block = kWave * S * Q;
    sh.grid = ntiles < max_blocks ? ntiles : max_blocks;
    if (sh.grid < 1) sh.grid = 1;
    return sh;
}

template <int FMT, int PRO, int EPI>
static hipError_t launch_m(int m, const GemvParams& p, const GemvShape& sh, int slots, hipStream_t st) {
    dim3 grid(sh.grid, slots), block(sh.block);
    if (FMT == FMT_Q4 && inst_m(m) == 1 && (p.K + kChunk - 1) / kChunk > kRow1Chunks) return hipErrorInvalidValue;
    switch (inst_m(m)) {
        case 1: hipLaunchKernelGGL((k_gemv<FMT, 1, PRO, EPI>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((k_gemv<FMT, 2, PRO, EPI>), grid, block, 0, st, p); break;
        case 4: hipLaunchKernelGGL((k_gemv<FMT, 4, PRO, EPI>), grid, block, 0, st, p); break;
        default: hipLaunchKernelGGL((k_gemv<FMT, 8, PRO, EPI>), grid, block, 0, st, p); break;
    }
    return hipGetLastError();
}

// The lm_head (argmax epilogue) at three or four rows: persistent matrix-core
// blocks.
static bool mma_head_path(int fmt, int epi, int m, const GemvParams& p) {
    return epi == EPI_ARGMAX && m >= 3 && m <= 4 && p.K == kChunk && p.nmat == 1 &&
           !p.slot_expert;
}

// Store and SwiGLU GEMVs at three or four rows over 1-3 chunks that are not
// persistent take the split-K matrix-core kernel, a block per unit.
static bool mma_sk_path(int fmt, int epi, int m, const GemvParams& p) {
    return fmt == FMT_Q4 && (epi == EPI_STORE || epi == EPI_SWIGLU) && m >= 3 && m <= 4 && !p.balance &&
           !p.slot_expert && p.nmat <= 3 && (p.K == kChunk || p.K == 2 * kChunk || p.K == 3 * kChunk);
}

// 16 waves per block while the units fit one block per compute unit (every
// SIMD then holds four of a block's waves), else 8 (three blocks of one
// chunk fit a compute unit's LDS).
template <int PRO, int EPI, int W>
static void launch_mma_sk_w(const GemvParams& p, dim3 grid, hipStream_t st) {
    const dim3 block(W * kWave);
    switch (p.K / kChunk) {
        case 1: hipLaunchKernelGGL((k_gemv_mma_sk<PRO, EPI, 1, W>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((k_gemv_mma_sk<PRO, EPI, 2, W>), grid, block, 0, st, p); break;
        default: hipLaunchKernelGGL((k_gemv_mma_sk<PRO, EPI, 3, W>), grid, block, 0, st, p); break;
    }
}

template <int PRO, int EPI>
static hipError_t launch_mma_sk(const GemvParams& p, hipStream_t st) {
    const int rows = EPI == EPI_SWIGLU ? kMmaRows / 2 : kMmaRows;
    const int units = (p.N + rows - 1) / rows;
    if (units <= device_cu_count())
        launch_mma_sk_w<PRO, EPI, 16>(p, dim3(units), st);
    else
        launch_mma_sk_w<PRO, EPI, 8>(p, dim3(units), st);
    return hipGetLastError();
}

// One 8-wave block per compute unit (fewer for a small matrix).
template <int FMT, int PRO>
static hipError_t launch_mma_head(const GemvParams& p, hipStream_t st) {
    const int units = (p.N + kMmaRows - 1) / kMmaRows;
    const int need = (units + kMaxWaves - 1) / kMaxWaves, cu = device_cu_count();
    hipLaunchKernelGGL((k_gemv_mma<FMT, PRO>), dim3(need < cu ? need : cu), dim3(64 * kMaxWaves), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_gemv(int fmt, int pro, int epi, int m, const GemvParams& p, const GemvShape& sh,
                       hipStream_t st) {
    if (p.slot_expert) return hipErrorInvalidValue;  // slot launches use launch_gemv_slots
    if (epi == EPI_ARGMAX && sh.grid > kHeadMaxBlocks) return hipErrorInvalidValue;
    if (mma_sk_path(fmt, epi, m, p)) {
        if (pro == PRO_PLAIN && epi == EPI_STORE) return launch_mma_sk<PRO_PLAIN, EPI_STORE>(p, st);
        if (pro == PRO_RMS && epi == EPI_STORE) return launch_mma_sk<PRO_RMS, EPI_STORE>(p, st);
        if (pro == PRO_CONCAT && epi == EPI_STORE) return launch_mma_sk<PRO_CONCAT, EPI_STORE>(p, st);
        if (pro == PRO_PLAIN && epi == EPI_SWIGLU) return launch_mma_sk<PRO_PLAIN, EPI_SWIGLU>(p, st);
        if (pro == PRO_RMS && epi == EPI_SWIGLU) return launch_mma_sk<PRO_RMS, EPI_SWIGLU>(p, st);
    }
    if (mma_head_path(fmt, epi, m, p) && pro == PRO_RMS)
        return fmt == FMT_Q4 ? launch_mma_head<FMT_Q4, PRO_RMS>(p, st) : launch_mma_head<FMT_Q8, PRO_RMS>(p, st);
    if (fmt == FMT_Q4) {
        if (pro == PRO_PLAIN && epi == EPI_STORE) return launch_m<FMT_Q4, PRO_PLAIN, EPI_STORE>(m, p, sh, 1, st);
        if (pro == PRO_RMS && epi == EPI_STORE) return launch_m<FMT_Q4, PRO_RMS, EPI_STORE>(m, p, sh, 1, st);
        if (pro == PRO_CONCAT && epi == EPI_STORE) return launch_m<FMT_Q4, PRO_CONCAT, EPI_STORE>(m, p, sh, 1, st);
        if (pro == PRO_PLAIN && epi == EPI_SWIGLU) return launch_m<FMT_Q4, PRO_PLAIN, EPI_SWIGLU>(m, p, sh, 1, st);
        if (pro == PRO_RMS && epi == EPI_SWIGLU) return launch_m<FMT_Q4, PRO_RMS, EPI_SWIGLU>(m, p, sh, 1, st);
        if (pro == PRO_RMS && epi == EPI_ARGMAX) return launch_m<FMT_Q4, PRO_RMS, EPI_ARGMAX>(m, p, sh, 1, st);
    } else {
        if (pro == PRO_PLAIN && epi == EPI_STORE) return launch_m<FMT_Q8, PRO_PLAIN, EPI_STORE>(m, p, sh, 1, st);
        if (pro == PRO_PLAIN && epi == EPI_SWIGLU) return launch_m<FMT_Q8, PRO_PLAIN, EPI_SWIGLU>(m, p, sh, 1, st);
        if (pro == PRO_RMS && epi == EPI_ARGMAX) return launch_m<FMT_Q8, PRO_RMS, EPI_ARGMAX>(m, p, sh, 1, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_slots(int fmt, int epi, int m, const GemvParams& p, const GemvShape& sh, int max_slots,
                             hipStream_t st) {
    if (fmt != FMT_Q8 || !p.slot_expert) return hipErrorInvalidValue;
    if (epi == EPI_SWIGLU) return launch_m<FMT_Q8, PRO_PLAIN, EPI_SWIGLU>(m, p, sh, max_slots, st);
    if (epi == EPI_STORE) return launch_m<FMT_Q8, PRO_PLAIN, EPI_STORE>(m, p, sh, max_slots, st);
    return hipErrorInvalidValue;
}

hipError_t launch_dequant(int fmt, const QMat& w, int k, float* out, hipStream_t st) {
    const int64_t threads = (int64_t)w.n * (k / kGroup);
    const int64_t blocks = (threads + 255) / 256;
    if (fmt == FMT_Q4)
        hipLaunchKernelGGL(k_dequant<FMT_Q4>, dim3((unsigned)blocks), dim3(256), 0, st, w, w.n, k, out);
    else
        hipLaunchKernelGGL(k_dequant<FMT_Q8>, dim3((unsigned)blocks), dim3(256), 0, st, w, w.n, k, out);
    return hipGetLastError();
}

}  // namespace mtp
