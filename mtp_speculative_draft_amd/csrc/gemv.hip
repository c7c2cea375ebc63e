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

template <bool SLOT>
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
    if constexpr (SLOT) {
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

// Row mi's input for the features of segment seg (PRO_CONCAT: 0 = the
// embedding row, or the token's table row, 1 = the hidden row; otherwise the
// one input row) and the matching gamma.
template <int PRO>
__device__ __forceinline__ const float* x_segment(const GemvParams& p, const View& v, int mi, int seg,
                                                  const float*& gam, int tok_in = INT_MIN) {
    if constexpr (PRO == PRO_CONCAT) {
        if (seg) {
            gam = p.g1;
            return p.x1 + (int64_t)mi * p.H;
        }
        gam = p.g0;
        if (p.tokens) {
            int tok = tok_in != INT_MIN ? tok_in : p.tokens[mi];  // tok_in: the row's token, already read
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

// Norm (for PRO_RMS / PRO_CONCAT) of the lane's features of row mi, then its
// fragment.  Every thread of the block calls it; it holds block barriers when
// several waves share one weight row (S > 1).
template <int FMT, int PRO>
__device__ __forceinline__ void norm_row(const GemvParams& p, const View& v, int wid, int lane, int S, int mi,
                                         int kk, bool active, float (&xv)[32], const float (&gv)[32], XFrag& xf,
                                         float (*nred)[2]) {
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
    make_frag<FMT>(xv, xf);
}

// One activation row.  Each wave loads its whole chunk s of the row in 1 KB
// pieces (lane l holds features 256 i + 4 l .. +3 of piece i), so every load
// instruction reads a contiguous kilobyte; the loads are requested before the
// first weight tiles (row1_load), with no branches, so that the setup waits
// for them alone, and consumed after (row1_finish): the norm (over the
// block's chunk waves through LDS when S > 1), then the pieces pass through a
// wave-private LDS region (groups 36 floats apart, so that both the writes
// and the group reads spread over all banks) to the lane that owns the group.
struct Row1Pieces {
    float4 x[8], g[8];
};
constexpr int kRow1Chunks = 4;  // K <= 8192
constexpr int kGroupStride = 36;  // floats between groups in the LDS transposes
constexpr int kRow1Floats = kWave * kGroupStride;

template <int PRO>
__device__ __forceinline__ void row1_load(const GemvParams& p, const View& v, int lane, int s, int tok0,
                                          Row1Pieces& rp) {
    const float *gam0 = nullptr, *gam1 = nullptr;
    const float* src0 = x_segment<PRO>(p, v, 0, 0, gam0, PRO == PRO_CONCAT ? tok0 : INT_MIN);
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

template <int FMT, int PRO>
__device__ __forceinline__ void row1_finish(const GemvParams& p, const View& v, int lane, int S, int s, int q,
                                            Row1Pieces& rp, float* xq, float (*part)[2], XFrag& xf) {
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
    // piece i, lane l -> group 8 i + l / 8, features 4 (l % 8) ..
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<float4*>(xq + (8 * i + (lane >> 3)) * kGroupStride + 4 * (lane & 7)) = rp.x[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float xv[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float4 t = *reinterpret_cast<const float4*>(xq + lane * kGroupStride + 4 * k);
        xv[4 * k] = t.x;
        xv[4 * k + 1] = t.y;
        xv[4 * k + 2] = t.z;
        xv[4 * k + 3] = t.w;
    }
    make_frag<FMT>(xv, xf);
}

// Four plain rows (the four-row pass): each wave loads its chunk of every
// row in 1 KB pieces as row1_load does (a load instruction covers eight whole
// lines, where each lane's own group would touch 64), rows past m reading row
// 0 (zeroed later), and passes them one row at a time through its LDS region
// to the lanes that own the groups.
__device__ __forceinline__ void rows4_load(const View& v, int lane, int s, int m, Row1Pieces (&rp)[4]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const float* src = v.x0 + (int64_t)(mi < m ? mi : 0) * v.K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int f = kChunk * s + 256 * i + 4 * lane;
            f = f < v.K ? f : 0;  // past the end: any valid address, zeroed in rows4_finish
            rp[mi].x[i] = *reinterpret_cast<const float4*>(src + f);
        }
    }
}

template <int FMT>
__device__ __forceinline__ void rows4_finish(const View& v, int lane, int s, int m, Row1Pieces (&rp)[4], float* xq,
                                             XFrag (&xf)[4]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        // piece i, lane l -> group 8 i + l / 8, features 4 (l % 8) ..
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool live = mi < m && kChunk * s + 256 * i + 4 * lane < v.K;
            *reinterpret_cast<float4*>(xq + (8 * i + (lane >> 3)) * kGroupStride + 4 * (lane & 7)) =
                live ? rp[mi].x[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float xv[32];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float4 t = *reinterpret_cast<const float4*>(xq + lane * kGroupStride + 4 * k);
            xv[4 * k] = t.x;
            xv[4 * k + 1] = t.y;
            xv[4 * k + 2] = t.z;
            xv[4 * k + 3] = t.w;
        }
        // every lane has read the row before the next one overwrites the region
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        make_frag<FMT>(xv, xf[mi]);
    }
}

// Weight fragments of one tile (R rows x P matrices) for this lane's group.
template <int FMT, int R, int P>
struct TileFrags {
    WFrag<FMT> f[R][P];
};

// MULTI: up to three matrices concatenated along n (P == 1); otherwise one
// matrix, or the SwiGLU pair (P == 2).
template <int FMT, int R, int P, bool MULTI>
__device__ __forceinline__ void load_tile(TileFrags<FMT, R, P>& tf, const View& v, int row0, int gc) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int row = row0 + r;
        row = row < v.N ? row : v.N - 1;  // tail rows are computed and dropped
        if constexpr (P == 2) {
            load_frag(tf.f[r][0], v.c0, v.s0, v.b0, row, v.G, gc);
            load_frag(tf.f[r][1], v.c1, v.s1, v.b1, row, v.G, gc);
        } else if constexpr (!MULTI) {
            load_frag(tf.f[r][0], v.c0, v.s0, v.b0, row, v.G, gc);
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
#pragma unroll
                for (int mi = 0; mi < M; ++mi) acc[(r * M + mi) * P + pp] = dot_q4(f.c, f.s, f.b, xf[mi]);
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
// In the shared mode wave w's first ns units are fixed (k = w, Q + w, ...), so
// that they can be requested before the block has set its counter up; the
// counter starts at ns * Q and start_claims() (after the block barrier that
// follows the counter's initialisation) puts the first claim in flight.
struct TileSeq {
    int base, step, NU, i;
    bool shared;
    int wid, Q, ns;
    int pend;  // claim in flight (valid in lane 0)

    __device__ void init(int b, int st, int nu) {
        base = b;
        step = st;
        NU = nu;
        i = 0;
        shared = false;
    }
    __device__ void init_shared(int b, int st, int nu, int w, int q, int nfixed) {
        init(b, st, nu);
        shared = true;
        wid = w;
        Q = q;
        ns = nfixed;
    }
    template <class Claim>
    __device__ void start_claims(Claim claim) {
        if (shared) pend = claim();
    }
    template <class Claim>
    __device__ int next(Claim claim) {
        int k;
        if (!shared) {
            k = i++;
        } else if (i < ns) {
            k = i++ * Q + wid;
        } else {
            k = __builtin_amdgcn_readfirstlane(pend);
            pend = claim();
        }
        const int u = base + step * k;
        return u < NU ? u : -1;
    }
};

// The launch parameters that the first requests of k_gemv depend on, named in
// one empty asm statement as scalar operands: the compiler then issues all
// their loads back to back and waits for them once, where it would otherwise
// load each group where it is first used and wait there (a division by S,
// then the pointers, ...), one round trip after another.
// The lm_head's, its epilogue's pointers included (the argmax state, the
// normed row and the logits are used by every wave at its end).
__device__ __forceinline__ void gather_head_params(const GemvParams& p, unsigned gx) {
    asm volatile("" ::"s"(p.w[0].codes), "s"(p.w[0].scales), "s"(p.w[0].biases), "s"(p.N), "s"(p.K), "s"(p.G),
                 "s"(p.S), "s"(p.m), "s"(gx), "s"(p.x0), "s"(p.g0), "s"(p.eps), "s"(p.balance), "s"(p.normed_out),
                 "s"(p.logits), "s"(p.head_keys), "s"(p.counter), "s"(p.ids));
}

template <int PRO, int EPI>
__device__ __forceinline__ void gather_params(const GemvParams& p, unsigned gx, unsigned* zero_words, int zero_n) {
    if constexpr (PRO == PRO_CONCAT)
        asm volatile("" ::"s"(p.w[0].codes), "s"(p.w[0].scales), "s"(p.w[0].biases), "s"(p.N), "s"(p.K), "s"(p.G),
                     "s"(p.S), "s"(p.m), "s"(gx), "s"(p.x0), "s"(p.x1), "s"(p.tokens), "s"(p.table), "s"(p.vocab),
                     "s"(p.H), "s"(p.g0), "s"(p.g1), "s"(p.eps), "s"(p.residual), "s"(zero_words), "s"(zero_n));
    else if constexpr (EPI == EPI_ARGMAX)
        gather_head_params(p, gx);
    else
        asm volatile("" ::"s"(p.w[0].codes), "s"(p.w[0].scales), "s"(p.w[0].biases), "s"(p.w[1].codes),
                     "s"(p.w[1].scales), "s"(p.w[1].biases), "s"(p.w[2].codes), "s"(p.w[2].scales),
                     "s"(p.w[2].biases), "s"(p.w[0].n), "s"(p.w[1].n), "s"(p.N), "s"(p.K), "s"(p.G), "s"(p.S),
                     "s"(p.m), "s"(gx), "s"(p.x0), "s"(p.g0), "s"(p.eps), "s"(p.residual));
}

// The same for the split-K matrix-core kernel, by prologue and epilogue.
template <int PRO, int EPI>
__device__ __forceinline__ void gather_sk_params(const GemvParams& p) {
    asm volatile("" ::"s"(p.w[0].codes), "s"(p.w[0].scales), "s"(p.w[0].biases), "s"(p.w[1].codes),
                 "s"(p.w[1].scales), "s"(p.w[1].biases), "s"(p.N), "s"(p.K), "s"(p.G), "s"(p.m), "s"(p.x0), "s"(p.y));
    if constexpr (PRO != PRO_PLAIN) asm volatile("" ::"s"(p.g0), "s"(p.eps));
    if constexpr (PRO == PRO_CONCAT)
        asm volatile("" ::"s"(p.x1), "s"(p.tokens), "s"(p.table), "s"(p.vocab), "s"(p.H), "s"(p.g1),
                     "s"(p.zero_words), "s"(p.zero_n));
    if constexpr (EPI == EPI_STORE)
        asm volatile("" ::"s"(p.w[2].codes), "s"(p.w[2].scales), "s"(p.w[2].biases), "s"(p.w[0].n), "s"(p.w[1].n),
                     "s"(p.residual));
}

// SLOT: the MoE slot launch (grid.y = slots, the matrices picked per slot).
// Nothing that depends on a launch parameter branches before the first
// requests (a branch waits for the parameter loads it depends on, and the
// loads after it would wait again), so the block pays one parameter round
// trip before it asks for its activations, weights and residuals.
template <int FMT, int M, int PRO, int EPI, bool SLOT>
__global__ void __launch_bounds__(block_waves(FMT, EPI, M) * 64) k_gemv(const GemvParams p) {
    constexpr int P = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int R = gemv_rows(M, P, EPI);
    constexpr int V = R * M * P;
    constexpr int kWaves = block_waves(FMT, EPI, M);  // waves per block, at most
    // matrices concatenated along n (q/k/v); the lm_head takes the same row
    // arithmetic (for one matrix it picks matrix 0 at run time), which
    // measured faster for its loop than the one-matrix form
    constexpr bool kMulti = (PRO == PRO_RMS && EPI == EPI_STORE) || EPI == EPI_ARGMAX;
    __shared__ float red[kWaves][kWave * 2];
    __shared__ float nred[kWaves][2];
    __shared__ int claim_ctr;

    View v;
    if (!resolve_view<SLOT>(p, v)) return;
    const unsigned gx = gridDim.x;
    constexpr bool kClears = PRO == PRO_CONCAT && EPI == EPI_STORE;  // zero_words: the eh_proj only
    unsigned* const zero_words = kClears ? p.zero_words : nullptr;
    const int zero_n = kClears ? p.zero_n : 0;
    if constexpr (!SLOT) gather_params<PRO, EPI>(p, gx, zero_words, zero_n);

    // the wave index is wave-uniform; saying so lets every row, pointer and
    // branch derived from it live in scalar registers
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int S = p.S;
    const int Q = S >= kWaves ? 1 : kWaves / S;  // the launch's S * Q waves per block
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
    // their latency overlaps it (two tiles where the loop double-buffers: the
    // persistent lm_head, whose waves take many units; the other launches
    // give each wave one unit, where a second tile would only be requests
    // that hold up the others)
    constexpr bool kDouble = EPI == EPI_ARGMAX && M <= 2 && P == 1;
    const bool active = g < v.G;
    const int kk = g * kGroup;
    const bool balanced = EPI == EPI_ARGMAX && S == 1 && p.balance;  // the persistent lm_head only
    auto claim = [&]() {
        int r = 0;
        if (lane == 0) r = atomicAdd(&claim_ctr, 1);
        return r;
    };
    TileSeq ts;
    if (balanced) {
        if (threadIdx.x == 0) claim_ctr = 0;
        __syncthreads();  // the counter is set before any wave claims from it
        ts.init_shared(blockIdx.x, (int)gx, NU, wid, Q, 0);
        ts.start_claims(claim);
    } else if (S == 1)
        ts.init(blockIdx.x * Q + q, (int)gx * Q, NU);
    else
        ts.init(blockIdx.x, (int)gx, NU);
    auto row0 = [&](int u) { return (u * per + qo) * R; };
    TileFrags<FMT, R, P> tf, tf2;
    XFrag xf[M];
    // the activations are requested before the first tiles, which are then
    // requested unconditionally (tile 0 stands in for none), so that the
    // setup waits for the activations only: one row in contiguous 1 KB
    // pieces, two rows as each lane's own group.  A token row's address
    // waits for the token id: only the waves whose features reach into the
    // embedding half request it and wait for it (their row still goes out
    // before their tiles: requested after the tiles, the row, which is what
    // these waves wait for longest, would queue behind their traffic).
    constexpr bool kRow1 = M == 1;  // S <= kRow1Chunks (checked at launch)
    constexpr bool kRows4 = M == 4 && PRO == PRO_PLAIN;  // the four-row pass
    // a wave whose features reach into the embedding half of the concat
    const bool tok_wave = kRow1 && PRO == PRO_CONCAT && kChunk * s < p.H;
    Row1Pieces rp;
    Row1Pieces rp4[kRows4 ? 4 : 1];
    float xv2[M][32], gv2[32];
    int tok0 = -1;
    if (tok_wave) tok0 = p.tokens ? p.tokens[0] : -1;
    if constexpr (kRow1) {
        row1_load<PRO>(p, v, lane, s, tok_wave ? tok0 : -1, rp);
    } else if constexpr (kRows4) {
        rows4_load(v, lane, s, p.m, rp4);
    } else {
#pragma unroll
        for (int mi = 0; mi < M; ++mi) load_x_row<PRO>(p, v, mi, kk, active, xv2[mi], gv2, mi == 0);
    }
    const int pos = reduce_base<V, P>(lane) / P;  // = r * M + mi of this lane's result
    const int r_l = pos / M, mi_l = pos % M;
    const bool writer = reduce_writer<V, P>(lane);
    // the residual a writer lane adds to its result, requested with the tile
    auto load_res = [&](int u) {
        float r = 0.0f;
        if constexpr (EPI == EPI_STORE) {
            const int row = row0(u) + r_l;
            if (p.residual && u >= 0 && writer && s == 0 && row < v.N && mi_l < p.m)
                r = p.residual[(int64_t)mi_l * v.N + row];
        }
        return r;
    };
    int wa = ts.next(claim), wb = -1;
    load_tile<FMT, R, P, kMulti>(tf, v, row0(wa >= 0 ? wa : 0), gc);
    float res_a = load_res(wa), res_b = 0.0f;
    if constexpr (kDouble) {
        if (wa >= 0) wb = ts.next(claim);
        load_tile<FMT, R, P, kMulti>(tf2, v, row0(wb >= 0 ? wb : 0), gc);
        res_b = load_res(wb);
    }
    if constexpr (kRow1) {
        __shared__ float xq1[kWaves][kRow1Floats];
        __shared__ float part1[kRow1Chunks][2];
        row1_finish<FMT, PRO>(p, v, lane, S, s, q, rp, xq1[wid], part1, xf[0]);
    } else if constexpr (kRows4) {
        __shared__ float xq4[kWaves][kRow1Floats];
        rows4_finish<FMT>(v, lane, s, p.m, rp4, xq4[wid], xf);
    } else {
#pragma unroll
        for (int mi = 0; mi < M; ++mi) norm_row<FMT, PRO>(p, v, wid, lane, S, mi, kk, active, xv2[mi], gv2, xf[mi], nred);
    }

    float best = -INFINITY;
    int best_i = INT_MAX;

    // reduce one tile's partials across the lanes (and the S chunk waves) and
    // apply the epilogue
    auto finish = [&](float (&acc)[V], int row0, float res) {
        reduce_transpose<V, P>(acc, lane);
        float v0 = acc[0];
        float v1 = (P == 2) ? acc[P - 1] : 0.0f;
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
                    if (writer) v.y[o] = p.residual ? v0 + res : v0;
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
                finish(acc, row0(wa), res_a);
            }
            if (wb < 0) break;
            wa = ts.next(claim);
            if (wa >= 0) {
                load_tile<FMT, R, P, kMulti>(tf, v, row0(wa), gc);
                res_a = load_res(wa);
            }
            {
                float acc[V];
                compute_tile<FMT, M, R, P>(tf2, xf, acc);
                finish(acc, row0(wb), res_b);
            }
            wb = wa >= 0 ? ts.next(claim) : -1;
            if (wb >= 0) {
                load_tile<FMT, R, P, kMulti>(tf2, v, row0(wb), gc);
                res_b = load_res(wb);
            }
        }
    } else {
        while (wa >= 0) {
            float acc[V];
            compute_tile<FMT, M, R, P>(tf, xf, acc);
            // next tile's loads fly while this one is reduced and stored
            const int nx = ts.next(claim);
            float res_n = 0.0f;
            if (nx >= 0) {
                load_tile<FMT, R, P, kMulti>(tf, v, row0(nx), gc);
                res_n = load_res(nx);
            }
            finish(acc, row0(wa), res_a);
            wa = nx;
            res_a = res_n;
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
    // the lm_head's argmax state, cleared by the layer's first launch (the
    // eh_proj; its readers run later on the same stream)
    if constexpr (kClears)
        if (zero_words && blockIdx.x == 0 && blockIdx.y == 0)
            for (int i = threadIdx.x; i < zero_n; i += kWave * S * Q) zero_words[i] = 0u;  // (the block's threads)
}

// ---------------------------------------------------------------------------
// Matrix-core GEMVs for three and four activation rows (f16 MFMA 16x16x32,
// one group of 32 features per MFMA).
//
// A (weights): 16 weight rows.  Lane (h = l/16, j = l%16) holds row j's
// k-slot h of the group as 8 f16 halves: the code subnormals of q4_halves
// (4-bit: word h of the group) or q8_halves (8-bit: words 2 rho(h), 2 rho(h)+1
// with rho = 0, 2, 1, 3), with no conversion.
// B (activations): the same k-slots in 12 columns; column 3 mi + t is term t
// of activation row mi, where v = x 2^(15-e) = hi + mid + lo in three f16
// values (2^e bounds the row's largest |x|, and features on 16c halves carry
// 1/16).  hi is v rounded to a fixed grid (16, or 1 for the 1/16 features),
// so all hi products of a group are multiples of one unit and their sum fits
// f32's 24 bits: the matrix core adds them exactly whatever its alignment
// and rounding.  mid and lo are the f16 remainder (|mid| <= 8), so x is
// represented down to 2^-34 of the row's largest value.  Every product is
// exact; the MFMA accumulates in f32.  Columns 12..15 read copies of
// other columns and their results are never used (each D column depends on
// its own B column only).
// The codes enter centred (4-bit c - 8, 8-bit c; see q4_operand).
// D: lane (h, c) holds rows 4h..4h+3 of column c.  Each group's D is scaled
// by its rows' group scales (staged per wave in LDS) into an f32 accumulator;
// the 4-bit bias, (b + 8 s) sum(x), is an f32 MFMA (16x16x4) over the group
// sums.  At the end every column is scaled back by 2^(9+e) (2^24 for the code
// subnormals times 2^(e-15)), and the three term columns of a row are added
// (DPP).
// ---------------------------------------------------------------------------
typedef float v4f_t __attribute__((ext_vector_type(4)));
constexpr int kMmaRows = 16;
constexpr int kMmaCols = 16;
constexpr int kBCols = 12;           // term columns: 4 rows x 3 terms
// B operands (u32x4) per group: 4 k-slots x 12 columns, and one entry of
// padding, so that the groups a wave writes at once start on different banks
constexpr int kBGroup = 4 * kBCols + 1;
constexpr int kStage = 20;           // floats per group in a wave's scale stage (16 rows, 16-byte aligned)

__device__ __forceinline__ void perm32_swap(unsigned& a, unsigned& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

__device__ __forceinline__ void perm16_swap(unsigned& a, unsigned& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// 4 x 4 transpose across the lane quarters: quarter q's word i becomes the
// word q that quarter i held.
__device__ __forceinline__ void quarter_transpose(unsigned& w0, unsigned& w1, unsigned& w2, unsigned& w3) {
    perm32_swap(w0, w2);
    perm32_swap(w1, w3);
    perm16_swap(w0, w1);
    perm16_swap(w2, w3);
}

__device__ __forceinline__ h8_t as_h8(unsigned a, unsigned b, unsigned c, unsigned d) {
    const u32x4 t = {a, b, c, d};
    return __builtin_bit_cast(h8_t, t);
}

__device__ __forceinline__ unsigned half_bits(float x) {
    return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)x);
}

// Two f32 values to an f16 pair (round to nearest even), and its bits.
typedef float f2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2_t pack_h2(float a, float b) {
    return __builtin_convertvector((f2_t){a, b}, h2_t);
}
__device__ __forceinline__ unsigned h2_bits(h2_t h) { return __builtin_bit_cast(unsigned, h); }

// Activation setup of the matrix-core kernels, shared by a block's waves:
// wave w takes activation row w % 4 and, of each of the S chunks, the 1 KB
// pieces NI (w / 4) .. NI (w / 4) + NI - 1 (lane l holds features
// 256 i + 4 l .. +3 of piece i), so that every load instruction reads one
// contiguous kilobyte.  The loads are issued first (mma_load_x), so that
// they overlap the weight requests that follow, and consumed by mma_setup.
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

// The rest of the setup: the norms (PRO_RMS, PRO_CONCAT) and the row maximum
// (of a normed row, a bound taken in the norm's pass), combined over the R
// waves of a row through part in one exchange, then the B operands
// (bq), the group sums (tx, column 3 mi of each group) and the scale-back
// factors (unsc).  Ends with a block barrier.
template <int FMT, int PRO, int S, int R>
__device__ __forceinline__ void mma_setup(const GemvParams& p, const View& v, int mi, int sub, int lane,
                                          XPieces<S, 8 / R>& xp, u32x4* bq, float (*tx)[kMmaCols], float* unsc,
                                          float (*part)[4][R]) {
    constexpr int NI = 8 / R;
    static_assert(FMT == FMT_Q4 || S == 1, "8-bit operands cover one chunk");
    const bool live = mi < p.m;
    float am = 0.0f;  // the row's largest |value|, or a bound just above it
    if constexpr (PRO != PRO_PLAIN) {
        // sum of squares and max |x gamma| of each segment in one pass and one
        // exchange: the normalised row's maximum is inv max |x gamma|
        float ss0 = 0.0f, ss1 = 0.0f, gm0 = 0.0f, gm1 = 0.0f;
#pragma unroll
        for (int c = 0; c < S; ++c)
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) {
                const float4 x = xp.x[c][ii], g = xp.g[c][ii];
                const float ss = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, x.w * x.w)));
                const float gm = fmaxf(fmaxf(fabsf(x.x * g.x), fabsf(x.y * g.y)),
                                       fmaxf(fabsf(x.z * g.z), fabsf(x.w * g.w)));
                if (PRO == PRO_CONCAT && kChunk * c + 256 * (sub * NI + ii) + 4 * lane >= p.H) {
                    ss1 += ss;
                    gm1 = fmaxf(gm1, gm);
                } else {
                    ss0 += ss;
                    gm0 = fmaxf(gm0, gm);
                }
            }
        ss0 = wave_sum(ss0);
        gm0 = wave_max(gm0);
        if constexpr (PRO == PRO_CONCAT) {
            ss1 = wave_sum(ss1);
            gm1 = wave_max(gm1);
        }
        if constexpr (R > 1) {
            if (lane == 0) {
                part[0][mi][sub] = ss0;
                part[1][mi][sub] = ss1;
                part[2][mi][sub] = gm0;
                part[3][mi][sub] = gm1;
            }
            __syncthreads();
            ss0 = 0.0f;
            ss1 = 0.0f;
#pragma unroll
            for (int q = 0; q < R; ++q) {
                ss0 += part[0][mi][q];
                ss1 += part[1][mi][q];
                gm0 = fmaxf(gm0, part[2][mi][q]);
                gm1 = fmaxf(gm1, part[3][mi][q]);
            }
        }
        const int nfeat = PRO == PRO_CONCAT ? p.H : v.K;
        const float inv0 = rsqrtf(ss0 / (float)nfeat + p.eps);
        const float inv1 = PRO == PRO_CONCAT ? rsqrtf(ss1 / (float)nfeat + p.eps) : inv0;
        // A normalised value (x inv) gamma and the bound inv max |x gamma|
        // differ by at most four roundings (< 2^-21 relative): the margin
        // 2^-20 keeps the bound above every |value|, so the term split's hi
        // parts stay within f16's exact range (a bound that crosses a power of
        // two costs one bit of the split's range, nothing else).
        am = fmaxf(inv0 * gm0, inv1 * gm1) * (1.0f + 0x1p-20f);
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
    } else {
#pragma unroll
        for (int c = 0; c < S; ++c)
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) {
                const float4 x = xp.x[c][ii];
                am = fmaxf(am, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
            }
        am = wave_max(am);
        if constexpr (R > 1) {
            if (lane == 0) part[2][mi][sub] = am;
            __syncthreads();
            am = part[2][mi][0];
#pragma unroll
            for (int q = 1; q < R; ++q) am = fmaxf(am, part[2][mi][q]);
        }
    }
    int e = 0;
    (void)frexpf(am, &e);  // am = m 2^e with m in [0.5, 1); e = 0 for am = 0
    const float sc = ldexpf(1.0f, 15 - e);
    if (sub == 0 && lane == 0) unsc[mi] = ldexpf(1.0f, 9 + e);
    const bool odd = lane & 1;
#pragma unroll
    for (int c = 0; c < S; ++c)
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
            const float4 x4 = xp.x[c][ii];
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
            const int gg = 64 * c + 8 * (sub * NI + ii) + (lane >> 3);  // group (all chunks)
            // the group's sum over its eight lanes
            float gs = (xv[0] + xv[1]) + (xv[2] + xv[3]);
            gs += dpp_partner<1>(gs);
            gs += dpp_partner<2>(gs);
            gs += dpp_partner<4>(gs);
            if ((lane & 7) < 3) tx[gg][3 * mi + (lane & 7)] = (lane & 7) == 0 ? gs : 0.0f;
            u32x4* grp = bq + gg * kBGroup;
            if constexpr (FMT == FMT_Q4) {
                // Lanes 2 k and 2 k + 1 hold features 0-3 and 4-7 of word k,
                // and operand word i of its k-slot pairs features (i, i + 4)
                // (q4_halves).  The pair swaps two values, so that lane 2 k + s
                // holds features 2 s, 2 s + 1, 2 s + 4, 2 s + 5 and forms the
                // words 2 s and 2 s + 1 alone; features 2 s + 1 and 2 s + 5 sit
                // on the 16c halves.
                const float r0 = dpp_partner<1>(odd ? xv[0] : xv[2]), r1 = dpp_partner<1>(odd ? xv[1] : xv[3]);
                const float pv[4] = {odd ? r0 : xv[0], odd ? r1 : xv[1], odd ? xv[2] : r0, odd ? xv[3] : r1};
                float hi[4], rm[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // term split of v = x 2^(15-e): hi is v on the grid 16 (1 for
                    // the 1/16 features), so every hi product lies on one grid
                    // and the MFMA sums them exactly; mid is the remainder rm
                    // rounded to f16 and lo the rest, in f16
                    const bool sixteenth = q & 1;
                    const float vq = pv[q] * sc * (sixteenth ? 0.0625f : 1.0f);
                    const float step = sixteenth ? 1.0f : 16.0f;
                    hi[q] = rintf(vq * (1.0f / step)) * step;  // |hi / step| <= 2^11: exact in f16
                    rm[q] = vq - hi[q];
                }
                const h2_t m0 = pack_h2(rm[0], rm[2]), m1 = pack_h2(rm[1], rm[3]);
                const h2_t l0 = pack_h2(rm[0] - (float)m0.x, rm[2] - (float)m0.y);
                const h2_t l1 = pack_h2(rm[1] - (float)m1.x, rm[3] - (float)m1.y);
                // term columns 3 mi .. 3 mi + 2 of k-slot (lane % 8) / 2: words 2 s, 2 s + 1
                unsigned* dst = reinterpret_cast<unsigned*>(grp + ((lane & 7) >> 1) * kBCols + 3 * mi) + 2 * odd;
                *reinterpret_cast<uint2*>(dst) = make_uint2(h2_bits(pack_h2(hi[0], hi[2])), h2_bits(pack_h2(hi[1], hi[3])));
                *reinterpret_cast<uint2*>(dst + 4) = make_uint2(h2_bits(m0), h2_bits(m1));
                *reinterpret_cast<uint2*>(dst + 8) = make_uint2(h2_bits(l0), h2_bits(l1));
            } else {
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    unsigned hb[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // term t of v = x 2^(15-e), split as for the 4-bit
                        // operands with the grid 16 for every feature
                        const float vq = xv[q] * sc;
                        const float hi = rintf(vq * (1.0f / 16.0f)) * 16.0f;
                        const float r1 = vq - hi;
                        const _Float16 h1 = (_Float16)r1;
                        const float r2 = r1 - (float)h1;
                        hb[q] = half_bits(t == 0 ? hi : (t == 1 ? (float)h1 : r2));
                    }
                    // 8-bit word lane % 8 of the group sits in k-slot rho(word / 2),
                    // halves 4 (word % 2) ..: pairs (feature 0, 2) and (1, 3)
                    const int wd = lane & 7, hq = ((wd >> 1) & 1) * 2 + (wd >> 2);
                    unsigned* dst = reinterpret_cast<unsigned*>(grp + hq * kBCols + 3 * mi + t) + 2 * (wd & 1);
                    *reinterpret_cast<uint2*>(dst) = make_uint2(hb[0] | (hb[2] << 16), hb[1] | (hb[3] << 16));
                }
            }
        }
    __syncthreads();
}

// A operands with centred codes: the f16 subnormal pairs shifted by an
// exact packed f16 subtraction, 4-bit c - 8 (16 (c - 8) on the 16c halves)
// and 8-bit c.  Centred, a group's product has no common part that the bias
// would cancel later, so the matrix core's accumulation error stays at the
// size of the result instead of the size of 8 sum(x) (4-bit) or 128 sum(x)
// (8-bit).
__device__ __forceinline__ unsigned sub_h2(unsigned r, unsigned k) {
    return __builtin_bit_cast(unsigned, as_h2(r) - as_h2(k));
}
constexpr unsigned kHalves8 = 0x00080008u;    // (8, 8) x 2^-24
constexpr unsigned kHalves128 = 0x00800080u;  // (128, 128) x 2^-24

__device__ __forceinline__ h8_t q8_operand(unsigned wa, unsigned wb) {
    const Q8Halves a = q8_halves(wa), b = q8_halves(wb);
    return as_h8(sub_h2(a.r[0], kHalves128), sub_h2(a.r[1], kHalves128), sub_h2(b.r[0], kHalves128),
                 sub_h2(b.r[1], kHalves128));
}

__device__ __forceinline__ h8_t q4_operand(unsigned w) {
    const Q4Halves q = q4_halves(w);
    return as_h8(sub_h2(q.r[0], kHalves8), sub_h2(q.r[1], kHalves128), sub_h2(q.r[2], kHalves8),
                 sub_h2(q.r[3], kHalves128));
}

// Sum of a lane's column and the next two (the three terms of an activation
// row land in the writer lane 3 mi).
__device__ __forceinline__ float add_terms(float x) {
    const float a = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x101, 0xF, 0xF, false));
    const float b = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x102, 0xF, 0xF, false));
    return x + a + b;
}

// The lm_head (argmax epilogue) at three or four rows, K = 2048: persistent,
// one 8-wave block per compute unit; a wave takes 16-row units claimed from
// its block's LDS counter.  The next unit's codes are requested register by
// register as the current unit consumes them (past the last unit, and for
// the first request, they go to unit 0, one small region that hits in L2,
// which keeps the loads unconditional).
template <int FMT, int PRO, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_mma(const GemvParams p) {
    static_assert(W >= 4, "waves 0-3 build the B operands");
    constexpr int R = 1;  // waves per activation row in the setup
    constexpr int NT = FMT == FMT_Q4 ? 16 : 32;  // 16-byte code loads per lane and unit
    __shared__ u32x4 bq[64 * kBGroup];               // 49 KB: B operands
    __shared__ float tx[64][kMmaCols];               // 4 KB: group sums in column 3 mi (4-bit bias)
    __shared__ float stage[W][64 * kStage];  // 5 KB per wave: its scales, [group][row]
    __shared__ float part[4][4][R];
    __shared__ float unsc[4];
    __shared__ int claim_ctr;

    View v;
    resolve_view<false>(p, v);
    gather_head_params(p, gridDim.x);
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
    ts.init_shared(blockIdx.x, gridDim.x, NU, wid, W, 0);
    ts.start_claims(claim);

    const int j = lane & 15, h = lane >> 4;
    const int mi_l = j / 3;
    const bool writer = j < kBCols && j % 3 == 0 && mi_l < p.m;
    const u32x4* bsrc = bq + h * kBCols + (j < kBCols ? j : j - 4);
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
    // Plain loads: a 4-bit load reads one half of a 128-byte line of each of
    // 16 rows and the next load the other half, so the line is better kept in
    // L2 than streamed past it.
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

    // Waves 0-3 build the B operands (activation row w each) while the
    // other waves request their first unit's weights at once.  A wave issues
    // its memory requests in order and stalls while the memory queues are
    // full, so a wave that requested weights first would start its setup only
    // once the weights drain; the barrier after the activation requests keeps
    // those ahead of every weight request of the block.
    XPieces<1, 8> xp;
    const bool setup_wave = wid < 4;
    if (setup_wave) mma_load_x<PRO, 1, 8>(p, v, wid, 0, lane, xp);
    __builtin_amdgcn_s_barrier();
    int u = ts.next(claim);
    auto first_loads = [&]() {
        const char* crow;
        const float *srow, *brow;
        row_ptrs(u >= 0 ? u : 0, crow, srow, brow);
#pragma unroll
        for (int t = 0; t < NT; ++t) load_codes(crow, t);
        load_sb(srow, brow);
    };
    if (setup_wave) {
        mma_setup<FMT, PRO, 1, 1>(p, v, wid, 0, lane, xp, bq, tx, unsc, part);  // ends with a block barrier
        first_loads();
    } else {
        first_loads();
        __syncthreads();  // the setup's closing barrier
    }
    const float cf = j < kBCols ? unsc[mi_l] : 0.0f;
    while (u >= 0) {
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
                if constexpr (FMT == FMT_Q4)
                    cb4[e & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(fmaf(8.0f, sv[t][e], bv[t][e]), tx[gg][j],
                                                                      cb4[e & 1], 0, 0, 0);
            }
        }
        load_sb(nsrow, nbrow);
        __builtin_amdgcn_wave_barrier();

        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
        auto group = [&](const h8_t& A, int gg) {
            const h8_t B = __builtin_bit_cast(h8_t, bsrc[gg * kBGroup]);
            const v4f_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, zero, 0, 0, 0);
            const float4 s4 = *reinterpret_cast<const float4*>(&st[gg * kStage + 4 * h]);
            acc[0] = fmaf(s4.x, D[0], acc[0]);
            acc[1] = fmaf(s4.y, D[1], acc[1]);
            acc[2] = fmaf(s4.z, D[2], acc[2]);
            acc[3] = fmaf(s4.w, D[3], acc[3]);
        };
        if constexpr (FMT == FMT_Q4) {
            // load t: lane quarter h holds group 4 t + h; after the transpose
            // word i is word h of group 4 t + i
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                unsigned w0 = cw[t].x, w1 = cw[t].y, w2 = cw[t].z, w3 = cw[t].w;
                quarter_transpose(w0, w1, w2, w3);
                load_codes(ncrow, t);  // the registers are free: the next unit's request
                group(q4_operand(w0), 4 * t);
                group(q4_operand(w1), 4 * t + 1);
                group(q4_operand(w2), 4 * t + 2);
                group(q4_operand(w3), 4 * t + 3);
            }
        } else {
            // load t: lane quarter h holds bytes 16 h .. of the group pair
            // 2 t, 2 t + 1 (quarters 0, 1 the first group); one swap gives each
            // quarter two words of both
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                unsigned w0 = cw[t].x, w1 = cw[t].y, w2 = cw[t].z, w3 = cw[t].w;
                perm32_swap(w0, w2);
                perm32_swap(w1, w3);
                load_codes(ncrow, t);
                group(q8_operand(w0, w1), 2 * t);
                group(q8_operand(w2, w3), 2 * t + 1);
            }
        }
        __builtin_amdgcn_wave_barrier();
        const v4f_t cb = cb4[0] + cb4[1];
        float res[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) res[r] = add_terms(fmaf(acc[r], cf, cb[r]));
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
        __shared__ float bv_s[W][8];
        __shared__ int bi_s[W][8];
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
        if (wid == 0) grid_argmax<4>(p, W, bv_s, bi_s, sink, lane);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core GEMV with the K range split over a block's W waves, for the
// 4-bit projections other than the lm_head: a block takes a unit (16 weight
// rows; 8 output rows of the SwiGLU pair, or 8 rows of a store with few
// units: HALF) over K = 2048 S with S <= 2.  A block per unit puts many more
// compute units to work than a wave per unit, and each wave's share (16 S / W
// loads of four groups) is short; with W = 16 every SIMD holds four waves,
// which hides the latency of both the activation setup and the loop.  The
// waves' partial sums meet in LDS, and wave r < 4 folds and stores register
// r.  PERSIST (more units than compute units): one block per compute unit
// builds the activation operands once and loops over its units, requesting
// the next unit's weights before each reduction.  Operands and arithmetic are
// those of k_gemv_mma.
// ---------------------------------------------------------------------------
template <int PRO, int EPI, int S, int W, bool PERSIST, bool HALF = false>
__global__ void __launch_bounds__(64 * W) k_gemv_mma_sk(const GemvParams p) {
    constexpr int R = W / 4;    // waves per activation row in the setup
    constexpr int NI = 8 / R;   // 1 KB pieces of each chunk per wave in the setup
    constexpr int T = 16 * S;   // loads (4 groups x 16 rows each) over K
    constexpr int TW = T / W;   // loads per wave
    constexpr int GW = 4 * TW;  // groups per wave
    constexpr int NE = GW / 4;  // groups per lane quarter
    static_assert(T % W == 0 && 8 % R == 0, "wave split");
    __shared__ u32x4 bq[64 * S * kBGroup];    // B operands, 49 KB per chunk
    __shared__ float tx[64 * S][kMmaCols];    // group sums, 4 KB per chunk
    __shared__ float stage[W][GW * kStage];   // each wave's scales, [group][row]
    __shared__ float red[PERSIST ? 2 : 1][W][4][kWave];  // the waves' partial sums (two areas in the loop)
    __shared__ float part[4][4][R];
    __shared__ float unsc[4];

    View v;
    resolve_view<false>(p, v);
    gather_sk_params<PRO, EPI>(p);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // HALF (store): 8-row units, lanes j and j + 8 on one row (twice the
    // blocks for the matrices that give fewer units than compute units)
    constexpr bool kHalfRows = EPI == EPI_SWIGLU || HALF;
    constexpr int kOutRows = kHalfRows ? kMmaRows / 2 : kMmaRows;
    const int NU = (v.N + kOutRows - 1) / kOutRows;
    int u = blockIdx.x;  // this block's units: blockIdx.x + gridDim.x k

    // ---- activations first (they come from L2 and are needed first)
    const int mi = wid & 3, sub = wid >> 2;
    XPieces<S, NI> xp;
    mma_load_x<PRO, S, NI>(p, v, mi, sub, lane, xp);

    // ---- this wave's weights of a unit
    const int j = lane & 15, h = lane >> 4;
    const int t0 = wid * TW, g0 = wid * GW;
    const int mi_l = j / 3;
    const bool writer = j < kBCols && j % 3 == 0 && mi_l < p.m;
    u32x4 cw[TW];
    float sv[NE], bv[NE];
    auto load_unit = [&](int uu) {
        int row = uu * kOutRows + (kHalfRows ? (j & 7) : j);
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
        const char* crow =
            static_cast<const char*>(v.c0) + in1 * v.dc1 + in2 * v.dc2 + (int64_t)lr * (v.K / 2) + 16 * h;
        const float* srow = reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.s0) + in1 * v.ds1 +
                                                           in2 * v.ds2) + (int64_t)lr * v.G + g0 + NE * h;
        const float* brow = reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.b0) + in1 * v.db1 +
                                                           in2 * v.db2) + (int64_t)lr * v.G + g0 + NE * h;
#pragma unroll
        for (int i = 0; i < TW; ++i) cw[i] = *reinterpret_cast<const u32x4*>(crow + 64 * (t0 + i));
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            sv[e] = __builtin_nontemporal_load(srow + e);
            bv[e] = __builtin_nontemporal_load(brow + e);
        }
    };
    // the residual that a storing lane (waves 0-3) adds, requested with the
    // weights
    auto load_res = [&](int uu) {
        float r = 0.0f;
        if constexpr (EPI == EPI_STORE) {
            const int orow = uu * kOutRows + 4 * h + wid;
            if (p.residual && wid < 4 && writer && (!HALF || h < 2) && orow < v.N)
                r = p.residual[(int64_t)mi_l * v.N + orow];
        }
        return r;
    };
    load_unit(u);
    float res = load_res(u);

    mma_setup<FMT_Q4, PRO, S, R>(p, v, mi, sub, lane, xp, bq, tx, unsc, part);
    // the lm_head's argmax state, cleared by the layer's first launch (the
    // eh_proj; its readers run later on the same stream)
    if constexpr (PRO == PRO_CONCAT)
        if (p.zero_words && blockIdx.x == 0)
            for (int i = threadIdx.x; i < p.zero_n; i += 64 * W) p.zero_words[i] = 0u;  // (64 W threads a block)

    float* st = stage[wid];
    const u32x4* bsrc = bq + h * kBCols + (j < kBCols ? j : j - 4);
    const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const float cf = j < kBCols ? unsc[j / 3] : 0.0f;
    for (int it = 0;; ++it) {
        // ---- bias sums and this wave's scale stage (lane quarter h holds
        // the scales of groups g0 + NE h .. of its row)
        v4f_t cb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int gl = NE * h + e;  // group within the wave's share
            st[gl * kStage + j] = sv[e];
            cb = __builtin_amdgcn_mfma_f32_16x16x4f32(fmaf(8.0f, sv[e], bv[e]), tx[g0 + gl][j], cb, 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();

        // ---- products
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int t = t0 + i;
            unsigned w[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
            quarter_transpose(w[0], w[1], w[2], w[3]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const h8_t B = __builtin_bit_cast(h8_t, bsrc[(4 * t + q) * kBGroup]);
                const v4f_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(q4_operand(w[q]), B, zero, 0, 0, 0);
                const float4 s4 = *reinterpret_cast<const float4*>(&st[(4 * i + q) * kStage + 4 * h]);
                acc[0] = fmaf(s4.x, D[0], acc[0]);
                acc[1] = fmaf(s4.y, D[1], acc[1]);
                acc[2] = fmaf(s4.z, D[2], acc[2]);
                acc[3] = fmaf(s4.w, D[3], acc[3]);
            }
        }
        // the next unit's weights go out now (past the last unit, this one's
        // again: cache hits, and the requests stay unconditional)
        const int un = u + (int)gridDim.x;
        float res_n = 0.0f;
        if constexpr (PERSIST) {
            load_unit(un < NU ? un : u);
            res_n = load_res(un < NU ? un : u);
        }
        float (*rb)[4][kWave] = red[PERSIST ? (it & 1) : 0];  // two areas: one barrier a unit
#pragma unroll
        for (int r = 0; r < 4; ++r) rb[wid][r][lane] = fmaf(acc[r], cf, cb[r]);
        __syncthreads();

        // ---- wave r < 4 sums, adds the terms and stores register r
        if (wid < 4) {
            const int r = wid;
            float x = 0.0f;
#pragma unroll
            for (int q = 0; q < W; ++q) x += rb[q][r][lane];
            x = add_terms(x);
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
                const int orow = u * kOutRows + 4 * h + r;
                if (writer && (!HALF || h < 2) && orow < v.N) {
                    const int64_t o = (int64_t)mi_l * v.N + orow;
                    v.y[o] = p.residual ? x + res : x;
                }
            }
        }
        if (!PERSIST || un >= NU) break;
        u = un;
        res = res_n;
    }
}

// Dequantize through the GEMV code path (load_frag + the code subnormals):
// one thread per (row, group).  The value is fmaf(s, c, b) (4-bit) or s c
// (8-bit), rounded once, computed as fmaf(s 2^24, c 2^-24, b) and
// fmaf(s 2^24, (c + 128) 2^-24, -128 s).
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
        dequant_q4_group(f, dst);
    } else {
        const unsigned c[8] = {f.c0.x, f.c0.y, f.c0.z, f.c0.w, f.c1.x, f.c1.y, f.c1.z, f.c1.w};
        const float s24 = f.s * kTwo24, off = -128.0f * f.s;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const Q8Halves q = q8_halves(c[j]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int slot = q8_slot(k);
                const h2_t hh = as_h2(q.r[slot >> 1]);
                dst[4 * j + k] = fmaf(s24, (float)((slot & 1) ? hh.y : hh.x), off);
            }
        }
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

// The vector kernel for one or two rows (SLOT: a MoE slot launch), or four
// on the vec4 path.
template <int FMT, int PRO, int EPI, bool SLOT = false>
static hipError_t launch_m(int m, const GemvParams& p, const GemvShape& sh, int slots, hipStream_t st) {
    dim3 grid(sh.grid, slots), block(sh.block);
    constexpr bool kFour = FMT == FMT_Q4 && PRO == PRO_PLAIN && EPI == EPI_STORE && !SLOT;
    if (m < 1 || m > (kFour ? 4 : 2)) return hipErrorInvalidValue;
    if (SLOT != (p.slot_expert != nullptr)) return hipErrorInvalidValue;
    if (p.zero_words && !(PRO == PRO_CONCAT && EPI == EPI_STORE)) return hipErrorInvalidValue;  // eh_proj only
    // matrices concatenated along n: the RMS-prologue store only (q/k/v)
    if (p.nmat != (EPI == EPI_SWIGLU ? 2 : 1) && !(PRO == PRO_RMS && EPI == EPI_STORE && p.nmat <= 3))
        return hipErrorInvalidValue;
    if (m == 1 && (p.K + kChunk - 1) / kChunk > kRow1Chunks) return hipErrorInvalidValue;
    if (m == 1)
        hipLaunchKernelGGL((k_gemv<FMT, 1, PRO, EPI, SLOT>), grid, block, 0, st, p);
    else if (m == 2)
        hipLaunchKernelGGL((k_gemv<FMT, 2, PRO, EPI, SLOT>), grid, block, 0, st, p);
    else if constexpr (kFour)
        hipLaunchKernelGGL((k_gemv<FMT, 4, PRO, EPI, SLOT>), grid, block, 0, st, p);
    return hipGetLastError();
}

// The lm_head (argmax epilogue) at three or four rows: persistent matrix-core
// blocks.
static bool mma_head_path(int fmt, int epi, int m, const GemvParams& p) {
    (void)fmt;
    return epi == EPI_ARGMAX && m >= 3 && m <= 4 && p.K == kChunk && p.nmat == 1 && !p.slot_expert;
}

// 4-bit store and SwiGLU GEMVs at three or four rows over one or two chunks
// that are not persistent take the split-K matrix-core kernel, a block per
// unit (three chunks of B operands would not fit the LDS).
static bool mma_sk_path(int fmt, int epi, int m, const GemvParams& p) {
    return fmt == FMT_Q4 && (epi == EPI_STORE || epi == EPI_SWIGLU) && m >= 3 && m <= 4 && !p.balance &&
           !p.slot_expert && p.nmat <= 3 && (p.K == kChunk || p.K == 2 * kChunk);
}

// 4-bit plain stores of three or four rows that neither matrix-core kernel
// takes (the dense down projection, K over two chunks): one pass of the
// vector kernel over four rows instead of two passes of two, so the weights
// are streamed once.
static bool vec4_path(int fmt, int pro, int epi, int m, const GemvParams& p) {
    return fmt == FMT_Q4 && pro == PRO_PLAIN && epi == EPI_STORE && m >= 3 && m <= 4 && p.nmat == 1 &&
           !p.slot_expert && !mma_sk_path(fmt, epi, m, p);
}

// 16 waves per block while the units fit one block per compute unit (every
// SIMD then holds four of a block's waves), else 8.
template <int PRO, int EPI, int W, bool HALF = false>
static void launch_mma_sk_w(const GemvParams& p, dim3 grid, hipStream_t st) {
    const dim3 block(W * kWave);
    constexpr bool kPersist = W == 8;  // the 8-wave launch runs over more units than blocks
    if (p.K == kChunk)
        hipLaunchKernelGGL((k_gemv_mma_sk<PRO, EPI, 1, W, kPersist, HALF>), grid, block, 0, st, p);
    else
        hipLaunchKernelGGL((k_gemv_mma_sk<PRO, EPI, 2, W, kPersist, HALF>), grid, block, 0, st, p);
}

// Blocks a compute unit of the split-K kernel when there are more units than
// compute units: one 8-wave block, which builds the activation operands once
// and then loops over its units (two blocks a unit, each over half as many
// units, measured slower).
constexpr int kSkBlocksPerCu = 1;

template <int PRO, int EPI>
static hipError_t launch_mma_sk(const GemvParams& p, hipStream_t st) {
    const int rows = EPI == EPI_SWIGLU ? kMmaRows / 2 : kMmaRows;
    const int units = (p.N + rows - 1) / rows;
    const int cu = device_cu_count();
    if (EPI == EPI_STORE && 2 * units <= cu)  // 8-row units: twice the blocks, still one a compute unit
        launch_mma_sk_w<PRO, EPI, 16, true>(p, dim3((p.N + kMmaRows / 2 - 1) / (kMmaRows / 2)), st);
    else if (units <= cu)
        launch_mma_sk_w<PRO, EPI, 16>(p, dim3(units), st);
    else  // persistent: kSkBlocksPerCu blocks a compute unit, each over several units
        launch_mma_sk_w<PRO, EPI, 8>(p, dim3(units < kSkBlocksPerCu * cu ? units : kSkBlocksPerCu * cu), st);
    return hipGetLastError();
}

// One 8-wave block per compute unit (fewer for a small matrix).
template <int FMT, int PRO>
static hipError_t launch_mma_head(const GemvParams& p, hipStream_t st) {
    constexpr int W = kMaxWaves;
    const int units = (p.N + kMmaRows - 1) / kMmaRows;
    const int need = (units + W - 1) / W, cu = device_cu_count();
    hipLaunchKernelGGL((k_gemv_mma<FMT, PRO, W>), dim3(need < cu ? need : cu), dim3(64 * W), 0, st, p);
    return hipGetLastError();
}

// The parameters of a pass over activation rows r0 .. r0 + pm - 1 (rows are
// independent in every prologue and epilogue, so a pass is the same GEMV on
// offset row pointers; the argmax state is left at zero by every pass).
static GemvParams row_pass(const GemvParams& p, int pro, int r0, int pm) {
    GemvParams q = p;
    q.m = pm;
    if (r0 == 0) return q;
    const int64_t xk = pro == PRO_CONCAT ? p.H : p.K;
    if (q.x0) q.x0 += r0 * xk;
    if (q.x1) q.x1 += (int64_t)r0 * p.H;
    if (q.tokens) q.tokens += r0;
    if (q.normed_out) q.normed_out += (int64_t)r0 * p.K;
    if (q.y) q.y += (int64_t)r0 * p.N;
    if (q.residual) q.residual += (int64_t)r0 * p.N;
    if (q.rowscale) q.rowscale += r0;
    if (q.logits) q.logits += (int64_t)r0 * p.N;
    if (q.ids) q.ids += r0;
    q.zero_words = nullptr;  // cleared by the first pass
    q.zero_n = 0;
    return q;
}

static hipError_t launch_pass(int fmt, int pro, int epi, int m, const GemvParams& p, int max_blocks,
                              hipStream_t st) {
    if (p.zero_words && !(pro == PRO_CONCAT && epi == EPI_STORE)) return hipErrorInvalidValue;  // eh_proj only
    if (mma_sk_path(fmt, epi, m, p)) {
        if (pro == PRO_PLAIN && epi == EPI_STORE) return launch_mma_sk<PRO_PLAIN, EPI_STORE>(p, st);
        if (pro == PRO_RMS && epi == EPI_STORE) return launch_mma_sk<PRO_RMS, EPI_STORE>(p, st);
        if (pro == PRO_CONCAT && epi == EPI_STORE) return launch_mma_sk<PRO_CONCAT, EPI_STORE>(p, st);
        if (pro == PRO_PLAIN && epi == EPI_SWIGLU) return launch_mma_sk<PRO_PLAIN, EPI_SWIGLU>(p, st);
        if (pro == PRO_RMS && epi == EPI_SWIGLU) return launch_mma_sk<PRO_RMS, EPI_SWIGLU>(p, st);
    }
    if (mma_head_path(fmt, epi, m, p) && pro == PRO_RMS && !p.zero_words)
        return fmt == FMT_Q4 ? launch_mma_head<FMT_Q4, PRO_RMS>(p, st) : launch_mma_head<FMT_Q8, PRO_RMS>(p, st);
    if (m > 2 && !vec4_path(fmt, pro, epi, m, p)) return hipErrorInvalidValue;
    const int waves = block_waves(fmt, epi, m);
    int maxb = max_blocks;
    if (epi == EPI_ARGMAX) {
        // persistent: one block of 8 waves per compute unit (two of 4 otherwise)
        maxb = device_cu_count() * (kMaxWaves / waves);
        if (maxb > kHeadMaxBlocks) maxb = kHeadMaxBlocks;
    }
    const GemvShape sh = gemv_shape(fmt, epi, m, p.N, p.K, maxb, waves);
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

// Rows in passes: up to four on the matrix-core kernels and the vec4 path,
// else up to two on the vector kernel.
hipError_t launch_gemv(int fmt, int pro, int epi, int m, const GemvParams& p, int max_blocks, hipStream_t st) {
    if (p.slot_expert) return hipErrorInvalidValue;  // slot launches use launch_gemv_slots
    for (int r0 = 0; r0 < m;) {
        const int left = m - r0;
        const int four = left < 4 ? left : 4;
        GemvParams q = row_pass(p, pro, r0, four);
        int pm = four;
        if (!(four >= 3 && (mma_sk_path(fmt, epi, four, q) || mma_head_path(fmt, epi, four, q) ||
                            vec4_path(fmt, pro, epi, four, q)))) {
            pm = left < 2 ? left : 2;
            q = row_pass(p, pro, r0, pm);
        }
        const hipError_t e = launch_pass(fmt, pro, epi, pm, q, max_blocks, st);
        if (e != hipSuccess) return e;
        r0 += pm;
    }
    return hipSuccess;
}

// MoE slots on the vector kernel (m <= 2; the MoE launcher runs larger row
// sets in passes).
hipError_t launch_gemv_slots(int fmt, int epi, int m, const GemvParams& p, int max_blocks, int max_slots,
                             hipStream_t st) {
    if (fmt != FMT_Q8 || !p.slot_expert || m < 1 || m > 2) return hipErrorInvalidValue;
    const int N = p.N > p.N_sh ? p.N : p.N_sh, K = p.K > p.K_sh ? p.K : p.K_sh;
    const GemvShape sh = gemv_shape(fmt, epi, m, N, K, max_blocks, block_waves(fmt, epi, m));
    if (epi == EPI_SWIGLU) return launch_m<FMT_Q8, PRO_PLAIN, EPI_SWIGLU, true>(m, p, sh, max_slots, st);
    if (epi == EPI_STORE) return launch_m<FMT_Q8, PRO_PLAIN, EPI_STORE, true>(m, p, sh, max_slots, st);
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
