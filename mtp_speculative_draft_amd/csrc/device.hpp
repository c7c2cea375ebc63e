// device.hpp -- shared device building blocks of libmtp's gfx950 kernels.
//
// Quantized GEMV scheme (all m <= 8 row kernels):
//   * one wave64 covers 64 consecutive groups of 32 input features (2048
//     features, a "chunk"); lane l owns group l of the chunk.  A weight row's
//     codes for a chunk are one contiguous 1 KB (4-bit) or 2 KB (8-bit) span,
//     so every load instruction of a wave reads whole 128-byte lines.
//   * the activation group held by a lane is quantized once per kernel to a
//     16-bit fixed-point value split into two int8 halves (hi, lo) with one
//     scale per (chunk, row): x ~= xs * (256*hi + lo).  The integer dot
//     products with the weight codes then run on v_dot4_i32_i8, exact in
//     int32; 4-bit codes only need a mask and a shift to become bytes.
//   * per (weight row, group) a lane returns s*A + b*sum(x^), A the exact
//     integer dot and x^ the quantized activations (see quantize_group); a
//     transposed butterfly reduces many rows' partials
//     across the 64 lanes at once, and the chunk result is xs * sum.
// Weight formats (hf2q 0.1.1, src/serve/forward_mlx_shared.rs,
// `MlxAffineExtra` / `MlxQWeight::from_mlx_affine_linear`): 4-bit codes u32
// [n][k/8], element k in nibble k%8 of word k/8; f32 scale and bias per group
// of 32.  8-bit: int8 codes [n][k], f32 scale per block of 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace mtp {

constexpr int kWave = 64;
constexpr int kGroup = 32;
constexpr int kChunk = kWave * kGroup;  // input features covered by one wave
constexpr float kQMax = 32512.0f;       // |q| bound so that hi = round(q/256) fits int8

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Cross-lane pairings by distance class D (gfx950).  D = 32 and 16 use the
// permlane swaps (the two 32-lane halves; the two 16-lane rows of each half),
// D = 8 and 4 the row mirrors (lane i with 15-i within 16, with 7-i within
// 8), D = 2 and 1 quad permutations (i^2, i^1).  Pairing D always flips lane
// bit D and keeps the bits of the larger classes, and the six together join
// all 64 lanes, so they serve both full reductions and the transposed
// butterfly below.  No LDS traffic.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ float dpp_partner(float x) {
    static_assert(D == 8 || D == 4 || D == 2 || D == 1, "row-local pairing");
    constexpr int ctrl = D == 8 ? 0x140 : (D == 4 ? 0x141 : (D == 2 ? 0x4E : 0xB1));
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), ctrl, 0xF, 0xF, false));
}
template <int D>
__device__ __forceinline__ int dpp_partner(int x) {
    return (int)__float_as_uint(dpp_partner<D>(__uint_as_float((unsigned)x)));
}

// Exchange across lane bit D for D = 32 (the wave's halves) or 16 (the two
// 16-lane rows of each half): afterwards r0 holds a from the lanes with bit D
// clear and b from the lanes with it set, r1 the partners' a and b in the
// same places, so a lane-wise combine of r0 and r1 gives a's pair result
// where bit D is clear and b's where it is set.
template <int D>
__device__ __forceinline__ void swap_halves(float a, float b, float& r0, float& r1) {
    static_assert(D == 32 || D == 16, "half swap");
    if constexpr (D == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    }
}

// One all-reduce step at class D with a commutative combine f.
template <int D, class F>
__device__ __forceinline__ float xor_step(float v, F f) {
    if constexpr (D >= 16) {
        float r0, r1;
        swap_halves<D>(v, v, r0, r1);
        return f(r0, r1);
    } else {
        return f(v, dpp_partner<D>(v));
    }
}

template <int FROM = 32, class F>
__device__ __forceinline__ float lanes_reduce(float v, F f) {
    if constexpr (FROM >= 32) v = xor_step<32>(v, f);
    if constexpr (FROM >= 16) v = xor_step<16>(v, f);
    v = xor_step<8>(v, f);
    v = xor_step<4>(v, f);
    v = xor_step<2>(v, f);
    return xor_step<1>(v, f);
}

__device__ __forceinline__ float wave_sum(float v) {
    return lanes_reduce(v, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ float wave_max(float v) {
    return lanes_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// Sum / max over each 32-lane half of the wave.
__device__ __forceinline__ float half_sum(float v) {
    return lanes_reduce<16>(v, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ float half_max(float v) {
    return lanes_reduce<16>(v, [](float a, float b) { return fmaxf(a, b); });
}

// Larger value wins; equal values go to the lower index; NaN never wins.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

template <int D>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
    if constexpr (D >= 16) {
        float v0, v1, i0, i1;
        swap_halves<D>(v, v, v0, v1);
        swap_halves<D>(__uint_as_float((unsigned)i), __uint_as_float((unsigned)i), i0, i1);
        v = v0;
        i = (int)__float_as_uint(i0);
        argmax_merge(v, i, v1, (int)__float_as_uint(i1));
    } else {
        argmax_merge(v, i, dpp_partner<D>(v), dpp_partner<D>(i));
    }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step<32>(v, i);
    argmax_step<16>(v, i);
    argmax_step<8>(v, i);
    argmax_step<4>(v, i);
    argmax_step<2>(v, i);
    argmax_step<1>(v, i);
}

// 64-bit argmax key: order-preserving bits of the value above the complement
// of the index, so an unsigned max picks the larger value and, among equal
// values, the lower index.  0 means "no candidate" (below every real key).
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
    const unsigned u = __float_as_uint(v);
    const unsigned hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)hi << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)i);
}

__device__ __forceinline__ int argmax_key_index(unsigned long long k) {
    return k == 0ull ? 0 : (int)(0xFFFFFFFFu - (unsigned)(k & 0xFFFFFFFFull));
}

// ---------------------------------------------------------------------------
// Activation fragment: one row of x restricted to this lane's group of 32.
// Q4 layout: word j of the group holds nibbles k = 8j..8j+7; the even
// nibbles (mask 0x0F0F0F0F) pair with hi[2j]/lo[2j] = x[8j+0,2,4,6], the odd
// nibbles (shift by 4, mask) with hi[2j+1]/lo[2j+1] = x[8j+1,3,5,7].
// Q8 layout: word j holds k = 4j..4j+3 in byte order, hi[j]/lo[j] likewise.
// ---------------------------------------------------------------------------
struct XFrag {
    int hi[8];
    int lo[8];
    float sxd;  // sum of the group's 32 quantized values (an integer), the bias factor of 4-bit rows
};

__device__ __forceinline__ int pack_bytes(int a, int b, int c, int d) {
    return (a & 0xFF) | ((b & 0xFF) << 8) | ((c & 0xFF) << 16) | ((unsigned)d << 24);
}

// Returns the 16-bit quantized value q = round(x*inv) as hi*256 + lo.
__device__ __forceinline__ int split16(float x, float inv, int& h, int& l) {
    const int q = __float2int_rn(x * inv);  // |q| <= 32512
    h = (q + 128) >> 8;                     // round(q / 256), in -127..127
    l = q - h * 256;                        // in -128..127
    return q;
}

// Quantizes the 32 values word by word (few live registers).
//
// 4-bit rows: with the group's quantized activations x^_k (x ~ xs * x^) a
// row's group term is computed as s * sum(c_k x^_k) + b * sum(x^_k), both
// sums exact integers; that is sum((s c_k + b) x^_k), the exact product of the
// row's weights with the quantized activations.  Its only error is the
// activation rounding weighted by the weights themselves, which are centred
// (the bias is about -8 s), so no error is shared by all rows.  (Summing the
// unrounded x/xs for the bias factor instead would leave the codes' mean 8
// times the rounding residual as such a shared error.)
template <int FMT>
__device__ __forceinline__ void quantize_group(const float (&xv)[32], float inv, float xs, XFrag& f) {
    (void)xs;
    int qs = 0;
    if constexpr (FMT == FMT_Q4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int h[8], l[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) qs += split16(xv[8 * j + i], inv, h[i], l[i]);
            f.hi[2 * j] = pack_bytes(h[0], h[2], h[4], h[6]);
            f.hi[2 * j + 1] = pack_bytes(h[1], h[3], h[5], h[7]);
            f.lo[2 * j] = pack_bytes(l[0], l[2], l[4], l[6]);
            f.lo[2 * j + 1] = pack_bytes(l[1], l[3], l[5], l[7]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int h[4], l[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split16(xv[4 * j + i], inv, h[i], l[i]);
            f.hi[j] = pack_bytes(h[0], h[1], h[2], h[3]);
            f.lo[j] = pack_bytes(l[0], l[1], l[2], l[3]);
        }
    }
    f.sxd = (float)qs;  // exact: |qs| <= 32 * 32512 < 2^24
}

// ---------------------------------------------------------------------------
// Weight fragments: one row's codes and group constants for one lane's group.
// ---------------------------------------------------------------------------
template <int FMT>
struct WFrag;

template <>
struct WFrag<FMT_Q4> {
    u32x4 c;
    float s, b;
};

template <>
struct WFrag<FMT_Q8> {
    u32x4 c0, c1;
    float s;
};

// 4-bit: codes row = G uint4 (4 words per group); scales/biases [n][G].
__device__ __forceinline__ void load_frag(WFrag<FMT_Q4>& w, const void* codes, const float* scales,
                                          const float* biases, int64_t row, int G, int g) {
    const int64_t gi = row * G + g;
    w.c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes) + gi);
    w.s = __builtin_nontemporal_load(scales + gi);
    w.b = __builtin_nontemporal_load(biases + gi);
}

// 8-bit: codes row = 2G uint4 (32 bytes per group); scales [n][G].
__device__ __forceinline__ void load_frag(WFrag<FMT_Q8>& w, const void* codes, const float* scales,
                                          const float*, int64_t row, int G, int g) {
    const int64_t gi = row * G + g;
    const u32x4* p = reinterpret_cast<const u32x4*>(codes) + 2 * gi;
    w.c0 = __builtin_nontemporal_load(p);
    w.c1 = __builtin_nontemporal_load(p + 1);
    w.s = __builtin_nontemporal_load(scales + gi);
}

// Nibbles of a 4-bit fragment as bytes: e[j] = even nibbles, o[j] = odd.
struct Nib {
    int e[4], o[4];
};

__device__ __forceinline__ Nib unpack_nibbles(const u32x4& c) {
    Nib n;
    const unsigned w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        n.e[j] = (int)(w[j] & 0x0F0F0F0Fu);
        n.o[j] = (int)((w[j] >> 4) & 0x0F0F0F0Fu);
    }
    return n;
}

__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// s*A + b*sxd for a 4-bit row against one activation fragment.
__device__ __forceinline__ float dot_q4(const Nib& n, float s, float b, const XFrag& x) {
    int ah = 0, al = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ah = sdot4(n.e[j], x.hi[2 * j], ah);
        ah = sdot4(n.o[j], x.hi[2 * j + 1], ah);
        al = sdot4(n.e[j], x.lo[2 * j], al);
        al = sdot4(n.o[j], x.lo[2 * j + 1], al);
    }
    const int a = ah * 256 + al;  // exact: |a| < 2^24
    return fmaf(s, (float)a, b * x.sxd);
}

// s*A for an 8-bit row against one activation fragment.
__device__ __forceinline__ float dot_q8(const WFrag<FMT_Q8>& w, const XFrag& x) {
    const int c[8] = {(int)w.c0.x, (int)w.c0.y, (int)w.c0.z, (int)w.c0.w,
                      (int)w.c1.x, (int)w.c1.y, (int)w.c1.z, (int)w.c1.w};
    int ah = 0, al = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ah = sdot4(c[j], x.hi[j], ah);
        al = sdot4(c[j], x.lo[j], al);
    }
    const int a = ah * 256 + al;  // |a| < 2^28
    return w.s * (float)a;
}

// ---------------------------------------------------------------------------
// Transposed butterfly: v[0..V) per lane -> after the call each lane holds in
// v[0..FINAL) the 64-lane sums of positions base..base+FINAL-1, where base is
// returned by reduce_base().  Positions are halved at the pairing classes 32,
// 16, ... (the lane keeping the upper half when its bit is set); once FINAL
// values remain the remaining classes are plain sums.
// ---------------------------------------------------------------------------
template <int V, int FINAL, int STEP>
struct Butterfly {
    __device__ __forceinline__ static void run(float* v, int lane) {
        if constexpr (STEP < 6) {
            constexpr int d = 32 >> STEP;
            if constexpr (V > FINAL) {
                constexpr int half = V / 2;
                if constexpr (d >= 16) {
                    // the swap hands each lane its own and its partner's copy
                    // of the half it keeps
#pragma unroll
                    for (int i = 0; i < half; ++i) {
                        float r0, r1;
                        swap_halves<d>(v[i], v[i + half], r0, r1);
                        v[i] = r0 + r1;
                    }
                } else {
                    const bool up = (lane & d) != 0;
#pragma unroll
                    for (int i = 0; i < half; ++i) {
                        const float send = up ? v[i] : v[i + half];
                        const float keep = up ? v[i + half] : v[i];
                        v[i] = keep + dpp_partner<d>(send);
                    }
                }
                Butterfly<half, FINAL, STEP + 1>::run(v, lane);
            } else {
#pragma unroll
                for (int i = 0; i < FINAL; ++i) v[i] = xor_step<d>(v[i], [](float a, float b) { return a + b; });
                Butterfly<V, FINAL, STEP + 1>::run(v, lane);
            }
        }
    }
};

template <int V, int FINAL>
__device__ __forceinline__ void reduce_transpose(float (&v)[V], int lane) {
    static_assert(V / FINAL <= 64 && (V & (V - 1)) == 0, "butterfly shape");
    Butterfly<V, FINAL, 0>::run(v, lane);
}

template <int V, int FINAL>
__device__ __forceinline__ int reduce_base(int lane) {
    int base = 0, cur = V;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        const int d = 32 >> step;
        if (cur > FINAL) {
            cur >>= 1;
            if (lane & d) base += cur;
        }
    }
    return base;
}

// Lanes that hold the first copy of each reduced position.
template <int V, int FINAL>
__device__ __forceinline__ bool reduce_writer(int lane) {
    constexpr int outs = V / FINAL;  // distinct positions across the wave
    constexpr int dup = 64 / outs;   // lanes holding each position
    return (lane & (dup - 1)) == 0;
}

template <int M>
__device__ __forceinline__ float select_m(const float (&a)[M], int i) {
    float r = a[0];
#pragma unroll
    for (int k = 1; k < M; ++k) r = (i == k) ? a[k] : r;
    return r;
}

__device__ __forceinline__ void load32(float (&xv)[32], const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float4 t = q[j];
        xv[4 * j] = t.x;
        xv[4 * j + 1] = t.y;
        xv[4 * j + 2] = t.z;
        xv[4 * j + 3] = t.w;
    }
}

__device__ __forceinline__ void store32(float* p, const float (&xv)[32]) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = make_float4(xv[4 * j], xv[4 * j + 1], xv[4 * j + 2], xv[4 * j + 3]);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace mtp
