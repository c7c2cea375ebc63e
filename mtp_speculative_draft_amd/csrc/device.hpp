// device.hpp -- shared device building blocks of libmtp's gfx950 kernels.
//
// Quantized GEMV arithmetic (every kernel, vector and matrix core):
//   * activations stay f32.  Weight codes become exact f16 operands without
//     any float conversion: a masked 4-bit code c (or 16c) in the low bits of
//     a 16-bit half is the f16 subnormal c * 2^-24 (16c * 2^-24), and an
//     8-bit code offset to c + 128 is the subnormal (c + 128) * 2^-24.  The
//     f32 FMA with an f16 operand (v_fma_mix_f32) and the f16 matrix cores
//     take these subnormals exactly (the kernels run with f16 subnormals
//     kept), so every product c * x is exact and only the f32 accumulation
//     rounds.
//   * per (weight row, group of 32) a 4-bit row contributes
//     (s * 2^24) * sum(c x 2^-24) + b * sum(x), which is sum((s c + b) x);
//     an 8-bit row s * (2^24 * sum((c + 128) x 2^-24) - 128 sum(x)).
//   * one wave64 covers 64 consecutive groups (2048 features, a "chunk");
//     lane l owns group l, so a weight row's codes for a chunk are one
//     contiguous 1 KB (4-bit) or 2 KB (8-bit) span and every load
//     instruction of a wave reads whole 128-byte lines.  A transposed
//     butterfly reduces many rows' partials across the 64 lanes at once.
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
constexpr float kTwo24 = 16777216.0f;   // 2^24: undoes the code subnormal scale

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

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Code words as f16 subnormal pairs.
// 4-bit word (codes c0..c7 of features 8j..8j+7, c_i in nibble i): four
// halves pairs, in feature order 0, 4 | 1, 5 | 2, 6 | 3, 7, where the pairs
// of features 1, 5 and 3, 7 hold 16 c (the nibble stays in bits 4-7), so
// their activations carry a factor 1/16.  Five integer ops, no conversion.
// ---------------------------------------------------------------------------
struct Q4Halves {
    unsigned r[4];
};

__device__ __forceinline__ Q4Halves q4_halves(unsigned w) {
    const unsigned w8 = w >> 8;
    return Q4Halves{{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u}};
}

// 8-bit word (codes of features 4j..4j+3 in byte order): (c + 128) of
// features 0, 2 | 1, 3 as two halves pairs.
struct Q8Halves {
    unsigned r[2];
};

__device__ __forceinline__ Q8Halves q8_halves(unsigned w) {
    const unsigned u = w ^ 0x80808080u;  // c + 128 in every byte
    return Q8Halves{{__builtin_amdgcn_perm(u, u, 0x0C020C00u), __builtin_amdgcn_perm(u, u, 0x0C030C01u)}};
}

__device__ __forceinline__ h2_t as_h2(unsigned r) { return __builtin_bit_cast(h2_t, r); }

// Position of feature f (0..7) of a 4-bit word in the halves order, and the
// activation factor that goes with it.
__host__ __device__ constexpr int q4_slot(int f) { return (f & 3) * 2 + (f >> 2); }
__host__ __device__ constexpr float q4_factor(int f) { return (f & 1) ? 0.0625f : 1.0f; }
// The same for feature f (0..3) of an 8-bit word.
__host__ __device__ constexpr int q8_slot(int f) { return (f & 1) * 2 + (f >> 1); }

// ---------------------------------------------------------------------------
// Activation fragment: one row of x restricted to this lane's group of 32,
// in the halves order of the group's code words (4-bit: word j's slots
// 8j + q4_slot(f) with the factor q4_factor(f); 8-bit: 4j + q8_slot(f)),
// and the group's sum (4-bit: sum x, the bias factor; 8-bit: -128 sum x).
// ---------------------------------------------------------------------------
struct XFrag {
    float v[32];
    float sum;
};

// xv: the group's 32 features in natural order.
template <int FMT>
__device__ __forceinline__ void make_frag(const float (&xv)[32], XFrag& f) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += xv[i];
    if constexpr (FMT == FMT_Q4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) f.v[8 * j + q4_slot(q)] = xv[8 * j + q] * q4_factor(q);
        f.sum = s;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) f.v[4 * j + q8_slot(q)] = xv[4 * j + q];
        f.sum = -128.0f * s;
    }
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

// 4-bit expert stacks with bf16 group constants (hf2q 0.1.1,
// `MlxAffineMoeStack`): a bf16 value is the upper half of an f32's bits, so
// widening it is a shift.
__device__ __forceinline__ float bf16_to_f32(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

__device__ __forceinline__ void load_frag_b16(WFrag<FMT_Q4>& w, const void* codes, const unsigned short* scales,
                                              const unsigned short* biases, int64_t row, int G, int g) {
    const int64_t gi = row * G + g;
    w.c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes) + gi);
    w.s = bf16_to_f32(__builtin_nontemporal_load(scales + gi));
    w.b = bf16_to_f32(__builtin_nontemporal_load(biases + gi));
}

// The 32 f32 weights of a 4-bit group, s c + b rounded once each: the code
// halves are c 2^-24 exactly (16 c 2^-24 times 1/16 for the upper nibbles of
// a byte), so fma(s 2^24, c 2^-24, b) is fma(s, c, b).
__device__ __forceinline__ void dequant_q4_group(const WFrag<FMT_Q4>& f, float* dst) {
    const unsigned c[4] = {f.c.x, f.c.y, f.c.z, f.c.w};
    const float s24 = f.s * kTwo24;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const Q4Halves q = q4_halves(c[j]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int slot = q4_slot(k);
            const h2_t hh = as_h2(q.r[slot >> 1]);
            const float cv = (float)((slot & 1) ? hh.y : hh.x) * q4_factor(k);
            dst[8 * j + k] = fmaf(s24, cv, f.b);
        }
    }
}

// (s c + b) . x over the group for a 4-bit row: 8 exact products per word
// accumulated in f32 (two chains), then the scale and the bias term.
__device__ __forceinline__ float dot_q4(const u32x4& c, float s, float b, const XFrag& x) {
    const unsigned w[4] = {c.x, c.y, c.z, c.w};
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const Q4Halves q = q4_halves(w[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h2_t h = as_h2(q.r[i]);
            float& a = (i & 1) ? a1 : a0;
            a = fmaf((float)h.x, x.v[8 * j + 2 * i], a);
            a = fmaf((float)h.y, x.v[8 * j + 2 * i + 1], a);
        }
    }
    return fmaf(s * kTwo24, a0 + a1, b * x.sum);
}

// (s c) . x over the group for an 8-bit row.
__device__ __forceinline__ float dot_q8(const WFrag<FMT_Q8>& w, const XFrag& x) {
    const unsigned c[8] = {w.c0.x, w.c0.y, w.c0.z, w.c0.w, w.c1.x, w.c1.y, w.c1.z, w.c1.w};
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const Q8Halves q = q8_halves(c[j]);
        const h2_t h0 = as_h2(q.r[0]), h1 = as_h2(q.r[1]);
        a0 = fmaf((float)h0.x, x.v[4 * j], a0);
        a1 = fmaf((float)h0.y, x.v[4 * j + 1], a1);
        a0 = fmaf((float)h1.x, x.v[4 * j + 2], a0);
        a1 = fmaf((float)h1.y, x.v[4 * j + 3], a1);
    }
    return w.s * fmaf(a0 + a1, kTwo24, x.sum);
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
