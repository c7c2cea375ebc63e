// launch.hpp -- host-side launchers of libmtp's kernels (internal; the public
// interface is include/mtp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

// One quantized matrix (device pointers). biases is unused for 8-bit.
struct QMat {
    const void* codes;
    const float* scales;
    const float* biases;
    int n;
};

enum Fmt { FMT_Q4 = 0, FMT_Q8 = 1 };
enum Pro { PRO_PLAIN = 0, PRO_RMS = 1, PRO_CONCAT = 2 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_ARGMAX = 2 };

// Parameters of one quantized GEMV launch over m activation rows.
//  weights: EPI_STORE / EPI_ARGMAX: up to three matrices with the same k,
//           concatenated along their output rows (w[0] rows first);
//           EPI_SWIGLU: w[0] = gate, w[1] = up, equal n.
//  prologue (the activation x[m][K] the GEMV consumes):
//           PRO_PLAIN  x = x0 [m][K]
//           PRO_RMS    x = rms(x0; g0, eps) over K; normed_out [m][K] optional
//           PRO_CONCAT x = [rms(e; g0) ; rms(x1; g1)], K = 2H, e row r is
//                      table[tokens[r]] when tokens && tokens[r] >= 0 else x0
//  epilogue: EPI_STORE  y[r][n] = v (+ residual[r][n])
//            EPI_SWIGLU y[r][n] = silu(a)*b (* rowscale[r] when given)
//            EPI_ARGMAX logits[r][n] = v when logits; the per-row argmax
//                       goes to ids[m] (see head_keys)
struct GemvParams {
    QMat w[3];
    int nmat;
    int m;  // activation rows actually present (the kernel may be built for more)
    int N, K, G, S;
    const float* x0;
    const float* x1;
    const int* tokens;
    const float* table;
    int vocab;
    const float* g0;
    const float* g1;
    float eps;
    int H;
    float* normed_out;
    float* y;
    const float* residual;
    const float* rowscale;
    float* logits;
    // EPI_ARGMAX: per-row 64-bit (value, index) keys merged with atomicMax,
    // row r's at head_keys[r * kKeyStride] so that each has a 128-byte line of
    // its own (atomics on one line are performed one after another), and the
    // block arrival counter on a line of its own; all zero on entry and zero
    // again on exit (the last block to arrive turns the keys into ids[m] and
    // clears them).
    unsigned long long* head_keys;
    unsigned* counter;
    int* ids;
    // The e/h concat store (eh_proj) only: when set, block (0, 0) stores zero
    // into zero_n words at zero_words (used to clear a later launch's argmax
    // state); other launches reject it.
    unsigned* zero_words;
    int zero_n;
    // Non-zero (S == 1 only): the waves of a block share its units and claim
    // them at run time from a block-local counter instead of taking a fixed
    // share each.
    int balance;
    // Expert slots (MoE): when slot_expert is set, blockIdx.y is a slot; slots
    // >= *n_slots exit at once.  Slot j uses expert e = slot_expert[j] of the
    // stacks in w[0..1] (byte stride ex_codes, float stride ex_scales), or the
    // shared matrices shw[0..1] (N_sh rows, K_sh features) when e < 0; x0 and y
    // advance by x_slot / y_slot elements per slot and rowscale by rs_slot.
    const int* slot_expert;
    const int* n_slots;
    int64_t ex_codes, ex_scales;
    QMat shw[2];
    int N_sh, K_sh;
    int64_t x_slot, y_slot, rs_slot;
};

// Weight rows a wave handles per loop iteration (the vector kernel, one or
// two activation rows): one row of a single matrix takes 4 rows per wave
// (for the small projections that doubles the blocks in flight, which
// shortens them), the SwiGLU pair 8; two rows keep 8 partial sums per lane.
constexpr int kRowsM1 = 4;    // M = 1, one matrix
constexpr int kRowsM1P2 = 4;  // M = 1, SwiGLU pair
// M = 4, one matrix (the vec4 path): as many rows as at two activation rows,
// so that the grid keeps its wave count (at its register use, about two
// waves a SIMD fit: twice the waves would run in two rounds)
constexpr int kRowsM4 = 4;
__host__ __device__ constexpr int gemv_rows(int M, int P, int epi) {
    return (void)epi, (M == 1 ? (P == 1 ? kRowsM1 : kRowsM1P2)
                              : (M == 4 && P == 1 ? kRowsM4 : (8 / (M * P) > 0 ? 8 / (M * P) : 1)));
}
// Row count of the kernel instantiation that serves m activation rows.
__host__ __device__ constexpr int inst_m(int m) { return m <= 1 ? 1 : (m <= 2 ? 2 : (m <= 4 ? 4 : 8)); }
// Argmax state: one 128-byte line per row key, then the counter's line.
constexpr int kKeyStride = 16;        // u64 between row keys
constexpr int kHeadRows = 8;          // activation rows at most (the C ABI's MTP_MAX_ROWS)
constexpr int kHeadMaxBlocks = 1024;  // lm_head grid cap
constexpr int kHeadStateBytes = (kHeadRows + 1) * kKeyStride * 8;
constexpr int kMaxWaves = 8;
// Waves per block of the vector kernel.  The 4-bit lm_head uses 8 (its
// persistent blocks take a whole compute unit each); everything else 4.
__host__ __device__ constexpr int block_waves(int fmt, int epi, int m) {
    return (fmt == FMT_Q4 && epi == EPI_ARGMAX && m <= 4) ? kMaxWaves : 4;
}

struct GemvShape {
    int grid, block, Q, R;
};

// Grid/block choice for a GEMV of N rows, K features (S chunks) at m rows.
GemvShape gemv_shape(int fmt, int epi, int m, int N, int K, int max_blocks, int waves = 4);
// Any m <= 8: the rows run in passes (up to four rows on the matrix-core
// kernels, up to two on the vector kernel).  max_blocks caps the grid of the
// non-persistent vector launches; the argmax epilogue is persistent.
hipError_t launch_gemv(int fmt, int pro, int epi, int m, const GemvParams& p, int max_blocks,
                       hipStream_t stream);
// MoE slot launch (m <= 2): grid.y = max_slots (blocks of unused slots exit at once).
hipError_t launch_gemv_slots(int fmt, int epi, int m, const GemvParams& p, int max_blocks, int max_slots,
                             hipStream_t stream);
hipError_t launch_dequant(int fmt, const QMat& w, int k, float* out, hipStream_t stream);
int device_cu_count();

// Attention (head_dim 128): RoPE + append + chunked partial softmax, then the
// log-sum-exp combine.
struct AttnParams {
    const float* qkv;  // [m][(qg * nh + 2 nkv) * d] pre-RoPE q (with gate rows when qg = 2), k and v
    float* k_cache;
    float* v_cache;
    int cache_len, capacity, m, nh, nkv, d;
    int vd;               // V head dims (d, or the wide geometry's narrower V heads)
    double log2_theta;  // inverse frequency i is 2^(-(2i/d) * log2_theta) = theta^(-2i/d)
    float* part;  // [chunks][nkv][group*m][d + 2]: p*V sums, chunk max, exp-sum
    float* o;     // [m][nh * d]
    int chunks;
    int qg;               // 1: q heads are d apart in qkv; 2: each q head is followed by its d gate values
    const float* gq;      // per-head RMSNorm weights [d] of q and k (NULL: none)
    const float* gk;
    float eps;
    int rot;              // rotary dims (a power of two <= d)
    int window;           // 0, or W: row at position p sees positions p-W+1 .. p
    const float* sinks;   // per query head softmax sink logits [nh] (NULL: none)
    int c0;               // first chunk any row sees; partials are stored from it
    const int* positions;  // [m][4] rotary position ids of the rows (NULL: row r at cache_len + r)
    int sec[4];            // their section sizes (rotary pair j takes id imrope_sec(j, sec))
};
// Position id of rotary pair j: ids 0, 1, 2 interleave pair by pair while
// each has pairs left (id k keeps the pairs j = k mod 3 with j < 3 sec[k]);
// the other pairs take id 3.
__host__ __device__ inline int imrope_sec(int j, const int (&sec)[4]) {
    const int k = j % 3;
    return j < 3 * sec[k] ? k : 3;
}
constexpr int kAttnChunk = 32;
hipError_t launch_attention(const AttnParams& p, hipStream_t stream);
// Cache catch-up: out [m][H] = (pending or 0, target rows 0 .. m-2); and the
// K/V side of the attention for m rows of kv [m][2 nkv d] at positions
// pos0 .. pos0+m-1 (fields used: k_cache, v_cache, capacity, nkv, log2_theta,
// gk, eps, rot).
hipError_t launch_shift_rows(const float* pending, const float* target, float* out, int m, int H,
                             hipStream_t stream);
hipError_t launch_append_kv(const AttnParams& p, const float* kv, int m, int pos0, hipStream_t stream);

// MoE (8-bit experts, or 4-bit experts with bf16 group constants when q4:
// then the QMat scales/biases fields of ge ... sd carry the bf16 arrays'
// addresses and are read as 16-bit values).
struct MoeParams {
    const float* x;      // [m][H] input rows
    const float* gamma;  // optional input norm
    float eps;
    float* f;            // [m][H] normalized rows (workspace)
    const float* router;  // [E][H]
    float* logits;        // [m][E]
    int E, H, top_k, m;
    int* expert_ids;      // [m][top_k] (workspace or caller)
    float* gates;         // [m][top_k]
    int* slot_expert;     // [max_slots]  (-1 = shared expert)
    float* slot_gate;     // [max_slots][m]
    int* n_slots;         // [1]
    int max_slots;
    QMat ge, ue, de;      // expert stacks (codes of expert 0; stride per expert below)
    QMat sg, su, sd;      // shared expert (codes NULL when absent)
    int inter, sh_inter;
    float* z;             // [max_slots][m][max(inter, sh_inter)]
    float* ypart;         // [max_slots][m][H]
    const float* residual;
    float* y;
    int q4;
};
hipError_t launch_moe(const MoeParams& p, hipStream_t stream);
hipError_t launch_dequant_q4e(const void* codes, const unsigned short* scales, const unsigned short* biases, int n,
                              int k, float* out, hipStream_t stream);

}  // namespace mtp
