// bench_stream.hip -- measurement support, not part of the draft layer: a
// plain HBM read stream that bench.py times to quote the box's practical read
// ceiling next to the 8 TB/s peak.  Built into libmtp_bench.so (loaded only by
// bench.py); libmtp.so does not contain it.
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
typedef float f4_t __attribute__((ext_vector_type(4)));

// Every 16-byte word of p[0 .. n4) is read once (nontemporal, as the weight
// streams are); each block writes one sum so the loads cannot be dropped.
__global__ void __launch_bounds__(kThreads) k_read_stream(const f4_t* __restrict__ p, size_t n4, float* out) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    float acc = 0.0f;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
        f4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n4; i += stride) {
        const f4_t v = __builtin_nontemporal_load(p + i);
        acc += (v.x + v.y) + (v.z + v.w);
    }
    __shared__ float red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

// The same read with contiguous shares: wave w of the grid reads whole tiles
// of 64 * U words (U KB) from its own contiguous range, U loads in flight per
// lane; wave 0 also reads the words past the last whole tile.
constexpr int kChunkThreads = 512;
template <int U>
__global__ void __launch_bounds__(kChunkThreads) k_read_chunks(const f4_t* __restrict__ p, size_t n4, float* out) {
    constexpr int kWaves = kChunkThreads / 64;
    const int lane = threadIdx.x & 63;
    const size_t waves = (size_t)gridDim.x * kWaves;
    const size_t w = (size_t)blockIdx.x * kWaves + threadIdx.x / 64;
    const size_t tiles = n4 / (64 * U);
    const size_t t0 = w * tiles / waves, t1 = (w + 1) * tiles / waves;
    float acc = 0.0f;
    for (size_t t = t0; t < t1; ++t) {
        const f4_t* q = p + t * 64 * U + lane;
        f4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(q + u * 64);
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    if (w == 0)
        for (size_t i = tiles * 64 * U + lane; i < n4; i += 64) {
            const f4_t v = __builtin_nontemporal_load(p + i);
            acc += (v.x + v.y) + (v.z + v.w);
        }
    __shared__ float red[kChunkThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kChunkThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

// bytes: a multiple of 16 (p 16-byte aligned); out: blocks floats.  mode 0:
// the grid-stride kernel (256 threads per block); mode 1: contiguous shares
// per wave, 4 KB tiles; mode 2: 8 KB tiles (512 threads per block).  Returns
// a hipError_t value (0 = success).
extern "C" int mtp_bench_read_stream(const void* p, size_t bytes, float* out, int blocks, int mode, void* stream) {
    if (!p || !out || blocks < 1 || (bytes & 15u) || (reinterpret_cast<size_t>(p) & 15u) || mode < 0 || mode > 2)
        return (int)hipErrorInvalidValue;
    const f4_t* q = static_cast<const f4_t*>(p);
    if (mode == 0)
        hipLaunchKernelGGL(k_read_stream, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, q, bytes / 16,
                           out);
    else if (mode == 1)
        hipLaunchKernelGGL(k_read_chunks<4>, dim3((unsigned)blocks), dim3(kChunkThreads), 0, (hipStream_t)stream, q,
                           bytes / 16, out);
    else
        hipLaunchKernelGGL(k_read_chunks<8>, dim3((unsigned)blocks), dim3(kChunkThreads), 0, (hipStream_t)stream, q,
                           bytes / 16, out);
    return (int)hipGetLastError();
}
