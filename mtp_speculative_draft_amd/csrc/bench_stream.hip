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

}  // namespace

// bytes: a multiple of 16 (p 16-byte aligned); out: blocks floats.  Returns a
// hipError_t value (0 = success).
extern "C" int mtp_bench_read_stream(const void* p, size_t bytes, float* out, int blocks, void* stream) {
    if (!p || !out || blocks < 1 || (bytes & 15u) || (reinterpret_cast<size_t>(p) & 15u)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_read_stream, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const f4_t*>(p), bytes / 16, out);
    return (int)hipGetLastError();
}
