// peak.hip -- measured ceilings on this device (matrix-core rates and a
// read-only HBM stream), for the benchmark's roofline (a measurement aid; no
// part of the matmul path).
//
// Each wave keeps 8 independent accumulator chains and issues `iters` rounds
// of one MFMA per chain, back to back, on operands held in registers: the
// matrix pipe of every SIMD is kept busy and nothing else runs.  One value per
// thread is written at the end so the work cannot be dropped.  Work per
// launch: blocks * 4 waves * iters * 8 MFMAs of 2*32*32*16 (f16) or
// 2*32*32*32 (int8) operations.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void k_peak_f16(float* __restrict__ out, int iters) {
    const int t = threadIdx.x;
    half8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)((t + i) & 7);
        b[i] = (_Float16)((t * 3 + i) & 7);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[(int64_t)blockIdx.x * blockDim.x + t] = s;
}

__global__ __launch_bounds__(256) void k_peak_i8(int* __restrict__ out, int iters) {
    const int t = threadIdx.x;
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = 0x01010101 * ((t + i) & 7);
        b[i] = 0x01010101 * ((t * 3 + i) & 7);
    }
    i32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[(int64_t)blockIdx.x * blockDim.x + t] = s;
}

// Read-only stream: each thread walks the buffer grid-stride in 16 B
// non-temporal loads (4 in flight) and writes one folded value at the end.
__global__ __launch_bounds__(256) void k_peak_read(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ out) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u4v v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(src + i + u * stride));
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(src + i));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[tid] = acc;
}

}  // namespace

extern "C" {

// MFMA chains per wave and waves per workgroup (the operation count per
// launch follows from these and the arguments).
int mmq_peak_chains(void) { return kChains; }

// out: device buffer of blocks * 256 floats (f16) or int32 (int8); blocks >= 1,
// 1 <= iters <= 1 << 20.  Returns 0, -1 for bad arguments, or the HIP error.
int mmq_peak_mfma_f16(float* out, int blocks, int iters, hipStream_t s) {
    if (out == nullptr || blocks < 1 || iters < 1 || iters > (1 << 20)) return -1;
    hipLaunchKernelGGL(k_peak_f16, dim3((unsigned)blocks), dim3(256), 0, s, out, iters);
    return (int)hipGetLastError();
}

int mmq_peak_mfma_i8(int* out, int blocks, int iters, hipStream_t s) {
    if (out == nullptr || blocks < 1 || iters < 1 || iters > (1 << 20)) return -1;
    hipLaunchKernelGGL(k_peak_i8, dim3((unsigned)blocks), dim3(256), 0, s, out, iters);
    return (int)hipGetLastError();
}

// src: device buffer of `bytes` bytes (bytes % 16 == 0), read once; out:
// device buffer of blocks * 256 uint32.  Returns 0, -1 for bad arguments, or
// the HIP error.
int mmq_peak_read(const void* src, int64_t bytes, unsigned* out, int blocks, hipStream_t s) {
    if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks < 1) return -1;
    hipLaunchKernelGGL(k_peak_read, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4*>(src), (int64_t)(bytes / 16), out);
    return (int)hipGetLastError();
}

}  // extern "C"
