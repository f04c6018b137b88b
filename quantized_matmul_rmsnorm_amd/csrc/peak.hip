// peak.hip -- measured ceilings on this device (matrix-core rates, the
// matmul's MFMA + rescale instruction mix without memory, and a read-only HBM
// stream), for the benchmark's roofline (a measurement aid; no part of the
// matmul path).
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

// The matmul's per-block instruction mix without memory traffic, in its
// launch shape (512 threads: 2 waves per SIMD).  Per block each wave issues 4
// MFMAs (two output tiles, two K-steps of 16) into one X buffer and 32 FMAs
// (acc += s * X, the per-block rescale) reading the X buffer of the previous
// block; the buffers alternate.  The first K-step accumulates onto the
// buffer's old contents (the matmul starts each block from zero; a zero start
// with fixed operands would be hoisted out of the loop).  That ties each
// block's MFMAs to the FMAs that last read their buffer, so this mix overlaps
// the two pipes less than the matmul's own flow can; k_mix_probe below
// measures the zero start with varying operands.  MODE 0: MFMAs only;
// 1: FMAs only; 2: both, in the matmul's order (the MFMAs of a block, then
// the FMAs of the one before).  MODE 3 is the same per-block work on int8
// MFMA: one v_mfma_i32_32x32x32_i8 per output tile and block (the whole
// 32-block in one instruction) and, per output, the three VALU operations an
// int32 block dot needs (convert, times the row's weight scale, FMA with the
// token scale).
template <int MODE>
__global__ __launch_bounds__(512) void k_peak_mix(float* __restrict__ out, int iters, float s_arg) {
    const int t = threadIdx.x;
    // a per-lane factor, as the matmul's token scale is: the rescale then
    // reads only VGPRs (an SGPR operand halves the VALU issue rate)
    const float s = s_arg * (1.0f + 0x1p-20f * (float)(t & 63));
    half8 a0, b0, a1, b1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0[i] = (_Float16)((t + i) & 7);
        b0[i] = (_Float16)((t * 3 + i) & 7);
        a1[i] = (_Float16)((t + 2 * i) & 7);
        b1[i] = (_Float16)((t * 5 + i) & 7);
    }
    f32x16 XA[2], XB[2], acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            XA[i][r] = (float)(r + i);
            XB[i][r] = (float)(r - i);
            acc[i][r] = 0.0f;
        }
    i32x4 ia0, ia1, ib0, ib1;
    i32x16 IA[2], IB[2];
    float wsc[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ia0[i] = 0x01010101 * ((t + i) & 7);
        ib0[i] = 0x01010101 * ((t * 3 + i) & 7);
        ia1[i] = 0x01010101 * ((t + 2 * i) & 7);
        ib1[i] = 0x01010101 * ((t * 5 + i) & 7);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        IA[0][r] = r; IA[1][r] = r + 1; IB[0][r] = r + 2; IB[1][r] = r + 3;
        wsc[r] = 1.0f + 0.125f * (float)r;
    }
    float dtok[2] = {s, 1.0f - s};   // the two tiles' token scales, a new value per block
    auto block_i8 = [&](i32x16* Iw, const i32x16* Ir) {
        Iw[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ia0, ib0, Iw[0], 0, 0, 0);
        Iw[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ia1, ib1, Iw[1], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            dtok[i] *= 0.999f;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(dtok[i] * wsc[r], (float)Ir[i][r], acc[i][r]);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // the block's MFMAs
        __builtin_amdgcn_sched_group_barrier(0x002, 98, 0);   // then its rescale
    };
    auto block = [&](f32x16* Xw, const f32x16* Xr) {
        if constexpr (MODE != 1) {
            Xw[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, Xw[0], 0, 0, 0);
            Xw[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, Xw[1], 0, 0, 0);
            Xw[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, a0, Xw[0], 0, 0, 0);
            Xw[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, a1, Xw[1], 0, 0, 0);
        }
        if constexpr (MODE != 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(s, Xr[i][r], acc[i][r]);
        }
        if constexpr (MODE == 2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);    // the block's MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);   // then the rescale FMAs
        }
    };
    for (int it = 0; it < iters; ++it) {
        if constexpr (MODE == 3) {
            block_i8(IA, IB);
            block_i8(IB, IA);
            continue;
        }
        block(XA, XB);
        block(XB, XA);
        if constexpr (MODE == 1) {   // the FMAs' inputs: registers the compiler cannot fold
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(XA[i][r]), "+v"(XB[i][r]));
        }
    }
    float v = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        v += XA[0][r] + XA[1][r] + XB[0][r] + XB[1][r] + acc[0][r] + acc[1][r];
        if constexpr (MODE == 3) v += (float)(IA[0][r] ^ IA[1][r] ^ IB[0][r] ^ IB[1][r]);
    }
    out[(int64_t)blockIdx.x * blockDim.x + t] = v;
}

// Overlap probes: what lets the matrix pipe and the VALU run at the same time.
// Per 32-block each wave issues, for each of its TILES output tiles, two
// v_mfma_f32_32x32x16_f16 (the block's two K-steps) and 16 FMAs (the tile's
// rescale, acc += s * X).  Variants:
//   MODE 0: MFMAs only; 1: FMAs only; 2: both from the same wave, the block's
//   MFMAs then the previous block's FMAs (the matmul's order); 3: split
//   waves -- in every SIMD one wave issues only the MFMAs and the other only
//   the FMAs (waves w and w + 4 of a 512-thread workgroup share a SIMD).
//   SRC 0: the FMAs read the previous block's MFMA results (the matmul's data
//   flow); 1: they read registers no MFMA writes, and no VALU reads an MFMA
//   result (the two pipes share nothing but the issue port and the register
//   file).
//   ZERO 1: each block's first K-step starts from zero (as the matmul does);
//   0: it accumulates onto the buffer's old contents.
// BS threads per workgroup and one workgroup per CU give BS / 256 waves per
// SIMD.  Work per launch: blocks * (BS / 64) * iters * 2 blocks * TILES * 2
// MFMAs of 2*32*32*16 operations (MODE 3: half the waves issue them).
// RND 1: the operands are random values in [-2, 2) (a hash of thread and
// index) in four sets that successive blocks rotate through, and each block's
// rescale factor differs, so the datapaths switch as they do on real data
// (iters rounded up to even); RND 0: small constant operands, the same every
// block.  The hash is Wellons' "lowbias32" integer mixer (hash-prospector).
__device__ __forceinline__ _Float16 probe_rand(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return (_Float16)((float)(x & 0xFFFFu) * (1.0f / 16384.0f) - 2.0f);
}

template <int BS, int TILES, int MODE, int SRC, int ZERO, int RND = 0>
__global__ __launch_bounds__(BS) void k_mix_probe(float* __restrict__ out, int iters, float s) {
    const int t = threadIdx.x;
    const int wave = t >> 6;
    // MODE 3: the first wave of each SIMD pair issues MFMAs, the second FMAs
    const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && ((wave >> 2) & 1) == 0);
    const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && ((wave >> 2) & 1) == 1);
    constexpr int NSET = RND ? 4 : 1;
    half8 a0[NSET], b0[NSET], a1[NSET], b1[NSET];
    float sv[NSET];
    const uint32_t seed = ((uint32_t)blockIdx.x * BS + (uint32_t)t) * 256u;
    // the rescale factor differs per lane, as the matmul's token scale does, so
    // the FMAs read three VGPRs (an SGPR operand would halve their issue rate)
    const float lane_s = s * (1.0f + 0x1p-20f * (float)(t & 63));
#pragma unroll
    for (int k = 0; k < NSET; ++k) {
        sv[k] = lane_s * (1.0f + 0.0078125f * (float)k);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (RND) {
                a0[k][i] = probe_rand(seed + 64u * k + i);
                b0[k][i] = probe_rand(seed + 64u * k + 8 + i);
                a1[k][i] = probe_rand(seed + 64u * k + 16 + i);
                b1[k][i] = probe_rand(seed + 64u * k + 24 + i);
            } else {
                a0[k][i] = (_Float16)((t + i) & 7);
                b0[k][i] = (_Float16)((t * 3 + i) & 7);
                a1[k][i] = (_Float16)((t + 2 * i) & 7);
                b1[k][i] = (_Float16)((t * 5 + i) & 7);
            }
        }
    }
    f32x16 XA[TILES], XB[TILES], acc[TILES], Y[TILES];
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            XA[i][r] = (float)(r + i);
            XB[i][r] = (float)(r - i);
            Y[i][r] = (float)(r * 3 - i);
            acc[i][r] = 0.0f;
        }
    auto block = [&](f32x16* Xw, const f32x16* Xr, int k) {
        if (do_m) {
            // operands opaque to the compiler, so a zero-started MFMA is not hoisted
            asm volatile("" : "+v"(a0[k]), "+v"(b0[k]), "+v"(a1[k]), "+v"(b1[k]));
#pragma unroll
            for (int i = 0; i < TILES; ++i) {
                const f32x16 zero = {};
                Xw[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(i ? a1[k] : a0[k], i ? b1[k] : b0[k],
                                                               ZERO ? zero : Xw[i], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < TILES; ++i)
                Xw[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(i ? b1[k] : b0[k], i ? a1[k] : a0[k], Xw[i],
                                                               0, 0, 0);
            // the unrolled RND loop overwrites a buffer two blocks later without
            // reading it: mark each block's results used so none is dropped
            if (RND) {
#pragma unroll
                for (int i = 0; i < TILES; ++i) asm volatile("" : : "v"(Xw[i]));
            }
        }
        if (do_v) {
#pragma unroll
            for (int i = 0; i < TILES; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(sv[k], SRC ? Y[i][r] : Xr[i][r], acc[i][r]);
        }
        if (MODE == 2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * TILES, 0);   // the block's MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 16 * TILES, 0);  // then the rescale FMAs
        }
    };
    // two blocks per iteration; with RND the loop is unrolled by two so that
    // four blocks walk the four operand sets with static register indices
    for (int it = 0; it < iters; it += RND ? 2 : 1) {
        block(XA, XB, 0);
        block(XB, XA, RND ? 1 : 0);
        if (RND) {
            block(XA, XB, RND ? 2 : 0);
            block(XB, XA, RND ? 3 : 0);
        }
        if (do_v && (SRC || !do_m)) {   // the FMAs' inputs: registers the compiler cannot fold
#pragma unroll
            for (int i = 0; i < TILES; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {   // element by element: no tuple copies
                    if (SRC) asm volatile("" : "+v"(Y[i][r]));
                    else asm volatile("" : "+v"(XA[i][r]), "+v"(XB[i][r]));
                }
        }
    }
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) v += XA[i][r] + XB[i][r] + acc[i][r] + Y[i][r];
    out[(int64_t)blockIdx.x * blockDim.x + t] = v;
}

struct ProbeInfo {
    const char* name;
    int bs, tiles, mode, src, zero;
    void (*fn)(float*, int, float);
};

#define PROBE(BS, T, M, S, Z, NAME) {NAME, BS, T, M, S, Z, k_mix_probe<BS, T, M, S, Z>}
#define PROBE_RND(BS, T, M, S, Z, NAME) {NAME, BS, T, M, S, Z, k_mix_probe<BS, T, M, S, Z, 1>}
const ProbeInfo kProbes[] = {
    PROBE(512, 2, 0, 0, 1, "w2_t2_mfma_only"),
    PROBE(512, 2, 1, 0, 1, "w2_t2_fma_only"),
    PROBE(512, 2, 2, 0, 1, "w2_t2_both_matmul_flow"),
    PROBE(512, 2, 2, 0, 0, "w2_t2_both_matmul_flow_accumulating"),
    PROBE(512, 2, 2, 1, 1, "w2_t2_both_independent"),
    PROBE(512, 2, 3, 1, 1, "w2_t2_split_waves"),
    PROBE(256, 2, 0, 0, 1, "w1_t2_mfma_only"),
    PROBE(256, 2, 1, 0, 1, "w1_t2_fma_only"),
    PROBE(256, 2, 2, 0, 1, "w1_t2_both_matmul_flow"),
    PROBE(256, 2, 2, 1, 1, "w1_t2_both_independent"),
    PROBE(1024, 1, 0, 0, 1, "w4_t1_mfma_only"),
    PROBE(1024, 1, 1, 0, 1, "w4_t1_fma_only"),
    PROBE(1024, 1, 2, 0, 1, "w4_t1_both_matmul_flow"),
    PROBE(1024, 1, 2, 1, 1, "w4_t1_both_independent"),
    PROBE(1024, 1, 3, 1, 1, "w4_t1_split_waves"),
    PROBE_RND(512, 2, 0, 0, 1, "r2_t2_mfma_only"),
    PROBE_RND(512, 2, 1, 0, 1, "r2_t2_fma_only"),
    PROBE_RND(512, 2, 2, 0, 1, "r2_t2_both_matmul_flow"),
    PROBE_RND(1024, 1, 0, 0, 1, "r4_t1_mfma_only"),
    PROBE_RND(1024, 1, 1, 0, 1, "r4_t1_fma_only"),
    PROBE_RND(1024, 1, 2, 0, 1, "r4_t1_both_matmul_flow"),
};
#undef PROBE
#undef PROBE_RND
constexpr int kNumProbes = sizeof(kProbes) / sizeof(kProbes[0]);

// Read-only stream: each thread walks the buffer grid-stride in 16 B
// non-temporal loads (4 in flight) and writes one folded value at the end.
template <int U>
__global__ __launch_bounds__(256) void k_peak_read(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ out) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u4v v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(src + i + u * stride));
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
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

// out: device buffer of blocks * 512 floats; blocks >= 1, 1 <= iters <=
// 1 << 20; mode 0 .. 3.  Returns 0, -1 for bad arguments, or the HIP error.
int mmq_peak_mix(float* out, int blocks, int iters, int mode, hipStream_t s) {
    if (out == nullptr || blocks < 1 || iters < 1 || iters > (1 << 20) || mode < 0 || mode > 3)
        return -1;
    const dim3 g((unsigned)blocks), b(512);
    if (mode == 0) hipLaunchKernelGGL(k_peak_mix<0>, g, b, 0, s, out, iters, 0.999f);
    else if (mode == 1) hipLaunchKernelGGL(k_peak_mix<1>, g, b, 0, s, out, iters, 0.999f);
    else if (mode == 2) hipLaunchKernelGGL(k_peak_mix<2>, g, b, 0, s, out, iters, 0.999f);
    else hipLaunchKernelGGL(k_peak_mix<3>, g, b, 0, s, out, iters, 0.999f);
    return (int)hipGetLastError();
}

int mmq_peak_probe_count(void) { return kNumProbes; }

// Description of probe i: name, threads per workgroup, tiles per wave, and the
// number of waves per workgroup that issue MFMAs (for the operation count).
// Returns 0, or -1 for an index out of range.
int mmq_peak_probe_info(int i, const char** name, int* threads, int* tiles, int* mfma_waves) {
    if (i < 0 || i >= kNumProbes || !name || !threads || !tiles || !mfma_waves) return -1;
    const ProbeInfo& p = kProbes[i];
    *name = p.name;
    *threads = p.bs;
    *tiles = p.tiles;
    *mfma_waves = p.mode == 1 ? 0 : (p.mode == 3 ? p.bs / 128 : p.bs / 64);
    return 0;
}

// out: device buffer of blocks * (threads of probe i) floats; blocks >= 1,
// 1 <= iters <= 1 << 20.  Returns 0, -1 for bad arguments, or the HIP error.
int mmq_peak_probe(int i, float* out, int blocks, int iters, hipStream_t s) {
    if (i < 0 || i >= kNumProbes || out == nullptr || blocks < 1 || iters < 1 || iters > (1 << 20))
        return -1;
    hipLaunchKernelGGL(kProbes[i].fn, dim3((unsigned)blocks), dim3((unsigned)kProbes[i].bs), 0, s,
                       out, iters, 0.999f);
    return (int)hipGetLastError();
}

// src: device buffer of `bytes` bytes (bytes % 16 == 0), read once; out:
// device buffer of blocks * 256 uint32.  Returns 0, -1 for bad arguments, or
// the HIP error.
int mmq_peak_read(const void* src, int64_t bytes, unsigned* out, int blocks, int unroll,
                  hipStream_t s) {
    if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks < 1) return -1;
    const uint4* p = static_cast<const uint4*>(src);
    const int64_t n16 = bytes / 16;
    switch (unroll) {
    case 4: hipLaunchKernelGGL(k_peak_read<4>, dim3((unsigned)blocks), dim3(256), 0, s, p, n16, out); break;
    case 8: hipLaunchKernelGGL(k_peak_read<8>, dim3((unsigned)blocks), dim3(256), 0, s, p, n16, out); break;
    case 16: hipLaunchKernelGGL(k_peak_read<16>, dim3((unsigned)blocks), dim3(256), 0, s, p, n16, out); break;
    default: return -1;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
