// quant.hip -- fused producers that quantise f32 activations in registers into
// a q8 plane (gfx950, wave64).
//
// Method: "55 · r52 — skip-write mode 2" (sections 2.2 and 3.2) and the decode
// RMSNorm of "72 · D3-7 ..." (Excerpt C).  Per row of d values (d % 256 == 0):
//   RMSNorm : y = (x * s) * w,  s = 1 / sqrt(sum(x^2) / d + eps)
//   SwiGLU  : y = (g / (1 + exp(-g))) * u
//   F32     : y = x                      (standalone quantise)
// then per 32-block: amax = max|y|, D = amax / 127, q = clamp(rint(y / D),
// -127, 127), S = sum(q); a block whose scale is zero (all zeros, or deep
// subnormals with amax <= 63 * 2^-149, where amax / 127 rounds to zero) has
// q = 0 and S = 0.
//
// Geometry.  One workgroup of W = 4 waves per row (per row segment for SwiGLU
// and the standalone quantise, whose rows need no row-wide reduction; W = 8
// for an RMSNorm of at most 4 rows); the row is swept in rounds of 256
// values, round r belonging to wave r % W: in round r lane l owns the float4
// at 256*r + 4*l, so each wave access is one contiguous 1 KiB (the pages'
// rule that a full-width coalesced access must
// never be broken), and the 8 consecutive lanes 8g..8g+7 hold exactly one
// 32-block.  amax and the code sum are reduced inside those 8 lanes with DPP
// (quad_perm xor-1, xor-2, then row_half_mirror).  Max and integer sums are
// exact in any order, so the plane does not depend on the lane grouping; the
// f32 y values themselves are computed by the same expressions whether or not
// y is stored, so write_y = 0, write_y = 1 and a standalone quantise of the
// stored y give byte-identical planes.
//
// SwiGLU's gate and up rows and the standalone quantise's input are read
// exactly once, with non-temporal loads; RMSNorm's x and weight vector are
// read with ordinary loads (the weight vector serves every row).
//
// RMSNorm accumulates sum(x^2) in f64 (products of f32 values are exact in
// f64): per lane, then across the wave, then the W wave sums in a fixed
// order through LDS; the scale is rounded once from f64, which makes it
// independent of the summation order to within one f64 rounding.  While a
// wave's share of the row fits (d <= W*256*MAXR) its x, and the matching
// rounds of the weight vector (loaded with x, before the row sum), stay in
// registers between the two passes; longer rows are re-read.
//
// Rows n .. rows-1 of the plane (the padding to a multiple of 32 rows) are
// written as zeros, so a plane's content never depends on what its slot held
// before.
#include <algorithm>

#include "mmq_internal.h"

namespace mmq {
namespace {

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i <- lane 7-i in each 8
constexpr int kRowMirror = 0x140;   // row_mirror: lane i <- lane 15-i in each 16

__device__ __forceinline__ float max8(float v) {
    v = fmaxf(v, __int_as_float(dpp<kQuadXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<kQuadXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<kHalfMirror>(__float_as_int(v))));
    return v;
}

__device__ __forceinline__ int sum8(int v) {
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kHalfMirror>(v);
    return v;
}

// Sum over the 64 lanes as a pairwise tree: lane pairs at distance 1, 2, 4
// and 8 by DPP on the two 32-bit halves (quad xor-1, quad xor-2, then the
// half-row and row mirrors, which pair the same groups as xor-4 and xor-8),
// then the 16- and 32-lane swaps.  Every lane ends with the same sum.
__device__ __forceinline__ double wave_sum_f64(double v) {
    auto step = [](double x, auto shuffle) {
        const long long b = __double_as_longlong(x);
        const int lo = shuffle((int)(b & 0xFFFFFFFFLL)), hi = shuffle((int)(b >> 32));
        return x + __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
    };
    v = step(v, [](int t) { return dpp<kQuadXor1>(t); });
    v = step(v, [](int t) { return dpp<kQuadXor2>(t); });
    v = step(v, [](int t) { return dpp<kHalfMirror>(t); });
    v = step(v, [](int t) { return dpp<kRowMirror>(t); });
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// q = clamp(rint(v / dsc), -127, 127) with the IEEE quotient.  Fast path:
// a = v * rcp(dsc) is within a few ulp of v / dsc (|v / dsc| <= 127, so within
// 2^-15 absolute); when a is farther than 2^-11 from a half-integer, rint(a)
// equals rint of the correctly rounded quotient.  Otherwise (and for a
// subnormal dsc) the quotient is computed exactly.
__device__ __forceinline__ int code(float v, float dsc, float rcp) {
    const float a = v * rcp;
    float r = rintf(a);
    if (!(fabsf(a - r) <= 0.5f - 0x1p-11f) || dsc < 0x1p-126f) r = rintf(v / dsc);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Quantise the 4 values of this lane; lanes 8g..8g+7 form one 32-block.
// Writes the 4 codes as one dword and, from the group's first lane, the
// block's (D, S) pair as one 8-byte store.
__device__ __forceinline__ void quant4(float4 v, int lane, uint32_t* qdst, uint2* dsdst) {
    float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    am = max8(am);
    const float dsc = am / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (dsc > 0.0f) {   // a zero scale (amax 0, or amax / 127 underflowing) leaves zero codes
        const float rcp = __builtin_amdgcn_rcpf(dsc);
        q0 = code(v.x, dsc, rcp); q1 = code(v.y, dsc, rcp);
        q2 = code(v.z, dsc, rcp); q3 = code(v.w, dsc, rcp);
    }
    *qdst = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
            ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
    const int s = sum8((q0 + q1) + (q2 + q3));
    if ((lane & 7) == 0) *dsdst = make_uint2(__float_as_uint(dsc), (uint32_t)s);
}

// A non-temporal 16-byte load, for inputs each workgroup reads exactly once.
__device__ __forceinline__ float4 stream_load(const float4* p) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    const float den = 1.0f + expf(-g);
    return (g / den) * u;
}

// One workgroup (4 waves) per row; round r of the row belongs to wave r % 4.
// MAXR > 0: a wave's rounds (at most MAXR) stay in registers between the
// RMSNorm passes.
template <int KIND, bool WRITE_Y, int MAXR, bool QUANT = true, int WV = 4>
__global__ __launch_bounds__(64 * WV) void k_producer(const float* __restrict__ a,
                                                  const float* __restrict__ b,
                                                  float* __restrict__ y, int n, int d,
                                                  float eps, int8_t* __restrict__ q,
                                                  uint2* __restrict__ ds, int rows,
                                                  int rps) {
    constexpr int W = WV;   // waves per row segment
    // rounds of one wave whose loads are in flight together (SwiGLU: its
    // segments give a wave at most 3 rounds, and the smaller buffer keeps
    // 8 waves per SIMD resident)
    constexpr int U = KIND == kProdSwiglu ? 4 : 8;
    __shared__ double s_ss[W];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const int nb = d / kBlock;
    // this workgroup's rounds: [r0, r0 + rcount); RMSNorm always takes the whole row
    const int r0 = blockIdx.y * rps;
    const int rcount = min(rps, d / kSuper - r0);
    const int my = (rcount - wave + W - 1) / W;   // rounds of this wave: r0 + wave + W*k, k < my
    uint32_t* q4 = reinterpret_cast<uint32_t*>(q + (int64_t)row * d) + 64 * r0;
    uint2* dsr = ds + (int64_t)row * nb + 8 * r0;
    const int g = lane >> 3;

    if (QUANT && row >= n) {  // padded tail rows: deterministic zeros
        for (int k = 0; k < my; ++k) {
            const int r = wave + W * k;
            q4[64 * r + lane] = 0u;
            if ((lane & 7) == 0) dsr[8 * r + g] = make_uint2(0u, 0u);
        }
        return;  // the whole workgroup takes this branch
    }

    const float4* a4 = reinterpret_cast<const float4*>(a + (int64_t)row * d) + 64 * r0;
    // RMSNorm: b is the weight vector (and r0 == 0); SwiGLU: b is the up row
    const float4* b4 = reinterpret_cast<const float4*>(
        KIND == kProdRms ? b : (KIND == kProdSwiglu ? b + (int64_t)row * d + 256 * r0 : nullptr));
    float4* y4 = reinterpret_cast<float4*>(y + (int64_t)row * d) + 64 * r0;

    float scale = 0.0f;
    float4 xr[MAXR > 0 ? MAXR : 1];
    float4 wr[MAXR > 0 ? MAXR : 1];   // RMSNorm register form: the weight rounds
    if constexpr (KIND == kProdRms) {
        double ss = 0.0;
        auto acc4 = [&](const float4& v) {
            ss += (double)v.x * (double)v.x;
            ss += (double)v.y * (double)v.y;
            ss += (double)v.z * (double)v.z;
            ss += (double)v.w * (double)v.w;
        };
        if constexpr (MAXR > 0) {
            // x and the weight rounds are loaded together, so the weight
            // loads are in flight across the row sum and its barrier
#pragma unroll
            for (int k = 0; k < MAXR; ++k)
                if (k < my) xr[k] = a4[64 * (wave + W * k) + lane];
#pragma unroll
            for (int k = 0; k < MAXR; ++k)
                if (k < my) wr[k] = b4[64 * (wave + W * k) + lane];
#pragma unroll
            for (int k = 0; k < MAXR; ++k)
                if (k < my) acc4(xr[k]);
        } else {
            for (int k0 = 0; k0 < my; k0 += U) {
                float4 t[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (k0 + u < my) t[u] = a4[64 * (wave + W * (k0 + u)) + lane];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (k0 + u < my) acc4(t[u]);
            }
        }
        ss = wave_sum_f64(ss);
        if (lane == 0) s_ss[wave] = ss;
        __syncthreads();
        double tot;
        if constexpr (W == 4) {
            tot = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
        } else {
            tot = s_ss[0];
#pragma unroll
            for (int i = 1; i < W; ++i) tot += s_ss[i];
        }
        scale = (float)(1.0 / sqrt(tot / (double)d + (double)eps));
    }

    auto finish = [&](int r, float4 xin, float4 bin) {
        float4 v;
        if constexpr (KIND == kProdRms) {
            v.x = (xin.x * scale) * bin.x;
            v.y = (xin.y * scale) * bin.y;
            v.z = (xin.z * scale) * bin.z;
            v.w = (xin.w * scale) * bin.w;
        } else if constexpr (KIND == kProdSwiglu) {
            v.x = silu_mul(xin.x, bin.x);
            v.y = silu_mul(xin.y, bin.y);
            v.z = silu_mul(xin.z, bin.z);
            v.w = silu_mul(xin.w, bin.w);
        } else {
            v = xin;
        }
        if constexpr (WRITE_Y) y4[64 * r + lane] = v;
        if constexpr (QUANT) quant4(v, lane, q4 + 64 * r + lane, dsr + 8 * r + g);
    };

    if constexpr (MAXR > 0) {
#pragma unroll
        for (int k0 = 0; k0 < MAXR; k0 += U) {
            if (k0 < my) {
                float4 tb[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (k0 + u < my)
                        tb[u] = KIND == kProdRms ? wr[k0 + u] : b4[64 * (wave + W * (k0 + u)) + lane];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (k0 + u < my) finish(wave + W * (k0 + u), xr[k0 + u], tb[u]);
            }
        }
    } else {
        for (int k0 = 0; k0 < my; k0 += U) {
            float4 ta[U], tb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = wave + W * (k0 + u);
                if (k0 + u < my) {
                    if constexpr (KIND == kProdRms) {   // x re-read, w shared by every row
                        ta[u] = a4[64 * r + lane];
                        tb[u] = b4[64 * r + lane];
                    } else {                            // read exactly once: streamed
                        ta[u] = stream_load(a4 + 64 * r + lane);
                        if constexpr (KIND == kProdSwiglu) tb[u] = stream_load(b4 + 64 * r + lane);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k0 + u < my) finish(wave + W * (k0 + u), ta[u], KIND != kProdF32 ? tb[u] : ta[u]);
        }
    }
}

template <int KIND, bool WY, bool QUANT = true>
hipError_t dispatch_maxr(const float* a, const float* b, float* y, int64_t n, int64_t d,
                         float eps, const PlaneView& pl, hipStream_t s) {
    const int64_t rows = QUANT ? pl.rows : n;   // without a plane there is no padding
    const int rounds = (int)(d / kSuper);
    const int per_wave = (rounds + 3) / 4;
    // Rows with no row-wide reduction (SwiGLU, standalone) are split into
    // segments: when there are few rows (decode), as many segments of at least
    // 4 rounds as it takes to fill the chip; rows of 16 rounds or more, up to 8
    // segments of at least 8 rounds (the last one may be shorter), so that the
    // workgroups of a large launch are short and its last round ends evenly.
    // RMSNorm keeps one workgroup per row.
    int segs = 1;
    if (KIND != kProdRms) {
        const int64_t fill = std::min<int64_t>((2048 + rows - 1) / rows, (rounds + 3) / 4);
        const int64_t split = std::min<int64_t>(8, rounds / 8);
        segs = (int)std::max<int64_t>(1, std::max(fill, split));
    }
    const int rps = (rounds + segs - 1) / segs;
    segs = (rounds + rps - 1) / rps;
    const dim3 grid((unsigned)rows, (unsigned)segs), block(256);
    // A few rows (decode): 8 waves per row, each with at most 8 rounds of it,
    // so the row's loads, sum and quantise finish sooner (1 x 5120: 3.9 ->
    // 3.3 us; the "wide block" of the decode RMSNorm).
    if (KIND == kProdRms && n <= 4 && rounds <= 64) {
        hipLaunchKernelGGL((k_producer<KIND, WY, 8, QUANT, 8>), grid, dim3(512), 0, s, a, b, y, (int)n,
                           (int)d, eps, pl.q, pl.ds, (int)rows, rps);
        return hipGetLastError();
    }
    if (KIND == kProdRms && per_wave <= 4) {
        hipLaunchKernelGGL((k_producer<KIND, WY, 4, QUANT>), grid, block, 0, s, a, b, y, (int)n,
                           (int)d, eps, pl.q, pl.ds, (int)rows, rps);
    } else if (KIND == kProdRms && per_wave <= 8) {
        hipLaunchKernelGGL((k_producer<KIND, WY, 8, QUANT>), grid, block, 0, s, a, b, y, (int)n,
                           (int)d, eps, pl.q, pl.ds, (int)rows, rps);
    } else if (KIND == kProdRms && per_wave <= 16) {
        hipLaunchKernelGGL((k_producer<KIND, WY, 16, QUANT>), grid, block, 0, s, a, b, y, (int)n,
                           (int)d, eps, pl.q, pl.ds, (int)rows, rps);
    } else {
        hipLaunchKernelGGL((k_producer<KIND, WY, 0, QUANT>), grid, block, 0, s, a, b, y, (int)n,
                           (int)d, eps, pl.q, pl.ds, (int)rows, rps);
    }
    return hipGetLastError();
}

// Export: the (D, S) pairs of `count` blocks into separate arrays.
__global__ __launch_bounds__(256) void k_plane_split(const uint2* __restrict__ ds,
                                                     float* __restrict__ D,
                                                     int32_t* __restrict__ S, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint2 v = ds[i];
        D[i] = __uint_as_float(v.x);
        S[i] = (int32_t)v.y;
    }
}

}  // namespace

hipError_t launch_plane_split(const uint2* ds, float* D, int32_t* S, int64_t count,
                              hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const int64_t want = (count + 255) / 256;
    const dim3 grid((unsigned)std::min<int64_t>(want, 4096));
    hipLaunchKernelGGL(k_plane_split, grid, dim3(256), 0, s, ds, D, S, count);
    return hipGetLastError();
}

hipError_t launch_producer(ProducerKind kind, const float* a, const float* b, float* y,
                           int64_t n, int64_t d, float eps, bool write_y,
                           const PlaneView& pl, hipStream_t s) {
    if (pl.q == nullptr) {   // unfused: y only, no plane (RMSNorm, SwiGLU)
        if (kind == kProdRms) return dispatch_maxr<kProdRms, true, false>(a, b, y, n, d, eps, pl, s);
        if (kind == kProdSwiglu)
            return dispatch_maxr<kProdSwiglu, true, false>(a, b, y, n, d, eps, pl, s);
        return hipErrorInvalidValue;
    }
    switch (kind) {
        case kProdRms:
            return write_y ? dispatch_maxr<kProdRms, true>(a, b, y, n, d, eps, pl, s)
                           : dispatch_maxr<kProdRms, false>(a, b, y, n, d, eps, pl, s);
        case kProdSwiglu:
            return write_y ? dispatch_maxr<kProdSwiglu, true>(a, b, y, n, d, eps, pl, s)
                           : dispatch_maxr<kProdSwiglu, false>(a, b, y, n, d, eps, pl, s);
        default:
            return dispatch_maxr<kProdF32, false>(a, nullptr, nullptr, n, d, eps, pl, s);
    }
}

}  // namespace mmq
