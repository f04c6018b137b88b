// gemm.hip -- q4_K / q6_K matmul over a q8 activation plane on gfx950 MFMA.
//
// Method ("64 · r60 ...", section 3.2; "55 · r52 ...", section 5): the prefill
// matmul multiplies the block-32 int8 activation plane by K-quant weights as
// integer block dots, rescaled per 32-block (q6_K: per 16-element half).  For
// token t, output o and 32-block b of superblock sb:
//   q4_K: out += D[t][b] * (d*sc_j * I  -  dmin*m_j * S[t][b]),  I = sum q_w*q
//   q6_K: out += D[t][b] * d * (sc0*I0 + sc1*I1),  I0/I1 = 16-element dots of
//         (q_w - 32) with q.
//
// How it maps onto CDNA4.  The integer dots run on v_mfma_f32_32x32x16_f16 with
// integer-valued f16 operands: the activation codes (|q| <= 127) and the
// registration-time weight values sc_j*q_w (q4_K, <= 945) or sc*(q_w-32) split
// into an even part and a 0/1 part (q6_K, |v| <= 4096) are exact in f16,
// every product is exact in f32 and every partial sum of one block stays below
// 2^24, so the MFMA returns the exact integer block dot as an f32.  Folding the
// weight's sub-scale into the operand leaves one FMA per output per block
// (acc += D[t][b] * X) with D constant per lane, because tokens sit on the
// MFMA's N axis (lane % 32) and outputs on its M axis (registers).  An int8
// MFMA would return int32 and need a convert, a sub-scale multiply and the FMA
// for every output of every block -- three VALU ops against the one here, and
// the VALU, not the matrix core, is what bounds this kernel.
// Per superblock the sum over its 8 blocks is scaled by d (one FMA per output);
// the q4_K min term sum_j (D*S)[t][j] * m_j is one extra MFMA per superblock
// with m_j exact in f16 and D*S split into two f16 parts (22 significant bits).
//
// Tiling.  Workgroup of 8 waves computes 128 outputs x 128 tokens; wave w owns
// output group w%4 (32 rows) and token groups 2*(w/4), 2*(w/4)+1 (2 x 32
// tokens).  Per 32-block the workgroup stages the weight fragments (copied,
// already in fragment order) and the 128 x 32 activation codes (converted
// int8 -> f16 once) in LDS; the next block's global loads are issued before the
// current block's MFMAs.  Plane rows beyond the plane's padded row count read
// as zero; outputs are stored only for t < n and o < rows.
#include "mmq_internal.h"

namespace mmq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;

__device__ __forceinline__ half8 i8x8_to_f16(uint2 v) {
    half8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = (_Float16)(float)(int8_t)(v.x >> (8 * i));
        h[4 + i] = (_Float16)(float)(int8_t)(v.y >> (8 * i));
    }
    return h;
}

template <bool Q4K>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(
    const half8* __restrict__ wa, const float* __restrict__ dmr,
    const half8* __restrict__ mfrag, const int8_t* __restrict__ Q,
    const float* __restrict__ Dp, const int32_t* __restrict__ Sp, int n, int plane_rows,
    int id, int od, int n_ttiles, float* __restrict__ out) {
    constexpr int NPART = Q4K ? 1 : 2;
    __shared__ half8 sA[4][2][NPART][64];   // [o group][k16][part][lane]
    __shared__ half8 sB[4][2][64];          // [t group][k16][lane]
    __shared__ float sD[128];
    __shared__ __attribute__((aligned(16))) _Float16 sP[4][64][8];  // q4_K: [t group][lane][block j]: D*S hi (lanes < 32) / lo

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ogl = wave & 3;
    const int th = wave >> 2;

    const int t_tile = blockIdx.x % n_ttiles;
    const int o_tile = blockIdx.x / n_ttiles;
    const int64_t t0 = (int64_t)t_tile * 128;
    const int64_t og0 = (int64_t)o_tile * 4;

    const int nb = id / kBlock;
    const int nsb = id / kSuper;
    const int64_t K16 = id / 16;

    // ---- staging assignment ----
    // A: q4_K 8 fragments (4 groups x 2 k16), q6_K 16 (x 2 parts): one or two per thread
    const int fa = tid >> 6;              // 0..7
    // B: thread -> token row tb, 8-byte chunk cb of the 32-byte block
    const int tb = tid >> 2;
    const int cb = tid & 3;
    const int64_t rowb = t0 + tb;
    const bool rowb_ok = rowb < plane_rows;
    const int8_t* qrow = Q + rowb * (int64_t)id + 8 * cb;

    half8 ra[NPART];
    uint2 rb;
    float rd = 0.0f;
    int32_t rs = 0;

    auto load_block = [&](int b) {
#pragma unroll
        for (int p = 0; p < NPART; ++p) {
            int64_t src;
            if (Q4K) {
                const int g = fa >> 1, k16 = fa & 1;
                src = ((og0 + g) * K16 + 2 * b + k16) * 64 + lane;
            } else {
                const int f = fa + 8 * p;           // 0..15 = g*4 + k16*2 + part
                const int g = f >> 2, k16 = (f >> 1) & 1, part = f & 1;
                src = (((og0 + g) * K16 + 2 * b + k16) * 2 + part) * 64 + lane;
            }
            ra[p] = wa[src];
        }
        rb = rowb_ok ? *reinterpret_cast<const uint2*>(qrow + (int64_t)b * kBlock)
                     : make_uint2(0u, 0u);
        if (tid < 128) {
            const int64_t r = t0 + tid;
            const bool ok = r < plane_rows;
            rd = ok ? Dp[r * nb + b] : 0.0f;
            if (Q4K) rs = ok ? Sp[r * nb + b] : 0;
        }
    };

    auto store_block = [&](int b) {
#pragma unroll
        for (int p = 0; p < NPART; ++p) {
            if (Q4K) {
                sA[fa >> 1][fa & 1][0][lane] = ra[p];
            } else {
                const int f = fa + 8 * p;
                sA[f >> 2][(f >> 1) & 1][f & 1][lane] = ra[p];
            }
        }
        sB[tb >> 5][cb >> 1][(tb & 31) + 32 * (cb & 1)] = i8x8_to_f16(rb);
        if (tid < 128) {
            sD[tid] = rd;
            if (Q4K) {
                const float P = rd * (float)rs;
                const _Float16 hi = (_Float16)P;
                const _Float16 lo = (_Float16)(P - (float)hi);
                const int j = b & 7;
                sP[tid >> 5][tid & 31][j] = hi;
                sP[tid >> 5][(tid & 31) + 32][j] = lo;
            }
        }
    };

    f32x16 acc[2], res[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { acc[i][r] = 0.0f; res[i][r] = 0.0f; }
    }

    load_block(0);
    for (int b = 0; b < nb; ++b) {
        __syncthreads();
        store_block(b);
        __syncthreads();
        if (b + 1 < nb) load_block(b + 1);

        const int j = b & 7;
        f32x16 X[2];
#pragma unroll
        for (int k16 = 0; k16 < 2; ++k16) {
            half8 a[NPART];
#pragma unroll
            for (int p = 0; p < NPART; ++p) a[p] = sA[ogl][k16][p][lane];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const half8 bf = sB[2 * th + i][k16][lane];
                if (k16 == 0) {
                    const f32x16 zero = {};
                    X[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], bf, zero, 0, 0, 0);
                } else {
                    X[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], bf, X[i], 0, 0, 0);
                }
                if (!Q4K) X[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[NPART - 1], bf, X[i], 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float da = sD[(2 * th + i) * 32 + (lane & 31)];
            if (j == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] = da * X[i][r];
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(da, X[i][r], acc[i][r]);
            }
        }

        if (j == 7) {  // superblock boundary
            const int sb = b >> 3;
            const int64_t og = og0 + ogl;
            const int half = lane >> 5;
            if (Q4K) {
                const float* dm = dmr + (og * nsb + sb) * 64;
                float dv[16], mv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    dv[r] = dm[half * 16 + r];
                    mv[r] = dm[32 + half * 16 + r];
                }
                const half8 mf = mfrag[(og * nsb + sb) * 64 + lane];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const half8 pf = *reinterpret_cast<const half8*>(&sP[2 * th + i][lane][0]);
                    const f32x16 zero = {};
                    const f32x16 mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(mf, pf, zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float v = fmaf(dv[r], acc[i][r], res[i][r]);
                        res[i][r] = fmaf(-mv[r], mn[r], v);
                    }
                }
            } else {
                const float* dm = dmr + (og * nsb + sb) * 32 + half * 16;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) res[i][r] = fmaf(dm[r], acc[i][r], res[i][r]);
            }
        }
    }

    // ---- store: lane holds token t, rows o = 8*(r/4) + 4*(lane/32) + r%4 ----
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = t0 + (2 * th + i) * 32 + (lane & 31);
        if (t >= n) continue;
        float* orow = out + t * (int64_t)od;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t o = (og0 + ogl) * 32 + 8 * q + 4 * (lane >> 5);
            if (o + 3 < od && (od & 3) == 0) {
                *reinterpret_cast<float4*>(orow + o) =
                    make_float4(res[i][4 * q], res[i][4 * q + 1], res[i][4 * q + 2], res[i][4 * q + 3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (o + e < od) orow[o + e] = res[i][4 * q + e];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                       hipStream_t s) {
    const int n_ttiles = (int)((n + 127) / 128);
    const int n_otiles = (int)(w.rows_pad / kTileO);
    const dim3 grid((unsigned)(n_ttiles * n_otiles)), block(kThreads);
    if (w.type == 12)
        hipLaunchKernelGGL(k_gemm<true>, grid, block, 0, s, (const half8*)w.wa, w.dmr,
                           (const half8*)w.mfrag, pl.q, pl.D, pl.S, (int)n, (int)pl.rows,
                           (int)w.cols, (int)w.rows, n_ttiles, out);
    else
        hipLaunchKernelGGL(k_gemm<false>, grid, block, 0, s, (const half8*)w.wa, w.dmr,
                           (const half8*)nullptr, pl.q, pl.D, pl.S, (int)n, (int)pl.rows,
                           (int)w.cols, (int)w.rows, n_ttiles, out);
    return hipGetLastError();
}

}  // namespace mmq
