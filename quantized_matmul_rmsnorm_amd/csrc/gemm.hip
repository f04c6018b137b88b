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
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kGroupO = 4;     // output tiles per raster group

// 4 int8 codes -> 4 exact f16: flip the sign bit (byte = q + 128), place each
// byte under the f16 exponent of 1024 (0x64xx = 1024 + byte) and subtract
// 1152 in packed f16 -- every value involved is an integer below 2048, so the
// result is exactly q.
__device__ __forceinline__ void i8x4_to_f16(uint32_t v, half2v& lo, half2v& hi) {
    v ^= 0x80808080u;
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u);
    const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = __builtin_bit_cast(half2v, a) + bias;
    hi = __builtin_bit_cast(half2v, b) + bias;
}

__device__ __forceinline__ half8 i8x8_to_f16(uint32_t x, uint32_t y) {
    half2v a, b, c, d;
    i8x4_to_f16(x, a, b);
    i8x4_to_f16(y, c, d);
    half8 h;
    h[0] = a[0]; h[1] = a[1]; h[2] = b[0]; h[3] = b[1];
    h[4] = c[0]; h[5] = c[1]; h[6] = d[0]; h[7] = d[1];
    return h;
}

// Hardware places workgroup i on XCD i % 8; give each XCD a contiguous range of
// logical tiles so that the workgroups resident on one XCD (and its L2) share
// weight and activation tiles.  Within the range, tiles are rastered in groups
// of kGroupO output tiles with the token tile varying slowest inside a group.
__device__ __forceinline__ void tile_of(int n_ttiles, int n_otiles, int& t_tile, int& o_tile) {
    const int nwg = gridDim.x;
    const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int L = xcd * per + min(xcd, rem) + li;
    const int gsize = kGroupO * n_ttiles;
    const int group = L / gsize, r = L % gsize;
    const int go = min(kGroupO, n_otiles - group * kGroupO);
    o_tile = group * kGroupO + r % go;
    t_tile = r / go;
}

template <bool Q4K, int CH>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(
    const half8* __restrict__ wa, const float* __restrict__ dmr,
    const half8* __restrict__ mfrag, const int8_t* __restrict__ Q,
    const float* __restrict__ Dp, const int32_t* __restrict__ Sp, int n, int plane_rows,
    int id, int od, int n_ttiles, int n_otiles, float* __restrict__ out) {
    constexpr int NPART = Q4K ? 1 : 2;
    constexpr int BPAD = 4;    // half8 of padding per B slot: keeps the 4 slots on distinct banks
    constexpr int DPAD = 16;   // floats of padding per D slot
    // Two LDS buffers of CH staged 32-blocks each (double buffering).
    __shared__ half8 sA[2][CH][4][2][NPART][64];   // [buf][block][o group][k16][part][lane]
    __shared__ half8 sB[2][CH][4 * 2 * 64 + BPAD]; // [buf][block][(t group, k16, lane)]
    __shared__ float sD[2][CH][128 + DPAD];
    // q4_K: D*S of the current and the next superblock: [sb&1][t group][lane][block j],
    // hi part in lanes < 32, lo part in lanes >= 32
    __shared__ __attribute__((aligned(16))) _Float16 sP[Q4K ? 2 : 1][4][64][8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ogl = wave & 3;
    const int th = wave >> 2;

    int t_tile, o_tile;
    tile_of(n_ttiles, n_otiles, t_tile, o_tile);
    const int64_t t0 = (int64_t)t_tile * 128;
    const int64_t og0 = (int64_t)o_tile * 4;

    const int nb = id / kBlock;
    const int nsb = id / kSuper;
    const int64_t K16 = id / 16;
    const int nch = nb / CH;

    // ---- staging assignment ----
    // A: per block q4_K has 8 fragments (4 groups x 2 k16), q6_K 16 (x 2 parts);
    //    thread tid copies fragment tid/64 (+ 8 for the second part) of each block.
    const int fa = tid >> 6;
    // B, D, S: CH == 4: thread -> token row tid/4, block tid%4 of the chunk (one
    // 32-byte block); CH == 2: thread -> row tid/4, block (tid/2)%2, 16-byte half tid%2.
    const int tb = tid >> 2;
    const int jb = CH == 4 ? (tid & 3) : ((tid >> 1) & 1);
    const int hb = CH == 4 ? -1 : (tid & 1);
    const int64_t rowb = t0 + tb;
    const bool rowb_ok = rowb < plane_rows;
    const uint4* qrow = reinterpret_cast<const uint4*>(Q + rowb * (int64_t)id);

    half8 ra[CH][NPART];
    uint4 rb0, rb1;
    float rd;
    int32_t rs;

    auto load_chunk = [&](int c) {
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
            const int b = c * CH + jj;
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
                ra[jj][p] = wa[src];
            }
        }
        const int b = c * CH + jb;
        if (rowb_ok) {
            if (CH == 4) {
                rb0 = qrow[2 * b];
                rb1 = qrow[2 * b + 1];
            } else {
                rb0 = qrow[2 * b + hb];
            }
            rd = Dp[rowb * nb + b];
            rs = Q4K ? Sp[rowb * nb + b] : 0;
        } else {
            rb0 = rb1 = make_uint4(0u, 0u, 0u, 0u);
            rd = 0.0f;
            rs = 0;
        }
    };

    auto store_chunk = [&](int c, int buf) {
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
#pragma unroll
            for (int p = 0; p < NPART; ++p) {
                if (Q4K) {
                    sA[buf][jj][fa >> 1][fa & 1][0][lane] = ra[jj][p];
                } else {
                    const int f = fa + 8 * p;
                    sA[buf][jj][f >> 2][(f >> 1) & 1][f & 1][lane] = ra[jj][p];
                }
            }
        }
        // codes of (row tb, block jb): 16 codes per k16, 8 per lane half
        const int tg = tb >> 5, tl = tb & 31;
        half8* sb = &sB[buf][jb][tg * 128];
        if (CH == 4) {
            sb[tl] = i8x8_to_f16(rb0.x, rb0.y);
            sb[tl + 32] = i8x8_to_f16(rb0.z, rb0.w);
            sb[64 + tl] = i8x8_to_f16(rb1.x, rb1.y);
            sb[64 + tl + 32] = i8x8_to_f16(rb1.z, rb1.w);
        } else {
            sb[64 * hb + tl] = i8x8_to_f16(rb0.x, rb0.y);
            sb[64 * hb + tl + 32] = i8x8_to_f16(rb0.z, rb0.w);
        }
        if (CH == 4 || hb == 0) {
            sD[buf][jb][tb] = rd;
            if (Q4K) {
                const float P = rd * (float)rs;
                const _Float16 hi = (_Float16)P;
                const _Float16 lo = (_Float16)(P - (float)hi);
                const int b = c * CH + jb;
                sP[(b >> 3) & 1][tg][tl][b & 7] = hi;
                sP[(b >> 3) & 1][tg][tl + 32][b & 7] = lo;
            }
        }
    };

    f32x16 acc[2], res[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { acc[i][r] = 0.0f; res[i][r] = 0.0f; }
    }

    load_chunk(0);
    store_chunk(0, 0);
    if (nch > 1) load_chunk(1);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        // stage chunk c+1 into the other buffer (its previous contents, chunk c-1,
        // were consumed before the barrier that ended the last iteration)
        if (c + 1 < nch) {
            store_chunk(c + 1, buf ^ 1);
            if (c + 2 < nch) load_chunk(c + 2);
        }

        // Software pipeline inside the chunk: the MFMAs of block jj are issued
        // before the epilogue FMAs of block jj-1, so the matrix core and the
        // VALU work on different blocks at the same time.
        f32x16 X[2][2];
        auto mfma_block = [&](int jj, f32x16* Xo) {
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16) {
                half8 a[NPART];
#pragma unroll
                for (int p = 0; p < NPART; ++p) a[p] = sA[buf][jj][ogl][k16][p][lane];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const half8 bf = sB[buf][jj][((2 * th + i) * 2 + k16) * 64 + lane];
                    if (k16 == 0) {
                        const f32x16 zero = {};
                        Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], bf, zero, 0, 0, 0);
                    } else {
                        Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], bf, Xo[i], 0, 0, 0);
                    }
                    if (!Q4K)
                        Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[NPART - 1], bf, Xo[i], 0, 0, 0);
                }
            }
        };
        auto epilogue_block = [&](int jj, const f32x16* Xi) {
            const int b = c * CH + jj;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float da = sD[buf][jj][(2 * th + i) * 32 + (lane & 31)];
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(da, Xi[i][r], acc[i][r]);
            }
            if ((b & 7) == 7) {  // superblock boundary
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
                        const half8 pf = *reinterpret_cast<const half8*>(&sP[sb & 1][2 * th + i][lane][0]);
                        const f32x16 zero = {};
                        const f32x16 mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(mf, pf, zero, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            float v = fmaf(dv[r], acc[i][r], res[i][r]);
                            res[i][r] = fmaf(-mv[r], mn[r], v);
                            acc[i][r] = 0.0f;
                        }
                    }
                } else {
                    const float* dm = dmr + (og * nsb + sb) * 32 + half * 16;
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            res[i][r] = fmaf(dm[r], acc[i][r], res[i][r]);
                            acc[i][r] = 0.0f;
                        }
                }
            }
        };
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
            mfma_block(jj, X[jj & 1]);
            if (jj > 0) epilogue_block(jj - 1, X[(jj - 1) & 1]);
        }
        epilogue_block(CH - 1, X[(CH - 1) & 1]);
        __syncthreads();
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
        hipLaunchKernelGGL((k_gemm<true, 4>), grid, block, 0, s, (const half8*)w.wa, w.dmr,
                           (const half8*)w.mfrag, pl.q, pl.D, pl.S, (int)n, (int)pl.rows,
                           (int)w.cols, (int)w.rows, n_ttiles, n_otiles, out);
    else
        hipLaunchKernelGGL((k_gemm<false, 2>), grid, block, 0, s, (const half8*)w.wa, w.dmr,
                           (const half8*)nullptr, pl.q, pl.D, pl.S, (int)n, (int)pl.rows,
                           (int)w.cols, (int)w.rows, n_ttiles, n_otiles, out);
    return hipGetLastError();
}

}  // namespace mmq
