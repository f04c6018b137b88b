// repack.hip -- registration-time repack of raw q4_K / q6_K superblocks into the
// device tiles the matmul and GEMV kernels read.
//
// The pages register every q4_K / q6_K weight once, before the first forward,
// and keep registration-time planes of them ("64 · r60 ...", section 3.1; the
// W_exp / W_dsc planes named in section 1).  Here a weight is copied to the
// device raw and this kernel rewrites it; it runs once per weight, outside any
// timed loop.
//
// Superblock formats (public GGUF K-quants, 256 weights each):
//   q4_K, 144 B: f16 d | f16 dmin | 12 B packed 6-bit (scale, min) x 8 | 128 B
//                4-bit quants; w = d*sc_j*q - dmin*m_j, j = sub-block of 32.
//   q5_K, 176 B: f16 d | f16 dmin | 12 B scales (as q4_K) | qh[32] | qs[128]
//                low nibbles (arranged as the q4_K quants); the fifth bit of
//                element 64*g + l (l < 32) is bit 2g of qh[l], that of
//                element 64*g + 32 + l bit 2g+1; w = d*sc_j*q - dmin*m_j,
//                q in [0, 31];
//   q6_K, 210 B: ql[128] | qh[64] | int8 scales[16] | f16 d;
//                w = d*sc[e/16]*(q - 32), q in [0, 63].
//
// Prefill tiles (read by gemm.hip).  Rows are padded to a multiple of 128
// with zero weights; og = row / 32, ol = row % 32; for k: k16 = k / 16,
// lane = ol + 32*((k % 16) / 8), e = k % 8 -- the A-operand fragment of
// v_mfma_f32_32x32x16_f16 (lane holds row lane%32, 8 consecutive k of the
// half lane/32), so a wave reads one fragment as 1 KiB contiguous.
//   q4_K: wa[og][k16][lane][e] = f16(sc_j * q)        (exact: <= 63*15 = 945)
//         dmr[og][sb][{d,dmin}][half][r] f32, r/half as the MFMA output row
//             of ol: ol = 8*(r/4) + 4*half + r%4
//         mfrag[og][sb][lane][j] = bf16(m_j) for both lane halves (exact)
//   q4_K packed (MMQ_USE_GEMM_PACKED): the same fragments as 4-bit codes,
//         wa4[og][b][lane] uint2 for 32-block b: .x holds the lane's 8 codes
//         of k16 = 2b, .y those of 2b + 1; code e sits at bits 4*(e/2) (e
//         even) or 16 + 4*(e/2) (e odd), so that one mask turns codes e and
//         e+1 into a pair of f16 subnormals (code * 2^-24);
//         wsc[og][sb][ol] uint4 = f16(sc_j * 2^10), j = 0..7 (exact: <= 64512),
//         so one packed multiply gives sc_j*q * 2^-14;
//         dmr as above with d times 2^14 (exact), mfrag as above
//   q6_K: wa[og][k16][lane][e] = f16(q - 32)     (exact; the matmul forms
//             sc * (q - 32), 13 bits, as two exact f16 parts in registers)
//         mfrag[og][sb][ol][i] = f16(sc_i), i = 0..15 (exact)
//         dmr[og][sb][half][r] = d
// One-token GEMV tiles (q6_K, read by mmvq.hip), per row o and 32-block b
// (weights w_0..w_31):
//   ql[o][b]  uint4: dword u holds w_8u..w_8u+7; byte i = low4(w_8u+i) |
//                    low4(w_8u+i+4) << 4
//   qh[o][b]  uint2: dword u holds w_16u..w_16u+15; byte i = hi2(w_i') |
//                    hi2(w_i'+4) << 2 | hi2(w_i'+8) << 4 | hi2(w_i'+12) << 6,
//                    i' = 16u + i
//   sc[o][b]  int16: low byte = sub-scale of w_0..15, high byte = of w_16..31
//   d[o][sb]  f32
// One-token GEMV tiles (q4_K), per row o and 32-block b = 8*sb + j:
//   ql[o][b]  uint4: the 4-bit codes, same byte order as the q6_K low nibbles
//   sc[o][b]  int16: sc_j | m_j << 8
//   d[o][sb]  f32 pair: d, dmin
// One-token GEMV tiles (q5_K): ql, sc and d as for q4_K (ql holds the low
// nibbles), plus
//   h5[o][b]  uint32: bit 8*i + g = fifth bit of w_{4g+i} (g = 0..7,
//             i = 0..3), so the bits of the 4 weights that one dot4 takes
//             from a nibble group g sit at bit g of each byte
#include "mmq_internal.h"

namespace mmq {
namespace {

__device__ __forceinline__ float f16f(const uint8_t* p) {
    const uint16_t bits = (uint16_t)(p[0] | (p[1] << 8));
    return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ void q4k_decode(const uint8_t* blk, float& d, float& dmin,
                                           int sc[8], int mn[8]) {
    d = f16f(blk);
    dmin = f16f(blk + 2);
    const uint8_t* s = blk + 4;
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        mn[j] = s[j + 4] & 63;
        sc[j + 4] = (s[j + 8] & 15) | ((s[j] >> 6) << 4);
        mn[j + 4] = (s[j + 8] >> 4) | ((s[j + 4] >> 6) << 4);
    }
}

__device__ __forceinline__ int q4k_quant(const uint8_t* blk, int e) {
    const uint8_t byte = blk[16 + 32 * (e / 64) + (e % 32)];
    return (e % 64) < 32 ? (byte & 15) : (byte >> 4);
}

__device__ __forceinline__ int q5k_quant(const uint8_t* blk, int e) {
    const int g = e / 64, i = e % 64;
    const uint8_t byte = blk[48 + 32 * g + (i % 32)];
    const int lo = i < 32 ? (byte & 15) : (byte >> 4);
    const int hi = (blk[16 + (i % 32)] >> (2 * g + (i >= 32 ? 1 : 0))) & 1;
    return lo | (hi << 4);
}

__device__ __forceinline__ int q6k_quant(const uint8_t* blk, int e) {
    const int h = e / 128, r = e % 128, s = r / 32, l = r % 32;
    const uint8_t lb = blk[64 * h + l + 32 * (s & 1)];
    const int lo = s < 2 ? (lb & 15) : (lb >> 4);
    const int hi = (blk[128 + 32 * h + l] >> (2 * s)) & 3;
    return lo | (hi << 4);
}

__device__ __forceinline__ void frag_pos(int64_t o, int64_t k, int64_t& og, int& lane, int& e,
                                         int64_t& k16) {
    og = o / 32;
    const int ol = (int)(o % 32);
    k16 = k / 16;
    lane = ol + 32 * (int)((k % 16) / 8);
    e = (int)(k % 8);
}

__device__ __forceinline__ int out_reg(int ol, int& half) {
    half = (ol % 8) / 4;
    return 4 * (ol / 8) + (ol % 4);
}

// One thread per (row, superblock) of the real rows.
__global__ void k_repack_q4k_gemm(const uint8_t* __restrict__ raw, int64_t rows, int64_t cols,
                                  _Float16* __restrict__ wa, float* __restrict__ dmr,
                                  _Float16* __restrict__ mfrag) {
    const int64_t nsb = cols / kSuper;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nsb) return;
    const int64_t o = idx / nsb, sb = idx % nsb;
    const uint8_t* blk = raw + idx * 144;
    float d, dmin;
    int sc[8], mn[8];
    q4k_decode(blk, d, dmin, sc, mn);
    const int64_t K16 = cols / 16;
    for (int e = 0; e < kSuper; ++e) {
        int64_t og, k16; int lane, el;
        frag_pos(o, sb * kSuper + e, og, lane, el, k16);
        wa[((og * K16 + k16) * 64 + lane) * 8 + el] = (_Float16)(float)(sc[e / 32] * q4k_quant(blk, e));
    }
    const int64_t og = o / 32;
    const int ol = (int)(o % 32);
    int half;
    const int r = out_reg(ol, half);
    float* dm = dmr + (og * nsb + sb) * 64;
    dm[half * 16 + r] = d;
    dm[32 + half * 16 + r] = dmin;
    // mins as bf16 bits (exact: at most 6 significant bits)
    uint16_t* mf = reinterpret_cast<uint16_t*>(mfrag) + (og * nsb + sb) * 512;
    for (int j = 0; j < 8; ++j) {
        const uint16_t bits = (uint16_t)(__float_as_uint((float)mn[j]) >> 16);
        mf[ol * 8 + j] = bits;
        mf[(ol + 32) * 8 + j] = bits;
    }
}

// Packed q4_K tiles: one thread per (row, superblock) of the real rows.  A
// row owns whole 32-bit words of wa4 (lanes ol and ol + 32), so no two
// threads write one word.
__global__ void k_repack_q4k_gemm_packed(const uint8_t* __restrict__ raw, int64_t rows,
                                         int64_t cols, uint32_t* __restrict__ wa4,
                                         uint4* __restrict__ wsc, float* __restrict__ dmr,
                                         _Float16* __restrict__ mfrag) {
    const int64_t nsb = cols / kSuper;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nsb) return;
    const int64_t o = idx / nsb, sb = idx % nsb;
    const uint8_t* blk = raw + idx * 144;
    float d, dmin;
    int sc[8], mn[8];
    q4k_decode(blk, d, dmin, sc, mn);
    const int64_t og = o / 32, nb = cols / kBlock;
    const int ol = (int)(o % 32);
    for (int j = 0; j < 8; ++j) {            // 32-block b = 8*sb + j
        const int64_t b = sb * 8 + j;
        for (int step = 0; step < 2; ++step) {
            for (int hl = 0; hl < 2; ++hl) {  // lane half: k % 16 in [8*hl, 8*hl + 8)
                uint32_t word = 0;
                for (int e = 0; e < 8; ++e) {
                    const int q = q4k_quant(blk, 32 * j + 16 * step + 8 * hl + e);
                    const int bit = (e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1);
                    word |= (uint32_t)q << bit;
                }
                const int lane = ol + 32 * hl;
                wa4[((og * nb + b) * 64 + lane) * 2 + step] = word;
            }
        }
    }
    uint32_t sp[4];
    for (int j = 0; j < 4; ++j) {
        const uint16_t lo = __builtin_bit_cast(uint16_t, (_Float16)(float)(sc[2 * j] * 1024));
        const uint16_t hi = __builtin_bit_cast(uint16_t, (_Float16)(float)(sc[2 * j + 1] * 1024));
        sp[j] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    wsc[(og * nsb + sb) * 32 + ol] = make_uint4(sp[0], sp[1], sp[2], sp[3]);
    int half;
    const int r = out_reg(ol, half);
    float* dm = dmr + (og * nsb + sb) * 64;
    dm[half * 16 + r] = d * 16384.0f;   // the block dots come out times 2^-14
    dm[32 + half * 16 + r] = dmin;
    uint16_t* mf = reinterpret_cast<uint16_t*>(mfrag) + (og * nsb + sb) * 512;
    for (int j = 0; j < 8; ++j) {
        const uint16_t bits = (uint16_t)(__float_as_uint((float)mn[j]) >> 16);
        mf[ol * 8 + j] = bits;
        mf[(ol + 32) * 8 + j] = bits;
    }
}

__global__ void k_repack_q6k_gemm(const uint8_t* __restrict__ raw, int64_t rows, int64_t cols,
                                  _Float16* __restrict__ wa, float* __restrict__ dmr,
                                  _Float16* __restrict__ wsc) {
    const int64_t nsb = cols / kSuper;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nsb) return;
    const int64_t o = idx / nsb, sb = idx % nsb;
    const uint8_t* blk = raw + idx * 210;
    const float d = f16f(blk + 208);
    const int8_t* scales = reinterpret_cast<const int8_t*>(blk + 192);
    const int64_t K16 = cols / 16;
    for (int e = 0; e < kSuper; ++e) {
        int64_t og, k16; int lane, el;
        frag_pos(o, sb * kSuper + e, og, lane, el, k16);
        wa[((og * K16 + k16) * 64 + lane) * 8 + el] = (_Float16)(float)(q6k_quant(blk, e) - 32);
    }
    const int64_t og = o / 32;
    const int ol = (int)(o % 32);
    for (int i = 0; i < 16; ++i) wsc[((og * nsb + sb) * 32 + ol) * 16 + i] = (_Float16)(float)scales[i];
    int half;
    const int r = out_reg(ol, half);
    dmr[(og * nsb + sb) * 32 + half * 16 + r] = d;
}

__global__ void k_repack_q6k_gemv(const uint8_t* __restrict__ raw, int64_t rows, int64_t cols,
                                  uint4* __restrict__ ql, uint2* __restrict__ qh,
                                  int16_t* __restrict__ scv, float* __restrict__ dv) {
    const int64_t nsb = cols / kSuper;
    const int64_t nb = cols / kBlock;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nsb) return;
    const int64_t o = idx / nsb, sb = idx % nsb;
    const uint8_t* blk = raw + idx * 210;
    const int8_t* scales = reinterpret_cast<const int8_t*>(blk + 192);
    dv[o * nsb + sb] = f16f(blk + 208);
    for (int j = 0; j < 8; ++j) {
        int q[32];
        for (int i = 0; i < 32; ++i) q[i] = q6k_quant(blk, 32 * j + i);
        uint32_t L[4], H[2];
        for (int u = 0; u < 4; ++u) {
            uint32_t v = 0;
            for (int i = 0; i < 4; ++i)
                v |= (uint32_t)((q[8 * u + i] & 15) | ((q[8 * u + i + 4] & 15) << 4)) << (8 * i);
            L[u] = v;
        }
        for (int u = 0; u < 2; ++u) {
            uint32_t v = 0;
            for (int i = 0; i < 4; ++i) {
                const int b0 = 16 * u + i;
                const uint32_t byte = (uint32_t)((q[b0] >> 4) | ((q[b0 + 4] >> 4) << 2) |
                                                 ((q[b0 + 8] >> 4) << 4) | ((q[b0 + 12] >> 4) << 6));
                v |= byte << (8 * i);
            }
            H[u] = v;
        }
        const int64_t b = sb * 8 + j;
        ql[o * nb + b] = make_uint4(L[0], L[1], L[2], L[3]);
        qh[o * nb + b] = make_uint2(H[0], H[1]);
        scv[o * nb + b] = (int16_t)(((uint16_t)(uint8_t)scales[2 * j]) |
                                    ((uint16_t)(uint8_t)scales[2 * j + 1] << 8));
    }
}

__global__ void k_repack_q4k_gemv(const uint8_t* __restrict__ raw, int64_t rows, int64_t cols,
                                  uint4* __restrict__ ql, int16_t* __restrict__ scv,
                                  float* __restrict__ dv) {
    const int64_t nsb = cols / kSuper;
    const int64_t nb = cols / kBlock;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nsb) return;
    const int64_t o = idx / nsb, sb = idx % nsb;
    const uint8_t* blk = raw + idx * 144;
    float d, dmin;
    int sc[8], mn[8];
    q4k_decode(blk, d, dmin, sc, mn);
    dv[2 * (o * nsb + sb)] = d;
    dv[2 * (o * nsb + sb) + 1] = dmin;
    for (int j = 0; j < 8; ++j) {
        uint32_t L[4];
        for (int u = 0; u < 4; ++u) {
            uint32_t v = 0;
            for (int i = 0; i < 4; ++i)
                v |= (uint32_t)(q4k_quant(blk, 32 * j + 8 * u + i) |
                                (q4k_quant(blk, 32 * j + 8 * u + i + 4) << 4)) << (8 * i);
            L[u] = v;
        }
        const int64_t b = sb * 8 + j;
        ql[o * nb + b] = make_uint4(L[0], L[1], L[2], L[3]);
        scv[o * nb + b] = (int16_t)((uint16_t)sc[j] | ((uint16_t)mn[j] << 8));
    }
}

__global__ void k_repack_q5k_gemv(const uint8_t* __restrict__ raw, int64_t rows, int64_t cols,
                                  uint4* __restrict__ ql, uint32_t* __restrict__ h5,
                                  int16_t* __restrict__ scv, float* __restrict__ dv) {
    const int64_t nsb = cols / kSuper;
    const int64_t nb = cols / kBlock;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nsb) return;
    const int64_t o = idx / nsb, sb = idx % nsb;
    const uint8_t* blk = raw + idx * 176;
    float d, dmin;
    int sc[8], mn[8];
    q4k_decode(blk, d, dmin, sc, mn);   // the header has the q4_K layout
    dv[2 * (o * nsb + sb)] = d;
    dv[2 * (o * nsb + sb) + 1] = dmin;
    for (int j = 0; j < 8; ++j) {
        uint32_t L[4];
        for (int u = 0; u < 4; ++u) {
            uint32_t v = 0;
            for (int i = 0; i < 4; ++i)
                v |= (uint32_t)((q5k_quant(blk, 32 * j + 8 * u + i) & 15) |
                                ((q5k_quant(blk, 32 * j + 8 * u + i + 4) & 15) << 4)) << (8 * i);
            L[u] = v;
        }
        uint32_t H = 0;
        for (int g = 0; g < 8; ++g)
            for (int i = 0; i < 4; ++i)
                H |= (uint32_t)(q5k_quant(blk, 32 * j + 4 * g + i) >> 4) << (8 * i + g);
        const int64_t b = sb * 8 + j;
        ql[o * nb + b] = make_uint4(L[0], L[1], L[2], L[3]);
        h5[o * nb + b] = H;
        scv[o * nb + b] = (int16_t)((uint16_t)sc[j] | ((uint16_t)mn[j] << 8));
    }
}

}  // namespace

hipError_t launch_repack_gemm(const uint8_t* raw_dev, const WeightDev& w, hipStream_t s) {
    const int64_t total = w.rows * (w.cols / kSuper);
    const dim3 block(128), grid((unsigned)((total + 127) / 128));
    if (w.type == 12 && w.packed)
        hipLaunchKernelGGL(k_repack_q4k_gemm_packed, grid, block, 0, s, raw_dev, w.rows, w.cols,
                           reinterpret_cast<uint32_t*>(w.wa), w.wsc, w.dmr, w.mfrag);
    else if (w.type == 12)
        hipLaunchKernelGGL(k_repack_q4k_gemm, grid, block, 0, s, raw_dev, w.rows, w.cols, w.wa,
                           w.dmr, w.mfrag);
    else
        hipLaunchKernelGGL(k_repack_q6k_gemm, grid, block, 0, s, raw_dev, w.rows, w.cols, w.wa,
                           w.dmr, w.mfrag);
    return hipGetLastError();
}

hipError_t launch_repack_gemv(const uint8_t* raw_dev, const WeightDev& w, hipStream_t s) {
    const int64_t total = w.rows * (w.cols / kSuper);
    const dim3 block(128), grid((unsigned)((total + 127) / 128));
    if (w.type == 12)
        hipLaunchKernelGGL(k_repack_q4k_gemv, grid, block, 0, s, raw_dev, w.rows, w.cols, w.gv_ql,
                           w.gv_sc, w.gv_d);
    else if (w.type == 13)
        hipLaunchKernelGGL(k_repack_q5k_gemv, grid, block, 0, s, raw_dev, w.rows, w.cols, w.gv_ql,
                           w.gv_h5, w.gv_sc, w.gv_d);
    else
        hipLaunchKernelGGL(k_repack_q6k_gemv, grid, block, 0, s, raw_dev, w.rows, w.cols, w.gv_ql,
                           w.gv_qh, w.gv_sc, w.gv_d);
    return hipGetLastError();
}

}  // namespace mmq
