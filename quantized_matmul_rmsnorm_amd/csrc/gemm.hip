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
// weight values.  For q4_K the weight value sc_j*q_w (<= 945) is folded at
// registration.  For q6_K, v = sc*(q_w-32) needs 13 bits (|v| <= 4096), so
// each wave forms it from the stored code q_w-32 and its f16 sub-scale as two
// exact f16 parts, hi = f16(v) and lo = v - hi (|lo| <= 1), with one packed
// multiply and one packed fma per pair; streaming the code rather than the two
// parts halves the bytes each wave loads per weight.  All operands are exact
// in f16, every product is exact in f32 and every partial sum of one block
// stays below 2^24, so the MFMA returns the exact integer block dot as an f32.
// With the sub-scale inside the operand, the rescale is one FMA per output
// per block (acc += D[t][b] * X), D constant per lane because tokens sit on
// the MFMA's N axis (lane % 32) and outputs on its M axis (registers).  An
// int8 MFMA would return int32 and need a convert, a sub-scale multiply and
// the FMA for every output of every block: three VALU ops against one, on the
// busier of the two arithmetic pipes here.
// Per superblock the sum over its 8 blocks is scaled by d (one FMA per output);
// the q4_K min term sum_j (D*S)[t][j] * m_j is two bf16 MFMAs per superblock
// with m_j exact in bf16 and D*S split exactly into three bf16 parts (bf16
// has f32's exponent range, so no activation scale overflows or underflows).
//
// Tiling.  A workgroup of 8 waves computes 128 outputs x 128 tokens; wave w
// owns output group w%4 (32 rows) and token groups 2*(w/4), 2*(w/4)+1.  Each
// wave streams its own weight fragments (stored in MFMA fragment order at
// registration) straight from L2 into a small register ring a few blocks
// ahead; the activation codes of the tile are staged per 4-block chunk
// through three LDS buffers, converted int8 -> f16 once per workgroup, and each
// block's B fragments are read from LDS one block ahead (the next chunk's
// first block included: one barrier in the middle of each chunk step makes
// that chunk visible, so no step starts by waiting on LDS).  All global reads use
// raw buffer loads with 32-bit offsets; plane rows past the plane's padded
// row count fall outside the buffer and read as zero.  Staging and prefetch
// indices are clamped instead of guarded, so a superblock's two chunks form
// one basic block the scheduler can interleave; each wave raises its priority
// while it issues a block's MFMAs, so the other wave on the SIMD runs its
// rescale FMAs in the gaps.  Outputs are stored
// only for t < n and o < rows.
//
// Packed q4_K tiles (k_gemm_da_packed).  A weight registered with its 4-bit
// codes streams 8 B per lane and block instead of 32 and the wave rebuilds
// the operand in registers: one mask turns two codes into the f16 subnormals
// q * 2^-24 (exact), and one packed multiply by the stored sc_j * 2^10 gives
// sc_j*q * 2^-14 exactly (a normal f16: sc_j*q <= 945).  The MFMAs then
// return each block dot times 2^-14, exactly, and registration stores the
// superblock scale d times 2^14, so every rescale rounds the same value
// scaled by a power of two: both forms return the same bits, as long as a
// superblock's partial sum stays above 2^-112 (it falls below only for block
// scales under about 2e-34).  Workgroups are mapped so that each XCD works
// on a contiguous group of output x token tiles (shared L2).
#include <algorithm>

#include "mmq_internal.h"

namespace mmq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Eight 4-bit codes of one fragment half (code e at bits 4*(e/2) for even e,
// 16 + 4*(e/2) for odd e) -> sc * code * 2^-14 as eight exact f16, given the
// pair s2 = (sc * 2^10, sc * 2^10): each masked code is the f16 subnormal
// code * 2^-24, and the product is exact (at most 945 * 2^-14, at least 2^-14
// when not zero).  This needs f16 denormals kept, the kernels' default mode
// (the build passes no flush or fast-math flag).
__device__ __forceinline__ half8 expand_q4(uint32_t x, half2v s2) {
    half8 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t w = (x >> (4 * k)) & 0x000F000Fu;
        const half2v p = __builtin_bit_cast(half2v, w) * s2;
        h[2 * k] = p[0];
        h[2 * k + 1] = p[1];
    }
    return h;
}

// bf16 bits of x, rounded to nearest even, and the value of such bits
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

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

// Token and output tile of logical tile L: tiles are rastered in groups of
// kGroupO output tiles with the token tile varying slowest inside a group.
__device__ __forceinline__ void raster(int L, int n_ttiles, int n_otiles, int& t_tile,
                                       int& o_tile) {
    const int gsize = kGroupO * n_ttiles;
    const int group = L / gsize, r = L % gsize;
    const int go = min(kGroupO, n_otiles - group * kGroupO);
    o_tile = group * kGroupO + r % go;
    t_tile = r / go;
}

// Hardware places workgroup i on XCD i % 8; give each XCD a contiguous range of
// logical indices so that the workgroups resident on one XCD (and its L2) share
// weight and activation tiles.  A launch covers `count` logical tiles from
// `base`; with a K split the logical index runs split-major, so the workgroups
// of one XCD share a split (its weight and plane columns).
__device__ __forceinline__ void tile_of(int base, int count, int n_ttiles, int n_otiles,
                                        int& t_tile, int& o_tile, int& split, int& local) {
    const int nwg = gridDim.x;
    const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    int L = xcd * per + min(xcd, rem) + li;
    split = L / count;
    local = L - split * count;
    raster(base + local, n_ttiles, n_otiles, t_tile, o_tile);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <typename T>
__device__ __forceinline__ T bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    else if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

struct GemmArgs {
    const half8* wa;      // weight fragments
    const float* dmr;     // per (row group, superblock) scales
    const half8* mfrag;   // q4_K mins (bf16) or q6_K sub-scales (f16)
    const int8_t* q;      // plane codes [plane_rows][id]
    const uint2* ds;      // plane (D, S) pairs [plane_rows][id/32]
    float* out;           // [n][od]
    uint32_t wa_bytes, dmr_bytes, mfrag_bytes, q_bytes, ds_bytes;
    int n, plane_rows, id, od, n_ttiles, n_otiles;
    int sb_per;           // superblocks per K split (all of them without a split)
    int64_t part_stride;  // floats between the partial outputs of two splits
    int tile_base, tile_count;  // logical tiles of this launch
    int compact;          // 1: partials go to part[split][tile][128][128]
};

// The packed q4_K matmul's arguments: the common ones plus the sub-scales.
struct GemmArgsPacked {
    GemmArgs g;
    const uint4* wsc;     // 8 f16 sub-scales per (row, superblock)
    uint32_t wsc_bytes;
};

// The matmul (Q4K: q4_K weights, else q6_K; PACKED: q4_K from 4-bit tiles).
template <bool Q4K, bool PACKED>
__device__ __forceinline__ void gemm_da(const GemmArgs& g, const uint4* wsc, uint32_t wsc_bytes) {
    static_assert(Q4K || !PACKED, "packed tiles are q4_K only");
    constexpr int CH = 4;                   // 32-blocks per staged activation chunk
    constexpr int SBCH = 8 / CH;
    constexpr int NDM = Q4K ? 2 : 1;
    constexpr int RA = 4;                   // weight-fragment ring depth (divides 8)
    constexpr int PD = RA - 1;              // prefetch distance in blocks
    constexpr int BPAD = 2, DPAD = 16;
    constexpr int NBUF = 3;
    constexpr int kBarAt = 1;               // the chunk step's barrier follows block 1
    static_assert(kBarAt < CH - 1, "the next chunk's first read must follow the barrier");
    __shared__ half8 sB[NBUF][CH][4 * 2 * 64 + BPAD];
    __shared__ float sD[NBUF][CH][128 + DPAD];
    // q4_K min term: D*S per (token, block) as three bf16 parts, B fragments of
    // two MFMAs: [hi | mid] and [lo | 0] over the superblock's 8 blocks
    __shared__ __attribute__((aligned(16))) uint16_t sP[Q4K ? 3 : 1][4][2][64][8];
    __shared__ __attribute__((aligned(16))) float sDM[2][kThreads];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ogl = wave & 3;
    const int th = wave >> 2;

    int t_tile, o_tile, split, local;
    tile_of(g.tile_base, g.tile_count, g.n_ttiles, g.n_otiles, t_tile, o_tile, split, local);
    const int t0 = t_tile * 128;
    const int og0 = o_tile * 4;
    const int id = g.id;
    const int nb = id / kBlock;
    const int nsb = id / kSuper;
    const int K16 = id / 16;

    const auto rA = rsrc(g.wa, g.wa_bytes);
    const auto rQ = rsrc(g.q, g.q_bytes);
    const auto rDS = rsrc(g.ds, g.ds_bytes);
    const auto rM = rsrc(g.dmr, g.dmr_bytes);
    const auto rF = rsrc(g.mfrag, g.mfrag_bytes);
    const auto rS = rsrc(wsc, wsc_bytes);

    // this wave's weight fragments: block b, half k16 at voffA + (2b + k16) KiB
    const uint32_t voffA = ((uint32_t)(og0 + ogl) * (uint32_t)K16) * 1024u + (uint32_t)lane * 16u;
    half8 ring[RA][2];
    // packed: block b's 4-bit codes at voffA4 + 512 b
    const uint32_t voffA4 = ((uint32_t)(og0 + ogl) * (uint32_t)nb) * 512u + (uint32_t)lane * 8u;
    uint2 ring4[RA];
    auto load_a = [&](int b, int slot) {
        if constexpr (PACKED) {
            ring4[slot] = bload<uint2>(rA, voffA4, (uint32_t)b * 512u);
        } else {
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16)
                ring[slot][k16] = bload<half8>(rA, voffA + (uint32_t)(k16 * 1024), (uint32_t)b * 2048u);
        }
    };

    const int tb = tid >> 2;
    const int jb = tid & 3;
    const int rowb = t0 + tb;
    const uint32_t rowq = rowb < g.plane_rows ? (uint32_t)rowb * (uint32_t)id : 0x80000000u;
    const uint32_t rowd = rowb < g.plane_rows ? (uint32_t)(rowb * nb + jb) * 8u : 0x80000000u;
    // superblock scales: thread tid stages entry tid % DMN (threads past DMN
    // duplicate an entry into a spare half of sDM, so every thread stores)
    constexpr int DMN = 4 * NDM * 32;
    const int dm_e = tid % DMN;
    const uint32_t dm_off = (uint32_t)(((og0 + dm_e / (NDM * 32)) * nsb) * (NDM * 32 * 4) +
                                       (dm_e % (NDM * 32)) * 4);

    uint4 rb0, rb1;
    float rd, rdm = 0.0f;
    int32_t rs;
    // Chunk c's codes, scales and sums (and, for a superblock's first chunk,
    // the superblock scales) into registers.  c is clamped by the caller, so
    // the loop body has no branch; a clamped repeat is never consumed.
    auto load_chunk = [&](int c, bool first) {
        const uint32_t sq = (uint32_t)(c * CH) * 32u;
        rb0 = bload<uint4>(rQ, rowq + (uint32_t)jb * 32u, sq);
        rb1 = bload<uint4>(rQ, rowq + (uint32_t)jb * 32u + 16u, sq);
        if constexpr (Q4K) {   // D and S in one load
            const uint2 v = bload<uint2>(rDS, rowd, (uint32_t)(c * CH) * 8u);
            rd = __uint_as_float(v.x);
            rs = (int32_t)v.y;
        } else {
            rd = bload<float>(rDS, rowd, (uint32_t)(c * CH) * 8u);
            rs = 0;
        }
        if (first) rdm = bload<float>(rM, dm_off, (uint32_t)((c / SBCH) * (NDM * 32 * 4)));
    };
    // real == false: a clamped repeat of the last chunk; its min-term operands
    // go to a spare slot of sP (the codes land in the idle sB buffer).
    auto store_chunk = [&](int c, int buf, bool first, bool real) {
        const int tg = tb >> 5, tl = tb & 31;
        half8* sbp = &sB[buf][jb][tg * 128];
        sbp[tl] = i8x8_to_f16(rb0.x, rb0.y);
        sbp[tl + 32] = i8x8_to_f16(rb0.z, rb0.w);
        sbp[64 + tl] = i8x8_to_f16(rb1.x, rb1.y);
        sbp[64 + tl + 32] = i8x8_to_f16(rb1.z, rb1.w);
        const int b = c * CH + jb;
        sD[buf][jb][tb] = rd;
        if (Q4K) {
            // P = hi + mid + lo exactly (three 8-bit significands hold the
            // 24 of an f32, and bf16 keeps f32's exponent range)
            const float P = rd * (float)rs;
            const uint16_t hi = bf16_bits(P);
            const float r1 = P - bf16_value(hi);
            const uint16_t mid = bf16_bits(r1);
            const uint16_t lo = bf16_bits(r1 - bf16_value(mid));
            const int slot = real ? ((b >> 3) & 1) : 2;
            sP[slot][tg][0][tl][b & 7] = hi;
            sP[slot][tg][0][tl + 32][b & 7] = mid;
            sP[slot][tg][1][tl][b & 7] = lo;
        }
        if (first) sDM[(c / SBCH) & 1][tid] = rdm;
    };

    // q6_K: this lane's row's 16 sub-scales of the current superblock as f16
    // pairs (sc[2j], sc[2j+1]) for block j, and those of the next superblock
    uint32_t scv[8], scn[8];
    auto load_sc = [&](int sbx, uint32_t* dst) {
        const uint32_t off = (uint32_t)((((og0 + ogl) * nsb + sbx) * 32 + (lane & 31)) * 32);
        const uint4 a = bload<uint4>(rF, off, 0u);
        const uint4 b = bload<uint4>(rF, off + 16u, 0u);
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
        dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
    };
    // packed q4_K: this lane's row's 8 sub-scales of superblock sbx, times
    // 2^10, as f16 pairs (sc[2j], sc[2j+1]) in dst[0..3]
    auto load_sc4 = [&](int sbx, uint32_t* dst) {
        const uint32_t off = (uint32_t)((((og0 + ogl) * nsb + sbx) * 32 + (lane & 31)) * 16);
        const uint4 a = bload<uint4>(rS, off, 0u);
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    };
    f32x16 acc[2], res[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[i][r] = 0.0f;

    // this workgroup's K range: superblocks [sb0, sb1), blocks [8*sb0, b_end),
    // chunks [c0, c_end); every split has at least one superblock
    const int sb0 = split * g.sb_per;
    const int sb1 = min(nsb, sb0 + g.sb_per);
    const int b_end = sb1 * 8;
    const int c0 = sb0 * SBCH, c_end = sb1 * SBCH;
#pragma unroll
    for (int b = 0; b < PD; ++b) load_a(8 * sb0 + b, b);   // 8 blocks per split > PD; slot b % RA
    if (!Q4K) {
        load_sc(sb0, scv);
        load_sc(min(sb0 + 1, sb1 - 1), scn);
    }
    if (PACKED) {
        load_sc4(sb0, scv);
        load_sc4(min(sb0 + 1, sb1 - 1), scn);
    }
    if (Q4K) {   // the zero half of the [lo | 0] fragments, never written again
        for (int e = tid; e < 3 * 4 * 32 * 8; e += kThreads)
            sP[e >> 10][(e >> 8) & 3][1][32 + ((e >> 3) & 31)][e & 7] = 0;
    }
    load_chunk(c0, true);
    store_chunk(c0, 0, true, true);
    load_chunk(c0 + 1, false);
    __syncthreads();

    half8 bfr[2][2][2];   // B fragments [ring][t group][k16], one block ahead
    auto read_b = [&](int bufi, int jj, half8 (*dst)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16)
                dst[i][k16] = sB[bufi][jj][((2 * th + i) * 2 + k16) * 64 + lane];
    };
    read_b(0, 0, bfr[0]);
    // three staging buffers: chunk c lives in buffer (c - c0) % 3.  Chunk c+1
    // is stored at the start of chunk c's step and one barrier follows in its
    // middle, so the first B fragments of chunk c+1 can be read before the
    // step ends, and the store of chunk c+2 never meets a read of chunk c-1.
    int bcur = 0;
    for (int sb = sb0; sb < sb1; ++sb) {
#pragma unroll
        for (int cc = 0; cc < SBCH; ++cc) {
            const int c = sb * SBCH + cc;
            const int bnext = bcur == NBUF - 1 ? 0 : bcur + 1;
            // stage chunk c+1 (loaded one chunk ago), load chunk c+2
            store_chunk(min(c + 1, c_end - 1), bnext, (cc + 1) % SBCH == 0, c + 1 < c_end);
            load_chunk(min(c + 2, c_end - 1), cc % SBCH == 0);
            bf16x8 mf;
            if (Q4K && cc == SBCH - 1)
                mf = bload<bf16x8>(rF, (uint32_t)((((og0 + ogl) * nsb + sb) * 64 + lane) * 16), 0u);
            f32x16 X[2][2];
            auto mfma_block = [&](int j, int slot, half8 (*bf)[2], f32x16* Xo) {
                if constexpr (Q4K) {
                    half8 A[2];
                    if constexpr (PACKED) {
                        const uint32_t sp = scv[j >> 1];
                        const half2v s2 = __builtin_bit_cast(
                            half2v, __builtin_amdgcn_perm(sp, sp, (j & 1) ? 0x03020302u : 0x01000100u));
                        A[0] = expand_q4(ring4[slot].x, s2);
                        A[1] = expand_q4(ring4[slot].y, s2);
                    } else {
                        A[0] = ring[slot][0];
                        A[1] = ring[slot][1];
                    }
#pragma unroll
                    for (int k16 = 0; k16 < 2; ++k16) {
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            if (k16 == 0) {
                                const f32x16 zero = {};
                                Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[0], bf[i][0], zero, 0, 0, 0);
                            } else {
                                Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[1], bf[i][1], Xo[i], 0, 0, 0);
                            }
                        }
                    }
                } else {
                    // A = sc * c split exactly into hi = f16(sc * c) and
                    // lo = sc * c - hi (|lo| <= 1): both are exact f16 integers
                    const uint32_t sp = scv[j];
                    const half2v s2[2] = {__builtin_bit_cast(half2v, __builtin_amdgcn_perm(sp, sp, 0x01000100u)),
                                          __builtin_bit_cast(half2v, __builtin_amdgcn_perm(sp, sp, 0x03020302u))};
#pragma unroll
                    for (int k16 = 0; k16 < 2; ++k16) {
                        const half8 c = ring[slot][k16];
                        half8 hi, lo;
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const half2v cp = {c[2 * p], c[2 * p + 1]};
                            const half2v h = cp * s2[k16];
                            const half2v l = __builtin_elementwise_fma(cp, s2[k16], -h);
                            hi[2 * p] = h[0]; hi[2 * p + 1] = h[1];
                            lo[2 * p] = l[0]; lo[2 * p + 1] = l[1];
                        }
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            if (k16 == 0) {
                                const f32x16 zero = {};
                                Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hi, bf[i][0], zero, 0, 0, 0);
                            } else {
                                Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hi, bf[i][1], Xo[i], 0, 0, 0);
                            }
                            Xo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(lo, bf[i][k16], Xo[i], 0, 0, 0);
                        }
                    }
                }
            };
            float dav[CH][2];
#pragma unroll
            for (int jj = 0; jj < CH; ++jj)
#pragma unroll
                for (int i = 0; i < 2; ++i) dav[jj][i] = sD[bcur][jj][(2 * th + i) * 32 + (lane & 31)];
            auto epilogue_block = [&](int jj, const f32x16* Xi) {
                const int j = cc * CH + jj;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float da = dav[jj][i];
                    if (j == 0) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[i][r] = da * Xi[i][r];
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(da, Xi[i][r], acc[i][r]);
                    }
                }
            };
#pragma unroll
            for (int jj = 0; jj < CH; ++jj) {
                const int j = cc * CH + jj;            // block within the superblock
                const int b = sb * 8 + j;
                load_a(min(b + PD, b_end - 1), (j + PD) % RA);   // clamped: no branch, in bounds
                if (jj + 1 < CH) read_b(bcur, jj + 1, bfr[(jj + 1) & 1]);
                else read_b(bnext, 0, bfr[0]);         // next chunk: stored at this step's start, past the barrier
                __builtin_amdgcn_s_setprio(1);   // wave priority only (not a queue priority)
                mfma_block(j, j % RA, bfr[jj & 1], X[jj & 1]);
                __builtin_amdgcn_s_setprio(0);
                if (jj > 0) epilogue_block(jj - 1, X[(jj - 1) & 1]);
                if (jj == kBarAt) __syncthreads();
            }
            epilogue_block(CH - 1, X[(CH - 1) & 1]);

            if (cc == SBCH - 1) {
                const int half = lane >> 5;
                const float* dmv = &sDM[sb & 1][ogl * (NDM * 32) + half * 16];
                if (Q4K) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const bf16x8 p0 = *reinterpret_cast<const bf16x8*>(&sP[sb & 1][2 * th + i][0][lane][0]);
                        const bf16x8 p1 = *reinterpret_cast<const bf16x8*>(&sP[sb & 1][2 * th + i][1][lane][0]);
                        const f32x16 zero = {};
                        f32x16 mn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mf, p0, zero, 0, 0, 0);
                        mn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mf, p1, mn, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float v = fmaf(dmv[r], acc[i][r], res[i][r]);
                            res[i][r] = fmaf(-dmv[32 + r], mn[r], v);
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) res[i][r] = fmaf(dmv[r], acc[i][r], res[i][r]);
                }
            }
            bcur = bnext;
        }
        if (!Q4K) {
#pragma unroll
            for (int i = 0; i < 8; ++i) scv[i] = scn[i];
            load_sc(min(sb + 2, sb1 - 1), scn);
        }
        if (PACKED) {
#pragma unroll
            for (int i = 0; i < 4; ++i) scv[i] = scn[i];
            load_sc4(min(sb + 2, sb1 - 1), scn);
        }
    }

    const int od = g.od;
    if (g.compact) {
        // the whole 128 x 128 tile, bounds applied by the tile reduce
        float* tp = g.out + ((int64_t)split * g.tile_count + local) * (128 * 128);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float* row = tp + ((2 * th + i) * 32 + (lane & 31)) * 128;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(row + ogl * 32 + 8 * q + 4 * (lane >> 5)) =
                    make_float4(res[i][4 * q], res[i][4 * q + 1], res[i][4 * q + 2], res[i][4 * q + 3]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = t0 + (2 * th + i) * 32 + (lane & 31);
        if (t >= g.n) continue;
        float* orow = g.out + split * g.part_stride + t * (int64_t)od;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t o = (int64_t)(og0 + ogl) * 32 + 8 * q + 4 * (lane >> 5);
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

template <bool Q4K>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_da(const GemmArgs g) {
    gemm_da<Q4K, false>(g, nullptr, 0u);
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_da_packed(const GemmArgsPacked p) {
    gemm_da<true, true>(p.g, p.wsc, p.wsc_bytes);
}

// Sum of the K-split partials in split order (deterministic): out[i] =
// part[0][i] + part[1][i] + ...
// Partial k starts at part + k * pstride (pstride a multiple of 64 floats).
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part,
                                                      float* __restrict__ out, int splits,
                                                      int64_t count, int64_t pstride) {
    const int64_t n4 = count / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 acc = reinterpret_cast<const float4*>(part)[i];
        for (int k = 1; k < splits; ++k) {
            const float4 v = reinterpret_cast<const float4*>(part + k * pstride)[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        reinterpret_cast<float4*>(out)[i] = acc;
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        float acc = part[i];
        for (int k = 1; k < splits; ++k) acc += part[k * pstride + i];
        out[i] = acc;
    }
}

// Sum of the compact partial tiles of the tail launch: out for tile `local`
// of the logical range [base, base + count) = sum over splits, in order.
// 16 workgroups per tile, 8 rows of 128 each (one float4 per thread).
__global__ __launch_bounds__(256) void k_tile_reduce(const float* __restrict__ part,
                                                     float* __restrict__ out, int splits,
                                                     int count, int base, int n_ttiles,
                                                     int n_otiles, int n, int od) {
    const int local = blockIdx.x >> 4, chunk = blockIdx.x & 15;
    int t_tile, o_tile;
    raster(base + local, n_ttiles, n_otiles, t_tile, o_tile);
    const int tt = chunk * 8 + (threadIdx.x >> 5);
    const int oo = (threadIdx.x & 31) * 4;
    const float* p = part + (int64_t)local * (128 * 128) + tt * 128 + oo;
    float4 acc = *reinterpret_cast<const float4*>(p);
    for (int k = 1; k < splits; ++k) {
        const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)k * count * (128 * 128));
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const int64_t t = (int64_t)t_tile * 128 + tt;
    const int64_t o = (int64_t)o_tile * 128 + oo;
    if (t >= n) return;
    float* orow = out + t * (int64_t)od;
    if (o + 3 < od && (od & 3) == 0) {
        *reinterpret_cast<float4*>(orow + o) = acc;
    } else {
        const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
        for (int e = 0; e < 4; ++e)
            if (o + e < od) orow[o + e] = a4[e];
    }
}

}  // namespace

// K splits for a matmul of n tokens: only when the output tiles fill less
// than one round of the chip, and then the count that minimises rounds per
// split (each split keeps at least 4 superblocks).
int gemm_splits(int64_t rows_pad, int64_t cols, int64_t n, int n_cu) {
    const int64_t tiles = ((n + 127) / 128) * (rows_pad / 128);
    if (n_cu <= 0 || tiles >= n_cu) return 1;
    const int64_t nsb = cols / kSuper;
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(64, nsb / 4));
    int best = 1;
    double best_cost = (double)((tiles + n_cu - 1) / n_cu);
    for (int64_t sp = 2; sp <= smax; ++sp) {
        const int64_t per = (nsb + sp - 1) / sp;
        const int64_t real = (nsb + per - 1) / per;
        const double cost = (double)((tiles * real + n_cu - 1) / n_cu) / (double)real;
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = (int)real;
        }
    }
    return best;
}

int64_t gemm_part_stride(int64_t n, int64_t rows) { return (n * rows + 63) / 64 * 64; }

// How a matmul is launched on n_cu compute units:
//  * few output tiles: K split across all of them (gemm_splits);
//  * many tiles whose last round would be nearly empty (under 1/8 full): the
//    full rounds run unsplit and the leftover tiles run K-split into compact
//    partial tiles that a tile reduce sums -- the leftover tiles then take a
//    fraction of a round instead of a whole one.
GemmPlan gemm_plan(const WeightDev& w, int64_t n, int n_cu) {
    GemmPlan p;
    const int64_t nsb = w.cols / kSuper;
    const int64_t tiles = ((n + 127) / 128) * (w.rows_pad / 128);
    p.splits = gemm_splits(w.rows_pad, w.cols, n, n_cu);
    if (p.splits > 1) {
        const int64_t per = (nsb + p.splits - 1) / p.splits;
        p.splits = (int)((nsb + per - 1) / per);
        p.part_floats = p.splits * gemm_part_stride(n, w.rows);
        return p;
    }
    const int64_t tail = n_cu > 0 ? tiles % n_cu : 0;
    if (n_cu > 0 && tiles > n_cu && tail > 0 && tail * 8 <= n_cu && nsb >= 2) {
        int64_t ts = std::min<int64_t>(nsb, std::max<int64_t>(2, n_cu / tail));
        const int64_t per = (nsb + ts - 1) / ts;
        ts = (nsb + per - 1) / per;
        if (ts >= 2) {
            p.tail_tiles = (int)tail;
            p.tail_splits = (int)ts;
            p.part_floats = ts * tail * 128 * 128;
        }
    }
    return p;
}

hipError_t launch_gemm(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                       float* part, const GemmPlan& plan, hipStream_t s) {
    GemmArgs a;
    a.wa = (const half8*)w.wa;
    a.dmr = w.dmr;
    a.mfrag = (const half8*)w.mfrag;
    a.q = pl.q;
    a.ds = pl.ds;
    const int64_t nsb = w.cols / kSuper, og = w.rows_pad / 32;
    a.wa_bytes = (uint32_t)(w.packed ? w.rows_pad * w.cols / 2 : w.rows_pad * w.cols * 2);
    a.dmr_bytes = (uint32_t)(og * nsb * (w.type == 12 ? 64 : 32) * 4);
    a.mfrag_bytes = (uint32_t)(og * nsb * (w.type == 12 ? 512 * 2 : 32 * 16 * 2));
    a.q_bytes = (uint32_t)(pl.rows * pl.d);
    a.ds_bytes = (uint32_t)(pl.rows * (pl.d / kBlock) * 8);
    a.n = (int)n;
    a.plane_rows = (int)pl.rows;
    a.id = (int)w.cols;
    a.od = (int)w.rows;
    a.n_ttiles = (int)((n + 127) / 128);
    a.n_otiles = (int)(w.rows_pad / 128);
    const int tiles = a.n_ttiles * a.n_otiles;
    auto go = [&](unsigned grid) {
        if (w.type == 12 && w.packed) {
            GemmArgsPacked ap;
            ap.g = a;
            ap.wsc = w.wsc;
            ap.wsc_bytes = (uint32_t)(w.rows_pad * nsb * 16);
            hipLaunchKernelGGL(k_gemm_da_packed, dim3(grid), dim3(kThreads), 0, s, ap);
        }
        else if (w.type == 12)
            hipLaunchKernelGGL((k_gemm_da<true>), dim3(grid), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((k_gemm_da<false>), dim3(grid), dim3(kThreads), 0, s, a);
    };
    const int splits = part != nullptr ? plan.splits : 1;
    if (splits > 1) {
        a.sb_per = (int)((nsb + splits - 1) / splits);
        a.out = part;
        a.part_stride = gemm_part_stride(n, w.rows);
        a.tile_base = 0;
        a.tile_count = tiles;
        a.compact = 0;
        go((unsigned)(tiles * splits));
        const int64_t count = n * w.rows;
        const int64_t want = (count / 4 + 255) / 256;
        const dim3 rg((unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 4096)));
        hipLaunchKernelGGL(k_split_reduce, rg, dim3(256), 0, s, part, out, splits, count,
                           a.part_stride);
        return hipGetLastError();
    }
    const int tail = part != nullptr ? plan.tail_tiles : 0;
    a.sb_per = (int)nsb;
    a.out = out;
    a.part_stride = 0;
    a.tile_base = 0;
    a.tile_count = tiles - tail;
    a.compact = 0;
    go((unsigned)(tiles - tail));
    if (tail > 0) {
        const int ts = plan.tail_splits;
        a.sb_per = (int)((nsb + ts - 1) / ts);
        a.out = part;
        a.tile_base = tiles - tail;
        a.tile_count = tail;
        a.compact = 1;
        go((unsigned)(tail * ts));
        hipLaunchKernelGGL(k_tile_reduce, dim3((unsigned)(tail * 16)), dim3(256), 0, s, part, out,
                           ts, tail, tiles - tail, a.n_ttiles, a.n_otiles, a.n, a.od);
    }
    return hipGetLastError();
}

}  // namespace mmq
