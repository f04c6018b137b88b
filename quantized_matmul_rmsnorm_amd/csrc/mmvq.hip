// mmvq.hip -- one-token q6_K / q4_K / q5_K GEMV over a q8 activation plane, and
// the q6_K GEMV on an f32 activation for small shapes (gfx950).
//
// Method ("72 · D3-7 ...", section 2 and Excerpts A, A2, B): at one token the
// matmul is a weight-streaming GEMV; the activation is quantised once into a
// q8 plane (shared through the plane cache by every consumer of the same
// buffer) and each output row is an integer dot of that plane with the row's
// packed weights, rescaled per block.  Each K-quant type has its own
// one-token arm:
//   q6_K: per 32-block, D * d * (sc0*I0 + sc1*I1), I0/I1 the dots of the
//         16-value halves of (q_w - 32) with the codes;
//   q4_K: per 32-block j of a superblock, D * (d*sc_j * I - dmin*m_j * S),
//         I = sum(q_w * q), S the plane's code sum of the block;
//   q5_K: the q4_K term with 5-bit codes q_w (the low nibble plus a fifth
//         bit stored apart; Excerpt B's q5_K arm).
//
// Design for CDNA4.  The kernel is bound by streaming the packed weights from
// HBM, so the weights are read exactly once, with non-temporal loads, in
// 1 KiB-per-wave coalesced pieces, and the integer work runs on
// v_dot4_i32_i8 (4 int8 products per instruction).  A wave takes one output
// row at a time -- lane l owns 32-blocks l, l+64, ... -- and issues all of the
// row's weight loads before it computes; per block the lane reads the block's
// packed codes (16 B of 4-bit codes, plus 8 B of high bit pairs for q6_K) and
// its scales (the registration layout of repack.hip), rebuilds packed bytes
// with masks and shifts and dots them with the plane's codes.  For q6_K the
// "- 32" of the code is applied through the activation: the dot accumulator
// starts at -32 * sum(q) of the half.  One f32 expression per block adds the
// block's term; a wave-wide sum per row finishes the output.  For rows of up
// to 768 blocks the plane is staged once per workgroup of 4 waves in LDS
// (40 B per block, the half sums included), while the waves' first rows are
// already streaming in; longer rows re-read the plane (from L2) once per pair
// of rows.
#include <algorithm>
#include <atomic>

#include "mmq_internal.h"

namespace mmq {
namespace {

// Raise a kernel's dynamic-LDS limit once on each device that launches it
// (the attribute is set with the device current; `done` holds one bit per
// device index).
template <class K>
void lds_limit_once(K kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return;
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    done.fetch_or(bit);
}

// Workgroups of `kernel` resident on the current device at once (per CU
// times CUs); a failed query counts one per CU and leaves no error behind.
// Call sites keep the result in a function-local static, whose
// initialisation C++ makes thread-safe.
template <class K>
int64_t resident_workgroups(K kernel, int threads, size_t lds) {
    int dev = 0, n_cu = 0, blk = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blk, kernel, threads, lds) != hipSuccess) {
        (void)hipGetLastError();
        blk = 1;
    }
    return (int64_t)(blk > 0 ? blk : 1) * (n_cu > 0 ? n_cu : 256);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 nt_load(const uint4* p) {
    const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 nt_load(const uint2* p) {
    const u2v v = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(p));
    return make_uint2(v.x, v.y);
}

struct MvArgs {
    const uint4* ql;      // [od][nb] packed 4-bit codes
    const uint2* qh;      // q6_K: [od][nb] high bit pairs
    const uint32_t* h5;   // q5_K: [od][nb] fifth bits
    const int16_t* sc;    // [od][nb] scales
    const float* dv;      // q6_K: [od][nsb] d; q4_K: [od][nsb][2] d, dmin
    const int8_t* Q;      // plane codes (row 0)
    const uint2* ds;      // plane (D, S) pairs
    int id, od;
    float* out;
};

// ---- q6_K arm ----
struct Q6 {
    struct Act {
        uint4 q0, q1;   // codes 0..15, 16..31
        float D;
        int c0, c1;     // -32 * sum of codes in each half
    };
    struct W {
        uint4 L;
        uint2 H;
        int16_t s;
        float d;
    };
    static __device__ __forceinline__ Act act(const MvArgs& g, int b) {
        Act a;
        const uint4* p = reinterpret_cast<const uint4*>(g.Q + (int64_t)b * kBlock);
        a.q0 = p[0];
        a.q1 = p[1];
        a.D = __uint_as_float(g.ds[b].x);
        const uint32_t ones = 0x01010101u;
        int s0 = dot4(a.q0.x, ones, 0); s0 = dot4(a.q0.y, ones, s0);
        s0 = dot4(a.q0.z, ones, s0);    s0 = dot4(a.q0.w, ones, s0);
        int s1 = dot4(a.q1.x, ones, 0); s1 = dot4(a.q1.y, ones, s1);
        s1 = dot4(a.q1.z, ones, s1);    s1 = dot4(a.q1.w, ones, s1);
        a.c0 = -32 * s0;
        a.c1 = -32 * s1;
        return a;
    }
    static __device__ __forceinline__ W load(const MvArgs& g, int64_t o, int b, int nb, int nsb) {
        W w;
        const int64_t i = o * nb + b;
        w.L = nt_load(g.ql + i);
        w.H = nt_load(g.qh + i);
        w.s = __builtin_nontemporal_load(g.sc + i);
        w.d = __builtin_nontemporal_load(g.dv + o * nsb + (b >> 3));
        return w;
    }
    static __device__ __forceinline__ float term(const Act& a, const W& w) {
        const uint32_t m4 = 0x0F0F0F0Fu, m2 = 0x30303030u;
        const uint4 L = w.L;
        const uint2 H = w.H;
        int i0 = a.c0;
        i0 = dot4((L.x & m4) | ((H.x << 4) & m2), a.q0.x, i0);
        i0 = dot4(((L.x >> 4) & m4) | ((H.x << 2) & m2), a.q0.y, i0);
        i0 = dot4((L.y & m4) | (H.x & m2), a.q0.z, i0);
        i0 = dot4(((L.y >> 4) & m4) | ((H.x >> 2) & m2), a.q0.w, i0);
        int i1 = a.c1;
        i1 = dot4((L.z & m4) | ((H.y << 4) & m2), a.q1.x, i1);
        i1 = dot4(((L.z >> 4) & m4) | ((H.y << 2) & m2), a.q1.y, i1);
        i1 = dot4((L.w & m4) | (H.y & m2), a.q1.z, i1);
        i1 = dot4(((L.w >> 4) & m4) | ((H.y >> 2) & m2), a.q1.w, i1);
        const int s0 = (int)(int8_t)(w.s & 0xFF);
        const int s1 = (int)(int8_t)((uint16_t)w.s >> 8);
        const int ic = s0 * i0 + s1 * i1;
        return (a.D * w.d) * (float)ic;
    }
};

// ---- q4_K arm ----
struct Q4 {
    struct Act {
        uint4 q0, q1;
        float D;
        int S;          // the plane's code sum of the block
    };
    struct W {
        uint4 L;
        int16_t s;      // sc | m << 8
        f2v dd;         // d, dmin
    };
    static __device__ __forceinline__ Act act(const MvArgs& g, int b) {
        Act a;
        const uint4* p = reinterpret_cast<const uint4*>(g.Q + (int64_t)b * kBlock);
        a.q0 = p[0];
        a.q1 = p[1];
        const uint2 v = g.ds[b];
        a.D = __uint_as_float(v.x);
        a.S = (int)v.y;
        return a;
    }
    static __device__ __forceinline__ W load(const MvArgs& g, int64_t o, int b, int nb, int nsb) {
        W w;
        const int64_t i = o * nb + b;
        w.L = nt_load(g.ql + i);
        w.s = __builtin_nontemporal_load(g.sc + i);
        w.dd = __builtin_nontemporal_load(reinterpret_cast<const f2v*>(g.dv) + o * nsb + (b >> 3));
        return w;
    }
    static __device__ __forceinline__ float term(const Act& a, const W& w) {
        const uint32_t m4 = 0x0F0F0F0Fu;
        const uint4 L = w.L;
        int i = dot4(L.x & m4, a.q0.x, 0);
        i = dot4((L.x >> 4) & m4, a.q0.y, i);
        i = dot4(L.y & m4, a.q0.z, i);
        i = dot4((L.y >> 4) & m4, a.q0.w, i);
        i = dot4(L.z & m4, a.q1.x, i);
        i = dot4((L.z >> 4) & m4, a.q1.y, i);
        i = dot4(L.w & m4, a.q1.z, i);
        i = dot4((L.w >> 4) & m4, a.q1.w, i);
        const float sc = (float)(w.s & 0xFF);
        const float mn = (float)(((uint16_t)w.s >> 8) & 0xFF);
        return a.D * ((w.dd.x * sc) * (float)i - (w.dd.y * mn) * (float)a.S);
    }
};

// ---- q5_K arm: the q4_K block term with a fifth code bit ----
struct Q5 {
    using Act = Q4::Act;
    struct W {
        uint4 L;
        uint32_t h;     // bit 8*i + g: fifth bit of the i-th weight of nibble group g
        int16_t s;      // sc | m << 8
        f2v dd;         // d, dmin
    };
    static __device__ __forceinline__ Act act(const MvArgs& g, int b) { return Q4::act(g, b); }
    static __device__ __forceinline__ W load(const MvArgs& g, int64_t o, int b, int nb, int nsb) {
        W w;
        const int64_t i = o * nb + b;
        w.L = nt_load(g.ql + i);
        w.h = __builtin_nontemporal_load(g.h5 + i);
        w.s = __builtin_nontemporal_load(g.sc + i);
        w.dd = __builtin_nontemporal_load(reinterpret_cast<const f2v*>(g.dv) + o * nsb + (b >> 3));
        return w;
    }
    static __device__ __forceinline__ float term(const Act& a, const W& w) {
        const uint32_t m4 = 0x0F0F0F0Fu, m5 = 0x10101010u;
        const uint4 L = w.L;
        const uint32_t h = w.h;
        // nibble group g takes bit g of each byte of h into bit 4
        int i = dot4((L.x & m4) | ((h << 4) & m5), a.q0.x, 0);
        i = dot4(((L.x >> 4) & m4) | ((h << 3) & m5), a.q0.y, i);
        i = dot4((L.y & m4) | ((h << 2) & m5), a.q0.z, i);
        i = dot4(((L.y >> 4) & m4) | ((h << 1) & m5), a.q0.w, i);
        i = dot4((L.z & m4) | (h & m5), a.q1.x, i);
        i = dot4(((L.z >> 4) & m4) | ((h >> 1) & m5), a.q1.y, i);
        i = dot4((L.w & m4) | ((h >> 2) & m5), a.q1.z, i);
        i = dot4(((L.w >> 4) & m4) | ((h >> 3) & m5), a.q1.w, i);
        const float sc = (float)(w.s & 0xFF);
        const float mn = (float)(((uint16_t)w.s >> 8) & 0xFF);
        return a.D * ((w.dd.x * sc) * (float)i - (w.dd.y * mn) * (float)a.S);
    }
};

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes: four DPP steps inside each row of 16 lanes
// (quad xor-1, quad xor-2, half-row mirror, row mirror), then two lane swaps.
__device__ __forceinline__ float wave_sum(float v) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    v += dppf<0x140>(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// Rows longer than 768 blocks: each wave walks pairs of rows grid-stride and
// re-reads its blocks of the plane (from L2) once per pair, so each read
// serves both rows.
template <class F>
__global__ __launch_bounds__(256) void k_mmvq_long(const MvArgs g) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int id = g.id, od = g.od;
    const int nb = id / kBlock;
    const int nsb = id / kSuper;
    const int rounds = (nb + 63) / 64;
    for (int o = wave; o < od; o += 2 * nwaves) {
        const int o2 = o + nwaves;
        float acc = 0.0f, acc2 = 0.0f;
        for (int r = 0; r < rounds; ++r) {
            const int b = 64 * r + lane;
            if (b < nb) {
                const typename F::Act a = F::act(g, b);
                acc += F::term(a, F::load(g, o, b, nb, nsb));
                if (o2 < od) acc2 += F::term(a, F::load(g, o2, b, nb, nsb));
            }
        }
        acc = wave_sum(acc);
        acc2 = wave_sum(acc2);
        if (lane == 0) {
            g.out[o] = acc;
            if (o2 < od) g.out[o2] = acc2;
        }
    }
}

// Workgroups of the long-row form: a wave per pair of rows while they fit in
// two rounds of resident waves, else exactly the resident waves.
template <class F>
int64_t mmvq_long_grid(int64_t rows) {
    static const int64_t resident = resident_workgroups(k_mmvq_long<F>, 256, 0);
    const int64_t want = (rows + 7) / 8;
    return want <= 2 * resident ? want : resident;
}

// ---- a few tokens at once (2 <= n <= 16, in passes of up to 8) ----
// One 32-block of one token, as staged in LDS (40 bytes, two arrays): the
// codes, then D and a sum word (q6_K: the two 16-value half sums as int16;
// q4_K: the block's code sum S).
struct ActRec {
    uint4 q0, q1;
    float D;
    int aux;
};
constexpr int kRecBytes = 32 + 8;

__device__ __forceinline__ Q6::Act to_act(const ActRec& r, Q6*) {
    Q6::Act a;
    a.q0 = r.q0; a.q1 = r.q1; a.D = r.D;
    a.c0 = -32 * (int)(int16_t)(r.aux & 0xFFFF);
    a.c1 = -32 * (r.aux >> 16);
    return a;
}
__device__ __forceinline__ Q4::Act to_act(const ActRec& r, Q4*) {
    Q4::Act a;
    a.q0 = r.q0; a.q1 = r.q1; a.D = r.D; a.S = r.aux;
    return a;
}

// Workgroups of 8 or 16 waves share the NT tokens' plane (tokens t0 ..
// t0+NT-1, missing tokens as zeros) staged once in LDS; each wave walks groups
// of R rows grid-stride, loads a block of the R rows per round (the next
// round's loads in flight) and applies it to all NT tokens.  out is [n][od].
template <class F, int NT, int R>
__global__ __launch_bounds__(1024) void k_mmvqn(const MvArgs g, int n, int t0) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    uint4* lds_q = reinterpret_cast<uint4*>(lds_raw);                      // [NT*nb][2]
    int2* lds_m = reinterpret_cast<int2*>(lds_raw + (size_t)NT * (g.id / kBlock) * 32);  // [NT*nb]
    const int lane = threadIdx.x & 63;
    const int wpb = blockDim.x >> 6;
    const int wave = blockIdx.x * wpb + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * wpb;
    const int id = g.id, od = g.od;
    const int nb = id / kBlock;
    const int nsb = id / kSuper;
    const int64_t plane_row = (int64_t)id;            // codes per plane row
    for (int rec = threadIdx.x; rec < NT * nb; rec += blockDim.x) {
        const int t = rec / nb, b = rec - t * nb;
        ActRec r;
        if (t0 + t < n) {
            const int8_t* qrow = g.Q + (int64_t)(t0 + t) * plane_row;
            const uint4* p = reinterpret_cast<const uint4*>(qrow + (int64_t)b * kBlock);
            r.q0 = p[0];
            r.q1 = p[1];
            const uint2 v = g.ds[(int64_t)(t0 + t) * nb + b];
            r.D = __uint_as_float(v.x);
            if constexpr (sizeof(typename F::Act) == sizeof(Q6::Act) &&
                          __is_same(F, Q6)) {
                const uint32_t ones = 0x01010101u;
                int s0 = dot4(r.q0.x, ones, 0); s0 = dot4(r.q0.y, ones, s0);
                s0 = dot4(r.q0.z, ones, s0);    s0 = dot4(r.q0.w, ones, s0);
                int s1 = dot4(r.q1.x, ones, 0); s1 = dot4(r.q1.y, ones, s1);
                s1 = dot4(r.q1.z, ones, s1);    s1 = dot4(r.q1.w, ones, s1);
                r.aux = (int)((uint32_t)(s0 & 0xFFFF) | ((uint32_t)s1 << 16));
            } else {
                r.aux = (int)v.y;
            }
        } else {
            r.q0 = make_uint4(0, 0, 0, 0);
            r.q1 = r.q0;
            r.D = 0.0f;
            r.aux = 0;
        }
        lds_q[2 * rec] = r.q0;
        lds_q[2 * rec + 1] = r.q1;
        lds_m[rec] = make_int2(__float_as_int(r.D), r.aux);
    }
    __syncthreads();

    const int rounds = (nb + 63) / 64;
    const int groups = (od + R - 1) / R;
    for (int grp = wave; grp < groups; grp += nwaves) {
        const int o0 = grp * R;
        float acc[R][NT];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[i][t] = 0.0f;
        typename F::W cur[R], nxt[R];
        auto load_round = [&](int r, typename F::W* dst) {
            const int b = 64 * r + lane;
            if (b < nb) {
#pragma unroll
                for (int i = 0; i < R; ++i)
                    if (o0 + i < od) dst[i] = F::load(g, o0 + i, b, nb, nsb);
            }
        };
        load_round(0, cur);
        for (int r = 0; r < rounds; ++r) {
            if (r + 1 < rounds) load_round(r + 1, nxt);
            const int b = 64 * r + lane;
            if (b < nb) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    ActRec rr;
                    rr.q0 = lds_q[2 * (t * nb + b)];
                    rr.q1 = lds_q[2 * (t * nb + b) + 1];
                    const int2 m = lds_m[t * nb + b];
                    rr.D = __int_as_float(m.x);
                    rr.aux = m.y;
                    const typename F::Act a = to_act(rr, (F*)nullptr);
#pragma unroll
                    for (int i = 0; i < R; ++i)
                        if (o0 + i < od) acc[i][t] += F::term(a, cur[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i) cur[i] = nxt[i];
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float v = wave_sum(acc[i][t]);
                if (lane == 0 && o0 + i < od && t0 + t < n)
                    g.out[(int64_t)(t0 + t) * od + o0 + i] = v;
            }
    }
}

__device__ __forceinline__ Q4::Act to_act(const ActRec& r, Q5*) { return to_act(r, (Q4*)nullptr); }

// One token, rows of up to RM * 64 blocks: the plane is staged once per
// workgroup of 4 waves in LDS as 40-byte records (for q6_K with the two half
// sums); each wave takes one row at a time grid-stride and issues all of the
// row's weight loads before it reads the plane -- the first row's right after
// the plane's own loads, so they stream in during the staging.  Per lane the
// block terms are added in round order, then the wave sum.
template <class F, int RM>
__global__ __launch_bounds__(256) void k_mmvq(const MvArgs g) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int id = g.id, od = g.od;
    const int nb = id / kBlock, nsb = id / kSuper;
    uint4* lds_q = reinterpret_cast<uint4*>(lds_raw);                 // [nb][2]
    int2* lds_m = reinterpret_cast<int2*>(lds_raw + (size_t)nb * 32);  // [nb]
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int rounds = (nb + 63) / 64;
    typename F::W w[RM];
    auto load_row = [&](int o) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int b = 64 * r + lane;
            if (r < rounds && b < nb) w[r] = F::load(g, o, b, nb, nsb);
        }
    };
    // The plane's loads are issued before the first row's weight loads:
    // loads complete in issue order, so the staging (and the barrier after
    // it) waits only for the plane, and each round of the row is then summed
    // as its weights arrive instead of after the whole row has.
    constexpr int SB = (RM * 64 + 255) / 256;   // plane blocks per thread (nb <= RM * 64)
    uint4 sq0[SB], sq1[SB];
    uint2 sv[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
        const int b = threadIdx.x + 256 * k;
        if (b < nb) {
            const uint4* p = reinterpret_cast<const uint4*>(g.Q + (int64_t)b * kBlock);
            sq0[k] = p[0];
            sq1[k] = p[1];
            sv[k] = g.ds[b];
        }
    }
    if (wave < od) load_row(wave);
#pragma unroll
    for (int k = 0; k < SB; ++k) {
        const int b = threadIdx.x + 256 * k;
        if (b >= nb) continue;
        const uint4 q0 = sq0[k], q1 = sq1[k];
        const uint2 v = sv[k];
        int aux;
        if constexpr (__is_same(F, Q6)) {
            const uint32_t ones = 0x01010101u;
            int s0 = dot4(q0.x, ones, 0); s0 = dot4(q0.y, ones, s0);
            s0 = dot4(q0.z, ones, s0);    s0 = dot4(q0.w, ones, s0);
            int s1 = dot4(q1.x, ones, 0); s1 = dot4(q1.y, ones, s1);
            s1 = dot4(q1.z, ones, s1);    s1 = dot4(q1.w, ones, s1);
            aux = (int)((uint32_t)(s0 & 0xFFFF) | ((uint32_t)s1 << 16));
        } else {
            aux = (int)v.y;
        }
        lds_q[2 * b] = q0;
        lds_q[2 * b + 1] = q1;
        lds_m[b] = make_int2((int)v.x, aux);
    }
    __syncthreads();
    for (int o = wave; o < od; o += nwaves) {
        if (o != wave) load_row(o);
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int b = 64 * r + lane;
            if (r < rounds && b < nb) {
                ActRec rr;
                rr.q0 = lds_q[2 * b];
                rr.q1 = lds_q[2 * b + 1];
                const int2 m = lds_m[b];
                rr.D = __int_as_float(m.x);
                rr.aux = m.y;
                acc += F::term(to_act(rr, (F*)nullptr), w[r]);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) g.out[o] = acc;
    }
}

template <class F, int RM>
void launch_rows(const MvArgs& g, int64_t rows, hipStream_t s) {
    const int64_t want = (rows + 3) / 4;
    const size_t lds = (size_t)(g.id / kBlock) * kRecBytes;
    hipLaunchKernelGGL((k_mmvq<F, RM>), dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 16384))),
                       dim3(256), lds, s, g);
}

template <class F>
hipError_t launch_mmvq(const WeightDev& w, const PlaneView& pl, float* out, hipStream_t s) {
    MvArgs g;
    g.ql = w.gv_ql;
    g.qh = w.gv_qh;
    g.h5 = w.gv_h5;
    g.sc = w.gv_sc;
    g.dv = w.gv_d;
    g.Q = pl.q;
    g.ds = pl.ds;
    g.id = (int)w.cols;
    g.od = (int)w.rows;
    g.out = out;
    // the row's weight registers sized to its rounds of 64 blocks (up to 12:
    // 768 blocks, 24576 columns, 30 KiB of plane records in LDS, about 160
    // VGPRs and 3 waves per SIMD; at 14 rounds, 2 waves per SIMD, it measured
    // slower than the re-reading form); longer rows
    // take the re-reading form
    const int64_t nb = w.cols / kBlock;
    switch ((nb + 63) / 64) {
    case 1: launch_rows<F, 1>(g, w.rows, s); break;
    case 2: launch_rows<F, 2>(g, w.rows, s); break;
    case 3: launch_rows<F, 3>(g, w.rows, s); break;
    case 4: launch_rows<F, 4>(g, w.rows, s); break;
    case 5: launch_rows<F, 5>(g, w.rows, s); break;
    case 6: launch_rows<F, 6>(g, w.rows, s); break;
    case 7: launch_rows<F, 7>(g, w.rows, s); break;
    case 8: launch_rows<F, 8>(g, w.rows, s); break;
    case 9: launch_rows<F, 9>(g, w.rows, s); break;
    case 10: launch_rows<F, 10>(g, w.rows, s); break;
    case 11: launch_rows<F, 11>(g, w.rows, s); break;
    case 12: launch_rows<F, 12>(g, w.rows, s); break;
    default:
        hipLaunchKernelGGL((k_mmvq_long<F>), dim3((unsigned)mmvq_long_grid<F>(w.rows)), dim3(256), 0, s, g);
    }
    return hipGetLastError();
}

// Tokens per pass: as many of {8, 4, 2} as the LDS holds (160 KiB).
int mmvqn_tokens(int64_t cols, int64_t n) {
    const int64_t rec = (cols / kBlock) * kRecBytes;
    int nt = n > 4 ? 8 : (n > 2 ? 4 : 2);
    while (nt > 2 && nt * rec > 160 * 1024) nt /= 2;
    return nt * rec <= 160 * 1024 ? nt : 0;
}

template <class F, int NT>
hipError_t launch_nt(const MvArgs& g, int64_t n, int64_t t0, int n_cu, hipStream_t s) {
    // One row per group: the register arrays stay small (57-94 VGPRs), so
    // several workgroups fit on a CU where the LDS allows; a plane of more
    // than 80 KiB (one workgroup per CU) is shared by 16 waves instead of 8.
    // Against 4 rows per group on 8-wave workgroups, one per CU: n = 2 is
    // 1.3-1.8x faster, n = 4 1.2-1.9x, n = 8 1.1-1.8x at the 7B and 14B shapes.
    constexpr int R = 1;
    const size_t lds = (size_t)NT * (g.id / kBlock) * kRecBytes;
    static std::atomic<uint64_t> attr{0};
    lds_limit_once(k_mmvqn<F, NT, R>, 160 * 1024, attr);
    const int threads = lds > 80 * 1024 ? 1024 : 512;
    const int64_t groups = (g.od + R - 1) / R;
    const int64_t want = (groups + threads / 64 - 1) / (threads / 64);
    const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 4 * (int64_t)n_cu)));
    hipLaunchKernelGGL((k_mmvqn<F, NT, R>), grid, dim3(threads), lds, s, g, (int)n, (int)t0);
    return hipGetLastError();
}

template <class F>
hipError_t launch_mmvqn(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                        int n_cu, hipStream_t s) {
    MvArgs g;
    g.ql = w.gv_ql;
    g.qh = w.gv_qh;
    g.h5 = w.gv_h5;
    g.sc = w.gv_sc;
    g.dv = w.gv_d;
    g.Q = pl.q;
    g.ds = pl.ds;
    g.id = (int)w.cols;
    g.od = (int)w.rows;
    g.out = out;
    const int nt = mmvqn_tokens(w.cols, n);
    if (nt == 0) return hipErrorInvalidValue;
    for (int64_t t0 = 0; t0 < n; t0 += nt) {
        hipError_t e = nt == 8   ? launch_nt<F, 8>(g, n, t0, n_cu, s)
                       : nt == 4 ? launch_nt<F, 4>(g, n, t0, n_cu, s)
                                 : launch_nt<F, 2>(g, n, t0, n_cu, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---- f32-activation q6_K GEMV: the decode arm's path for small shapes ----
// ("72 · D3-7 ...", section 2 and Excerpt A: below an od*id gate the q6_K
// decode arm runs a kernel on the f32 activation instead of quantising it.)
// out[o] = sum_k w[o][k] * x[k] with w dequantised in f32 from the GEMV tiles:
// per 32-block and 16-value half h, (d * sc_h) * sum (q - 32) * x.  Every
// (q - 32) and d * sc_h is exact in f32, so only the products and sums round.
// x (id floats) is staged once per workgroup in LDS; each wave takes rows
// grid-stride and lane l owns 32-blocks l, l + 64, ...
__global__ __launch_bounds__(256) void k_gemv_f32_q6(const MvArgs g, const float* __restrict__ x) {
    extern __shared__ float4 sx[];   // [id / 4]
    const int id = g.id, od = g.od;
    const int nb = id / kBlock, nsb = id / kSuper;
    for (int i = threadIdx.x; i < id / 4; i += blockDim.x)
        sx[i] = reinterpret_cast<const float4*>(x)[i];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const uint32_t m4 = 0x0F0F0F0Fu, m2 = 0x30303030u;
    for (int o = wave; o < od; o += nwaves) {
        float acc = 0.0f;
        for (int b = lane; b < nb; b += 64) {
            const int64_t i = (int64_t)o * nb + b;
            const uint4 L = nt_load(g.ql + i);
            const uint2 H = nt_load(g.qh + i);
            const int16_t sc = __builtin_nontemporal_load(g.sc + i);
            const float d = __builtin_nontemporal_load(g.dv + (int64_t)o * nsb + (b >> 3));
            // word w holds the 6-bit codes of values 4w .. 4w+3, one per byte
            const uint32_t c[8] = {(L.x & m4) | ((H.x << 4) & m2), ((L.x >> 4) & m4) | ((H.x << 2) & m2),
                                   (L.y & m4) | (H.x & m2),        ((L.y >> 4) & m4) | ((H.x >> 2) & m2),
                                   (L.z & m4) | ((H.y << 4) & m2), ((L.z >> 4) & m4) | ((H.y << 2) & m2),
                                   (L.w & m4) | (H.y & m2),        ((L.w >> 4) & m4) | ((H.y >> 2) & m2)};
            const float4* xb = sx + (int64_t)b * 8;
            float h[2] = {0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const float4 xv = xb[w];
                float& hs = h[w >> 2];
                hs = fmaf((float)(c[w] & 0xFF) - 32.0f, xv.x, hs);
                hs = fmaf((float)((c[w] >> 8) & 0xFF) - 32.0f, xv.y, hs);
                hs = fmaf((float)((c[w] >> 16) & 0xFF) - 32.0f, xv.z, hs);
                hs = fmaf((float)(c[w] >> 24) - 32.0f, xv.w, hs);
            }
            const float s0 = d * (float)(int)(int8_t)(sc & 0xFF);
            const float s1 = d * (float)(int)(int8_t)((uint16_t)sc >> 8);
            acc = fmaf(s0, h[0], acc);
            acc = fmaf(s1, h[1], acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) g.out[o] = acc;
    }
}

}  // namespace

// The GEMV path pays off while one pass holds all n tokens (each further
// pass streams the weights again); the crossover against the split-K matmul
// was measured at the 7B/14B shapes for n = 1..8.
int mmvqn_passes(int64_t cols, int64_t n) {
    const int nt = n >= 1 ? mmvqn_tokens(cols, n) : 0;
    return nt > 0 ? (int)((n + nt - 1) / nt) : 0;
}

hipError_t launch_mmvqn_q6k(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                            int n_cu, hipStream_t s) {
    return launch_mmvqn<Q6>(w, pl, n, out, n_cu, s);
}

hipError_t launch_mmvqn_q4k(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                            int n_cu, hipStream_t s) {
    return launch_mmvqn<Q4>(w, pl, n, out, n_cu, s);
}

hipError_t launch_mmvq_q6k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s) {
    return launch_mmvq<Q6>(w, pl, out, s);
}

hipError_t launch_mmvq_q4k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s) {
    return launch_mmvq<Q4>(w, pl, out, s);
}

hipError_t launch_mmvq_q5k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s) {
    return launch_mmvq<Q5>(w, pl, out, s);
}

// The f32-activation q6_K GEMV: one launch, x read once per workgroup into
// LDS (cols <= kGemvF32MaxCols, so it fits the default 64 KiB).  Grid: a wave
// per row while the rows fit two rounds of resident waves, else exactly the
// resident waves.
hipError_t launch_gemv_f32_q6k(const WeightDev& w, const float* x, float* out, hipStream_t s) {
    if (w.cols > kGemvF32MaxCols || w.cols % kSuper != 0) return hipErrorInvalidValue;
    MvArgs g{};
    g.ql = w.gv_ql;
    g.qh = w.gv_qh;
    g.sc = w.gv_sc;
    g.dv = w.gv_d;
    g.id = (int)w.cols;
    g.od = (int)w.rows;
    g.out = out;
    const size_t lds = (size_t)w.cols * 4;
    static std::atomic<uint64_t> attr{0};
    lds_limit_once(k_gemv_f32_q6, (int)(kGemvF32MaxCols * 4), attr);
    // counted at the largest staged x, so the grid never exceeds what fits
    static const int64_t resident =
        resident_workgroups(k_gemv_f32_q6, 256, (size_t)kGemvF32MaxCols * 4);
    const int64_t want = (w.rows + 3) / 4;
    const int64_t grid = want <= 2 * resident ? want : resident;
    hipLaunchKernelGGL(k_gemv_f32_q6, dim3((unsigned)grid), dim3(256), lds, s, g, x);
    return hipGetLastError();
}

}  // namespace mmq
