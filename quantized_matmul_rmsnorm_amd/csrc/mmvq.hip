// mmvq.hip -- one-token q6_K GEMV over a q8 activation plane (gfx950).
//
// Method ("72 · D3-7 ...", section 2 and Excerpts A/A2): at one token the
// matmul is a weight-streaming GEMV; the activation is quantised once into a
// q8 plane (shared through the plane cache by every consumer of the same
// buffer) and each output row is an integer dot of that plane with the row's
// 6-bit weights, rescaled per 16-element half by the int8 sub-scale and per
// 32-block by D * d.
//
// Design for CDNA4.  The kernel is bound by streaming the packed weights from
// HBM, so the weights are read exactly once, in 1 KiB-per-wave coalesced
// pieces, and the integer work runs on v_dot4_i32_i8 (4 int8 products per
// instruction).  Each wave keeps its slice of the activation plane in
// registers for its whole lifetime -- lane l owns 32-blocks l, l+64, ... -- and
// walks output rows grid-stride; per row and block the lane reads 16 B of low
// nibbles, 8 B of high bit pairs and 2 B of sub-scales (the registration
// layout of repack.hip), rebuilds four packed dwords of 6-bit codes per
// 16-element half with masks and shifts, and dots them with its codes.  The
// "- 32" of the q6_K code is applied through the activation: the dot
// accumulator starts at -32 * sum(q) of the half, computed once per lane.
// One f32 FMA per block adds (D * d) * (sc0*I0 + sc1*I1); a wave-wide sum per
// row finishes the output.
#include "mmq_internal.h"

namespace mmq {
namespace {

struct ActBlock {
    uint4 q0, q1;   // codes 0..15, 16..31
    float D;
    int c0, c1;     // -32 * sum of codes in each half
};

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ ActBlock load_act(const int8_t* Q, const float* Dp, int b, int nb) {
    ActBlock a;
    if (b < nb) {
        const uint4* p = reinterpret_cast<const uint4*>(Q + (int64_t)b * kBlock);
        a.q0 = p[0];
        a.q1 = p[1];
        a.D = Dp[b];
        const uint32_t ones = 0x01010101u;
        int s0 = dot4(a.q0.x, ones, 0); s0 = dot4(a.q0.y, ones, s0);
        s0 = dot4(a.q0.z, ones, s0);    s0 = dot4(a.q0.w, ones, s0);
        int s1 = dot4(a.q1.x, ones, 0); s1 = dot4(a.q1.y, ones, s1);
        s1 = dot4(a.q1.z, ones, s1);    s1 = dot4(a.q1.w, ones, s1);
        a.c0 = -32 * s0;
        a.c1 = -32 * s1;
    } else {
        a.q0 = make_uint4(0, 0, 0, 0);
        a.q1 = a.q0;
        a.D = 0.0f;
        a.c0 = a.c1 = 0;
    }
    return a;
}

// (D * d) * (sc0 * I0 + sc1 * I1) for one 32-block of one row.
__device__ __forceinline__ float block_term(const ActBlock& a, uint4 L, uint2 H, int16_t sc,
                                            float d) {
    const uint32_t m4 = 0x0F0F0F0Fu, m2 = 0x30303030u;
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
    const int s0 = (int)(int8_t)(sc & 0xFF);
    const int s1 = (int)(int8_t)((uint16_t)sc >> 8);
    const int ic = s0 * i0 + s1 * i1;
    return (a.D * d) * (float)ic;
}

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

// MAXR > 0: the lane's activation blocks stay in registers (nb <= 64 * MAXR),
// and the weights of the wave's next row are loaded block by block as soon as
// the current row's registers for that block are consumed, so a row's loads
// are in flight while the previous row is reduced.
// MAXR == 0: blocks are re-read from the plane for every row (any length).
template <int MAXR>
__global__ __launch_bounds__(256) void k_mmvq_q6k(const uint4* __restrict__ ql,
                                                  const uint2* __restrict__ qh,
                                                  const int16_t* __restrict__ sc,
                                                  const float* __restrict__ dv,
                                                  const int8_t* __restrict__ Q,
                                                  const float* __restrict__ Dp, int id, int od,
                                                  float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int nb = id / kBlock;
    const int nsb = id / kSuper;
    const int rounds = (nb + 63) / 64;

    if constexpr (MAXR > 0) {
        ActBlock act[MAXR];
        uint4 L[MAXR];
        uint2 H[MAXR];
        int16_t S[MAXR];
        float Dw[MAXR];
#pragma unroll
        for (int r = 0; r < MAXR; ++r)
            if (r < rounds) act[r] = load_act(Q, Dp, 64 * r + lane, nb);
        auto load_block = [&](int o, int r) {
            const int b = 64 * r + lane;
            const int64_t rb = (int64_t)o * nb;
            {
                typedef uint32_t u4v __attribute__((ext_vector_type(4)));
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                const u4v l4 = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(ql) + rb + b);
                const u2v h2 = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(qh) + rb + b);
                L[r] = make_uint4(l4.x, l4.y, l4.z, l4.w);
                H[r] = make_uint2(h2.x, h2.y);
            }
            S[r] = __builtin_nontemporal_load(&sc[rb + b]);
            Dw[r] = __builtin_nontemporal_load(&dv[(int64_t)o * nsb + (b >> 3)]);
        };
        int o = wave;
        if (o < od) {
#pragma unroll
            for (int r = 0; r < MAXR; ++r)
                if (r < rounds && 64 * r + lane < nb) load_block(o, r);
        }
        for (; o < od; o += nwaves) {
            const int on = o + nwaves;
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < MAXR; ++r) {
                if (r < rounds && 64 * r + lane < nb) {
                    acc += block_term(act[r], L[r], H[r], S[r], Dw[r]);
                    if (on < od) load_block(on, r);
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) out[o] = acc;
        }
    } else {
        for (int o = wave; o < od; o += nwaves) {
            const int64_t rb = (int64_t)o * nb;
            float acc = 0.0f;
            for (int r = 0; r < rounds; ++r) {
                const int b = 64 * r + lane;
                if (b < nb) {
                    const ActBlock a = load_act(Q, Dp, b, nb);
                    acc += block_term(a, ql[rb + b], qh[rb + b], sc[rb + b],
                                      dv[(int64_t)o * nsb + (b >> 3)]);
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) out[o] = acc;
        }
    }
}

// Workgroups of one launch: every row gets a wave when the rows fit in two
// rounds of resident waves; larger matrices get exactly the resident waves
// (each then walks rows grid-stride with its plane slice loaded once).
template <int MAXR>
int64_t mmvq_grid(int64_t rows) {
    static int per_cu = -1, n_cu = 0;
    if (per_cu < 0) {
        int dev = 0, blk = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blk, k_mmvq_q6k<MAXR>, 256, 0) != hipSuccess)
            blk = 1;
        per_cu = blk > 0 ? blk : 1;
        if (n_cu <= 0) n_cu = 256;
    }
    const int64_t resident = (int64_t)per_cu * n_cu;
    const int64_t want = (rows + 3) / 4;
    return want <= 2 * resident ? want : resident;
}

}  // namespace

hipError_t launch_mmvq_q6k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s) {
    const int64_t nb = w.cols / kBlock;
    const int id = (int)w.cols, od = (int)w.rows;
    const dim3 block(256);
    if (nb <= 64 * 4) {
        const dim3 grid((unsigned)mmvq_grid<4>(w.rows));
        hipLaunchKernelGGL(k_mmvq_q6k<4>, grid, block, 0, s, w.gv_ql, w.gv_qh, w.gv_sc, w.gv_d,
                           pl.q, pl.D, id, od, out);
    } else if (nb <= 64 * 8) {
        const dim3 grid((unsigned)mmvq_grid<8>(w.rows));
        hipLaunchKernelGGL(k_mmvq_q6k<8>, grid, block, 0, s, w.gv_ql, w.gv_qh, w.gv_sc, w.gv_d,
                           pl.q, pl.D, id, od, out);
    } else {
        const dim3 grid((unsigned)mmvq_grid<0>(w.rows));
        hipLaunchKernelGGL(k_mmvq_q6k<0>, grid, block, 0, s, w.gv_ql, w.gv_qh, w.gv_sc, w.gv_d,
                           pl.q, pl.D, id, od, out);
    }
    return hipGetLastError();
}

}  // namespace mmq
