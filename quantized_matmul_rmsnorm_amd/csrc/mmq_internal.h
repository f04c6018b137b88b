// mmq_internal.h -- launcher interface between the host library (host.cpp)
// and the gfx950 kernels (quant.hip, repack.hip, gemm.hip, mmvq.hip).
// Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

// Plane of n tokens x d values: rows padded to kPlaneRows, two arrays in one
// allocation: q int8 [rows][d] and ds [rows][d/32] of (D f32 bits, S int32)
// pairs, so that one 8-byte load fetches a block's scale and code sum.
constexpr int kPlaneRows = 32;
constexpr int kBlock = 32;     // activation block (one f32 scale, one int sum)
constexpr int kSuper = 256;    // K-quant superblock

struct PlaneView {
    int8_t* q;
    uint2* ds;      // .x = D (f32 bits), .y = S
    int64_t rows;   // padded row count
    int64_t d;
};

// Matmul tiles: weights are padded to kTileO output rows (zero weights).
constexpr int kTileO = 128;

// Registered weight, device side.  Layouts are written by repack.hip and read
// by gemm.hip / mmvq.hip; they are described there.
struct WeightDev {
    int type = 0;             // 12 = q4_K, 13 = q5_K (GEMV only), 14 = q6_K
    int64_t rows = 0, cols = 0, rows_pad = 0;
    unsigned uses = 0;
    // prefill matmul tiles
    bool packed = false;      // q4_K registered with MMQ_USE_GEMM_PACKED
    _Float16* wa = nullptr;   // f16 integer-valued A fragments (q4_K sc*q, q6_K q-32);
                              // packed: the 4-bit codes, 8 B per lane and block
    uint4* wsc = nullptr;     // packed: [row group][superblock][32 rows] 8 f16 sub-scales
    float* dmr = nullptr;     // per (row group, superblock) scales, fragment order
    _Float16* mfrag = nullptr;// q4_K: 6-bit mins as f16, fragment order;
                              // q6_K: [row group][superblock][32 rows][16] f16 sub-scales
    // one-token GEMV
    uint4* gv_ql = nullptr;   // [rows][cols/32] 4-bit codes (q5_K, q6_K: their low nibbles)
    uint2* gv_qh = nullptr;   // q6_K: [rows][cols/32] high bit pairs
    uint32_t* gv_h5 = nullptr;// q5_K: [rows][cols/32] fifth bits
    int16_t* gv_sc = nullptr; // [rows][cols/32] q6_K: two int8 sub-scales; q4_K, q5_K: sc | m << 8
    float* gv_d = nullptr;    // q6_K: [rows][cols/256] d; q4_K, q5_K: [rows][cols/256][2] d, dmin
    int64_t bytes = 0;
};

// ---- producers (quant.hip); a PlaneView with q == nullptr: RMSNorm / SwiGLU
// write y only (the unfused tier) ----
enum ProducerKind { kProdRms = 0, kProdSwiglu = 1, kProdF32 = 2 };
hipError_t launch_producer(ProducerKind kind, const float* a, const float* b, float* y,
                           int64_t n, int64_t d, float eps, bool write_y,
                           const PlaneView& pl, hipStream_t s);
// Plane scales and sums into separate arrays (count blocks), for export.
hipError_t launch_plane_split(const uint2* ds, float* D, int32_t* S, int64_t count,
                              hipStream_t s);

// ---- registration repack (repack.hip): raw superblocks already on device ----
hipError_t launch_repack_gemm(const uint8_t* raw_dev, const WeightDev& w, hipStream_t s);
hipError_t launch_repack_gemv(const uint8_t* raw_dev, const WeightDev& w, hipStream_t s);

// ---- consumers ----
// K splits the matmul uses for n tokens on n_cu compute units (1: none);
// with splits > 1 the partials go to part [splits][stride] and are summed
// into out in split order by a second kernel.
int gemm_splits(int64_t rows_pad, int64_t cols, int64_t n, int n_cu);
int64_t gemm_part_stride(int64_t n, int64_t rows);   // floats per partial (16-byte aligned)
// The launch plan: a K split of every tile (splits > 1), or a K split of
// only the tail tiles that would leave the last round nearly empty
// (tail_tiles > 0, partials as compact 128 x 128 tiles); part_floats is the
// scratch it needs (0: none).
struct GemmPlan {
    int splits = 1;
    int tail_tiles = 0, tail_splits = 0;
    int64_t part_floats = 0;
};
GemmPlan gemm_plan(const WeightDev& w, int64_t n, int n_cu);
hipError_t launch_gemm(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                       float* part, const GemmPlan& plan, hipStream_t s);
hipError_t launch_mmvq_q6k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s);
hipError_t launch_mmvq_q4k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s);
hipError_t launch_mmvq_q5k(const WeightDev& w, const PlaneView& pl, float* out,
                           hipStream_t s);
// q6_K GEMV on the f32 activation x [cols] (no plane): out [rows].
constexpr int64_t kGemvF32MaxCols = 16384;   // x is staged whole in 64 KiB of LDS
hipError_t launch_gemv_f32_q6k(const WeightDev& w, const float* x, float* out, hipStream_t s);
// A few tokens at once over the GEMV tiles (out [n][rows]); used when the n
// tokens' plane fits the LDS in one pass.
// Launches (passes of up to 8 tokens) the few-token GEMV takes for n tokens
// of width cols; 0 if not even 2 tokens fit the LDS.
int mmvqn_passes(int64_t cols, int64_t n);
hipError_t launch_mmvqn_q6k(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                            int n_cu, hipStream_t s);
hipError_t launch_mmvqn_q4k(const WeightDev& w, const PlaneView& pl, int64_t n, float* out,
                            int n_cu, hipStream_t s);

}  // namespace mmq
