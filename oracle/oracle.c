/*
 * oracle.c -- the CPU oracle for the q8-plane producers and the q4_K / q5_K /
 * q6_K integer-dot matmuls.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no source,
 * header, table or helper with the HIP library under
 * quantized_matmul_rmsnorm_amd/csrc/, and the product path never calls it.
 *
 * Plain scalar loops, compiled with -O2 -ffp-contract=off so that every f32
 * expression below rounds exactly where it is written.  OpenMP only splits
 * independent output rows across threads; it does not change any result.
 *
 * Sources (titles of the engineering-log pages this follows):
 *   [r52]  "55 · r52 — skip-write mode 2", sections 2.2 and 3.2
 *   [r60]  "64 · r60 — the coronation: flipping the verified gate set to
 *          default-on", section 3.2
 *   [d37]  "72 · D3-7 — attn_v-q6K MMVQ routing ...", Excerpts A, A2, C
 * The K-quant superblock layouts are not on those pages; they follow the
 * public GGUF q4_K / q5_K / q6_K definitions (256 weights per superblock).
 * The pages name a q5_K one-token arm beside the q6_K one [d37 Excerpt B].
 *
 * Pinned by tests/test_oracle_pins.py: brute-force f64 dequantised matmul on
 * tiny shapes, the integer special case (unit scales -> exact int matmul),
 * quantiser invariants, the RMSNorm and SwiGLU closed forms, and an
 * independent field encoder for the three superblock formats.
 *
 * Parity unpinned: (1) bit-compatibility of the two superblock byte layouts
 * with real GGUF files (no such file is available; the layouts are this
 * project's reading of the public format, pinned only for self-consistency
 * by the encoder round trips); (2) agreement with a worked numeric example
 * from the pages, which print none for the plane or the matmul.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define QK 32          /* activation block: 32 values, one f32 scale, one int sum */
#define QKK 256        /* K-quant superblock */
#define Q4K_BYTES 144
#define Q5K_BYTES 176
#define Q6K_BYTES 210

/* IEEE half -> float, written out from the binary16 definition. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);              /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25); /* (1 + man/1024) * 2^(exp-15) */
    return (float)(sign ? -v : v);
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/*
 * q4_K superblock (144 B): f16 d, f16 dmin, 12 B of packed 6-bit
 * (scale, min) pairs for the eight 32-element sub-blocks, 128 B of 4-bit
 * quants.  Element e belongs to sub-block j = e / 32; weight value is
 * d * scale_j * q_e - dmin * min_j.
 */
void oracle_q4k_fields(const uint8_t* blk, float* d, float* dmin,
                       uint8_t sc[8], uint8_t mn[8], uint8_t q[256])
{
    const uint8_t* s = blk + 4;
    const uint8_t* qs = blk + 16;
    *d = oracle_f16_to_f32(rd16(blk));
    *dmin = oracle_f16_to_f32(rd16(blk + 2));
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            sc[j] = (uint8_t)((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4));
            mn[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
        }
    }
    for (int e = 0; e < 256; e++) {
        int g = e / 64, i = e % 64;
        uint8_t byte = qs[32 * g + (i % 32)];
        q[e] = (i < 32) ? (byte & 15) : (byte >> 4);
    }
}

/*
 * q5_K superblock (176 B): f16 d, f16 dmin, the same 12 B of packed 6-bit
 * (scale, min) pairs as q4_K, 32 B of high bits, 128 B of low nibbles.
 * Quants are 5-bit: element e = 64 g + i (g = 0..3) takes its low nibble
 * from byte 32 g + (i % 32) of the nibbles (low half for i < 32, high half
 * otherwise) and its fifth bit from bit 2 g + (i >= 32) of high-bit byte
 * i % 32.  Weight value is d * scale_j * q_e - dmin * min_j, j = e / 32.
 */
void oracle_q5k_fields(const uint8_t* blk, float* d, float* dmin,
                       uint8_t sc[8], uint8_t mn[8], uint8_t q[256])
{
    const uint8_t* qh = blk + 16;
    const uint8_t* qs = blk + 48;
    /* the header (d, dmin, scales) has the q4_K layout */
    uint8_t head[144];
    uint8_t unused[256];
    memcpy(head, blk, 16);
    memset(head + 16, 0, 128);
    oracle_q4k_fields(head, d, dmin, sc, mn, unused);
    for (int e = 0; e < 256; e++) {
        int g = e / 64, i = e % 64;
        uint8_t byte = qs[32 * g + (i % 32)];
        int lo = (i < 32) ? (byte & 15) : (byte >> 4);
        int hi = (qh[i % 32] >> (2 * g + (i >= 32))) & 1;
        q[e] = (uint8_t)(lo + 16 * hi);
    }
}

/*
 * q6_K superblock (210 B): ql[128] low nibbles, qh[64] high 2-bit pairs,
 * 16 int8 sub-scales (one per 16 elements), f16 d.  Weight value is
 * d * scale[e / 16] * (q_e - 32), q_e in [0, 63].
 */
void oracle_q6k_fields(const uint8_t* blk, float* d, int8_t sc[16], uint8_t q[256])
{
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    const int8_t* scales = (const int8_t*)(blk + 192);
    *d = oracle_f16_to_f32(rd16(blk + 208));
    for (int i = 0; i < 16; i++) sc[i] = scales[i];
    for (int e = 0; e < 256; e++) {
        int h = e / 128, r = e % 128, s = r / 32, l = r % 32;
        uint8_t lb = ql[64 * h + l + 32 * (s % 2)];
        int lo = (s < 2) ? (lb & 15) : (lb >> 4);
        int hi = (qh[32 * h + l] >> (2 * s)) & 3;
        q[e] = (uint8_t)(lo + 16 * hi);
    }
}

/* Dequantised weights in f64 (used by the brute-force pins). w: [rows][cols]. */
void oracle_dequant_q4k(const uint8_t* raw, int64_t rows, int64_t cols, double* w)
{
    int64_t nsb = cols / QKK;
    for (int64_t o = 0; o < rows; o++)
        for (int64_t sb = 0; sb < nsb; sb++) {
            float d, dmin; uint8_t sc[8], mn[8], q[256];
            oracle_q4k_fields(raw + (o * nsb + sb) * Q4K_BYTES, &d, &dmin, sc, mn, q);
            for (int e = 0; e < 256; e++)
                w[o * cols + sb * 256 + e] =
                    (double)d * sc[e / 32] * q[e] - (double)dmin * mn[e / 32];
        }
}

void oracle_dequant_q5k(const uint8_t* raw, int64_t rows, int64_t cols, double* w)
{
    int64_t nsb = cols / QKK;
    for (int64_t o = 0; o < rows; o++)
        for (int64_t sb = 0; sb < nsb; sb++) {
            float d, dmin; uint8_t sc[8], mn[8], q[256];
            oracle_q5k_fields(raw + (o * nsb + sb) * Q5K_BYTES, &d, &dmin, sc, mn, q);
            for (int e = 0; e < 256; e++)
                w[o * cols + sb * 256 + e] =
                    (double)d * sc[e / 32] * q[e] - (double)dmin * mn[e / 32];
        }
}

void oracle_dequant_q6k(const uint8_t* raw, int64_t rows, int64_t cols, double* w)
{
    int64_t nsb = cols / QKK;
    for (int64_t o = 0; o < rows; o++)
        for (int64_t sb = 0; sb < nsb; sb++) {
            float d; int8_t sc[16]; uint8_t q[256];
            oracle_q6k_fields(raw + (o * nsb + sb) * Q6K_BYTES, &d, sc, q);
            for (int e = 0; e < 256; e++)
                w[o * cols + sb * 256 + e] = (double)d * sc[e / 16] * ((int)q[e] - 32);
        }
}

/*
 * RMSNorm producer math [r52 3.2; d37 Excerpt C]: ss = sum x^2,
 * scale = 1/sqrt(ss/d + eps), y = (x * scale) * w -- two f32 multiplies in
 * that order.  The oracle accumulates ss in f64 and rounds scale once
 * (the pages use an f32 lane-serial chain and rsqrtf; that difference is
 * covered by the fused-producer tolerance).
 */
void oracle_rmsnorm(const float* x, const float* w, int64_t n, int64_t d,
                    float eps, float* y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; t++) {
        const float* xr = x + t * d;
        double ss = 0.0;
        for (int64_t i = 0; i < d; i++) ss += (double)xr[i] * (double)xr[i];
        float scale = (float)(1.0 / sqrt(ss / (double)d + (double)eps));
        for (int64_t i = 0; i < d; i++) {
            float a = xr[i] * scale;
            y[t * d + i] = a * w[i];
        }
    }
}

/* SwiGLU producer math [r52 3.2]: y = (g / (1 + exp(-g))) * u in f32. */
void oracle_swiglu(const float* g, const float* u, int64_t n, int64_t d, float* y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; t++)
        for (int64_t i = 0; i < d; i++) {
            float gv = g[t * d + i];
            float den = 1.0f + expf(-gv);
            float s = gv / den;
            y[t * d + i] = s * u[t * d + i];
        }
}

/*
 * Block-32 quantisation [r52 2.2, 3.2; d37 Excerpt C]: per block of 32
 * values, amax = max |y|, scale D = amax / 127 (f32 IEEE divide), codes
 * q = clamp(rint(y / D), -127, 127) with round-half-even and the IEEE
 * quotient, S = sum q (int).  A block whose scale is zero has q = 0 and
 * S = 0: the all-zero block, and also a block of deep subnormals whose
 * quotient amax / 127 rounds to zero (amax <= 63 * 2^-149).  With D = 0 the
 * block's values D * q are zero whatever the codes, so the zero codes of the
 * all-zero block (and of a padded row) are the reading that keeps D, q and S
 * consistent; it also keeps y / 0 out of the arithmetic.
 * q: [n][d] int8, D and S: [n][d/32].
 */
void oracle_quantize(const float* y, int64_t n, int64_t d,
                     int8_t* q, float* D, int32_t* S)
{
    int64_t nb = d / QK;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; t++)
        for (int64_t b = 0; b < nb; b++) {
            const float* yb = y + t * d + b * QK;
            float amax = 0.0f;
            for (int i = 0; i < QK; i++) {
                float a = fabsf(yb[i]);
                if (a > amax) amax = a;
            }
            float dsc = amax / 127.0f;
            int32_t sum = 0;
            for (int i = 0; i < QK; i++) {
                int v = 0;
                if (dsc != 0.0f) {
                    float r = rintf(yb[i] / dsc);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    v = (int)r;
                }
                q[t * d + b * QK + i] = (int8_t)v;
                sum += v;
            }
            D[t * nb + b] = dsc;
            S[t * nb + b] = sum;
        }
}

/*
 * q4_K integer-dot matmul over a q8 plane [r60 3.2: int8 MMA over the
 * plane, k32 chunks].  For output (t, o) and 32-block b in superblock sb
 * with sub-block j:
 *   I    = sum_{k in b} q_w[o][k] * Q[t][k]                (exact int32)
 *   term = D[t][b] * (d * sc_j) * I  -  D[t][b] * S[t][b] * (dmin * m_j)
 * The factoring per block is exact, so the result is, up to rounding, the
 * product of the plane's values D * q with the dequantised weight; the oracle
 * evaluates that plain definition with every term in f64 (d*sc_j, dmin*m_j and
 * D*d*sc_j are exact; the product with I rounds once, at 2^-53), sums the
 * terms over blocks in f64 and stores the sum as f32.  mag (may be NULL)
 * receives, per output, the sum over blocks of |first part| + |second part|:
 * the magnitude any f32 evaluation of the per-block rescale rounds against.
 * Computes out[i][j] for t = tok[i], o = outs[j]; out and mag are
 * [ntok][nout].  Q: [*][id] int8 row-major, D/S: [*][id/32]; raw: [od][id/256]
 * superblocks.
 */
void oracle_gemm_q4k(const int8_t* Q, const float* D, const int32_t* S,
                     const uint8_t* raw, int64_t id,
                     const int64_t* tok, int64_t ntok,
                     const int64_t* outs, int64_t nout, float* out, double* mag)
{
    int64_t nb = id / QK, nsb = id / QKK;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t jo = 0; jo < nout; jo++) {
        int64_t o = outs[jo];
        for (int64_t it = 0; it < ntok; it++) {
            int64_t t = tok[it];
            double acc = 0.0, sabs = 0.0;
            for (int64_t sb = 0; sb < nsb; sb++) {
                float d, dmin; uint8_t sc[8], mn[8], qw[256];
                oracle_q4k_fields(raw + (o * nsb + sb) * Q4K_BYTES, &d, &dmin, sc, mn, qw);
                for (int j = 0; j < 8; j++) {
                    int64_t b = sb * 8 + j;
                    int32_t I = 0;
                    for (int l = 0; l < QK; l++)
                        I += (int32_t)qw[j * QK + l] * (int32_t)Q[t * id + b * QK + l];
                    double Da = (double)D[t * nb + b];
                    double dsc = (double)d * (double)sc[j];
                    double dmn = (double)dmin * (double)mn[j];
                    double t1 = Da * dsc * (double)I;
                    double t2 = Da * (double)S[t * nb + b] * dmn;
                    acc += t1 - t2;
                    sabs += fabs(t1) + fabs(t2);
                }
            }
            out[it * nout + jo] = (float)acc;
            if (mag) mag[it * nout + jo] = sabs;
        }
    }
}

/*
 * q5_K integer-dot matmul over a q8 plane: the q4_K expression with 5-bit
 * quants (the one-token arm of d37 Excerpt B is this with ntok = 1):
 *   I    = sum_{k in b} q_w[o][k] * Q[t][k]                (exact int32)
 *   term = D[t][b] * (d * sc_j) * I  -  D[t][b] * S[t][b] * (dmin * m_j)
 * evaluated as for q4_K (f64 terms, f64 sum, f32 result; mag as there).
 */
void oracle_gemm_q5k(const int8_t* Q, const float* D, const int32_t* S,
                     const uint8_t* raw, int64_t id,
                     const int64_t* tok, int64_t ntok,
                     const int64_t* outs, int64_t nout, float* out, double* mag)
{
    int64_t nb = id / QK, nsb = id / QKK;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t jo = 0; jo < nout; jo++) {
        int64_t o = outs[jo];
        for (int64_t it = 0; it < ntok; it++) {
            int64_t t = tok[it];
            double acc = 0.0, sabs = 0.0;
            for (int64_t sb = 0; sb < nsb; sb++) {
                float d, dmin; uint8_t sc[8], mn[8], qw[256];
                oracle_q5k_fields(raw + (o * nsb + sb) * Q5K_BYTES, &d, &dmin, sc, mn, qw);
                for (int j = 0; j < 8; j++) {
                    int64_t b = sb * 8 + j;
                    int32_t I = 0;
                    for (int l = 0; l < QK; l++)
                        I += (int32_t)qw[j * QK + l] * (int32_t)Q[t * id + b * QK + l];
                    double Da = (double)D[t * nb + b];
                    double dsc = (double)d * (double)sc[j];
                    double dmn = (double)dmin * (double)mn[j];
                    double t1 = Da * dsc * (double)I;
                    double t2 = Da * (double)S[t * nb + b] * dmn;
                    acc += t1 - t2;
                    sabs += fabs(t1) + fabs(t2);
                }
            }
            out[it * nout + jo] = (float)acc;
            if (mag) mag[it * nout + jo] = sabs;
        }
    }
}

/*
 * q6_K integer-dot matmul over a q8 plane [r60 3.2: "k32 chunks with dual
 * 16-sub rescale"]: each 32-block spans two 16-element sub-blocks with their
 * own int8 scales sc0, sc1:
 *   I0, I1 = 16-element int dots of (q_w - 32) with Q     (exact int32)
 *   Ic     = sc0 * I0 + sc1 * I1                          (exact int32)
 *   term   = D[t][b] * d * Ic
 * in f64 (D*d exact, the product with Ic rounded once at 2^-53), summed over
 * blocks in f64, stored as f32: the plain dequantised product, as for q4_K.
 * mag (may be NULL) receives the sum of |term| per output.  The one-token
 * GEMV is this function with ntok = 1 [d37 Excerpt A].
 */
void oracle_gemm_q6k(const int8_t* Q, const float* D,
                     const uint8_t* raw, int64_t id,
                     const int64_t* tok, int64_t ntok,
                     const int64_t* outs, int64_t nout, float* out, double* mag)
{
    int64_t nb = id / QK, nsb = id / QKK;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t jo = 0; jo < nout; jo++) {
        int64_t o = outs[jo];
        for (int64_t it = 0; it < ntok; it++) {
            int64_t t = tok[it];
            double acc = 0.0, sabs = 0.0;
            for (int64_t sb = 0; sb < nsb; sb++) {
                float d; int8_t sc[16]; uint8_t qw[256];
                oracle_q6k_fields(raw + (o * nsb + sb) * Q6K_BYTES, &d, sc, qw);
                for (int j = 0; j < 8; j++) {
                    int64_t b = sb * 8 + j;
                    int32_t I0 = 0, I1 = 0;
                    for (int l = 0; l < 16; l++)
                        I0 += ((int32_t)qw[j * QK + l] - 32) * (int32_t)Q[t * id + b * QK + l];
                    for (int l = 16; l < 32; l++)
                        I1 += ((int32_t)qw[j * QK + l] - 32) * (int32_t)Q[t * id + b * QK + l];
                    int32_t Ic = (int32_t)sc[2 * j] * I0 + (int32_t)sc[2 * j + 1] * I1;
                    double term = (double)D[t * nb + b] * (double)d * (double)Ic;
                    acc += term;
                    sabs += fabs(term);
                }
            }
            out[it * nout + jo] = (float)acc;
            if (mag) mag[it * nout + jo] = sabs;
        }
    }
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n); }
#else
int oracle_threads(void) { return 1; }
void oracle_set_threads(int n) { (void)n; }
#endif
