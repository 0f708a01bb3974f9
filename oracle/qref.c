/*
 * qref.c — the oracle (see qref.h). TEST INFRASTRUCTURE ONLY: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * What it follows, page by page:
 *  - Bit layout and dequantization: emily lib/emily/quantization.ex,
 *    `dequantize_defn/1` docs and `dequantize_impl` (lane i sits at bit
 *    offset i*bits of the row's u32 stream, masked to `bits` bits; group
 *    g = i div group_size; w = lane * scales[g] + biases[g]), and the
 *    cross-word unpack (`unpack_cross_word_lanes`, `build_word_indices`:
 *    read the word holding the lane and the next one, clamped to the last
 *    word, as one 64-bit value, shift right by i*bits mod 32, mask).
 *  - Quantizer: the pages call MLX's quantizer without printing its body
 *    (ollama x/create/client/quantize.go, `loadAndQuantizeArray`; emily
 *    `QuantizedWeight.from_dense/2` in the `quantized_matmul/2` example).
 *    The formula used here is the plain affine one: per group,
 *    scale = (max - min) / (2^bits - 1), bias = min, q = round((w-bias)/scale).
 *    The readings where the pages are silent follow the per-tensor int8
 *    quantizer of mlex src/quant.rs (`quantize_dynamic_int8`): the scale is
 *    floored at FLT_EPSILON, codes use round-half-away-from-zero and are
 *    clamped to the code range. Codes are computed from the scale and bias
 *    AS STORED (rounded to the storage type, a zero bias stored as +0), so
 *    dequantization sees the nearest grid point.
 *    Parity with MLX's own quantizer: parity unpinned (no values printed).
 *  - The product: emily `quantized_matmul/2` docs (x @ W^T with the packed
 *    W laid out [N, K], transpose = true).
 *  - MoE: ferrum-kernels src/stacked_expert.rs, `gemv_moe_id` and
 *    `gemv_moe_id_batched` docs (pair p reads a[(p/top_k)*outer +
 *    (p%top_k)*inner] and expert ids[p]), and the CPU fallback in the module
 *    docs (per-expert Linear calls): here, one dot product per pair and row.
 *    `gemv_moe_id_gate_up_silu` docs: SiLU(gate) * up.
 *  - Per-tensor dynamic-range int8: mlex src/quant.rs (`quantize_dynamic_int8`,
 *    `dequantize_dynamic_int8`).
 *  - Microscaled modes: emily `dequantize_defn/1` docs and its mxfp4 / mxfp8
 *    / nvfp4 implementations (lane and scale formats below).
 *
 * Arithmetic: fp32 for quantize and dequantize (compiled with
 * -ffp-contract=off, so a*b+c is a multiply then an add), fp64 for every
 * product sum. The dense weight in the scales' own type (the pages'
 * `dequantize_impl`, which casts the codes to the scales' type) rounds the
 * product and then the sum to that type, each exactly once. Each output's sum runs sequentially in k order, so the OpenMP
 * loops over outputs give the same bits at any thread count.
 */
#include "qref.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Floating-point formats                                              */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round a >= 0 (finite) to the nearest integer multiple of `quantum` (a power
 * of two), ties to the even multiple. Every step is exact in fp64 for the
 * fp32 inputs used here. */
static double round_to_multiple_even(double a, double quantum)
{
    double t = a / quantum;
    double lo = floor(t);
    double frac = t - lo;
    double r;
    if (frac > 0.5)
        r = lo + 1.0;
    else if (frac < 0.5)
        r = lo;
    else
        r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
    return r * quantum;
}

/* A binary format with `mant_bits` explicit mantissa bits, exponent bias
 * `bias`, and `exp_bits` exponent bits (IEEE layout, subnormals, inf/NaN). */
struct fmt16 { int mant_bits, exp_bits, bias; };
static const struct fmt16 FMT_BF16 = {7, 8, 127};
static const struct fmt16 FMT_F16 = {10, 5, 15};

/* x (an fp64 value) rounded to format F, nearest with ties to even. */
static uint16_t encode_rne_d(double x, struct fmt16 F)
{
    uint16_t sign = (uint16_t)(signbit(x) ? 0x8000u : 0u);
    uint16_t exp_all_ones = (uint16_t)(((1u << F.exp_bits) - 1u) << F.mant_bits);
    if (isnan(x))
        return (uint16_t)(sign | exp_all_ones | (1u << (F.mant_bits - 1)));
    double a = fabs(x);
    if (isinf(x))
        return (uint16_t)(sign | exp_all_ones);
    if (a == 0.0)
        return sign;
    int emin = 1 - F.bias;                    /* smallest normal exponent */
    int emax = (1 << F.exp_bits) - 2 - F.bias; /* largest finite exponent */
    int e2;
    (void)frexp(a, &e2);                      /* a = f * 2^e2, 0.5 <= f < 1 */
    int e = e2 - 1;                           /* a = m * 2^e, 1 <= m < 2 */
    if (e < emin)
        e = emin;                             /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - F.mant_bits);
    double v = round_to_multiple_even(a, quantum);
    if (v >= ldexp(1.0, emax + 1))            /* rounded past the largest finite */
        return (uint16_t)(sign | exp_all_ones);
    if (v < ldexp(1.0, emin)) {               /* subnormal (or zero) */
        uint32_t mant = (uint32_t)(v / ldexp(1.0, emin - F.mant_bits));
        return (uint16_t)(sign | mant);
    }
    (void)frexp(v, &e2);
    e = e2 - 1;
    uint32_t mant = (uint32_t)((v / ldexp(1.0, e) - 1.0) * ldexp(1.0, F.mant_bits));
    return (uint16_t)(sign | ((uint32_t)(e + F.bias) << F.mant_bits) | mant);
}

static uint16_t encode_rne(float f, struct fmt16 F) { return encode_rne_d((double)f, F); }

uint16_t qref_f32_to_bf16(float f) { return encode_rne(f, FMT_BF16); }
uint16_t qref_f32_to_f16(float f) { return encode_rne(f, FMT_F16); }

/* bf16 is, by definition, the upper 16 bits of an fp32. */
float qref_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

float qref_f16_to_f32(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

void qref_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = qref_f32_to_bf16(in[i]);
}

void qref_f32_to_f16_n(const float* in, uint16_t* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = qref_f32_to_f16(in[i]);
}

void qref_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = qref_bf16_to_f32(in[i]);
}

void qref_f16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = qref_f16_to_f32(in[i]);
}

/* Value of element `idx` of an array of element type `dtype`. */
static float load_elem(const void* p, int dtype, int64_t idx)
{
    switch (dtype) {
    case QREF_F32: return ((const float*)p)[idx];
    case QREF_F16: return qref_f16_to_f32(((const uint16_t*)p)[idx]);
    case QREF_BF16: return qref_bf16_to_f32(((const uint16_t*)p)[idx]);
    }
    abort();
}

/* Round fp32 `v` to element type `dtype`, store it, and return the stored value. */
static float store_elem(void* p, int dtype, int64_t idx, float v)
{
    switch (dtype) {
    case QREF_F32: ((float*)p)[idx] = v; return v;
    case QREF_F16: {
        uint16_t h = qref_f32_to_f16(v);
        ((uint16_t*)p)[idx] = h;
        return qref_f16_to_f32(h);
    }
    case QREF_BF16: {
        uint16_t h = qref_f32_to_bf16(v);
        ((uint16_t*)p)[idx] = h;
        return qref_bf16_to_f32(h);
    }
    }
    abort();
}

/* ------------------------------------------------------------------ */
/* Packing                                                             */
/* ------------------------------------------------------------------ */

static int bits_ok(int bits)
{
    return bits == 2 || bits == 3 || bits == 4 || bits == 6 || bits == 8;
}

/* Packed row length; the packing needs k*bits to be a multiple of 32. */
static int64_t words_per_row(int64_t k, int bits) { return k * bits / 32; }

/* Lane i of a row: word i*bits div 32 and the next word (clamped to the
 * row's last word) read as one 64-bit value, shifted right by
 * i*bits mod 32, masked to `bits` bits. For bits dividing 32 the lane never
 * leaves its word and this is the plain (word >> (lane*bits)) & mask. */
static uint32_t unpack_lane(const uint32_t* row, int64_t words, int64_t i, int bits)
{
    int64_t w = (i * bits) / 32;
    int64_t w_next = (w + 1 < words) ? w + 1 : words - 1;
    uint64_t window = (uint64_t)row[w] | ((uint64_t)row[w_next] << 32);
    uint64_t shifted = window >> ((i * bits) % 32);
    return (uint32_t)(shifted & ((1u << bits) - 1u));
}

int qref_pack(const uint8_t* codes, int64_t n, int64_t k, int bits, uint32_t* wq)
{
    if (!bits_ok(bits) || n < 0 || k < 0 || (k * bits) % 32 != 0)
        return -1;
    int64_t words = words_per_row(k, bits);
    for (int64_t r = 0; r < n; ++r) {
        uint32_t* row = wq + r * words;
        for (int64_t w = 0; w < words; ++w)
            row[w] = 0;
        for (int64_t i = 0; i < k; ++i) {
            uint32_t q = codes[r * k + i] & ((1u << bits) - 1u);
            int64_t bit = i * bits;
            int64_t w = bit / 32;
            int off = (int)(bit % 32);
            row[w] |= q << off;
            if (off + bits > 32) /* the lane runs on into the next word */
                row[w + 1] |= q >> (32 - off);
        }
    }
    return 0;
}

int qref_unpack(const uint32_t* wq, int64_t n, int64_t k, int bits, uint8_t* codes)
{
    if (!bits_ok(bits) || n < 0 || k < 0 || (k * bits) % 32 != 0)
        return -1;
    int64_t words = words_per_row(k, bits);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < k; ++i)
            codes[r * k + i] = (uint8_t)unpack_lane(wq + r * words, words, i, bits);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Quantize / dequantize                                               */
/* ------------------------------------------------------------------ */

static int args_ok(int64_t n, int64_t k, int bits, int group_size, int dtype)
{
    if (!bits_ok(bits) || n < 0 || k < 0 || group_size <= 0)
        return 0;
    if (k % group_size != 0 || (k * bits) % 32 != 0)
        return 0;
    return dtype == QREF_F32 || dtype == QREF_F16 || dtype == QREF_BF16;
}

int qref_quantize(const float* w, int64_t n, int64_t k, int bits, int group_size,
                  int sb_dtype, uint32_t* wq, void* scales, void* biases)
{
    if (!args_ok(n, k, bits, group_size, sb_dtype))
        return -1;
    int64_t groups = k / group_size;
    int64_t words = words_per_row(k, bits);
    float qmax = (float)((1 << bits) - 1);
    int failed = 0;
    /* Rows are independent; each thread packs its own rows. */
#pragma omp parallel reduction(| : failed)
    {
    uint8_t* codes = (uint8_t*)malloc((size_t)(k > 0 ? k : 1));
    if (!codes)
        failed = 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        if (!codes)
            continue;
        const float* wr = w + r * k;
        for (int64_t g = 0; g < groups; ++g) {
            const float* wg = wr + g * group_size;
            float mn = wg[0], mx = wg[0];
            for (int i = 1; i < group_size; ++i) {
                if (wg[i] < mn) mn = wg[i];
                if (wg[i] > mx) mx = wg[i];
            }
            float s = (mx - mn) / qmax;
            if (!(s >= FLT_EPSILON)) /* constant group: floor the scale */
                s = FLT_EPSILON;
            float sq = store_elem(scales, sb_dtype, r * groups + g, s);
            float bq = store_elem(biases, sb_dtype, r * groups + g, mn);
            if (bq == 0.0f) /* a zero bias is stored as +0 */
                bq = store_elem(biases, sb_dtype, r * groups + g, 0.0f);
            for (int i = 0; i < group_size; ++i) {
                float t = roundf((wg[i] - bq) / sq);
                if (t < 0.0f) t = 0.0f;
                if (t > qmax) t = qmax;
                codes[g * group_size + i] = (uint8_t)t;
            }
        }
        qref_pack(codes, 1, k, bits, wq + r * words);
    }
    free(codes);
    }
    return failed ? -1 : 0;
}

/* Dequantized weight (n_row's element i) in fp32: fp32(q) * s' + b'. */
static float dequant_elem(const uint32_t* row_wq, int64_t words, const void* scales,
                          const void* biases, int sb_dtype, int64_t sb_row_off, int64_t i,
                          int bits, int group_size)
{
    uint32_t q = unpack_lane(row_wq, words, i, bits);
    int64_t g = i / group_size;
    float s = load_elem(scales, sb_dtype, sb_row_off + g);
    float b = load_elem(biases, sb_dtype, sb_row_off + g);
    float prod = (float)q * s;
    return prod + b;
}

int qref_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                    int sb_dtype, int64_t n, int64_t k, int bits, int group_size,
                    float* w_out)
{
    if (!args_ok(n, k, bits, group_size, sb_dtype))
        return -1;
    int64_t groups = k / group_size, words = words_per_row(k, bits);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < k; ++i)
            w_out[r * k + i] = dequant_elem(wq + r * words, words, scales, biases, sb_dtype,
                                            r * groups, i, bits, group_size);
    return 0;
}

/* v rounded to nearest, ties to even, in element type `dtype`; the rounded
 * value is returned and, when `out` is non-null, stored at out[idx]. */
static double round_to_type(double v, int dtype, void* out, int64_t idx)
{
    switch (dtype) {
    case QREF_F32: {
        float f = (float)v; /* C's double -> float conversion rounds to nearest even */
        if (out)
            ((float*)out)[idx] = f;
        return f;
    }
    case QREF_F16: {
        uint16_t h = encode_rne_d(v, FMT_F16);
        if (out)
            ((uint16_t*)out)[idx] = h;
        return qref_f16_to_f32(h);
    }
    case QREF_BF16: {
        uint16_t h = encode_rne_d(v, FMT_BF16);
        if (out)
            ((uint16_t*)out)[idx] = h;
        return qref_bf16_to_f32(h);
    }
    }
    abort();
}

/* The dense weight in the scales' own type T (emily `dequantize_impl`: the
 * unpacked codes are cast to the scales' type, then multiplied by the scale
 * and added to the bias as two operations of that type). Each operation is
 * taken exactly in fp64 and rounded once to T: q < 2^8 times a scale of at
 * most 24 significant bits is exact in fp64, and so is the sum of two values
 * of T unless their exponents lie more than 29 apart, where the one fp64
 * rounding cannot change the nearest value of T (53 >= 2 * 24 + 2). */
int qref_dequantize_typed(const uint32_t* wq, const void* scales, const void* biases,
                          int sb_dtype, int64_t n, int64_t k, int bits, int group_size,
                          void* w_out)
{
    if (!args_ok(n, k, bits, group_size, sb_dtype))
        return -1;
    int64_t groups = k / group_size, words = words_per_row(k, bits);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < k; ++i) {
            double q = (double)unpack_lane(wq + r * words, words, i, bits);
            int64_t g = r * groups + i / group_size;
            double s = (double)load_elem(scales, sb_dtype, g);
            double b = (double)load_elem(biases, sb_dtype, g);
            double prod = round_to_type(q * s, sb_dtype, NULL, 0);
            round_to_type(prod + b, sb_dtype, w_out, r * k + i);
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Products                                                            */
/* ------------------------------------------------------------------ */

/* One output: sum over k of x_row[k] * w'[row, k] (fp64, k order). */
static void dot_row(const void* x, int x_dtype, int64_t x_off, const uint32_t* row_wq,
                    const void* scales, const void* biases, int sb_dtype, int64_t sb_off,
                    int64_t k, int bits, int group_size, double* y, double* S)
{
    int64_t words = words_per_row(k, bits);
    double acc = 0.0, mag = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        double xv = (double)load_elem(x, x_dtype, x_off + i);
        double wv = (double)dequant_elem(row_wq, words, scales, biases, sb_dtype, sb_off, i,
                                         bits, group_size);
        acc += xv * wv;
        mag += fabs(xv) * fabs(wv);
    }
    *y = acc;
    *S = mag;
}

int qref_qmatmul(const void* x, int x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                 const void* scales, const void* biases, int sb_dtype, int64_t n, int bits,
                 int group_size, double* y, double* S)
{
    if (!args_ok(n, k, bits, group_size, sb_dtype) || m < 0 || x_dtype < 0 || x_dtype > 2)
        return -1;
    int64_t groups = k / group_size, words = words_per_row(k, bits);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < n; ++c)
            dot_row(x, x_dtype, r * k, wq + c * words, scales, biases, sb_dtype, c * groups, k,
                    bits, group_size, &y[r * n + c], &S[r * n + c]);
    return 0;
}

int qref_qmatmul_sampled(const void* x, int x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                         const void* scales, const void* biases, int sb_dtype, int64_t n,
                         int bits, int group_size, const int64_t* mi, const int64_t* ni,
                         int64_t count, double* y, double* S)
{
    if (!args_ok(n, k, bits, group_size, sb_dtype) || m < 0 || x_dtype < 0 || x_dtype > 2)
        return -1;
    for (int64_t c = 0; c < count; ++c)
        if (mi[c] < 0 || mi[c] >= m || ni[c] < 0 || ni[c] >= n)
            return -1;
    int64_t groups = k / group_size, words = words_per_row(k, bits);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < count; ++c)
        dot_row(x, x_dtype, mi[c] * k, wq + ni[c] * words, scales, biases, sb_dtype,
                ni[c] * groups, k, bits, group_size, &y[c], &S[c]);
    return 0;
}

static int moe_args_ok(const int32_t* ids, int64_t pairs, int64_t num_experts)
{
    for (int64_t p = 0; p < pairs; ++p)
        if (ids[p] < 0 || ids[p] >= num_experts)
            return 0;
    return 1;
}

int qref_moe(const void* a, int a_dtype, const int32_t* ids, int64_t n_tokens, int64_t top_k,
             int64_t a_outer, int64_t a_inner, const uint32_t* wq, const void* scales,
             const void* biases, int sb_dtype, int64_t num_experts, int64_t n_rows,
             int64_t n_cols, int bits, int group_size, double* out, double* S)
{
    if (!args_ok(n_rows, n_cols, bits, group_size, sb_dtype) || n_tokens < 0 || top_k < 0)
        return -1;
    int64_t pairs = n_tokens * top_k;
    if (!moe_args_ok(ids, pairs, num_experts))
        return -2;
    int64_t groups = n_cols / group_size, words = words_per_row(n_cols, bits);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < pairs; ++p)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t a_off = (p / top_k) * a_outer + (p % top_k) * a_inner;
            int64_t row = (int64_t)ids[p] * n_rows + r; /* expert-major row index */
            dot_row(a, a_dtype, a_off, wq + row * words, scales, biases, sb_dtype,
                    row * groups, n_cols, bits, group_size, &out[p * n_rows + r],
                    &S[p * n_rows + r]);
        }
    return 0;
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

int qref_moe_gate_up_silu(const void* a, int a_dtype, const int32_t* ids, int64_t n_tokens,
                          int64_t top_k, int64_t a_outer, int64_t a_inner,
                          const uint32_t* gate_wq, const void* gate_s, const void* gate_b,
                          const uint32_t* up_wq, const void* up_s, const void* up_b,
                          int sb_dtype, int64_t num_experts, int64_t n_rows, int64_t n_cols,
                          int bits, int group_size, double* silu_out, double* g, double* u,
                          double* Sg, double* Su)
{
    int rc = qref_moe(a, a_dtype, ids, n_tokens, top_k, a_outer, a_inner, gate_wq, gate_s,
                      gate_b, sb_dtype, num_experts, n_rows, n_cols, bits, group_size, g, Sg);
    if (rc)
        return rc;
    rc = qref_moe(a, a_dtype, ids, n_tokens, top_k, a_outer, a_inner, up_wq, up_s, up_b,
                  sb_dtype, num_experts, n_rows, n_cols, bits, group_size, u, Su);
    if (rc)
        return rc;
    int64_t total = n_tokens * top_k * n_rows;
    for (int64_t i = 0; i < total; ++i)
        silu_out[i] = silu(g[i]) * u[i];
    return 0;
}

/* ------------------------------------------------------------------ */
/* The transpose = false layout                                        */
/* ------------------------------------------------------------------ */
/* emily `quantized_matmul/2` with transpose = false (the AWQ convention):
 * the packed weight is W [k, n], quantized along its last axis, so row i
 * holds n lanes with n / group_size groups, and y = x @ W':
 *   y[m, j] = sum_i x[m, i] * w'[i, j],  w'[i, j] = q[i, j] * s'[i, j/gs] + b'[i, j/gs]
 * with w' the fp32 dequantized weight of qref_dequantize (row i, lane j). */
int qref_qmatmul_t(const void* x, int x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                   const void* scales, const void* biases, int sb_dtype, int64_t n, int bits,
                   int group_size, double* y, double* S)
{
    if (!args_ok(k, n, bits, group_size, sb_dtype) || m < 0)
        return -1;
    int64_t groups = n / group_size, words = words_per_row(n, bits);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                double xv = (double)load_elem(x, x_dtype, mi * k + i);
                double wv = (double)dequant_elem(wq + i * words, words, scales, biases, sb_dtype,
                                                 i * groups, j, bits, group_size);
                double t_ij = xv * wv;
                acc += t_ij;
                mag += fabs(t_ij);
            }
            y[mi * n + j] = acc;
            S[mi * n + j] = mag;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Per-tensor dynamic-range int8                                       */
/* ------------------------------------------------------------------ */
/* mlex src/quant.rs, `quantize_dynamic_int8` / `dequantize_dynamic_int8`:
 * one output range [lo, hi] for the whole tensor; the signed int8 code q maps
 * affinely onto it, w = (q + 128) * ((hi - lo) / 255) + lo, each step an fp32
 * operation (cast, add, multiply, add). The quantizer takes lo / hi as the
 * tensor's min / max, floors its step at FLT_EPSILON, and codes
 * q = clamp(round((w - lo) / step) - 128, -128, 127), round half away. */
int qref_quantize_int8_tensor(const float* w, int64_t count, int8_t* q, float* range)
{
    if (count < 0)
        return -1;
    float lo = INFINITY, hi = -INFINITY;
    for (int64_t i = 0; i < count; ++i) {
        lo = fminf(lo, w[i]);
        hi = fmaxf(hi, w[i]);
    }
    float step = (hi - lo) / 255.0f;
    if (!(step >= FLT_EPSILON))
        step = FLT_EPSILON;
    for (int64_t i = 0; i < count; ++i) {
        float t = roundf((w[i] - lo) / step) - 128.0f;
        if (t < -128.0f) t = -128.0f;
        if (t > 127.0f) t = 127.0f;
        q[i] = (int8_t)t;
    }
    range[0] = lo;
    range[1] = hi;
    return 0;
}

static float int8_tensor_weight(int8_t q, float step, float lo)
{
    float shifted = (float)q + 128.0f;
    float scaled = shifted * step;
    return scaled + lo;
}

int qref_dequantize_int8_tensor(const int8_t* q, int64_t count, const float* range, float* w)
{
    if (count < 0)
        return -1;
    float step = (range[1] - range[0]) / 255.0f;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        w[i] = int8_tensor_weight(q[i], step, range[0]);
    return 0;
}

/* y[m,n] = sum_k x[m,k] * w[n,k] (fp64, k order) with w the dequantized
 * int8 weight [n, k]; S = sum |x||w|. */
int qref_qmatmul_int8_tensor(const void* x, int x_dtype, int64_t m, int64_t k, const int8_t* q,
                             const float* range, int64_t n, double* y, double* S)
{
    if (m < 0 || k < 0 || n < 0)
        return -1;
    float step = (range[1] - range[0]) / 255.0f;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t ni = 0; ni < n; ++ni) {
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                double xv = (double)load_elem(x, x_dtype, mi * k + i);
                double wv = (double)int8_tensor_weight(q[ni * k + i], step, range[0]);
                acc += xv * wv;
                mag += fabs(xv * wv);
            }
            y[mi * n + ni] = acc;
            S[mi * n + ni] = mag;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* MoE feed-forward block                                              */
/* ------------------------------------------------------------------ */
/* One MoE FFN block over stacked experts, as the ferrum-kernels MoE calls
 * chain (`gemv_moe_id_gate_up_silu` into `gemv_moe_id_batched`, each storing
 * its output in the activation type), closed by the weighted sum over each
 * token's top_k slots, which the pages leave to the caller:
 *   h[p]   = RNE_dt(SiLU(a_t Wg[e]^T) * (a_t Wu[e]^T)),   p = t*top_k + j, e = ids[p]
 *   o[p]   = RNE_dt(h[p] Wd[e]^T)
 *   out[t] = sum_j rw[t*top_k + j] * o[t*top_k + j]       (fp64, j in order)
 * a: [n_tokens, d_model]; gate / up: [E, d_ff, d_model*bits/32]; down:
 * [E, d_model, d_ff*bits/32]. h_out [P, d_ff] and o_out [P, d_model] receive
 * the rounded intermediates (storage of a_dtype); out is [n_tokens, d_model]. */
int qref_moe_ffn(const void* a, int a_dtype, const int32_t* ids, const float* rw,
                 int64_t n_tokens, int64_t top_k, const uint32_t* gate_wq, const void* gate_s,
                 const void* gate_b, const uint32_t* up_wq, const void* up_s, const void* up_b,
                 const uint32_t* down_wq, const void* down_s, const void* down_b, int sb_dtype,
                 int64_t num_experts, int64_t d_model, int64_t d_ff, int bits, int group_size,
                 double* out, void* h_out, void* o_out)
{
    int64_t P = n_tokens * top_k;
    size_t nh = (size_t)(P * d_ff > 0 ? P * d_ff : 1), no = (size_t)(P * d_model > 0 ? P * d_model : 1);
    double* silu_v = (double*)malloc(nh * sizeof(double));
    double* g = (double*)malloc(nh * sizeof(double));
    double* u = (double*)malloc(nh * sizeof(double));
    double* Sg = (double*)malloc(nh * sizeof(double));
    double* Su = (double*)malloc(nh * sizeof(double));
    double* o = (double*)malloc(no * sizeof(double));
    double* So = (double*)malloc(no * sizeof(double));
    int rc = -1;
    if (!silu_v || !g || !u || !Sg || !Su || !o || !So)
        goto done;
    rc = qref_moe_gate_up_silu(a, a_dtype, ids, n_tokens, top_k, d_model, 0, gate_wq, gate_s,
                               gate_b, up_wq, up_s, up_b, sb_dtype, num_experts, d_ff, d_model,
                               bits, group_size, silu_v, g, u, Sg, Su);
    if (rc)
        goto done;
    for (int64_t i = 0; i < P * d_ff; ++i)
        round_to_type(silu_v[i], a_dtype, h_out, i);
    rc = qref_moe(h_out, a_dtype, ids, n_tokens, top_k, top_k * d_ff, d_ff, down_wq, down_s,
                  down_b, sb_dtype, num_experts, d_model, d_ff, bits, group_size, o, So);
    if (rc)
        goto done;
    for (int64_t i = 0; i < P * d_model; ++i)
        round_to_type(o[i], a_dtype, o_out, i);
    for (int64_t t = 0; t < n_tokens; ++t)
        for (int64_t d = 0; d < d_model; ++d) {
            double acc = 0.0;
            for (int64_t j = 0; j < top_k; ++j) {
                int64_t p = t * top_k + j;
                acc += (double)rw[p] * (double)load_elem(o_out, a_dtype, p * d_model + d);
            }
            out[t * d_model + d] = acc;
        }
done:
    free(silu_v); free(g); free(u); free(Sg); free(Su); free(o); free(So);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Microscaled modes                                                   */
/* ------------------------------------------------------------------ */
/* emily lib/emily/quantization.ex, `dequantize_mxfp4_impl`,
 * `dequantize_mxfp8_impl`, `dequantize_nvfp4_impl`: no biases; each group of
 * gs lanes along a row shares one scale byte; w = lane_value * scale_value.
 *   mxfp4: 4-bit lanes, FP4-E2M1; gs 32; E8M0 scales.
 *   mxfp8: 8-bit lanes, FP8-E4M3 as MLX decodes it; gs 32; E8M0 scales.
 *   nvfp4: 4-bit lanes, FP4-E2M1; gs 16; FP8-E4M3 scales (MLX decode).
 * Group sizes: ollama x/create/client/quantize.go `quantizeParams` (nvfp4
 * 16, mxfp8 32) and the mxfp4 docs (one scale per 32 lanes). */

int qref_mx_params(int mode, int* bits, int* group_size)
{
    switch (mode) {
    case QREF_MXFP4: *bits = 4; *group_size = 32; return 0;
    case QREF_MXFP8: *bits = 8; *group_size = 32; return 0;
    case QREF_NVFP4: *bits = 4; *group_size = 16; return 0;
    }
    return -1;
}

/* FP4-E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; an
 * exponent field of 0 is subnormal (value = mantissa * 2^-1). */
double qref_fp4_e2m1(uint32_t c)
{
    double sign = (c & 8u) ? -1.0 : 1.0;
    int e = (int)((c >> 1) & 3u), m = (int)(c & 1u);
    double mag = e == 0 ? m * 0.5 : (1.0 + m / 2.0) * ldexp(1.0, e - 1);
    return sign * mag;
}

/* FP8-E4M3 as MLX decodes it (the pages' `fp8_e4m3_lut`): sign bit 7,
 * exponent bits 6..3 (bias 7), mantissa bits 2..0; an exponent field of 0 is
 * subnormal (mantissa * 2^-9). No code is NaN: 0x7F / 0xFF are +-480. */
double qref_fp8_e4m3(uint32_t b)
{
    double sign = (b & 0x80u) ? -1.0 : 1.0;
    int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
    double mag = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return sign * mag;
}

/* FP8-E8M0: 2^(s - 127) (the pages' `e8m0_lut`; s = 255 gives 2^128). */
double qref_e8m0(uint32_t s) { return ldexp(1.0, (int)s - 127); }

/* Element i of row r's dense weight, exactly (fp64 holds every product). */
static double mx_weight(const uint32_t* row_wq, int64_t words, const uint8_t* row_scales, int mode,
                        int bits, int group_size, int64_t i)
{
    uint32_t q = unpack_lane(row_wq, words, i, bits);
    uint32_t sb = row_scales[i / group_size];
    double lane = mode == QREF_MXFP8 ? qref_fp8_e4m3(q) : qref_fp4_e2m1(q);
    double scale = mode == QREF_NVFP4 ? qref_fp8_e4m3(sb) : qref_e8m0(sb);
    return lane * scale;
}

static int mx_args_ok(int mode, int64_t n, int64_t k, int* bits, int* group_size)
{
    if (qref_mx_params(mode, bits, group_size) != 0 || n < 0 || k < 0)
        return 0;
    return k % *group_size == 0 && (k * *bits) % 32 == 0;
}

int qref_mx_dequantize(const uint32_t* wq, const uint8_t* scales, int mode, int64_t n, int64_t k,
                       int out_dtype, void* w_out)
{
    int bits, gs;
    if (!mx_args_ok(mode, n, k, &bits, &gs))
        return -1;
    if (out_dtype != QREF_F32 && out_dtype != QREF_F16 && out_dtype != QREF_BF16)
        return -1;
    int64_t words = words_per_row(k, bits), groups = k / gs;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < k; ++i)
            round_to_type(mx_weight(wq + r * words, words, scales + r * groups, mode, bits, gs, i),
                          out_dtype, w_out, r * k + i);
    return 0;
}

int qref_mx_qmatmul(const void* x, int x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                    const uint8_t* scales, int mode, int64_t n, double* y, double* S)
{
    int bits, gs;
    if (!mx_args_ok(mode, n, k, &bits, &gs) || m < 0)
        return -1;
    if (x_dtype != QREF_F32 && x_dtype != QREF_F16 && x_dtype != QREF_BF16)
        return -1;
    int64_t words = words_per_row(k, bits), groups = k / gs;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t ni = 0; ni < n; ++ni) {
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                double xv = (double)load_elem(x, x_dtype, mi * k + i);
                double wv = mx_weight(wq + ni * words, words, scales + ni * groups, mode, bits,
                                      gs, i);
                double term = xv * wv;
                acc += term;
                mag += fabs(term);
            }
            y[mi * n + ni] = acc;
            S[mi * n + ni] = mag;
        }
    return 0;
}

int qref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
