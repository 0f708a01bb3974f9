/*
 * qref.h — the oracle: a plain, slow CPU implementation of affine group
 * quantization, bit packing, dequantization and the quantized matmul / MoE
 * products.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do. It shares no code, header or table with
 * the HIP library.
 *
 * Element-type codes used by every function below (the oracle's own
 * numbering, independent of the library's):
 *   0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16 (top half of an fp32).
 *
 * Parity pins: every function here is pinned by the CPU tests (closed forms,
 * printed examples, brute force, library routines), except agreement with the
 * MLX quantizer itself, which the pages never print values for ("parity
 * unpinned": the readings in qref.c fix our own quantizer, not MLX's).
 */
#ifndef QREF_H
#define QREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QREF_F32 = 0, QREF_F16 = 1, QREF_BF16 = 2 };

/* Scalar conversions. fp32 -> 16-bit formats round to nearest, ties to even. */
uint16_t qref_f32_to_bf16(float f);
uint16_t qref_f32_to_f16(float f);
float qref_bf16_to_f32(uint16_t h);
float qref_f16_to_f32(uint16_t h);
/* Bulk forms (for exhaustive checks). */
void qref_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n);
void qref_f32_to_f16_n(const float* in, uint16_t* out, int64_t n);
void qref_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n);
void qref_f16_to_f32_n(const uint16_t* in, float* out, int64_t n);

/* Codes <-> packed little-endian u32 stream, row by row.
 * codes: [n, k] u8 (values < 2^bits); wq: [n, k*bits/32] u32. */
int qref_pack(const uint8_t* codes, int64_t n, int64_t k, int bits, uint32_t* wq);
int qref_unpack(const uint32_t* wq, int64_t n, int64_t k, int bits, uint8_t* codes);

/* Affine group quantization of w[n,k] (fp32) into packed codes plus one
 * scale and one bias per group, stored in element type sb_dtype.
 * scales, biases: [n, k/group_size]. Returns 0, or -1 on bad arguments. */
int qref_quantize(const float* w, int64_t n, int64_t k, int bits, int group_size,
                  int sb_dtype, uint32_t* wq, void* scales, void* biases);

/* Dequantize to fp32: w'[n,k] = fp32(q) * s' + b' (multiply, then add). */
int qref_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                    int sb_dtype, int64_t n, int64_t k, int bits, int group_size,
                    float* w_out);

/* Dense weight in the scales' own element type sb_dtype (w_out: [n,k] of that
 * type): cast the code to that type, then multiply by the scale and add the
 * bias, each operation rounded to nearest even in that type. For fp32 scales
 * this equals qref_dequantize. */
int qref_dequantize_typed(const uint32_t* wq, const void* scales, const void* biases,
                          int sb_dtype, int64_t n, int64_t k, int bits, int group_size,
                          void* w_out);

/* y[m,n] = sum_k x[m,k] * w'[n,k] in fp64, in k order, plus
 * S[m,n] = sum_k |x[m,k]| * |w'[n,k]| (the scale of the error bound).
 * x: [m,k] of element type x_dtype. y, S: [m,n] fp64. */
int qref_qmatmul(const void* x, int x_dtype, int64_t m, int64_t k,
                 const uint32_t* wq, const void* scales, const void* biases,
                 int sb_dtype, int64_t n, int bits, int group_size,
                 double* y, double* S);

/* The same product at `count` sampled output positions (mi[c], ni[c]). */
int qref_qmatmul_sampled(const void* x, int x_dtype, int64_t m, int64_t k,
                         const uint32_t* wq, const void* scales, const void* biases,
                         int sb_dtype, int64_t n, int bits, int group_size,
                         const int64_t* mi, const int64_t* ni, int64_t count,
                         double* y, double* S);

/* MoE over stacked experts, one (token, slot) pair at a time.
 * Pair p = t*top_k + j reads the activation row a + t*a_outer + j*a_inner
 * (element offsets) and expert ids[p]'s weights:
 *   wq: [E, n_rows, n_cols*bits/32], scales/biases: [E, n_rows, n_cols/gs].
 * out, S: [n_tokens*top_k, n_rows] fp64. Returns -2 if an id is out of range. */
int qref_moe(const void* a, int a_dtype, const int32_t* ids, int64_t n_tokens,
             int64_t top_k, int64_t a_outer, int64_t a_inner,
             const uint32_t* wq, const void* scales, const void* biases, int sb_dtype,
             int64_t num_experts, int64_t n_rows, int64_t n_cols, int bits,
             int group_size, double* out, double* S);

/* Fused gate/up: silu_out[p,r] = SiLU(g) * u with g, u the gate and up
 * products of pair p, row r (fp64). Also returns g, u and their S terms. */
int qref_moe_gate_up_silu(const void* a, int a_dtype, const int32_t* ids,
                          int64_t n_tokens, int64_t top_k, int64_t a_outer,
                          int64_t a_inner,
                          const uint32_t* gate_wq, const void* gate_s, const void* gate_b,
                          const uint32_t* up_wq, const void* up_s, const void* up_b,
                          int sb_dtype, int64_t num_experts, int64_t n_rows,
                          int64_t n_cols, int bits, int group_size,
                          double* silu_out, double* g, double* u, double* Sg, double* Su);

/* transpose = false: wq packs W [k, n] along n (wq: [k, n*bits/32], scales /
 * biases: [k, n/gs]); y[m, j] = sum_i x[m, i] * w'[i, j] in fp64, in i order,
 * and S = sum |x||w'|. */
int qref_qmatmul_t(const void* x, int x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                   const void* scales, const void* biases, int sb_dtype, int64_t n, int bits,
                   int group_size, double* y, double* S);

/* Per-tensor dynamic-range int8 (one range [lo, hi] = range[0..1] for the
 * whole tensor): w = (q + 128) * ((hi - lo) / 255) + lo in fp32 steps. The
 * quantizer sets the range to the tensor's min / max. */
int qref_quantize_int8_tensor(const float* w, int64_t count, int8_t* q, float* range);
int qref_dequantize_int8_tensor(const int8_t* q, int64_t count, const float* range, float* w);
int qref_qmatmul_int8_tensor(const void* x, int x_dtype, int64_t m, int64_t k, const int8_t* q,
                             const float* range, int64_t n, double* y, double* S);

/* MoE FFN block: gate+up+SiLU, down, then out[t] = sum_j rw[t*top_k+j] *
 * o[t*top_k+j] in fp64, with the intermediates h [P, d_ff] and o [P, d_model]
 * rounded to a_dtype (returned in h_out / o_out). out: [n_tokens, d_model]. */
int qref_moe_ffn(const void* a, int a_dtype, const int32_t* ids, const float* rw,
                 int64_t n_tokens, int64_t top_k, const uint32_t* gate_wq, const void* gate_s,
                 const void* gate_b, const uint32_t* up_wq, const void* up_s, const void* up_b,
                 const uint32_t* down_wq, const void* down_s, const void* down_b, int sb_dtype,
                 int64_t num_experts, int64_t d_model, int64_t d_ff, int bits, int group_size,
                 double* out, void* h_out, void* o_out);

/* Microscaled modes: no biases, one scale byte per group of lanes.
 *   mode 1 = mxfp4 (4-bit FP4-E2M1 lanes, gs 32, E8M0 scales),
 *   mode 2 = mxfp8 (8-bit FP8-E4M3 lanes as MLX decodes them, gs 32, E8M0),
 *   mode 3 = nvfp4 (4-bit FP4-E2M1 lanes, gs 16, FP8-E4M3 scales).
 * wq: [n, k*bits/32] packed as above; scales: [n, k/gs] u8. */
enum { QREF_MXFP4 = 1, QREF_MXFP8 = 2, QREF_NVFP4 = 3 };
int qref_mx_params(int mode, int* bits, int* group_size);
double qref_fp4_e2m1(uint32_t code);
double qref_fp8_e4m3(uint32_t byte);
double qref_e8m0(uint32_t byte);
/* Dense weight lane * scale (exact in fp64), rounded to nearest even in
 * out_dtype (0/1/2 as above); w_out: [n, k]. */
int qref_mx_dequantize(const uint32_t* wq, const uint8_t* scales, int mode, int64_t n,
                       int64_t k, int out_dtype, void* w_out);
/* y[m,n] = sum_k x[m,k] * w[n,k] in fp64 in k order, and S = sum |x||w|. */
int qref_mx_qmatmul(const void* x, int x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                    const uint8_t* scales, int mode, int64_t n, double* y, double* S);

/* Number of OpenMP threads the oracle's parallel loops use. */
int qref_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
