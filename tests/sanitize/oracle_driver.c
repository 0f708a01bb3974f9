/*
 * oracle_driver.c — runs every oracle entry point once on small, ragged
 * shapes with buffers of exactly the documented sizes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize_host.py).
 * It checks return codes and a few identities; the numerical pins live in the
 * Python tests. Exit status 0 means every call returned what it should.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/qref.h"

static int failures = 0;
#define CHECK(cond, ...)                                                              \
    do {                                                                              \
        if (!(cond)) {                                                                \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);                      \
            fprintf(stderr, __VA_ARGS__);                                             \
            fprintf(stderr, "\n");                                                    \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 16);
}
static float next_f32(void) { return ((float)(next_u32() & 0xFFFFFF) / 16777216.0f) * 2.0f - 1.0f; }

static void* xmalloc(size_t n) { return malloc(n ? n : 1); }

static size_t esize(int dt) { return dt == QREF_F32 ? 4 : 2; }

/* Activations of element type dt, [m, k]. */
static void* make_x(int dt, int64_t m, int64_t k)
{
    void* x = xmalloc((size_t)(m * k) * esize(dt));
    for (int64_t i = 0; i < m * k; ++i) {
        const float v = next_f32();
        if (dt == QREF_F32)
            ((float*)x)[i] = v;
        else if (dt == QREF_F16)
            ((uint16_t*)x)[i] = qref_f32_to_f16(v);
        else
            ((uint16_t*)x)[i] = qref_f32_to_bf16(v);
    }
    return x;
}

static void dense(int bits, int gs, int dt, int64_t n, int64_t k, int64_t m)
{
    const int64_t words = k * bits / 32, groups = k / gs;
    float* w = xmalloc((size_t)(n * k) * 4);
    for (int64_t i = 0; i < n * k; ++i)
        w[i] = 0.02f * next_f32();
    uint32_t* wq = xmalloc((size_t)(n * words) * 4);
    void* s = xmalloc((size_t)(n * groups) * esize(dt));
    void* b = xmalloc((size_t)(n * groups) * esize(dt));
    CHECK(qref_quantize(w, n, k, bits, gs, dt, wq, s, b) == 0, "quantize b%d gs%d", bits, gs);

    uint8_t* codes = xmalloc((size_t)(n * k));
    uint32_t* wq2 = xmalloc((size_t)(n * words) * 4);
    CHECK(qref_unpack(wq, n, k, bits, codes) == 0, "unpack");
    CHECK(qref_pack(codes, n, k, bits, wq2) == 0, "pack");
    CHECK(memcmp(wq, wq2, (size_t)(n * words) * 4) == 0, "pack(unpack) b%d", bits);

    float* wd = xmalloc((size_t)(n * k) * 4);
    void* wt = xmalloc((size_t)(n * k) * esize(dt));
    CHECK(qref_dequantize(wq, s, b, dt, n, k, bits, gs, wd) == 0, "dequantize");
    CHECK(qref_dequantize_typed(wq, s, b, dt, n, k, bits, gs, wt) == 0, "dequantize_typed");

    void* x = make_x(dt, m, k);
    double* y = xmalloc((size_t)(m * n) * 8);
    double* S = xmalloc((size_t)(m * n) * 8);
    CHECK(qref_qmatmul(x, dt, m, k, wq, s, b, dt, n, bits, gs, y, S) == 0, "qmatmul");
    /* The product against the dequantized weights, recomputed here. */
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                const double xv = dt == QREF_F32 ? ((float*)x)[i * k + c]
                                  : dt == QREF_F16 ? qref_f16_to_f32(((uint16_t*)x)[i * k + c])
                                                   : qref_bf16_to_f32(((uint16_t*)x)[i * k + c]);
                acc += xv * (double)wd[j * k + c];
            }
            CHECK(fabs(acc - y[i * n + j]) <= 1e-9 * (1.0 + S[i * n + j]), "qmatmul (%ld, %ld)",
                  (long)i, (long)j);
        }
    int64_t mi[3] = {0, m - 1, m / 2}, ni[3] = {n - 1, 0, n / 2};
    double ys[3], Ss[3];
    CHECK(qref_qmatmul_sampled(x, dt, m, k, wq, s, b, dt, n, bits, gs, mi, ni, 3, ys, Ss) == 0,
          "qmatmul_sampled");
    for (int c = 0; c < 3; ++c)
        CHECK(ys[c] == y[mi[c] * n + ni[c]], "sampled %d", c);

    /* Transposed layout: W [k, n] packed along n (n a multiple of gs). */
    if (n % gs == 0) {
        const int64_t kt = n, nt = k;   /* reuse sizes: x [m, kt] */
        uint32_t* tq = xmalloc((size_t)(kt * (nt * bits / 32)) * 4);
        void* ts = xmalloc((size_t)(kt * (nt / gs)) * esize(dt));
        void* tb = xmalloc((size_t)(kt * (nt / gs)) * esize(dt));
        float* wt2 = xmalloc((size_t)(kt * nt) * 4);
        for (int64_t i = 0; i < kt * nt; ++i)
            wt2[i] = 0.02f * next_f32();
        CHECK(qref_quantize(wt2, kt, nt, bits, gs, dt, tq, ts, tb) == 0, "quantize t");
        void* xt = make_x(dt, m, kt);
        double* yt = xmalloc((size_t)(m * nt) * 8);
        double* St = xmalloc((size_t)(m * nt) * 8);
        CHECK(qref_qmatmul_t(xt, dt, m, kt, tq, ts, tb, dt, nt, bits, gs, yt, St) == 0, "qmatmul_t");
        free(tq); free(ts); free(tb); free(wt2); free(xt); free(yt); free(St);
    }
    CHECK(qref_quantize(w, n, k, 5, gs, dt, wq, s, b) != 0, "bits 5 rejected");
    free(w); free(wq); free(s); free(b); free(codes); free(wq2); free(wd); free(wt); free(x);
    free(y); free(S);
}

static void moe(int bits, int gs, int dt)
{
    const int64_t E = 5, R = 7, C = 2 * gs, T = 3, K = 2, P = T * K;
    const int64_t words = C * bits / 32, groups = C / gs;
    float* w = xmalloc((size_t)(E * R * C) * 4);
    uint32_t* gq = xmalloc((size_t)(E * R * words) * 4);
    uint32_t* uq = xmalloc((size_t)(E * R * words) * 4);
    void* gsc = xmalloc((size_t)(E * R * groups) * esize(dt));
    void* gb = xmalloc((size_t)(E * R * groups) * esize(dt));
    void* us = xmalloc((size_t)(E * R * groups) * esize(dt));
    void* ub = xmalloc((size_t)(E * R * groups) * esize(dt));
    for (int64_t i = 0; i < E * R * C; ++i)
        w[i] = 0.02f * next_f32();
    CHECK(qref_quantize(w, E * R, C, bits, gs, dt, gq, gsc, gb) == 0, "moe quantize gate");
    CHECK(qref_quantize(w, E * R, C, bits, gs, dt, uq, us, ub) == 0, "moe quantize up");
    void* a = make_x(dt, T, C);
    int32_t ids[6] = {4, 0, 2, 2, 1, 3};
    double* out = xmalloc((size_t)(P * R) * 8);
    double* S = xmalloc((size_t)(P * R) * 8);
    CHECK(qref_moe(a, dt, ids, T, K, C, 0, gq, gsc, gb, dt, E, R, C, bits, gs, out, S) == 0, "moe");
    double *so = xmalloc((size_t)(P * R) * 8), *g = xmalloc((size_t)(P * R) * 8),
           *u = xmalloc((size_t)(P * R) * 8), *Sg = xmalloc((size_t)(P * R) * 8),
           *Su = xmalloc((size_t)(P * R) * 8);
    CHECK(qref_moe_gate_up_silu(a, dt, ids, T, K, C, 0, gq, gsc, gb, uq, us, ub, dt, E, R, C, bits,
                                gs, so, g, u, Sg, Su) == 0, "moe gate_up");
    for (int64_t i = 0; i < P * R; ++i)
        CHECK(g[i] == out[i], "gate product equals the plain product at %ld", (long)i);
    int32_t bad[6] = {4, 0, 5, 2, 1, 3};
    CHECK(qref_moe(a, dt, bad, T, K, C, 0, gq, gsc, gb, dt, E, R, C, bits, gs, out, S) == -2,
          "moe rejects an out-of-range id");

    /* FFN block: d_model = C, d_ff = R rounded to the group size. */
    const int64_t dff = gs, dm = C;
    float* wf = xmalloc((size_t)(E * dff * dm) * 4);
    for (int64_t i = 0; i < E * dff * dm; ++i)
        wf[i] = 0.02f * next_f32();
    const int64_t wg = dm * bits / 32, gg = dm / gs, wd = dff * bits / 32, gd = dff / gs;
    uint32_t* fq = xmalloc((size_t)(E * dff * wg) * 4);
    void* fs = xmalloc((size_t)(E * dff * gg) * esize(dt));
    void* fb = xmalloc((size_t)(E * dff * gg) * esize(dt));
    uint32_t* dq = xmalloc((size_t)(E * dm * wd) * 4);
    void* ds = xmalloc((size_t)(E * dm * gd) * esize(dt));
    void* db = xmalloc((size_t)(E * dm * gd) * esize(dt));
    CHECK(qref_quantize(wf, E * dff, dm, bits, gs, dt, fq, fs, fb) == 0, "ffn quantize gate/up");
    CHECK(qref_quantize(wf, E * dm, dff, bits, gs, dt, dq, ds, db) == 0, "ffn quantize down");
    float rw[6] = {0.5f, 0.5f, 0.25f, 0.75f, 1.0f, 0.0f};
    double* fo = xmalloc((size_t)(T * dm) * 8);
    void* h = xmalloc((size_t)(P * dff) * esize(dt));
    void* o = xmalloc((size_t)(P * dm) * esize(dt));
    CHECK(qref_moe_ffn(a, dt, ids, rw, T, K, fq, fs, fb, fq, fs, fb, dq, ds, db, dt, E, dm, dff,
                       bits, gs, fo, h, o) == 0, "moe_ffn");
    free(w); free(gq); free(uq); free(gsc); free(gb); free(us); free(ub); free(a); free(out);
    free(S); free(so); free(g); free(u); free(Sg); free(Su); free(wf); free(fq); free(fs);
    free(fb); free(dq); free(ds); free(db); free(fo); free(h); free(o);
}

static void int8_tensor(void)
{
    const int64_t n = 9, k = 40, m = 3;
    float* w = xmalloc((size_t)(n * k) * 4);
    for (int64_t i = 0; i < n * k; ++i)
        w[i] = next_f32();
    int8_t* q = xmalloc((size_t)(n * k));
    float range[2];
    float* back = xmalloc((size_t)(n * k) * 4);
    CHECK(qref_quantize_int8_tensor(w, n * k, q, range) == 0, "int8 quantize");
    CHECK(qref_dequantize_int8_tensor(q, n * k, range, back) == 0, "int8 dequantize");
    void* x = make_x(QREF_BF16, m, k);
    double* y = xmalloc((size_t)(m * n) * 8);
    double* S = xmalloc((size_t)(m * n) * 8);
    CHECK(qref_qmatmul_int8_tensor(x, QREF_BF16, m, k, q, range, n, y, S) == 0, "int8 qmatmul");
    free(w); free(q); free(back); free(x); free(y); free(S);
}

static void mx(int mode)
{
    int bits = 0, gs = 0;
    CHECK(qref_mx_params(mode, &bits, &gs) == 0, "mx params %d", mode);
    const int64_t n = 5, k = 3 * gs, m = 2;
    uint32_t* wq = xmalloc((size_t)(n * k * bits / 32) * 4);
    uint8_t* sc = xmalloc((size_t)(n * k / gs));
    for (int64_t i = 0; i < n * k * bits / 32; ++i)
        wq[i] = next_u32();
    for (int64_t i = 0; i < n * k / gs; ++i)
        sc[i] = (uint8_t)(mode == QREF_NVFP4 ? (next_u32() % 0x70) : (120 + next_u32() % 16));
    uint16_t* wd = xmalloc((size_t)(n * k) * 2);
    CHECK(qref_mx_dequantize(wq, sc, mode, n, k, QREF_BF16, wd) == 0, "mx dequantize %d", mode);
    void* x = make_x(QREF_BF16, m, k);
    double* y = xmalloc((size_t)(m * n) * 8);
    double* S = xmalloc((size_t)(m * n) * 8);
    CHECK(qref_mx_qmatmul(x, QREF_BF16, m, k, wq, sc, mode, n, y, S) == 0, "mx qmatmul %d", mode);
    free(wq); free(sc); free(wd); free(x); free(y); free(S);
}

int main(void)
{
    const int bits[5] = {2, 3, 4, 6, 8};
    const int gss[3] = {32, 64, 128};
    for (int bi = 0; bi < 5; ++bi)
        for (int gi = 0; gi < 3; ++gi)
            for (int dt = 0; dt < 3; ++dt) {
                dense(bits[bi], gss[gi], dt, 3, 2 * gss[gi], 2);
                dense(bits[bi], gss[gi], dt, gss[gi], gss[gi], 3);   /* square: the transposed form */
            }
    for (int bi = 0; bi < 5; ++bi)
        for (int dt = 0; dt < 3; ++dt)
            moe(bits[bi], 32, dt);
    int8_tensor();
    for (int mode = 1; mode <= 3; ++mode)
        mx(mode);
    uint16_t h[4];
    float f[4] = {1.0f, -0.0f, 65504.0f, 1e-8f}, g2[4];
    qref_f32_to_bf16_n(f, h, 4);
    qref_bf16_to_f32_n(h, g2, 4);
    qref_f32_to_f16_n(f, h, 4);
    qref_f16_to_f32_n(h, g2, 4);
    CHECK(qref_num_threads() >= 1, "threads");
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all calls clean\n");
    return 0;
}
