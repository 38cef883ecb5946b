/*
 * mlap_oracle.c -- plain CPU oracle for the MLA Prolog.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code with the HIP path.
 *
 * It computes, one token row at a time, exactly what the method defines, in the
 * order the pages give and with the casts at the points they give:
 *
 *   GEMM  : Y = bf16(fp32(sum_k X[k] * W[n,k]))      products and sum in fp64
 *           ("PyPTO-Gym 算子设计模式 AT-10 ... MLAProlog 实战", section 二 and
 *            section 五: matmul with BF16 output dtype, weight laid out [N,K]).
 *   RMSNorm (variant B, sqrt then divide), fp32:
 *           x^2 -> *(1/D) -> row sum -> +eps -> sqrt -> 1/std -> x*rstd,
 *           then *fp32(gamma) and cast to bf16
 *           (same page, section 三 variant B; section 五 gamma applied by the caller
 *            in fp32, then cast to BF16).
 *   RoPE  : rotate-half, out = x*cos + rotate_half(x)*sin, rotate_half(x1,x2) = (-x2,x1),
 *           fp32 math, cast back to bf16
 *           ("PyPTO Operator 深度解析 (DeepSeek-V3.2-Exp)", section 3.3 QuantRope;
 *            "DeepSeek-V2-Lite-Chat MLA KV Prolog 迁移指南", section 精度验证).
 *   Quant : per row, fp32: amax = max|z|, m = 127/amax, code = rint(z*m) (half to even),
 *           saturated to [-127,127]; stored scale = amax/127
 *           ("PyPTO Operator 深度解析", section 3.1 PrologQuant;
 *            "PyPTO Gym 中的 grouped_matmul_swiglu_quant", sections 算子语义与数学公式
 *            and 实现特点 5).
 *   W8A8  : per-token activation quant (as above) -> int8 x int8 -> exact int32 ->
 *           dequant bf16(fp32(acc) * (x_scale[t] * w_scale[n]))
 *           ("PyPTO-Gym 算子设计模式 AT-10", section 四, INT8 W8A8 mode).
 *
 * Readings where the pages leave a step open are listed in the design notes; the
 * ones that shape the arithmetic here: head-major q_b/kv_b output with
 * [nope | rope] (q) or [nope | v] (kv_b) inside a head; kv_a output ordered
 * [c_kv | k_pe]; one q scale per token over all heads, taken after RoPE; an
 * all-zero row quantises to codes 0 and scale 0.
 *
 * Parity pins: every function here is pinned by the not-gpu tests against
 * closed forms, invariants, library routines or brute force; see tests/.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------- bf16 ---- */

/* Exact widening: a bf16 value is the top 16 bits of an IEEE fp32. */
static float orc_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t orc_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/*
 * fp32 -> bf16, round to nearest, ties to even, from the definition: take the
 * two bf16 neighbours of v (truncation and one unit up, in magnitude), compare
 * the distances exactly in fp64 and keep the nearer; on a tie keep the one whose
 * last mantissa bit is 0. Overflow past the largest finite bf16 rounds to inf
 * under the same rule. NaN stays NaN (quiet).
 */
ORC_API uint16_t orc_bf16(float v) {
    uint32_t u = orc_bits(v);
    if (isnan(v)) return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(v)) return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);              /* |lo| <= |v| (truncation) */
    if ((u & 0xffffu) == 0) return lo;              /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);               /* next magnitude up, same sign */
    double dv = (double)v;
    double dl = fabs(dv - (double)orc_f32(lo));
    double dh;
    if ((hi & 0x7f80u) == 0x7f80u) {
        /* hi is inf: measure against the value one ulp above the max finite */
        double maxf = (double)orc_f32((uint16_t)(lo | 0x7f7fu));
        double ulp = ldexp(1.0, 127 - 7);
        dh = fabs(fabs(dv) - (fabs(maxf) + ulp));
    } else {
        dh = fabs(dv - (double)orc_f32(hi));
    }
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1u) ? hi : lo;
}

ORC_API void orc_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16(in[i]);
}

/* ---------------------------------------------------------------- GEMM ---- */

/* One output: bf16(fp32(sum_k fp64(x_k) * fp64(w_k))). bf16 x bf16 products are
 * exact in fp64 (16 significant bits), so the fp64 sum is the exact sum up to
 * fp64 rounding; it is rounded once to fp32 (the accumulator type), then to bf16. */
static float orc_dot_bf16(const uint16_t* x, const uint16_t* w, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += (double)orc_f32(x[k]) * (double)orc_f32(w[k]);
    return (float)acc;
}

/* Y[m,n] = bf16(X[m,:] . W[n,:]); X [M,K], W [N,K], Y [M,N], all row-major. */
ORC_API void orc_gemm_bf16(const uint16_t* X, const uint16_t* W, int64_t M, int64_t N,
                           int64_t K, uint16_t* Y) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = orc_bf16(orc_dot_bf16(X + m * K, W + n * K, K));
}

/* C[m,n] = sum_k A[m,k] * B[n,k] exactly (int64 sum, checked to fit int32). */
ORC_API int orc_gemm_i8(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K,
                        int32_t* C) {
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
            if (acc > INT32_MAX || acc < INT32_MIN) bad = 1;
            C[m * N + n] = (int32_t)acc;
        }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------- RMSNorm ---- */

/* Variant B in fp32, step by step: sq_k = (y_k*y_k)*(1/D) each rounded to fp32,
 * mean_sq = their sum (fp64, rounded once to fp32), std = sqrt(mean_sq + eps),
 * rstd = 1/std, out_k = bf16((y_k*rstd)*f32(gamma_k)). gamma may be NULL (no gamma). */
ORC_API void orc_rmsnorm_row(const uint16_t* v, const uint16_t* gamma, int64_t D, float eps,
                             uint16_t* out) {
    const float invD = 1.0f / (float)D;
    double s = 0.0;
    for (int64_t k = 0; k < D; ++k) {
        float y = orc_f32(v[k]);
        float sq = y * y;
        float sqd = sq * invD;
        s += (double)sqd;
    }
    float mean_sq = (float)s;
    float var = mean_sq + eps;
    float stdv = sqrtf(var);
    float rstd = 1.0f / stdv;
    for (int64_t k = 0; k < D; ++k) {
        float y = orc_f32(v[k]) * rstd;
        if (gamma) y = y * orc_f32(gamma[k]);
        out[k] = orc_bf16(y);
    }
}

/* Variant A ([AT-10] section 三, AT-03 rsqrt_mode): sum of the squares (fp64, rounded once to
 * fp32), times 1/D in fp32 (= mean_sq), + eps, rstd = 1/sqrt(var) rounded once to fp32 (the
 * rsqrt), out_k = bf16((y_k*rstd)*f32(gamma_k)). */
ORC_API void orc_rmsnorm_row_rsqrt(const uint16_t* v, const uint16_t* gamma, int64_t D, float eps,
                                   uint16_t* out) {
    const float invD = 1.0f / (float)D;
    double s = 0.0;
    for (int64_t k = 0; k < D; ++k) {
        float y = orc_f32(v[k]);
        float sq = y * y;
        s += (double)sq;
    }
    float mean_sq = (float)s * invD;
    float var = mean_sq + eps;
    float rstd = (float)(1.0 / sqrt((double)var));
    for (int64_t k = 0; k < D; ++k) {
        float y = orc_f32(v[k]) * rstd;
        if (gamma) y = y * orc_f32(gamma[k]);
        out[k] = orc_bf16(y);
    }
}

/* ---------------------------------------------------------------- RoPE ---- */

/* Rotate-half RoPE of one R-wide slice u (bf16) with the token's cos/sin rows:
 * out_i     = u_i * c_i       + (-u_{i+h}) * s_i        (i < h = R/2)
 * out_{i+h} = u_{i+h} * c_{i+h} + u_i * s_{i+h}
 * each product rounded to fp32, then the fp32 sum, then bf16. */
ORC_API void orc_rope_row(const uint16_t* u, const float* c, const float* s, int64_t R,
                          uint16_t* out) {
    int64_t h = R / 2;
    for (int64_t i = 0; i < h; ++i) {
        float x1 = orc_f32(u[i]), x2 = orc_f32(u[i + h]);
        float a = x1 * c[i];
        float b = (-x2) * s[i];
        float lo = a + b;
        float d = x2 * c[i + h];
        float e = x1 * s[i + h];
        float hi = d + e;
        out[i] = orc_bf16(lo);
        out[i + h] = orc_bf16(hi);
    }
}

/* The QuantRope3D form ([V32] section 3.3): the slice is viewed as R/CHUNK chunks of CHUNK
 * values, the two axes are transposed, and rotate-half is applied to the result. With
 * CHUNK = 2 the transpose de-interleaves adjacent pairs (u_0 u_2 u_4 ... | u_1 u_3 ...), so
 * pair (2i, 2i+1) rotates with the cos/sin of columns i and i + R/2; the output keeps the
 * transposed (half-split) order. orc_rope_transpose is the first step on its own: t = the
 * [R/chunk, chunk] -> [chunk, R/chunk] transpose of u (t must not alias u). */
static void orc_rope_transpose(const uint16_t* u, int64_t R, int64_t chunk, uint16_t* t) {
    const int64_t nch = R / chunk;
    for (int64_t a = 0; a < nch; ++a)
        for (int64_t b = 0; b < chunk; ++b) t[b * nch + a] = u[a * chunk + b];
}

ORC_API void orc_rope_row_chunked(const uint16_t* u, const float* c, const float* s, int64_t R,
                                  int64_t chunk, uint16_t* out) {
    uint16_t t[1024];
    orc_rope_transpose(u, R, chunk, t);
    orc_rope_row(t, c, s, R, out);
}

/* --------------------------------------------------------------- Quant ---- */

/* Per-row symmetric dynamic INT8 quant of n bf16 values z (fp32 math). */
ORC_API void orc_quant_row(const uint16_t* z, int64_t n, int8_t* codes, float* scale) {
    float amax = 0.0f;
    for (int64_t k = 0; k < n; ++k) {
        float a = fabsf(orc_f32(z[k]));
        if (a > amax) amax = a;
    }
    if (!(amax > 0.0f)) {
        for (int64_t k = 0; k < n; ++k) codes[k] = 0;
        *scale = 0.0f;
        return;
    }
    float m = 127.0f / amax;
    for (int64_t k = 0; k < n; ++k) {
        float p = orc_f32(z[k]) * m;
        float r = rintf(p); /* default rounding mode: nearest, ties to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        codes[k] = (int8_t)r;
    }
    *scale = amax / 127.0f;
}

/* ------------------------------------------------------------- MXFP8 ---- */

/* The MXFP8 format of the grouped_matmul_swiglu_quant page (section 算子语义): FP8 E4M3 data
 * (OCP E4M3FN: sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities, 0x7F and
 * 0xFF are NaN) and one E8M0 scale 2^(e-127) per 32-element block along K. */
ORC_API double orc_e4m3_value(uint8_t c) {
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                 /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* Nearest E4M3 value to v, ties to even, saturating at +-448 (the largest finite value). */
ORC_API double orc_e4m3_round(double v) {
    const double a = fabs(v);
    double q;
    if (a >= 448.0) {
        q = 448.0;
    } else if (a < 0x1p-6) {
        q = nearbyint(a * 512.0) / 512.0;        /* subnormal grid: steps of 2^-9 */
    } else {
        int e;
        frexp(a, &e);                            /* a in [2^(e-1), 2^e) */
        const double step = ldexp(1.0, e - 1 - 3);
        q = nearbyint(a / step) * step;
        if (q > 448.0) q = 448.0;
    }
    return v < 0 ? -q : q;
}

/* MX conversion of one row of n bf16 values (n a multiple of 32), block by block: the
 * shared exponent is floor(log2(amax)) - 8 (8 = the largest exponent of E4M3), clamped to
 * E8M0's range, and each value divided by 2^shared rounds to E4M3. Writes the dequantised
 * values (code * 2^shared, exact in bf16 within its exponent range) and the E8M0 bytes. */
ORC_API void orc_mx_quant_row(const uint16_t* v, int64_t n, uint16_t* deq, uint8_t* scales) {
    for (int64_t b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int k = 0; k < 32; ++k) {
            const double a = fabs((double)orc_f32(v[b * 32 + k]));
            if (a > amax) amax = a;
        }
        int sh = -127;
        if (amax > 0.0) {
            int e;
            frexp(amax, &e);
            sh = (e - 1) - 8;
            if (sh < -127) sh = -127;
            if (sh > 127) sh = 127;
        }
        if (scales) scales[b] = (uint8_t)(sh + 127);
        for (int k = 0; k < 32; ++k) {
            const double x = (double)orc_f32(v[b * 32 + k]);
            const double q = amax > 0.0 ? orc_e4m3_round(ldexp(x, -sh)) : 0.0;
            deq[b * 32 + k] = orc_bf16((float)ldexp(q, sh));
        }
    }
}

/* Dequant of one int32 accumulator: bf16(fp32(acc) * (xs * ws)). */
static uint16_t orc_dequant(int32_t acc, float xs, float ws) {
    float sc = xs * ws;
    float y = (float)acc * sc;
    return orc_bf16(y);
}

/* --------------------------------------------------------------- Prolog --- */

typedef struct {
    int32_t hidden, q_lora, kv_lora, rope_dim, nope_dim, v_dim, n_heads, max_pos;
    float eps;
    int32_t w8a8;
    int32_t norm_rsqrt;       /* RMSNorm variant A instead of B */
    int32_t rope_chunk;       /* 0: rotate-half on the slice as is; else the QuantRope3D form */
    int32_t q_quant_per_head; /* q codes and scales per (token, head) instead of per token */
    int32_t q_head_norm;      /* RMSNorm (no gamma) of every q head after q_b, before RoPE */
    int32_t mxfp8;            /* MXFP8 projections: E4M3 weights with E8M0 block scales */
} orc_cfg;

typedef struct {
    const uint16_t* x;        /* [T, hidden] bf16 */
    const int32_t* positions; /* [T] */
    const void* w_qa;         /* [q_lora, hidden]: bf16, or int8 when w8a8 */
    const void* w_qb;         /* [H*(nope+rope), q_lora] */
    const void* w_kva;        /* [kv_lora+rope, hidden] */
    const void* w_kvb;        /* [H*(nope+v), kv_lora] */
    const float* ws_qa;       /* W8A8 per-output-channel scales [N] */
    const float* ws_qb;
    const float* ws_kva;
    const float* ws_kvb;
    const uint16_t* gamma_q;  /* [q_lora] bf16 */
    const uint16_t* gamma_kv; /* [kv_lora] bf16 */
    const float* cos;         /* [max_pos, rope] fp32 */
    const float* sin;
    const uint8_t* ms_qa;     /* MXFP8: E8M0 block scales [N, K/32] of each weight */
    const uint8_t* ms_qb;
    const uint8_t* ms_kva;
    const uint8_t* ms_kvb;
} orc_inputs;

typedef struct { /* every array is [nrows, ...] in the order of rows[] */
    uint16_t* q_nope;   /* [nrows, H, nope] */
    uint16_t* q_pe;     /* [nrows, H, rope] */
    uint16_t* kv_norm;  /* [nrows, kv_lora] */
    uint16_t* k_pe;     /* [nrows, rope] */
    uint16_t* k_nope;   /* [nrows, H, nope] (kv_b) */
    uint16_t* value;    /* [nrows, H, v] (kv_b) */
    uint16_t* q_norm;   /* [nrows, q_lora] */
    int8_t* q_i8;       /* [nrows, H, nope+rope] */
    float* q_scale;     /* [nrows], or [nrows, H] per head */
    int8_t* kv_i8;      /* [nrows, kv_lora] */
    float* kv_scale;    /* [nrows] */
} orc_outputs;

static void orc_norm(const orc_cfg* cfg, const uint16_t* v, const uint16_t* gamma, int64_t D,
                     uint16_t* out) {
    if (cfg->norm_rsqrt)
        orc_rmsnorm_row_rsqrt(v, gamma, D, cfg->eps, out);
    else
        orc_rmsnorm_row(v, gamma, D, cfg->eps, out);
}

/* A raw rope slice put in the order the rotate-half takes it, in place: the QuantRope3D
 * transpose when the configuration uses that form, else nothing. */
static void orc_rope_order(const orc_cfg* cfg, uint16_t* u, int64_t R) {
    if (cfg->rope_chunk <= 0) return;
    uint16_t t[1024];
    orc_rope_transpose(u, R, cfg->rope_chunk, t);
    memcpy(u, t, sizeof(uint16_t) * (size_t)R);
}

/* One projection of one bf16 row v (length K) through W [N,K]: bf16, W8A8 or MXFP8
 * (the AT-09 Linear modes of the AT-10 card, section 四). MXFP8: scaled_mm with an fp32
 * result, sum_k deq(x_k) * deq(w_nk) with x converted to MX block by block, then the bf16
 * cast point of the projection. */
static void orc_project(const orc_cfg* cfg, const uint16_t* v, int64_t K, const void* W,
                        const float* ws, const uint8_t* ms, int64_t N, uint16_t* out,
                        int8_t* tmp_codes) {
    if (cfg->mxfp8) {
        uint16_t* xd = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)K);
        orc_mx_quant_row(v, K, xd, NULL);
        const uint8_t* Wc = (const uint8_t*)W;
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double w = ldexp(orc_e4m3_value(Wc[n * K + k]), (int)ms[n * (K / 32) + k / 32] - 127);
                s += (double)orc_f32(xd[k]) * w;
            }
            out[n] = orc_bf16((float)s);
        }
        free(xd);
        return;
    }
    if (!cfg->w8a8) {
        const uint16_t* Wb = (const uint16_t*)W;
        for (int64_t n = 0; n < N; ++n) out[n] = orc_bf16(orc_dot_bf16(v, Wb + n * K, K));
        return;
    }
    const int8_t* Wq = (const int8_t*)W;
    float xs;
    orc_quant_row(v, K, tmp_codes, &xs);
    for (int64_t n = 0; n < N; ++n) {
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k) acc += (int64_t)tmp_codes[k] * (int64_t)Wq[n * K + k];
        out[n] = orc_dequant((int32_t)acc, xs, ws[n]);
    }
}

/* Rows that stand in for the oracle's own intermediate results of the same rows, so a caller
 * can check one step of the chain on exactly the inputs another implementation fed that step
 * (every array optional, [nrows, ...] bf16 in the order of rows[]). Every rope slice in these
 * rows (and in the taps below) is in the order the rotate-half takes it: with the QuantRope3D
 * form, already transposed (orc_rope_transpose). */
typedef struct {
    const uint16_t* a;    /* [nrows, Lq + Lkv + R]: the down projection [q_a | c_kv | k_pe raw] */
    const uint16_t* qn;   /* [nrows, Lq]: q_norm, the input of the q_b projection */
    const uint16_t* kvn;  /* [nrows, Lkv]: kv_norm, the input of the kv_b projection */
    const uint16_t* qraw; /* [nrows, H, Dn + R]: the q_b projection per head, before any head norm */
    const uint16_t* qpe;  /* [nrows, H, R]: each head's rope slice just before RoPE */
} orc_given;

/* The oracle's own intermediate results (every array optional, [nrows, ...] bf16). */
typedef struct {
    uint16_t* a_proj; /* [nrows, Lq + Lkv + R]: the down projection */
    uint16_t* q_proj; /* [nrows, H, Dn + R]: the q_b projection of the q_b input in use */
    uint16_t* q_pre;  /* [nrows, H, R]: each head's rope slice just before RoPE (after the head
                         norm when there is one) */
} orc_taps;

/* Full prolog for the token rows listed in rows[0..nrows). NULL outputs are skipped. `given`
 * (optional) replaces intermediate rows as described above: everything downstream of a given
 * row is computed from it, the rest of the chain is unchanged. `taps` (optional) receives
 * intermediate rows. Returns 0, or -1 on an argument the oracle does not accept. */
ORC_API int orc_prolog_staged(const orc_cfg* cfg, const orc_inputs* in, const int32_t* rows,
                              int32_t nrows, const orc_given* given, const orc_outputs* out,
                              const orc_taps* taps) {
    const int64_t Hd = cfg->hidden, Lq = cfg->q_lora, Lkv = cfg->kv_lora, R = cfg->rope_dim;
    const int64_t Dn = cfg->nope_dim, Dv = cfg->v_dim, H = cfg->n_heads;
    const int64_t QH = Dn + R, KH = Dn + Dv, N1 = Lq + Lkv + R;
    static const orc_given no_given;
    static const orc_taps no_taps;
    if (!given) given = &no_given;
    if (!taps) taps = &no_taps;
    if (R <= 0 || (R & 1) || Lkv <= 0 || Hd <= 0) return -1;
    if (cfg->rope_chunk < 0 || (cfg->rope_chunk > 0 && (R % cfg->rope_chunk || R > 1024))) return -1;
    for (int32_t i = 0; i < nrows; ++i) {
        int32_t p = in->positions[rows[i]];
        if (p < 0 || p >= cfg->max_pos) return -1;
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t i = 0; i < nrows; ++i) {
        const int64_t t = rows[i];
        const uint16_t* x = in->x + t * Hd;
        const int64_t p = in->positions[t];
        const float* c = in->cos + p * R;
        const float* s = in->sin + p * R;
        int64_t maxK = Hd > Lq ? Hd : Lq;
        if (Lkv > maxK) maxK = Lkv;
        int64_t maxN = H * (QH > KH ? QH : KH);
        if (N1 > maxN) maxN = N1;
        uint16_t* A = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N1);
        uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)maxN);
        uint16_t* qn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(Lq > 0 ? Lq : 1));
        uint16_t* kvn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)Lkv);
        uint16_t* qrow = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(H * QH));
        int8_t* codes = (int8_t*)malloc((size_t)(maxK > H * QH ? maxK : H * QH));
        if (!A || !y || !qn || !kvn || !qrow || !codes) {
            bad = 1;
            free(A); free(y); free(qn); free(kvn); free(qrow); free(codes);
            continue;
        }

        /* down projection A = [q_a | c_kv | k_pe raw]: x . W_qa^T and x . W_kva^T */
        if (given->a) {
            memcpy(A, given->a + i * N1, sizeof(uint16_t) * (size_t)N1);
        } else {
            if (Lq > 0) orc_project(cfg, x, Hd, in->w_qa, in->ws_qa, in->ms_qa, Lq, A, codes);
            orc_project(cfg, x, Hd, in->w_kva, in->ws_kva, in->ms_kva, Lkv + R, A + Lq, codes);
            orc_rope_order(cfg, A + Lq + Lkv, R);
        }
        if (taps->a_proj) memcpy(taps->a_proj + i * N1, A, sizeof(uint16_t) * (size_t)N1);

        /* kv branch: RMSNorm of c_kv, RoPE of k_pe, quant of kv_norm */
        const uint16_t* ckv = A + Lq;
        orc_norm(cfg, ckv, in->gamma_kv, Lkv, kvn);
        if (out->kv_norm) memcpy(out->kv_norm + i * Lkv, kvn, sizeof(uint16_t) * (size_t)Lkv);
        if (out->k_pe) orc_rope_row(ckv + Lkv, c, s, R, out->k_pe + i * R);
        if (out->kv_i8 || out->kv_scale) {
            float sc;
            orc_quant_row(kvn, Lkv, codes, &sc);
            if (out->kv_i8) memcpy(out->kv_i8 + i * Lkv, codes, (size_t)Lkv);
            if (out->kv_scale) out->kv_scale[i] = sc;
        }
        if (Dv > 0) { /* kv_b projection of the normalised compressed KV */
            const uint16_t* kv_src = given->kvn ? given->kvn + i * Lkv : kvn;
            orc_project(cfg, kv_src, Lkv, in->w_kvb, in->ws_kvb, in->ms_kvb, H * KH, y, codes);
            for (int64_t h = 0; h < H; ++h) {
                if (out->k_nope)
                    memcpy(out->k_nope + (i * H + h) * Dn, y + h * KH, sizeof(uint16_t) * (size_t)Dn);
                if (out->value)
                    memcpy(out->value + (i * H + h) * Dv, y + h * KH + Dn, sizeof(uint16_t) * (size_t)Dv);
            }
        }

        /* q branch: RMSNorm*gamma of q_a -> q_b projection -> split, [head norm], RoPE -> quant */
        if (Lq > 0) {
            orc_norm(cfg, A, in->gamma_q, Lq, qn);
            if (out->q_norm) memcpy(out->q_norm + i * Lq, qn, sizeof(uint16_t) * (size_t)Lq);
            const uint16_t* q_src = given->qn ? given->qn + i * Lq : qn;
            orc_project(cfg, q_src, Lq, in->w_qb, in->ws_qb, in->ms_qb, H * QH, y, codes);
            for (int64_t h = 0; h < H; ++h) orc_rope_order(cfg, y + h * QH + Dn, R);
            if (taps->q_proj) memcpy(taps->q_proj + i * H * QH, y, sizeof(uint16_t) * (size_t)(H * QH));
            if (given->qraw) memcpy(y, given->qraw + i * H * QH, sizeof(uint16_t) * (size_t)(H * QH));
            if (cfg->q_head_norm) /* [AT-10] section 九: q_b -> reshape (heads, head_dim) -> RMSNorm */
                for (int64_t h = 0; h < H; ++h) orc_norm(cfg, y + h * QH, NULL, QH, y + h * QH);
            for (int64_t h = 0; h < H; ++h) {
                const uint16_t* head = y + h * QH;
                uint16_t* qh = qrow + h * QH;
                const uint16_t* pe = given->qpe ? given->qpe + (i * H + h) * R : head + Dn;
                if (taps->q_pre) memcpy(taps->q_pre + (i * H + h) * R, head + Dn, sizeof(uint16_t) * (size_t)R);
                memcpy(qh, head, sizeof(uint16_t) * (size_t)Dn);
                orc_rope_row(pe, c, s, R, qh + Dn);
                if (out->q_nope) memcpy(out->q_nope + (i * H + h) * Dn, qh, sizeof(uint16_t) * (size_t)Dn);
                if (out->q_pe) memcpy(out->q_pe + (i * H + h) * R, qh + Dn, sizeof(uint16_t) * (size_t)R);
            }
            if ((out->q_i8 || out->q_scale) && cfg->q_quant_per_head) {
                for (int64_t h = 0; h < H; ++h) {  /* each head's [nope | pe] row on its own */
                    float sc;
                    orc_quant_row(qrow + h * QH, QH, codes, &sc);
                    if (out->q_i8) memcpy(out->q_i8 + (i * H + h) * QH, codes, (size_t)QH);
                    if (out->q_scale) out->q_scale[i * H + h] = sc;
                }
            } else if (out->q_i8 || out->q_scale) {
                float sc;
                orc_quant_row(qrow, H * QH, codes, &sc);
                if (out->q_i8) memcpy(out->q_i8 + i * H * QH, codes, (size_t)(H * QH));
                if (out->q_scale) out->q_scale[i] = sc;
            }
        }
        free(A); free(y); free(qn); free(kvn); free(qrow); free(codes);
    }
    return bad ? -1 : 0;
}

ORC_API int orc_prolog(const orc_cfg* cfg, const orc_inputs* in, const int32_t* rows,
                       int32_t nrows, const orc_outputs* out) {
    return orc_prolog_staged(cfg, in, rows, nrows, NULL, out, NULL);
}

/* ------------------------------------------------------------ KV cache --- */

/* The KV cache write: the prolog's per-token rows placed at their tokens' cache rows, the
 * ScatterUpdate of the results into the K cache named in the [V32] page (section 2.4) and
 * the caching of the per-row quantised rows in step 2 of the [BLOG] page. Row t of src
 * (row_bytes each) goes to row slots[t] of dst when 0 <= slots[t] < n_slots; every other
 * row of dst is left as it was. Returns -1 if two in-range slots of the run coincide (the
 * caller's contract), else 0. */
ORC_API int orc_cache_scatter(const int32_t* slots, int32_t T, int32_t n_slots, const void* src,
                              int64_t row_bytes, void* dst) {
    for (int32_t t = 0; t < T; ++t) {
        const int32_t s = slots[t];
        if (s < 0 || s >= n_slots) continue;
        for (int32_t u = 0; u < t; ++u)
            if (slots[u] == s) return -1;
        memcpy((char*)dst + (size_t)s * (size_t)row_bytes, (const char*)src + (size_t)t * (size_t)row_bytes,
               (size_t)row_bytes);
    }
    return 0;
}

/* Threads the OpenMP loops use from now on (the CPU-baseline timing runs the oracle on all
 * host cores and on one). */
ORC_API void orc_set_num_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
