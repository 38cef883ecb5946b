/*
 * mlap.h -- C ABI of the MI355X (gfx950) MLA Prolog library, libmlap.so.
 *
 * The MLA Prolog is the per-token stage in front of DeepSeek's multi-head latent
 * attention. For every token row it computes
 *
 *   A      = x . [W_qa ; W_kva]^T                 bf16 out, fp32 accumulate
 *   q_norm = bf16(RMSNorm(A[:, :q_lora]) * gamma_q)
 *   kv_norm= bf16(RMSNorm(A[:, q_lora:q_lora+kv_lora]) * gamma_kv)
 *   k_pe   = RoPE(A[:, q_lora+kv_lora:])
 *   Q      = q_norm . W_qb^T  -> per head [q_nope | q_pe_raw], q_pe = RoPE(q_pe_raw)
 *   KVB    = kv_norm . W_kvb^T -> per head [k_nope | value]      (KV-Prolog mode)
 *   q_i8, q_scale  = per-token INT8 quant of all heads' [q_nope | q_pe]
 *   kv_i8, kv_scale= per-token INT8 quant of kv_norm
 *
 * Passages this follows (page title, section):
 *   - the q_a -> RMSNorm -> *gamma -> bf16 -> q_b chain and the parallel kv branch:
 *     "PyPTO-Gym 算子设计模式 AT-10：RMSNorm + Linear 融合（V→C 排布）的原理与 MLAProlog
 *     实战", section 五 (MLAProlog, DeepSeek-V4 source walk-through) and section 二
 *     (norm in FP32, cast to BF16, matmul with BF16 out, weight [N, K]);
 *   - RMSNorm variant B (sqrt, then divide): same page, section 三;
 *   - the KV Prolog flow kv_a -> split -> RMSNorm -> kv_b -> reshape/split -> RoPE:
 *     "DeepSeek-V2-Lite-Chat MLA KV Prolog 迁移指南", sections 背景 and 源码级原理;
 *   - rotate-half RoPE with one cos/sin row per token: "PyPTO Operator 深度解析
 *     (DeepSeek-V3.2-Exp)", section 3.3 QuantRope;
 *   - per-token symmetric INT8 quant (127/amax multiplier, round half to even,
 *     scale = amax/127): same page, section 3.1 PrologQuant; and "PyPTO Gym 中的
 *     grouped_matmul_swiglu_quant", sections 算子语义与数学公式 and 实现特点 5;
 *   - the INT8 W8A8 linear (per-token activation quant, int8 x int8 -> int32,
 *     dequant with x_scale * w_scale): AT-10 page, section 四.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major. Weights are [N, K] (output channel major, K contiguous).
 *   - bf16 tensors are passed as raw 16-bit patterns (void pointers).
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them past the call. They must be 16-byte
 *     aligned (a misaligned pointer is MLAP_ERR_INVALID_ARG; the MXFP8 scale
 *     tensors ms_* need 4 bytes) and must not overlap (inputs may alias other inputs).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     on it; no call synchronises the host except where stated.
 *   - Errors are returned as status codes (mlap_status); nothing aborts and no
 *     C++ exception crosses the ABI. A kernel launch failure is reported as
 *     MLAP_ERR_HIP; a device fault surfaces at the caller's next synchronisation.
 */
#ifndef MLAP_H
#define MLAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef MLAP_API
#define MLAP_API __attribute__((visibility("default")))
#endif

typedef enum {
    MLAP_OK = 0,
    MLAP_ERR_INVALID_ARG = 1, /* NULL required pointer, T out of [0, t_max], bad handle */
    MLAP_ERR_UNSUPPORTED = 2, /* dimensions the kernels do not support */
    MLAP_ERR_WORKSPACE = 3,   /* workspace missing or smaller than mlap_workspace_size */
    MLAP_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
    MLAP_ERR_NO_MEMORY = 5    /* a host allocation failed (mlap_create) */
} mlap_status;

/* Configuration flags. */
#define MLAP_W8A8 0x1u /* int8 weights + per-output-channel fp32 scales; W8A8 GEMMs */
/* Numeric variants the pages describe besides the default path:
 * MLAP_NORM_RSQRT: RMSNorm variant A of the AT-10 card (section 三): sum of squares, times
 *   1/D, + eps, rsqrt; the default is variant B (x^2/D summed, sqrt, divide).
 * MLAP_ROPE_INTERLEAVED: the QuantRope3D form of the [V32] page (section 3.3) with chunk 2:
 *   each raw rope slice (q_pe per head, k_pe) is de-interleaved (u0 u2 ... | u1 u3 ...) before
 *   rotate-half; the outputs keep the split-half order. cos/sin as for the default.
 * MLAP_QUANT_Q_PER_HEAD: q codes and scales per (token, head): the per-row max of [V32]
 *   section 3.1 over the last axis of the [T, H, Dn+R] q tensor; q_scale is then [T, H].
 *   Needs H <= 1024 and H*(Dn+R) <= 32768. */
#define MLAP_NORM_RSQRT 0x2u
#define MLAP_ROPE_INTERLEAVED 0x4u
#define MLAP_QUANT_Q_PER_HEAD 0x8u
/* MLAP_Q_HEAD_NORM: the V4-shape prolog of the AT-10 card (sections 五, 九): after q_b the q
 *   row is reshaped to its heads and every head (Dn + R values) goes through RMSNorm without
 *   gamma (the configured variant) before RoPE. bf16 only; Dn and Dn + R multiples of 64,
 *   H <= 1024, H*(Dn+R) <= 32768, H*R <= 8192. */
#define MLAP_Q_HEAD_NORM 0x10u
/* MLAP_MXFP8: MXFP8 projections (the third Linear mode of the AT-10 card, section 四:
 *   scaled_mm with an fp32 result; the format of the grouped_matmul_swiglu_quant page,
 *   section 算子语义: E4M3 data and one E8M0 scale 2^(e-127) per 32 values along K). The
 *   weights w_* are E4M3FN bytes [N, K] with scales ms_* [N, K/32]; the activations (x, q_norm,
 *   kv_norm) are converted block by block (shared exponent floor(log2(amax)) - 8, values
 *   rounded to E4M3, saturating at 448). Not with MLAP_W8A8. */
#define MLAP_MXFP8 0x20u
/* MLAP_MXFP8_MFMA (with MLAP_MXFP8): run the projections on gfx950's block-scaled MFMA
 * (E4M3 operands with their E8M0 scales, 64 values of K per instruction) instead of decoding
 * the weights to bf16. Faster, but the instruction's own sum of 64 products is not exact (up to
 * ~5e-5 of the sum of |products| on prolog-like operands), so bf16 outputs more often land one
 * ulp away: INT8 codes measured 99.86-99.94% exact at V3 sizes, against >= 99.9% on the default
 * route, where the MXFP8 products and sums are exact up to the fp32 accumulation. Needs hidden,
 * q_lora and (with kv_b) kv_lora multiples of 128; otherwise the decoded path runs. */
#define MLAP_MXFP8_MFMA 0x40u

typedef struct {
    int32_t t_max;    /* largest token count a run may pass (sizes nothing on device) */
    int32_t hidden;   /* model width (K of the down projection); multiple of 64 (128 with W8A8) */
    int32_t q_lora;   /* q low-rank width; 0 = no q branch (KV-Prolog mode); multiple of 64 (128) */
    int32_t kv_lora;  /* compressed-KV width; multiple of 8 (64, or 128 with W8A8, if v_dim > 0) */
    int32_t rope_dim; /* RoPE slice width of q and k; multiple of 16 */
    int32_t nope_dim; /* per-head non-rotary width of q (and of k_nope); multiple of 8 */
    int32_t v_dim;    /* per-head value width of kv_b; 0 = no kv_b projection; multiple of 8 */
    int32_t n_heads;  /* attention heads */
    int32_t max_pos;  /* rows of the cos/sin tables */
    float eps;        /* RMSNorm epsilon (added to the mean square) */
    uint32_t flags;   /* MLAP_W8A8 | MLAP_NORM_RSQRT | MLAP_ROPE_INTERLEAVED | MLAP_QUANT_Q_PER_HEAD |
                         MLAP_Q_HEAD_NORM | MLAP_MXFP8 | MLAP_MXFP8_MFMA */
} mlap_config;

/*
 * Inputs of one run (device pointers). Shapes use T = tokens of this run,
 * Hd = hidden, Lq = q_lora, Lkv = kv_lora, R = rope_dim, Dn = nope_dim,
 * Dv = v_dim, H = n_heads.
 */
typedef struct {
    int32_t T;                 /* tokens in this run, 0 <= T <= t_max */
    const void* x;             /* [T, Hd] bf16 token activations */
    const int32_t* positions;  /* [T] position of each token in [0, max_pos); values outside
                                  are clamped into range (a violated precondition) */
    const void* w_qa;          /* [Lq, Hd]          bf16 (int8 with W8A8, E4M3 with MXFP8); unused if Lq == 0 */
    const void* w_qb;          /* [H*(Dn+R), Lq]    bf16 (int8); per head [nope | rope] rows */
    const void* w_kva;         /* [Lkv+R, Hd]       bf16 (int8); rows [c_kv | k_pe] */
    const void* w_kvb;         /* [H*(Dn+Dv), Lkv]  bf16 (int8); per head [nope | v]; if Dv > 0 */
    const float* ws_qa;        /* W8A8 only: per-output-channel weight scales, [Lq] */
    const float* ws_qb;        /* W8A8 only: [H*(Dn+R)] */
    const float* ws_kva;       /* W8A8 only: [Lkv+R] */
    const float* ws_kvb;       /* W8A8 only: [H*(Dn+Dv)] */
    const void* gamma_q;       /* [Lq] bf16 RMSNorm weight of the q branch */
    const void* gamma_kv;      /* [Lkv] bf16 RMSNorm weight of the kv branch */
    const float* cos;          /* [max_pos, R] fp32, the rotate-half table (both halves) */
    const float* sin;          /* [max_pos, R] fp32 */
    /* KV cache write (optional; the caches are in mlap_outputs). slot_mapping[t] is the cache
       row of token t: a flat slot index (for a paged cache, block * block_size + offset). A
       negative slot, or one >= cache_slots, leaves the caches untouched for that token
       (padding). Slots of one run must be distinct; with duplicates the row holds one of the
       tokens' entries. Needed (with cache_slots > 0) when any cache pointer is set. */
    const int32_t* slot_mapping; /* [T] int32 */
    int32_t cache_slots;         /* rows of every cache */
    const uint8_t* ms_qa;        /* MLAP_MXFP8 only: E8M0 block scales [Lq, Hd/32] of w_qa; every
                                    ms_* pointer 4-byte aligned */
    const uint8_t* ms_qb;        /* [H*(Dn+R), Lq/32] */
    const uint8_t* ms_kva;       /* [Lkv+R, Hd/32] */
    const uint8_t* ms_kvb;       /* [H*(Dn+Dv), Lkv/32] */
} mlap_inputs;

/*
 * Outputs of one run (device pointers, caller-allocated). A NULL output is not
 * produced. Token-major layouts; per-head tensors are [T, H, d].
 */
typedef struct {
    void* q_nope;     /* [T, H, Dn] bf16                      (needs Lq > 0) */
    void* q_pe;       /* [T, H, R]  bf16, after RoPE          (needs Lq > 0) */
    void* kv_norm;    /* [T, Lkv]   bf16 */
    void* k_pe;       /* [T, R]     bf16, after RoPE */
    void* k_nope;     /* [T, H, Dn] bf16                      (needs Dv > 0) */
    void* value;      /* [T, H, Dv] bf16                      (needs Dv > 0) */
    void* q_norm;     /* [T, Lq]    bf16, the normalised q_a projection (optional) */
    int8_t* q_i8;     /* [T, H, Dn+R] int8 codes of [q_nope | q_pe] per head */
    float* q_scale;   /* [T] fp32, amax/127 over the token's H*(Dn+R) values ([T, H] per head) */
    int8_t* kv_i8;    /* [T, Lkv] int8 codes of kv_norm */
    float* kv_scale;  /* [T] fp32 */
    /* KV cache rows written at mlap_inputs.slot_mapping: the ScatterUpdate of the prolog's kv
       results into the cache ([V32] page, section 2.4; the [BLOG] page's step 2 caches the
       per-row quantised rows). Each is optional and holds exactly what the same-named
       per-token output holds, at row slot_mapping[t] instead of t; other rows are untouched. */
    void* kv_cache;         /* [cache_slots, Lkv] bf16 kv_norm */
    int8_t* kv_cache_i8;    /* [cache_slots, Lkv] int8 codes of kv_norm */
    float* kv_cache_scale;  /* [cache_slots] fp32 kv scale */
    void* kr_cache;         /* [cache_slots, R] bf16 k_pe, after RoPE */
    /* Diagnostic taps (optional), for checking the path one step at a time against a reference
       that can start from given intermediate rows:
       a_proj: [T, Lq+Lkv+R] bf16, the down projection [q_a | c_kv | k_pe raw] exactly as the
         row stage takes it (each value at the projection's bf16 cast point; with
         MLAP_ROPE_INTERLEAVED the k_pe slice already de-interleaved, the order the rotate-half
         reads it in);
       q_proj: [T, H, Dn+R] bf16, the q up projection per head before the per-head norm (rope
         slice in rotate-half order as above); only with MLAP_Q_HEAD_NORM, where it needs the
         q_nope and q_pe outputs too. */
    void* a_proj;
    void* q_proj;
} mlap_outputs;

typedef struct mlap_prolog* mlap_handle;

/* Validate `cfg` and create a host-side handle (no device allocation, no sync).
 * Returns MLAP_ERR_UNSUPPORTED for dimensions the kernels do not handle (among them a
 * rope_dim above 4096) and MLAP_ERR_NO_MEMORY if the handle cannot be allocated. */
MLAP_API int mlap_create(const mlap_config* cfg, mlap_handle* out);

/* Bytes of device workspace a run with T tokens needs (GEMM intermediates, the
 * per-tile partial amax of q, the W8A8 int8 activations; with MXFP8 also the decoded
 * bf16 weights and converted activations). The caller allocates it. */
MLAP_API int mlap_workspace_size(mlap_handle h, int32_t T, size_t* bytes);

/* Enqueue the whole prolog for in->T tokens on `stream`. `ws` must hold at least
 * mlap_workspace_size(h, in->T) bytes, 256-byte aligned. T == 0 is a no-op.
 * Runs on one handle must not overlap in time unless they use distinct workspaces, and a
 * handle is not for concurrent calls from several host threads. All work is enqueued on
 * `stream` (no host synchronisation), so a run can be captured into a HIP graph. */
MLAP_API int mlap_run(mlap_handle h, void* stream, const mlap_inputs* in, const mlap_outputs* out,
             void* ws, size_t ws_bytes);

/*
 * mlap_run for callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, with the library's own device scratch in
 * place of the caller's workspace. That scratch is one array of MLAP_STATIC_SCRATCH_BYTES
 * (64 MiB) per GPU, part of the library's code object: it is loaded with the library on each GPU
 * the library runs on and held until the process ends. A run whose mlap_workspace_size exceeds
 * it returns MLAP_ERR_WORKSPACE (V3 bf16: up to T = 8192 fits). Nothing here allocates: no
 * device or host buffer, stream or event. Every call on
 * one GPU shares that GPU's array, from any handle: calls that overlap in time on one GPU race
 * and give wrong results; order them on one stream or serialise them. No run needs the array
 * cleared (each run writes every workspace byte it reads).
 */
#define MLAP_STATIC_SCRATCH_BYTES (64u << 20)
MLAP_API int mlap_run_static(mlap_handle h, void* stream, const mlap_inputs* in, const mlap_outputs* out);

/* Free the handle (host memory and timing events). NULL is allowed. */
MLAP_API void mlap_destroy(mlap_handle h);

/* Static description of a status code. */
MLAP_API const char* mlap_status_str(int status);

/*
 * Test export of the W8A8 matmul core (AT-10 page, section 四: int8 x int8 ->
 * int32): C[m, n] = sum_k A[m, k] * B[n, k], exact int32, on the kernel and tiles the
 * W8A8 prolog runs for a batch of M tokens: for M > 512 the LDS-DMA GEMM with 256 x 256
 * tiles (a column remainder that is a multiple of 64 on 64 x 64 tiles), as the W8A8 down
 * and q up projections of large batches; for M <= 512 the register-staged GEMM with the
 * small-batch projections' tiles (128 x 192 when N is a multiple of 192, as the q up
 * projection, else 256 x 64, as the down projection). Only the epilogue differs: the
 * accumulators are stored instead of dequantised. A [M, K] int8, B [N, K] int8, C [M, N]
 * int32, device pointers (16-byte aligned); K must be a multiple of 128. Enqueued on `stream`.
 */
MLAP_API int mlap_gemm_i8_i32(void* stream, const int8_t* A, const int8_t* B, int32_t* C, int32_t M,
                     int32_t N, int32_t K);

/*
 * Test export of the bf16 matmul core (AT-10 page, sections 二 and 五: matmul with
 * BF16 output, weight [N, K]): C = bf16(A . B^T) with fp32 accumulation. A [M, K],
 * B [N, K], C [M, N] bf16, device pointers; K must be a multiple of 64.
 */
MLAP_API int mlap_gemm_bf16(void* stream, const void* A, const void* B, void* C, int32_t M, int32_t N,
                   int32_t K);

/*
 * Test export of the block-scaled MFMA core (MLAP_MXFP8_MFMA; the MXFP8 scaled_mm of the AT-10
 * card, section 四, with an fp32 result): C[m, n] = sum_k deq(A[m, k]) * deq(B[n, k]) where
 * deq(code) = E4M3 value of the byte times 2^(scale - 127), one scale byte per 32 values of K
 * (A_scale [M, K/32], B_scale [N, K/32], both 4-byte aligned). A [M, K], B [N, K] E4M3 bytes,
 * C [M, N] fp32, device pointers; K a multiple of 128, N of 4. Enqueued on `stream`.
 */
MLAP_API int mlap_gemm_mxfp8_f32(void* stream, const uint8_t* A, const uint8_t* A_scale, const uint8_t* B,
                                 const uint8_t* B_scale, float* C, int32_t M, int32_t N, int32_t K);

/*
 * Per-kernel timing (measurement support). Kernel ids: see mlap_kernel_name.
 * mlap_timing_begin arms HIP events around every launch of kernel `kernel_id`
 * in the next `max_launches` runs of `h` (events are created here). The events
 * are recorded on the run's stream, so they time exactly that kernel.
 * mlap_timing_end waits for the recorded events (host sync), writes up to `cap`
 * per-launch durations in milliseconds to `ms`, stores the count in *n and
 * disarms timing.
 */
MLAP_API int mlap_timing_begin(mlap_handle h, int32_t kernel_id, int32_t max_launches);
MLAP_API int mlap_timing_end(mlap_handle h, float* ms, int32_t cap, int32_t* n);

/* Shader clock of the timed kernel (measurement support): while timing is armed, every
 * launch of the armed kernel that runs on the LDS-DMA GEMM (gemm_down, gemm_up_q, gemm_up_kv
 * past the weight-streaming batches or on its tiles) adds, for every 16th workgroup, the
 * shader-clock cycles and the constant 100 MHz clock ticks it ran for into counters[0] and
 * counters[1] (device memory, two uint64, caller-owned, zeroed by the caller; 8-byte aligned).
 * Their ratio times 100 MHz is the average shader clock while that kernel ran. NULL disarms. */
MLAP_API int mlap_timing_clock(mlap_handle h, unsigned long long* counters);

/* Bounds checks of the debug build (the library compiled with MLAP_DEBUG; a test and
 * development aid, not part of the path): the kernels check their operand rows, K ranges,
 * output indexes and input positions as they go and set a bit for every check that failed
 * on the current device, without stopping (the accesses are clamped or guarded anyway).
 * This call synchronizes the device, stores the bits collected since the last reset in
 * *flags (0: every check held) and clears them when `reset` is nonzero. Bits: 1 GEMM
 * activation row, 2 GEMM weight row, 4 GEMM K range, 8 output index, 16 row-kernel index,
 * 32 q-quant index, 64 an input position outside [0, max_pos) (a precondition of mlap_run
 * that the kernels clamp). Release builds store 0 and return MLAP_ERR_UNSUPPORTED. */
MLAP_API int mlap_debug_flags(unsigned int* flags, int32_t reset);

/* Name of kernel `kernel_id` ("gemm_down", "norm_rope", "gemm_up_q", ...), or NULL
 * past the last one. */
MLAP_API const char* mlap_kernel_name(int32_t kernel_id);

/* Library version string. */
MLAP_API const char* mlap_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLAP_H */
