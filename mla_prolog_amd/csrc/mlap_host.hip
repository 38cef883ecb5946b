// mlap_host.hip -- the C ABI of libmlap.so: validation, per-run plan and launches.
//
// The run is a fixed chain of kernels on the caller's stream (no host sync):
//   [W8A8: act_quant(x)] -> gemm_down (x . [W_qa; W_kva]^T, bf16 out)
//   -> norm_rope (RMSNorm*gamma -> bf16 for q_a and c_kv, RoPE of k_pe, kv quant)
//   -> gemm_up_q (q_norm . W_qb^T; per head: q_nope, RoPE'd q_pe, partial amax)
//   -> gemm_up_kv (kv_norm . W_kvb^T; per head: k_nope, value)   [KV-Prolog mode]
//   -> quant_q (per-token INT8 codes and scale of all heads' q)
// The chain follows the MLAProlog walk-through of the AT-10 card ("PyPTO-Gym 算子设计
// 模式 AT-10 ... MLAProlog 实战", section 五) and the KV Prolog flow of the V2-Lite
// migration guide ("DeepSeek-V2-Lite-Chat MLA KV Prolog 迁移指南", section 背景).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <mutex>
#include <vector>

#include "../../include/mlap.h"
#include "launch.hpp"

using namespace mlap;

// Workspace of mlap_run_static (see static_scratch below).
static __device__ __align__(256) char scratch[size_t(MLAP_STATIC_SCRATCH_BYTES)];

#ifdef MLAP_DEBUG
// The debug build's bounds-check word (MLAP_CHECK): each GPU's copy collects the bits of the
// checks that failed there until mlap_debug_flags reads and clears it.
static __device__ unsigned int dbg_flags_word;
#endif

namespace {

enum KernelId : int32_t {
    kKActQuant = 0,
    kKGemmDown = 1,
    kKNormRope = 2,
    kKGemmUpQ = 3,
    kKGemmUpKv = 4,
    kKQuantQ = 5,
    kKQHeadNorm = 6,
    kKMxConvert = 7,
    kKCount = 8
};
const char* const kKernelNames[kKCount] = {"act_quant", "gemm_down", "norm_rope", "gemm_up_q",
                                           "gemm_up_kv", "quant_q", "q_head_norm", "mx_convert"};

constexpr size_t kAlign = 256;
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kSmallBatch = 512;  // token counts up to this use the weight-streaming tiles
constexpr int kGroupM = 4;        // M-tiles per group in the XCD-aware tile order
constexpr int kGroupNq = 8;       // N-tiles per group for the q up projection (N-major split)

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Split-K factor for `tiles` output tiles over `nk` K-tiles: the largest divisor of nk (at
// most max_splits) that keeps the grid within one round of the 256 CUs -- a grid just past 256
// workgroups runs a second, nearly empty round -- or 1 if the tiles alone fill a round.
int one_round_splits(int tiles, int nk, int max_splits = 16) {
    int best = 1;
    for (int c = 1; c <= max_splits; ++c)
        if (nk % c == 0 && tiles * c <= kCUs) best = c;
    return best;
}

// Widest supported up-projection tile that holds whole heads.
int heads_tile(int head_w) {
    static const int cand[] = {256, 192, 128, 64};
    for (int bn : cand)
        if (bn % head_w == 0) return bn;
    return 0;
}

// Kernel shapes for one run of T tokens: the counterpart of a tile table bucketed by token
// count. Small batches stream the weights (the projections are bound by reading them):
// tiles that span the whole batch (256 rows, or 64 at most 64 tokens) with three stages in
// flight, a split-K down projection whose fp32 partial sums the row kernel adds up, half-head
// q tiles and 32-column kv_b tiles so every CU has work. Large batches are bound by MFMA
// throughput: 256 x 256 tiles. The int8 small-batch projections keep the register-staged
// kernel of gemm.hpp (GemmTile fields).
struct Plan {
    GemmTile down;
    Epi down_epi;
    int down_splits;
    GemmTile up_q, up_kv;
    bool big_down = false, big_q = false, big_kv = false;  // large-batch kernel (gemm_big.hpp)
    // bf16 large batches: the down projection's columns past the last whole 256-wide tile
    // (the k_pe slice at V3 and V2-Lite widths) run as a split-K GEMM with fp32 partials
    // that the row kernel sums, instead of a second, mostly idle round of tiles.
    int tail_c0 = 0, tail_splits = 0;
    // ... or, in bf16 and int8 when the slice is eight columns per 256-wide tile (the k_pe
    // slice at V3 width: 64 columns over 8 tiles), as eight extra columns of every tile
    // (kStoreBf16X), from the activation rows already staged: x is read once
    bool x_fuse = false;
    BigShape down_shape = BigShape::kWide, q_shape = BigShape::kWide, kv_shape = BigShape::kWide;
    int nt_q = 0;  // per-token partial amax entries of q (N tiles of the q up projection)
    int hn_groups = 1;  // per-head q norm: workgroups per token (each writes one partial amax)
    // MXFP8 on the block-scaled MFMA (E4M3 operands in the GEMMs); else, with MXFP8, the
    // weights are decoded to bf16 for the bf16 GEMMs
    bool mx_native = false;
};

struct Timer {
    int32_t kernel = -1;
    int32_t cap = 0;
    int32_t used = 0;
    std::vector<hipEvent_t> ev;  // 2 per launch
    unsigned long long* clk = nullptr;  // shader-clock counters of the timed kernel, or null
};

// Workspace carve-up for T tokens.
struct WsLayout {
    size_t a1 = 0, tail = 0, qn = 0, kvn = 0, qpart = 0, xq = 0, xs = 0, qnq = 0, qns = 0, kvq = 0, kvs = 0;
    size_t wd_down = 0, wd_qb = 0, wd_kvb = 0, xm = 0, qnm = 0, kvnm = 0;  // MXFP8 operands
    size_t total = 0;
};

}  // namespace

struct mlap_prolog {
    mlap_config cfg;
    bool w8a8;
    bool mx;      // MXFP8 projections
    bool mx_mfma;  // ... on the block-scaled MFMA where the shapes allow
    int N1;       // down-projection width
    int QH, KH;   // q head width (nope + rope), kv_b head width (nope + v)
    int bn_q, bn_kv;
    Timer timer;

    bool head_norm() const { return (cfg.flags & MLAP_Q_HEAD_NORM) && cfg.q_lora > 0; }

    // MXFP8 runs on the block-scaled MFMA when asked for and every projection fits the LDS-DMA
    // kernel (whole 128-value K stages), else through the decoded bf16 weights.
    Plan plan(int T) const {
        if (mx && mx_mfma) {
            Plan p = plan_for(T, InType::kFp8);
            if (p.big_down && (cfg.q_lora == 0 || p.big_q) && (cfg.v_dim == 0 || p.big_kv)) {
                p.mx_native = true;
                return p;
            }
        }
        return plan_for(T, w8a8 ? InType::kInt8 : InType::kBf16);
    }

    Plan plan_for(int T, InType it) const {
        Plan p{};
        const bool small = T <= kSmallBatch;
        const bool i8 = it == InType::kInt8;
        const int kb = it == InType::kBf16 ? 64 : 128;  // elements per 128-byte K-tile
        const int nk = cfg.hidden / kb;
        if (!i8 && small) {
            p.down = {256, 64, 3};
            p.down_epi = Epi::kStoreF32;
            // at most 8 splits: the row kernel then sums the partials in one round trip (16
            // splits at the V2-Lite shape cost it a second one: 20.2 -> 18.4 us per step at 8)
            p.down_splits = one_round_splits(((T + 255) / 256) * ((N1 + 63) / 64), nk, 8);
        } else {
            p.down = (cfg.q_lora % 192 == 0 && !small) ? GemmTile{256, 192, 1} : GemmTile{256, 64, 1};
            p.down_epi = Epi::kStoreBf16;
            p.down_splits = 1;
        }
        p.up_q = {small ? 128 : 256, bn_q, small ? 3 : 1};
        p.up_kv = {small ? 128 : 256, bn_kv, small ? 3 : 1};
        if (!small) {
            // MFMA-bound: the large-batch kernel wherever the shapes suit it
            GemmArgs d{};
            d.K = cfg.hidden;
            d.N = N1;
            d.ldo = N1;
            p.big_down = gemm_big_fits(d, it, Epi::kStoreBf16);
            if (p.big_down) {
                p.down_epi = Epi::kStoreBf16;
                p.down_splits = 1;
                const int c0 = N1 / kBigTile * kBigTile;
                if (it != InType::kFp8 && c0 > 0 && N1 - c0 == 8 * (c0 / kBigTile)) {
                    p.tail_c0 = c0;
                    p.x_fuse = true;
                } else if (!i8 && c0 > 0 && c0 < N1 && (N1 - c0) % 64 == 0) {
                    p.tail_c0 = c0;
                    p.tail_splits = one_round_splits((T + 255) / 256 * ((N1 - c0) / 64), nk);
                }
            }
            if (cfg.q_lora > 0) {
                GemmArgs u{};
                u.K = cfg.q_lora;
                u.head_w = QH;
                u.d0 = cfg.nope_dim;
                u.d1 = cfg.rope_dim;
                u.rope = head_norm() ? 0 : 1;
                p.big_q = gemm_big_fits(u, it, Epi::kHeads);
            }
            if (cfg.v_dim > 0) {
                GemmArgs u{};
                u.K = cfg.kv_lora;
                u.head_w = KH;
                u.d0 = cfg.nope_dim;
                u.d1 = cfg.v_dim;
                u.rope = 0;
                p.big_kv = gemm_big_fits(u, it, Epi::kHeads);
            }
        } else if (!i8) {
            // weight streaming: the LDS-DMA kernel with split-K fp32 partials for the down
            // projection and half-head tiles spanning the whole batch for the q up projection
            GemmArgs d{};
            d.K = cfg.hidden;
            d.N = N1;
            d.ldo = N1;
            d.k_splits = p.down_splits;
            if (gemm_big_fits(d, it, Epi::kStoreF32, BigShape::kSplitK)) {
                p.big_down = true;
                p.down_shape = BigShape::kSplitK;
            }
            if (cfg.q_lora > 0) {
                GemmArgs u{};
                u.K = cfg.q_lora;
                u.head_w = QH;
                u.d0 = cfg.nope_dim;
                u.d1 = cfg.rope_dim;
                u.rope = head_norm() ? 0 : 1;
                if (gemm_big_fits(u, it, Epi::kHeads, BigShape::kHalfHead)) {
                    p.big_q = true;
                    p.q_shape = BigShape::kHalfHead;
                } else if (head_norm() && gemm_big_fits(u, it, Epi::kHeads, BigShape::kNarrowHeads)) {
                    p.big_q = true;  // raw heads: no rope slice to keep whole
                    p.q_shape = BigShape::kNarrowHeads;
                }
            }
            if (cfg.v_dim > 0) {
                GemmArgs u{};
                u.K = cfg.kv_lora;
                u.head_w = KH;
                u.d0 = cfg.nope_dim;
                u.d1 = cfg.v_dim;
                u.rope = 0;
                if (gemm_big_fits(u, it, Epi::kHeads, BigShape::kNarrowHeads)) {
                    p.big_kv = true;
                    p.kv_shape = BigShape::kNarrowHeads;
                }
            }
        }
        if (cfg.q_lora > 0) {
            const int nq = cfg.n_heads * QH;
            const int bn = p.big_q ? big_tile_n(p.q_shape) : bn_q;
            p.nt_q = (nq + bn - 1) / bn;
            // small batches split each token's heads over up to 16 workgroups (whole heads, at
            // most one workgroup per CU in all), one partial amax each
            if (head_norm())
                for (int g = 16; g > 1; g >>= 1)
                    if (cfg.n_heads % g == 0 && g <= p.nt_q && T * g <= kCUs) {
                        p.hn_groups = g;
                        break;
                    }
        }
        return p;
    }

    WsLayout layout(int T) const {
        WsLayout L;
        const Plan p = plan(T);
        size_t off = 0;
        auto take = [&](size_t bytes) {
            size_t o = off;
            off += align_up(bytes);
            return o;
        };
        const size_t t = static_cast<size_t>(T);
        L.a1 = take(p.down_epi == Epi::kStoreF32 ? t * N1 * 4 * p.down_splits : t * N1 * 2);
        if (p.tail_splits) L.tail = take(t * (N1 - p.tail_c0) * 4 * p.tail_splits);
        if (cfg.q_lora > 0) L.qn = take(t * cfg.q_lora * 2);
        if (cfg.v_dim > 0) L.kvn = take(t * cfg.kv_lora * 2);
        if (cfg.q_lora > 0) L.qpart = take(t * p.nt_q * 4);
        if (w8a8) {
            L.xq = take(t * cfg.hidden);
            L.xs = take(t * 4);
            if (cfg.q_lora > 0) {
                L.qnq = take(t * cfg.q_lora);
                L.qns = take(t * 4);
            }
            if (cfg.v_dim > 0) {
                L.kvq = take(t * cfg.kv_lora);
                L.kvs = take(t * 4);
            }
        }
        if (mx && p.mx_native) {  // E4M3 codes and E8M0 block scales of the GEMM inputs
            L.xq = take(t * cfg.hidden);
            L.xs = take(t * (cfg.hidden / 32));
            if (cfg.q_lora > 0) {
                L.qnq = take(t * cfg.q_lora);
                L.qns = take(t * (cfg.q_lora / 32));
            }
            if (cfg.v_dim > 0) {
                L.kvq = take(t * cfg.kv_lora);
                L.kvs = take(t * (cfg.kv_lora / 32));
            }
        } else if (mx) {  // decoded weights and converted activations for the bf16 GEMMs
            L.wd_down = take(static_cast<size_t>(N1) * cfg.hidden * 2);
            L.xm = take(t * cfg.hidden * 2);
            if (cfg.q_lora > 0) {
                L.wd_qb = take(static_cast<size_t>(cfg.n_heads) * QH * cfg.q_lora * 2);
                L.qnm = take(t * cfg.q_lora * 2);
            }
            if (cfg.v_dim > 0) {
                L.wd_kvb = take(static_cast<size_t>(cfg.n_heads) * KH * cfg.kv_lora * 2);
                L.kvnm = take(t * cfg.kv_lora * 2);
            }
        }
        L.total = std::max<size_t>(off, kAlign);
        return L;
    }

    // the clock counters for a launch of kernel k (while it is the timed one)
    unsigned long long* clock_for(int32_t k) const {
        return (timer.kernel == k && timer.used < timer.cap) ? timer.clk : nullptr;
    }

    void tick(int32_t k, hipStream_t s, bool begin) {
        Timer& tm = timer;
        if (tm.kernel != k || tm.used >= tm.cap) return;
        (void)hipEventRecord(tm.ev[2 * tm.used + (begin ? 0 : 1)], s);
        if (!begin) ++tm.used;
    }
};

namespace {

int validate(const mlap_config* c) {
    const bool w8 = (c->flags & MLAP_W8A8) != 0;
    if (c->flags & ~(MLAP_W8A8 | MLAP_NORM_RSQRT | MLAP_ROPE_INTERLEAVED | MLAP_QUANT_Q_PER_HEAD |
                     MLAP_Q_HEAD_NORM | MLAP_MXFP8 | MLAP_MXFP8_MFMA))
        return MLAP_ERR_INVALID_ARG;
    if ((c->flags & MLAP_MXFP8_MFMA) && !(c->flags & MLAP_MXFP8)) return MLAP_ERR_INVALID_ARG;
    if ((c->flags & MLAP_W8A8) && (c->flags & MLAP_MXFP8)) return MLAP_ERR_INVALID_ARG;
    const bool head_norm = (c->flags & MLAP_Q_HEAD_NORM) && c->q_lora > 0;
    if (c->t_max < 1 || c->hidden < 1 || c->kv_lora < 1 || c->rope_dim < 1 || c->n_heads < 1 ||
        c->max_pos < 1 || c->q_lora < 0 || c->v_dim < 0 || c->nope_dim < 0 || !(c->eps >= 0.f))
        return MLAP_ERR_INVALID_ARG;
    const int kmul = w8 ? 128 : 64;  // K of every GEMM: whole 128-byte K-tiles
    if (c->hidden % kmul) return MLAP_ERR_UNSUPPORTED;
    if (c->q_lora % kmul) return MLAP_ERR_UNSUPPORTED;
    if (c->kv_lora % 8 || (c->v_dim > 0 && c->kv_lora % kmul)) return MLAP_ERR_UNSUPPORTED;
    if (c->rope_dim % 16 || c->rope_dim > 4096) return MLAP_ERR_UNSUPPORTED;  // row kernels: R/16 <= 256
    if (c->nope_dim % 8 || c->v_dim % 8) return MLAP_ERR_UNSUPPORTED;
    if (c->q_lora > 8192 || c->kv_lora > 8192) return MLAP_ERR_UNSUPPORTED;  // row kernel
    if (c->q_lora > 0 && !head_norm && heads_tile(c->nope_dim + c->rope_dim) == 0) return MLAP_ERR_UNSUPPORTED;
    // per-head q norm: raw heads from the LDS-DMA GEMM (32-column tiles at small batches,
    // 256 x 256 at large), then the head-norm row kernel
    if (head_norm && (w8 || c->nope_dim % 64 || (c->nope_dim + c->rope_dim) % 64 || c->n_heads > kMaxQuantHeads ||
                      c->n_heads * (c->nope_dim + c->rope_dim) > kHeadNormChunks * 8 * 256 ||
                      c->n_heads * (c->rope_dim >> 3) > kHeadNormPeChunks))
        return MLAP_ERR_UNSUPPORTED;
    if (c->v_dim > 0 && heads_tile(c->nope_dim + c->v_dim) == 0) return MLAP_ERR_UNSUPPORTED;
    if ((c->flags & MLAP_QUANT_Q_PER_HEAD) && c->q_lora > 0 &&
        (c->n_heads > kMaxQuantHeads ||
         c->n_heads * (c->nope_dim + c->rope_dim) > kQuantHeadChunks * 8 * 256))
        return MLAP_ERR_UNSUPPORTED;
    // GEMM sizes and grid dimensions are 32-bit in the kernels
    if (c->t_max > (1 << 24) || c->hidden > (1 << 20) || c->n_heads > 4096 || c->max_pos > (1 << 26))
        return MLAP_ERR_UNSUPPORTED;
    return MLAP_OK;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int run_impl(mlap_handle h, void* stream, const mlap_inputs* in, const mlap_outputs* out, void* ws,
             size_t ws_bytes);

// The allocation-free entry point's workspace: a device array of kStaticScratchBytes in every
// GPU's copy of this code object. Host code must never pass `scratch` itself to a kernel or a
// copy (it names a host-side stand-in); it uses the per-device address from static_scratch().
// Nothing in the prolog needs its workspace cleared: every byte a run reads, the same run wrote
// first (the down-projection output and its split-K partials, q_norm / kv_norm, the per-tile
// partial amax, the int8 and MX activations), so the contents a previous call left are inert.
constexpr size_t kStaticScratchBytes = size_t(MLAP_STATIC_SCRATCH_BYTES);

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device.
int static_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MLAP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MLAP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLAP_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *ptr = g_scratch_addr[dev];
    return MLAP_OK;
}

#ifdef MLAP_DEBUG
std::mutex g_dbg_mu;
unsigned int* g_dbg_addr[kMaxDevices] = {};
#endif

}  // namespace

// The bounds-check word of the current device (debug build), looked up once per device; null in
// release builds or when the lookup fails (the checks are then skipped).
unsigned int* mlap::debug_word() {
#ifdef MLAP_DEBUG
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_dbg_mu);
    if (!g_dbg_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_flags_word)) != hipSuccess) return nullptr;
        g_dbg_addr[dev] = static_cast<unsigned int*>(p);
    }
    return g_dbg_addr[dev];
#else
    return nullptr;
#endif
}

namespace {

// A tensor pointer the kernels cannot use: the 16-byte vector accesses and global->LDS copies
// need 16-byte alignment (NULL passes: optional tensors are checked separately).
inline bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

}  // namespace

extern "C" {

MLAP_API const char* mlap_version(void) { return "mlap 0.1 gfx950"; }

MLAP_API const char* mlap_status_str(int status) {
    switch (status) {
        case MLAP_OK: return "ok";
        case MLAP_ERR_INVALID_ARG: return "invalid argument";
        case MLAP_ERR_UNSUPPORTED: return "unsupported dimensions";
        case MLAP_ERR_WORKSPACE: return "workspace missing or too small";
        case MLAP_ERR_HIP: return "HIP runtime error";
        case MLAP_ERR_NO_MEMORY: return "host allocation failed";
        default: return "unknown status";
    }
}

MLAP_API const char* mlap_kernel_name(int32_t kernel_id) {
    return (kernel_id >= 0 && kernel_id < kKCount) ? kKernelNames[kernel_id] : nullptr;
}

MLAP_API int mlap_create(const mlap_config* cfg, mlap_handle* out) {
    if (!cfg || !out) return MLAP_ERR_INVALID_ARG;
    *out = nullptr;
    const int v = validate(cfg);
    if (v != MLAP_OK) return v;
    mlap_prolog* h = new (std::nothrow) mlap_prolog();
    if (!h) return MLAP_ERR_NO_MEMORY;
    h->cfg = *cfg;
    h->w8a8 = (cfg->flags & MLAP_W8A8) != 0;
    h->mx = (cfg->flags & MLAP_MXFP8) != 0;
    h->mx_mfma = (cfg->flags & MLAP_MXFP8_MFMA) != 0;
    h->N1 = cfg->q_lora + cfg->kv_lora + cfg->rope_dim;
    h->QH = cfg->nope_dim + cfg->rope_dim;
    h->KH = cfg->nope_dim + cfg->v_dim;
    h->bn_q = cfg->q_lora > 0 ? heads_tile(h->QH) : 0;
    h->bn_kv = cfg->v_dim > 0 ? heads_tile(h->KH) : 0;
    *out = h;
    return MLAP_OK;
}

MLAP_API void mlap_destroy(mlap_handle h) {
    if (!h) return;
    for (hipEvent_t e : h->timer.ev) (void)hipEventDestroy(e);
    delete h;
}

MLAP_API int mlap_workspace_size(mlap_handle h, int32_t T, size_t* bytes) {
    if (!h || !bytes || T < 0 || T > h->cfg.t_max) return MLAP_ERR_INVALID_ARG;
    *bytes = h->layout(T).total;
    return MLAP_OK;
}

MLAP_API int mlap_timing_begin(mlap_handle h, int32_t kernel_id, int32_t max_launches) {
    if (!h || kernel_id < 0 || kernel_id >= kKCount || max_launches < 1 || max_launches > 100000)
        return MLAP_ERR_INVALID_ARG;
    Timer& tm = h->timer;
    while (static_cast<int32_t>(tm.ev.size()) < 2 * max_launches) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return MLAP_ERR_HIP;
        tm.ev.push_back(e);
    }
    tm.kernel = kernel_id;
    tm.cap = max_launches;
    tm.used = 0;
    return MLAP_OK;
}

MLAP_API int mlap_debug_flags(unsigned int* flags, int32_t reset) {
    if (!flags) return MLAP_ERR_INVALID_ARG;
#ifdef MLAP_DEBUG
    unsigned int* w = mlap::debug_word();
    if (!w) return MLAP_ERR_HIP;
    if (hipDeviceSynchronize() != hipSuccess) return MLAP_ERR_HIP;
    if (hipMemcpy(flags, w, sizeof(unsigned int), hipMemcpyDeviceToHost) != hipSuccess) return MLAP_ERR_HIP;
    if (reset) {
        const unsigned int zero = 0;
        if (hipMemcpy(w, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return MLAP_ERR_HIP;
    }
    return MLAP_OK;
#else
    (void)reset;
    *flags = 0;
    return MLAP_ERR_UNSUPPORTED;
#endif
}

MLAP_API int mlap_timing_clock(mlap_handle h, unsigned long long* counters) {
    if (!h || (reinterpret_cast<uintptr_t>(counters) & 7)) return MLAP_ERR_INVALID_ARG;
    h->timer.clk = counters;
    return MLAP_OK;
}

MLAP_API int mlap_timing_end(mlap_handle h, float* ms, int32_t cap, int32_t* n) {
    if (!h || !n || (cap > 0 && !ms)) return MLAP_ERR_INVALID_ARG;
    Timer& tm = h->timer;
    int rc = MLAP_OK;
    int32_t k = 0;
    for (int32_t i = 0; i < tm.used; ++i) {
        if (hipEventSynchronize(tm.ev[2 * i + 1]) != hipSuccess) {
            rc = MLAP_ERR_HIP;
            break;
        }
        float v = 0.f;
        if (hipEventElapsedTime(&v, tm.ev[2 * i], tm.ev[2 * i + 1]) != hipSuccess) {
            rc = MLAP_ERR_HIP;
            break;
        }
        if (k < cap) ms[k++] = v;
    }
    *n = k;
    tm.kernel = -1;
    tm.cap = tm.used = 0;
    return rc;
}

MLAP_API int mlap_run(mlap_handle h, void* stream, const mlap_inputs* in, const mlap_outputs* out,
             void* ws, size_t ws_bytes) {
    return run_impl(h, stream, in, out, ws, ws_bytes);
}

// The allocation-free run: the workspace is the file-scope device array `scratch` (one per GPU,
// loaded with the library and held until the process ends), reached through its device address,
// which hipGetSymbolAddress gives once per device (in host code the array's name is a host-side
// stand-in, not a device address). No call here allocates: no buffer, stream or event.
MLAP_API int mlap_run_static(mlap_handle h, void* stream, const mlap_inputs* in, const mlap_outputs* out) {
    if (!h || !in || !out) return MLAP_ERR_INVALID_ARG;
    if (in->T < 0 || in->T > h->cfg.t_max) return MLAP_ERR_INVALID_ARG;
    if (in->T == 0) return MLAP_OK;
    if (h->layout(in->T).total > kStaticScratchBytes) return MLAP_ERR_WORKSPACE;  // beyond the array
    void* ptr = nullptr;
    const int rc = static_scratch(&ptr);
    if (rc != MLAP_OK) return rc;
    return run_impl(h, stream, in, out, ptr, kStaticScratchBytes);
}

}  // extern "C"

namespace {

int run_impl(mlap_handle h, void* stream, const mlap_inputs* in, const mlap_outputs* out, void* ws,
             size_t ws_bytes) {
    if (!h || !in || !out) return MLAP_ERR_INVALID_ARG;
    const mlap_config& c = h->cfg;
    const int T = in->T;
    if (T < 0 || T > c.t_max) return MLAP_ERR_INVALID_ARG;
    if (T == 0) return MLAP_OK;
    const bool has_q = c.q_lora > 0, has_kvb = c.v_dim > 0, w8 = h->w8a8;
    // required inputs
    if (!in->x || !in->positions || !in->w_kva || !in->gamma_kv || !in->cos || !in->sin)
        return MLAP_ERR_INVALID_ARG;
    if (has_q && (!in->w_qa || !in->w_qb || !in->gamma_q)) return MLAP_ERR_INVALID_ARG;
    if (has_kvb && !in->w_kvb) return MLAP_ERR_INVALID_ARG;
    const bool mx = h->mx;
    if (mx && (!in->ms_kva || (has_q && (!in->ms_qa || !in->ms_qb)) || (has_kvb && !in->ms_kvb)))
        return MLAP_ERR_INVALID_ARG;
    if (mx && ((reinterpret_cast<uintptr_t>(in->ms_qa) | reinterpret_cast<uintptr_t>(in->ms_qb) |
                reinterpret_cast<uintptr_t>(in->ms_kva) | reinterpret_cast<uintptr_t>(in->ms_kvb)) & 3))
        return MLAP_ERR_INVALID_ARG;  // the GEMMs read four block scales per 32-bit load
    if (w8 && (!in->ws_kva || (has_q && (!in->ws_qa || !in->ws_qb)) || (has_kvb && !in->ws_kvb)))
        return MLAP_ERR_INVALID_ARG;
    // outputs that need a branch this configuration lacks
    if (!has_q && (out->q_nope || out->q_pe || out->q_norm || out->q_i8 || out->q_scale))
        return MLAP_ERR_INVALID_ARG;
    if (!has_kvb && (out->k_nope || out->value)) return MLAP_ERR_INVALID_ARG;
    // a KV cache write needs the slots and the cache size
    const bool cache = out->kv_cache || out->kv_cache_i8 || out->kv_cache_scale || out->kr_cache;
    if (cache && (!in->slot_mapping || in->cache_slots <= 0)) return MLAP_ERR_INVALID_ARG;
    // the q quant reads the q tensors back
    const bool quant_q = out->q_i8 || out->q_scale;
    const int per_head = (c.flags & MLAP_QUANT_Q_PER_HEAD) ? 1 : 0;
    const bool head_norm = h->head_norm();
    if (quant_q && out->q_i8 && (!out->q_nope || !out->q_pe)) return MLAP_ERR_INVALID_ARG;
    // the per-head quant reads every head's values back, and the per-head norm rewrites the
    // raw heads in place: both need the two q tensors, for any q output
    const bool need_q = has_q && (out->q_nope || out->q_pe || quant_q || out->q_proj);
    if ((head_norm && need_q) || (quant_q && per_head))
        if (!out->q_nope || !out->q_pe) return MLAP_ERR_INVALID_ARG;
    if (out->q_proj && !head_norm) return MLAP_ERR_INVALID_ARG;  // the tap exists with the head norm only
    // 16-byte alignment of every tensor the kernels touch (the MXFP8 scales: 4 bytes, above)
    {
        const void* ptrs[] = {in->x, in->positions, in->w_qa, in->w_qb, in->w_kva, in->w_kvb,
                              in->ws_qa, in->ws_qb, in->ws_kva, in->ws_kvb, in->gamma_q, in->gamma_kv,
                              in->cos, in->sin, in->slot_mapping, out->q_nope, out->q_pe, out->kv_norm,
                              out->k_pe, out->k_nope, out->value, out->q_norm, out->q_i8, out->q_scale,
                              out->kv_i8, out->kv_scale, out->kv_cache, out->kv_cache_i8,
                              out->kv_cache_scale, out->kr_cache, out->a_proj, out->q_proj};
        for (const void* p : ptrs)
            if (misaligned16(p)) return MLAP_ERR_INVALID_ARG;
    }
    const WsLayout L = h->layout(T);
    if (!ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) % kAlign))
        return MLAP_ERR_WORKSPACE;

    char* wsb = static_cast<char*>(ws);
    hipStream_t s = as_stream(stream);
    const int Lq = c.q_lora, Lkv = c.kv_lora, R = c.rope_dim, H = c.n_heads;
    uint16_t* a1 = reinterpret_cast<uint16_t*>(wsb + L.a1);
    uint16_t* qn = has_q ? (out->q_norm ? static_cast<uint16_t*>(out->q_norm)
                                        : reinterpret_cast<uint16_t*>(wsb + L.qn))
                         : nullptr;
    // kv_norm is the kv_b input in KV-Prolog mode: write it to the output when the caller
    // wants it, else to the workspace.
    uint16_t* kvn = out->kv_norm ? static_cast<uint16_t*>(out->kv_norm)
                                 : (has_kvb ? reinterpret_cast<uint16_t*>(wsb + L.kvn) : nullptr);
    hipError_t e = hipSuccess;
#define MLAP_LAUNCH(kid, call)       \
    do {                             \
        h->tick(kid, s, true);       \
        e = (call);                  \
        h->tick(kid, s, false);      \
        if (e != hipSuccess) return MLAP_ERR_HIP; \
    } while (0)

    const Plan plan = h->plan(T);
    // 0. MXFP8: x converted block by block to E4M3 codes and E8M0 scales for the block-scaled
    // MFMA, or (shapes it does not take) the weights decoded to bf16 and x converted to its
    // exactly representable bf16 values, for the bf16 GEMMs
    const bool mxn = plan.mx_native;
    const bool mxd = mx && !mxn;
    uint16_t* wd_down = mxd ? reinterpret_cast<uint16_t*>(wsb + L.wd_down) : nullptr;
    uint16_t* xm = mxd ? reinterpret_cast<uint16_t*>(wsb + L.xm) : nullptr;
    if (mxn)
        MLAP_LAUNCH(kKMxConvert, launch_mx_act_codes(static_cast<const uint16_t*>(in->x), T, c.hidden,
                                                     reinterpret_cast<uint8_t*>(wsb + L.xq),
                                                     reinterpret_cast<uint8_t*>(wsb + L.xs), s));
    if (mxd) {
        if (has_q)
            MLAP_LAUNCH(kKMxConvert, launch_mx_dequant(static_cast<const uint8_t*>(in->w_qa), in->ms_qa, Lq,
                                                      c.hidden, wd_down, s));
        MLAP_LAUNCH(kKMxConvert, launch_mx_dequant(static_cast<const uint8_t*>(in->w_kva), in->ms_kva, Lkv + R,
                                                  c.hidden, wd_down + static_cast<size_t>(Lq) * c.hidden, s));
        if (has_q)
            MLAP_LAUNCH(kKMxConvert, launch_mx_dequant(static_cast<const uint8_t*>(in->w_qb), in->ms_qb, H * h->QH,
                                                      Lq, reinterpret_cast<uint16_t*>(wsb + L.wd_qb), s));
        if (has_kvb)
            MLAP_LAUNCH(kKMxConvert, launch_mx_dequant(static_cast<const uint8_t*>(in->w_kvb), in->ms_kvb, H * h->KH,
                                                      Lkv, reinterpret_cast<uint16_t*>(wsb + L.wd_kvb), s));
        MLAP_LAUNCH(kKMxConvert, launch_mx_act(static_cast<const uint16_t*>(in->x), T, c.hidden, xm, s));
    }

    // 1. down projection x . [W_qa ; W_kva]^T -> a1 [T, N1] bf16
    GemmArgs g{};
    g.M = T;
    g.N = h->N1;
    g.K = c.hidden;
    g.lda = c.hidden;
    g.ldb = c.hidden;
    g.B0 = mxd ? static_cast<const void*>(wd_down) : (has_q ? in->w_qa : in->w_kva);
    g.B1 = mxd ? static_cast<const void*>(wd_down + static_cast<size_t>(Lq) * c.hidden) : in->w_kva;
    g.b_split = Lq;
    if (c.flags & MLAP_ROPE_INTERLEAVED) {  // the k_pe slice of [q_a | c_kv | k_pe]
        g.pe_period = h->N1;
        g.pe_off = Lq + Lkv;
        g.pe_w = R;
    }
    g.k_splits = plan.down_splits;
    g.group_m = kGroupM;
    g.clk = h->clock_for(kKGemmDown);
    g.out = a1;
    g.ldo = h->N1;
    if (w8) {
        int8_t* xq = reinterpret_cast<int8_t*>(wsb + L.xq);
        float* xs = reinterpret_cast<float*>(wsb + L.xs);
        MLAP_LAUNCH(kKActQuant, launch_act_quant(static_cast<const uint16_t*>(in->x), T, c.hidden,
                                                 xq, xs, s));
        g.A = xq;
        g.a_scale = xs;
        g.b_scale0 = has_q ? in->ws_qa : in->ws_kva;
        g.b_scale1 = in->ws_kva;
        if (plan.x_fuse) {  // the k_pe columns as eight extra columns of every 256 x 256 tile
            g.N = plan.tail_c0;
            MLAP_LAUNCH(kKGemmDown, launch_gemm_big(g, InType::kInt8, Epi::kStoreBf16X, s));
            g.N = h->N1;
        } else {
            MLAP_LAUNCH(kKGemmDown, plan.big_down
                                        ? launch_gemm_big(g, InType::kInt8, Epi::kStoreBf16, s)
                                        : launch_gemm(g, InType::kInt8, plan.down, plan.down_epi, s));
        }
    } else if (plan.x_fuse) {
        // columns [0, tail_c0) as 256 x 256 tiles, each with eight of [tail_c0, N1) as extras
        g.A = mxd ? static_cast<const void*>(xm) : in->x;
        g.N = plan.tail_c0;
        MLAP_LAUNCH(kKGemmDown, launch_gemm_big(g, InType::kBf16, Epi::kStoreBf16X, s));
        g.N = h->N1;
    } else if (plan.tail_splits) {
        const InType it = mxn ? InType::kFp8 : InType::kBf16;
        const size_t eb = mxn ? 1 : 2;                                   // bytes per weight
        const size_t mxrow = static_cast<size_t>(c.hidden / 32);         // E8M0 bytes per row
        if (mxn) {
            g.A = wsb + L.xq;
            g.a_mx = reinterpret_cast<const uint8_t*>(wsb + L.xs);
            g.b_mx0 = has_q ? in->ms_qa : in->ms_kva;
            g.b_mx1 = in->ms_kva;
        } else {
            g.A = mxd ? static_cast<const void*>(xm) : in->x;
        }
        GemmArgs r = g;  // columns [tail_c0, N1): split-K fp32 partials
        r.N = h->N1 - plan.tail_c0;
        r.pe_c0 = plan.tail_c0;
        r.k_splits = plan.tail_splits;
        if (plan.tail_c0 >= g.b_split) {
            const size_t rows = static_cast<size_t>(plan.tail_c0 - g.b_split);
            r.B0 = r.B1 = static_cast<const char*>(g.B1) + rows * g.ldb * eb;
            if (mxn) r.b_mx0 = r.b_mx1 = g.b_mx1 + rows * mxrow;
            r.b_split = r.N;
        } else {
            const size_t rows = static_cast<size_t>(plan.tail_c0);
            r.B0 = static_cast<const char*>(g.B0) + rows * g.ldb * eb;
            if (mxn) r.b_mx0 = g.b_mx0 + rows * mxrow;
            r.b_split = g.b_split - plan.tail_c0;
        }
        r.out = wsb + L.tail;
        r.ldo = r.N;
        g.N = plan.tail_c0;
        MLAP_LAUNCH(kKGemmDown, launch_gemm_big(g, it, Epi::kStoreBf16, s) != hipSuccess
                                    ? hipErrorInvalidValue
                                    : gemm_big_fits(r, it, Epi::kStoreF32, BigShape::kSplitK)
                                          ? launch_gemm_big(r, it, Epi::kStoreF32, s, BigShape::kSplitK)
                                          : launch_gemm(r, it, GemmTile{256, 64, 3}, Epi::kStoreF32, s));
        g.N = h->N1;
    } else if (mxn) {
        g.A = wsb + L.xq;
        g.a_mx = reinterpret_cast<const uint8_t*>(wsb + L.xs);
        g.b_mx0 = has_q ? in->ms_qa : in->ms_kva;
        g.b_mx1 = in->ms_kva;
        MLAP_LAUNCH(kKGemmDown, launch_gemm_big(g, InType::kFp8, plan.down_epi, s, plan.down_shape));
    } else {
        g.A = mxd ? static_cast<const void*>(xm) : in->x;
        MLAP_LAUNCH(kKGemmDown, plan.big_down
                                    ? launch_gemm_big(g, InType::kBf16, plan.down_epi, s, plan.down_shape)
                                    : launch_gemm(g, InType::kBf16, plan.down, plan.down_epi, s));
    }

    // 2. row stage
    NormArgs na{};
    na.T = T;
    na.Lq = Lq;
    na.Lkv = Lkv;
    na.R = R;
    na.N1 = h->N1;
    na.k_splits = plan.down_splits;
    if (plan.tail_splits) {
        na.tail_f32 = reinterpret_cast<const float*>(wsb + L.tail);
        na.tail_c0 = plan.tail_c0;
        na.tail_splits = plan.tail_splits;
    }
    if (plan.down_epi == Epi::kStoreF32)
        na.a_f32 = reinterpret_cast<const float*>(a1);
    else
        na.a_bf16 = a1;
    na.gamma_q = static_cast<const uint16_t*>(in->gamma_q);
    na.gamma_kv = static_cast<const uint16_t*>(in->gamma_kv);
    na.eps = c.eps;
    na.rsqrt = (c.flags & MLAP_NORM_RSQRT) ? 1 : 0;
    na.positions = in->positions;
    na.cos = in->cos;
    na.sin = in->sin;
    na.max_pos = c.max_pos;
    na.q_norm = qn;
    na.kv_norm = static_cast<uint16_t*>(out->kv_norm);
    na.k_pe = static_cast<uint16_t*>(out->k_pe);
    na.kv_i8 = out->kv_i8;
    na.kv_scale = out->kv_scale;
    if (cache) {
        na.slots = in->slot_mapping;
        na.n_slots = in->cache_slots;
        na.kv_cache = static_cast<uint16_t*>(out->kv_cache);
        na.kv_cache_i8 = out->kv_cache_i8;
        na.kv_cache_scale = out->kv_cache_scale;
        na.kr_cache = static_cast<uint16_t*>(out->kr_cache);
    }
    na.a_proj = static_cast<uint16_t*>(out->a_proj);
    const bool need_kvb = has_kvb && (out->k_nope || out->value);
    if (need_kvb && !w8) na.kv_norm = kvn;  // the bf16 kv_b reads it
    if (w8 && need_q) {
        na.qn_i8 = reinterpret_cast<int8_t*>(wsb + L.qnq);
        na.qn_scale = reinterpret_cast<float*>(wsb + L.qns);
    }
    if (w8 && need_kvb) {
        na.kv_i8_b = reinterpret_cast<int8_t*>(wsb + L.kvq);
        na.kv_scale_b = reinterpret_cast<float*>(wsb + L.kvs);
    }
    MLAP_LAUNCH(kKNormRope, launch_norm(na, s));

    // 3. q up projection with split / RoPE / partial amax epilogue
    if (need_q) {
        GemmArgs u{};
        u.M = T;
        u.N = H * h->QH;
        u.K = Lq;
        u.lda = Lq;
        u.ldb = Lq;
        u.B0 = u.B1 = mxd ? static_cast<const void*>(wsb + L.wd_qb) : in->w_qb;
        u.b_split = u.N;
        u.k_splits = 1;
        u.group_m = kGroupM;
        u.n_major = 1;   // B (75 MB at V3) dwarfs A: give each XCD a 1/8 share of B
        u.group_m = kGroupNq;
        u.clk = h->clock_for(kKGemmUpQ);
        u.head_w = h->QH;
        u.d0 = c.nope_dim;
        u.d1 = R;
        u.rope = head_norm ? 0 : 1;  // with the per-head norm, RoPE follows it in the row kernel
        if (c.flags & MLAP_ROPE_INTERLEAVED) {  // the rope slice of every q head
            u.pe_period = h->QH;
            u.pe_off = c.nope_dim;
            u.pe_w = R;
        }
        u.n_heads = H;
        u.out0 = out->q_nope;
        u.out1 = out->q_pe;
        u.positions = in->positions;
        u.cos = in->cos;
        u.sin = in->sin;
        u.max_pos = c.max_pos;
        // per-token q quant: the epilogue's per-tile partial amax (per-head quant reads the rows)
        u.part_amax = quant_q && !per_head && !head_norm ? reinterpret_cast<float*>(wsb + L.qpart) : nullptr;
        u.n_tiles = plan.nt_q;
        const InType it = w8 ? InType::kInt8 : mxn ? InType::kFp8 : InType::kBf16;
        if (w8) {
            u.A = na.qn_i8;
            u.a_scale = na.qn_scale;
            u.b_scale0 = u.b_scale1 = in->ws_qb;
        } else if (mxn) {  // q_norm as E4M3 codes with E8M0 block scales
            MLAP_LAUNCH(kKMxConvert, launch_mx_act_codes(qn, T, Lq, reinterpret_cast<uint8_t*>(wsb + L.qnq),
                                                         reinterpret_cast<uint8_t*>(wsb + L.qns), s));
            u.A = wsb + L.qnq;
            u.a_mx = reinterpret_cast<const uint8_t*>(wsb + L.qns);
            u.b_mx0 = u.b_mx1 = in->ms_qb;
        } else if (mx) {  // the MX conversion of q_norm
            uint16_t* qnm = reinterpret_cast<uint16_t*>(wsb + L.qnm);
            MLAP_LAUNCH(kKMxConvert, launch_mx_act(qn, T, Lq, qnm, s));
            u.A = qnm;
        } else {
            u.A = qn;
        }
        MLAP_LAUNCH(kKGemmUpQ, plan.big_q ? launch_gemm_big(u, it, Epi::kHeads, s, plan.q_shape)
                                          : launch_gemm(u, it, plan.up_q, Epi::kHeads, s));
        if (head_norm) {
            QHeadNormArgs hn{};
            hn.T = T;
            hn.H = H;
            hn.Dn = c.nope_dim;
            hn.R = R;
            hn.eps = c.eps;
            hn.rsqrt = (c.flags & MLAP_NORM_RSQRT) ? 1 : 0;
            hn.positions = in->positions;
            hn.cos = in->cos;
            hn.sin = in->sin;
            hn.max_pos = c.max_pos;
            hn.q_nope = static_cast<uint16_t*>(out->q_nope);
            hn.q_pe = static_cast<uint16_t*>(out->q_pe);
            hn.part_amax = quant_q && !per_head ? reinterpret_cast<float*>(wsb + L.qpart) : nullptr;
            hn.groups = plan.hn_groups;
            hn.q_proj = static_cast<uint16_t*>(out->q_proj);
            MLAP_LAUNCH(kKQHeadNorm, launch_q_head_norm(hn, s));
        }
    }

    // 4. kv_b up projection (KV-Prolog mode): per head [k_nope | value]
    if (need_kvb) {
        GemmArgs u{};
        u.M = T;
        u.N = H * h->KH;
        u.K = Lkv;
        u.lda = Lkv;
        u.ldb = Lkv;
        u.B0 = u.B1 = mxd ? static_cast<const void*>(wsb + L.wd_kvb) : in->w_kvb;
        u.b_split = u.N;
        u.k_splits = 1;
        u.group_m = kGroupM;
        u.clk = h->clock_for(kKGemmUpKv);
        u.head_w = h->KH;
        u.d0 = c.nope_dim;
        u.d1 = c.v_dim;
        u.rope = 0;
        u.n_heads = H;
        u.out0 = out->k_nope;
        u.out1 = out->value;
        const InType it = w8 ? InType::kInt8 : mxn ? InType::kFp8 : InType::kBf16;
        if (w8) {
            u.A = na.kv_i8_b;
            u.a_scale = na.kv_scale_b;
            u.b_scale0 = u.b_scale1 = in->ws_kvb;
        } else if (mxn) {  // kv_norm as E4M3 codes with E8M0 block scales
            MLAP_LAUNCH(kKMxConvert, launch_mx_act_codes(kvn, T, Lkv, reinterpret_cast<uint8_t*>(wsb + L.kvq),
                                                         reinterpret_cast<uint8_t*>(wsb + L.kvs), s));
            u.A = wsb + L.kvq;
            u.a_mx = reinterpret_cast<const uint8_t*>(wsb + L.kvs);
            u.b_mx0 = u.b_mx1 = in->ms_kvb;
        } else if (mx) {  // the MX conversion of kv_norm
            uint16_t* kvnm = reinterpret_cast<uint16_t*>(wsb + L.kvnm);
            MLAP_LAUNCH(kKMxConvert, launch_mx_act(kvn, T, Lkv, kvnm, s));
            u.A = kvnm;
        } else {
            u.A = kvn;
        }
        MLAP_LAUNCH(kKGemmUpKv, plan.big_kv ? launch_gemm_big(u, it, Epi::kHeads, s, plan.kv_shape)
                                            : launch_gemm(u, it, plan.up_kv, Epi::kHeads, s));
    }

    // 5. per-token INT8 quant of q (after RoPE), one scale over all heads
    if (has_q && quant_q) {
        QuantQArgs qa{};
        qa.T = T;
        qa.H = H;
        qa.Dn = c.nope_dim;
        qa.R = R;
        qa.n_tiles = head_norm ? plan.hn_groups : plan.nt_q;  // head norm: one partial per group
        qa.part_amax = reinterpret_cast<const float*>(wsb + L.qpart);
        qa.per_head = per_head;
        qa.q_nope = static_cast<const uint16_t*>(out->q_nope);
        qa.q_pe = static_cast<const uint16_t*>(out->q_pe);
        qa.q_i8 = out->q_i8;
        qa.q_scale = out->q_scale;
        MLAP_LAUNCH(kKQuantQ, launch_quant_q(qa, s));
    }
#undef MLAP_LAUNCH
    return MLAP_OK;
}

}  // namespace

extern "C" {

MLAP_API int mlap_gemm_i8_i32(void* stream, const int8_t* A, const int8_t* B, int32_t* C, int32_t M,
                     int32_t N, int32_t K) {
    if (M < 0 || N < 0 || K <= 0) return MLAP_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MLAP_OK;
    if (!A || !B || !C) return MLAP_ERR_INVALID_ARG;
    if (K % 128) return MLAP_ERR_UNSUPPORTED;
    if (misaligned16(A) || misaligned16(B) || misaligned16(C)) return MLAP_ERR_INVALID_ARG;
    GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = A;
    g.lda = K;
    g.B0 = g.B1 = B;
    g.b_split = N;
    g.ldb = K;
    g.k_splits = 1;
    g.group_m = kGroupM;
    g.out = C;
    g.ldo = N;
    // The W8A8 prolog's own tiles for a batch of M tokens: past the weight-streaming bucket the
    // LDS-DMA 256 x 256 tiles (with 64 x 64 tiles for a column remainder that is a multiple of
    // 64), else the register-staged tiles of the small-batch projections (128 x 192 as for the
    // q up projection when N is a whole number of 192-wide heads, else the down projection's
    // 256 x 64).
    hipError_t e;
    if (M > kSmallBatch)
        e = launch_gemm_big(g, InType::kInt8, Epi::kStoreI32, as_stream(stream));
    else if (N % 192 == 0)
        e = launch_gemm(g, InType::kInt8, GemmTile{128, 192, 3}, Epi::kStoreI32, as_stream(stream));
    else
        e = launch_gemm(g, InType::kInt8, GemmTile{256, 64, 1}, Epi::kStoreI32, as_stream(stream));
    return e == hipSuccess ? MLAP_OK : MLAP_ERR_HIP;
}

MLAP_API int mlap_gemm_bf16(void* stream, const void* A, const void* B, void* C, int32_t M, int32_t N,
                   int32_t K) {
    if (M < 0 || N < 0 || K <= 0) return MLAP_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MLAP_OK;
    if (!A || !B || !C) return MLAP_ERR_INVALID_ARG;
    if (K % 64 || N % 8) return MLAP_ERR_UNSUPPORTED;
    GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = A;
    g.lda = K;
    g.B0 = g.B1 = B;
    g.b_split = N;
    g.ldb = K;
    g.k_splits = 1;
    g.group_m = kGroupM;
    g.out = C;
    g.ldo = N;
    return launch_gemm(g, InType::kBf16, GemmTile{128, 128, 1}, Epi::kStoreBf16, as_stream(stream)) == hipSuccess
               ? MLAP_OK
               : MLAP_ERR_HIP;
}

MLAP_API int mlap_gemm_mxfp8_f32(void* stream, const uint8_t* A, const uint8_t* A_scale, const uint8_t* B,
                                 const uint8_t* B_scale, float* C, int32_t M, int32_t N, int32_t K) {
    if (M < 0 || N < 0 || K <= 0) return MLAP_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MLAP_OK;
    if (!A || !A_scale || !B || !B_scale || !C) return MLAP_ERR_INVALID_ARG;
    if (K % 128 || N % 4) return MLAP_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(A_scale) | reinterpret_cast<uintptr_t>(B_scale)) & 3) return MLAP_ERR_INVALID_ARG;
    GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = A;
    g.lda = K;
    g.B0 = g.B1 = B;
    g.b_split = N;
    g.ldb = K;
    g.k_splits = 1;
    g.group_m = kGroupM;
    g.out = C;
    g.ldo = N;
    g.a_mx = A_scale;
    g.b_mx0 = g.b_mx1 = B_scale;
    return launch_gemm_big(g, InType::kFp8, Epi::kStoreF32, as_stream(stream), BigShape::kSplitK) == hipSuccess
               ? MLAP_OK
               : MLAP_ERR_HIP;
}

}  // extern "C"
