// C-ABI of libbeam_moe: argument validation, the launch plan, workspace
// carve-up and the stage sequence (declared in include/beam_moe.h).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "beam_moe.h"
#include "kernels.h"

using namespace beam;

// Workspace of beam_moe_forward_noalloc: one copy on every GPU the library
// runs on, allocated when the code object is loaded and held until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol): the device address of each GPU's copy
// comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) unsigned char scratch[BEAM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

namespace beam {
int device_cus() {
    static int n = 0;
    static std::once_flag once;
    std::call_once(once, [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            n = cus;
        if (n <= 0) n = 256;
    });
    return n;
}
}  // namespace beam

namespace {

bool aligned(const void *p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validate a descriptor and build the plan (host only).
int make_plan(const beam_moe_desc *desc, Plan &p) {
    if (!desc) return fail(BEAM_EINVAL, "desc is NULL");
    const beam_moe_desc &D = *desc;
    if (D.T < 0 || D.d <= 0 || D.E <= 0 || D.K <= 0 || D.I <= 0)
        return fail(BEAM_EINVAL, "sizes must satisfy T >= 0 and d, E, K, I > 0 (T=%d d=%d E=%d K=%d I=%d)",
                    D.T, D.d, D.E, D.K, D.I);
    if (D.K > D.E) return fail(BEAM_EINVAL, "K=%d exceeds E=%d", D.K, D.E);
    if (D.dtype != BEAM_F32 && D.dtype != BEAM_BF16)
        return fail(BEAM_EINVAL, "dtype %d is neither BEAM_F32 nor BEAM_BF16", D.dtype);
    if (D.block_m != 0 && D.block_m != 16 && D.block_m != 32 && D.block_m != 64 &&
        D.block_m != 128 && D.block_m != 256)
        return fail(BEAM_EINVAL, "block_m %d is not 0, 16, 32, 64, 128 or 256", D.block_m);
    if (D.flags & ~(BEAM_FORCE_DECODE | BEAM_FORCE_PREFILL))
        return fail(BEAM_EINVAL, "unknown flag bits 0x%x", D.flags);
    if ((D.flags & BEAM_FORCE_DECODE) && (D.flags & BEAM_FORCE_PREFILL))
        return fail(BEAM_EINVAL, "BEAM_FORCE_DECODE and BEAM_FORCE_PREFILL are exclusive");
    if (!(D.tau == 0.f || (D.tau > 0.f && D.tau < 1.f)))
        return fail(BEAM_EINVAL, "tau must be 0 (meaning 0.5) or lie in (0, 1)");
    if (D.n_shared < 0) return fail(BEAM_EINVAL, "n_shared=%d is negative", D.n_shared);
    if (D.reserved[0] || D.reserved[1])
        return fail(BEAM_EINVAL, "reserved fields must be 0");

    if (D.E + D.n_shared > 256)
        return fail(BEAM_EUNSUPPORTED, "E + n_shared = %d > 256", D.E + D.n_shared);
    if (D.K > 16) return fail(BEAM_EUNSUPPORTED, "K=%d > 16", D.K);
    if (D.dtype == BEAM_BF16 && (D.d % 128 != 0 || D.I % 64 != 0 || D.I > 2040))
        return fail(BEAM_EUNSUPPORTED,
                    "bf16 layer needs d %% 128 == 0, I %% 64 == 0 and I <= 2040 (d=%d I=%d)", D.d, D.I);
    const long long TK = (long long)D.T * D.K;
    const long long PT = (long long)D.T * (D.K + D.n_shared);
    if (PT > (1ll << 30)) return fail(BEAM_EUNSUPPORTED, "T*(K+n_shared)=%lld too large", PT);
    // the tiled (prefill) path: bf16, 128-position blocks, d % 256, I % 128;
    // its kernels address x and h with 32-bit byte offsets (below 2^31)
    const long long max_act_tiled = PT < D.E + D.n_shared ? PT : D.E + D.n_shared;
    const long long cap_tiled = (PT + max_act_tiled * 127 + 127) / 128 * 128;
    const bool offsets32 = (long long)D.T * D.d * 2 < (1ll << 31) &&
                           cap_tiled * D.I * 2 < (1ll << 31);
    const bool gemm_ok = D.dtype == BEAM_BF16 && D.d % 256 == 0 && D.I % 128 == 0 &&
                         (D.block_m == 0 || D.block_m == 128) && offsets32;
    if ((D.flags & BEAM_FORCE_PREFILL) && !gemm_ok)
        return fail(BEAM_EUNSUPPORTED,
                    "the tiled path needs bf16, d %% 256 == 0, I %% 128 == 0, block_m 0 or 128, "
                    "and x and the intermediate rows below 2 GiB");

    p.T = D.T; p.d = D.d; p.E = D.E; p.K = D.K; p.I = D.I;
    p.S = D.n_shared; p.E2 = D.E + D.n_shared; p.PT = (int)PT;
    p.dtype = D.dtype;
    // decode (weight streaming) for small batches, tiled grouped GEMM above
    p.path = (D.flags & BEAM_FORCE_PREFILL) ||
                     (!(D.flags & BEAM_FORCE_DECODE) && gemm_ok && D.T > 512)
                 ? 1
                 : 0;
    p.bm = p.path == 1 ? 128 : (D.block_m ? D.block_m : 16);
    // with few active pairs per expert the weights stream faster through the
    // streaming kernels than through mostly empty 256-row GEMM tiles; the
    // device decides per call from the routed counts
    p.split = p.path == 1 ? ((D.flags & BEAM_FORCE_PREFILL) ? 0 : 1) : INT_MAX;
    const float tau = D.tau == 0.f ? 0.5f : D.tau;
    // m = [sigmoid(z) >= tau]  <=>  z >= ln(tau / (1 - tau)); exactly 0 at tau = 0.5
    p.thr = tau == 0.5f ? 0.f : (float)std::log((double)tau / (1.0 - (double)tau));

    // small decode batches: routing + up projection in one launch, down
    // projection + combine in one (x and the token's h rows fit LDS)
    p.small = D.dtype == BEAM_BF16 && p.path == 0 && D.T <= SMALL_DECODE_T &&
              D.K + D.n_shared <= SMALL_SLOTS && (long long)D.T * D.d * 2 <= 48 * 1024 &&
              (long long)(D.K + D.n_shared) * D.I * 2 <= 48 * 1024;
    p.s_ts = 64;
    p.n_tiles = (D.T + 63) / 64;
    p.fuse_scatter = D.T <= ROUTE_SMALL_T;
    p.max_active = (int)(PT < p.E2 ? PT : p.E2);
    // the streaming kernels number their units (position blocks of <= 32 x
    // column groups of 16 units up / 32 channels down) in int
    if (D.dtype == BEAM_BF16) {
        const long long blocks = (long long)p.max_active + PT / 32 + 1;
        const long long groups = D.I / 16 > D.d / 32 ? D.I / 16 : D.d / 32;
        if (blocks * groups >= (1ll << 31))
            return fail(BEAM_EUNSUPPORTED, "T=%d is too large for the streaming kernels", D.T);
    }
    const long long cap_raw = PT + (long long)p.max_active * (p.bm - 1);
    p.cap = (cap_raw + p.bm - 1) / p.bm * p.bm;
    p.n_blocks_cap = p.cap / p.bm;

    const size_t elt = p.dtype == BEAM_BF16 ? 2 : 4;
    size_t off = 0;
    p.off_tile_mask = off; off = align_up(off + (size_t)p.n_tiles * p.E2 * 8, 256);
    p.off_tile_base = off; off = align_up(off + (size_t)p.n_tiles * p.E2 * 4, 256);
    p.off_cnt = off;       off = align_up(off + (size_t)p.E2 * 4, 256);
    p.off_pair_pos = off;  off = align_up(off + (size_t)PT * 4, 256);
    p.off_meta = off;      off = align_up(off + 16, 256);
    // position blocks of <= 32: at most one partial block per active expert
    p.off_pbt = off;       off = align_up(off + (size_t)(p.max_active + PT / 32 + 1) * 16, 256);
    // sorted tokens, plus 32 slack entries read (not used) past a block end
    p.off_stok = off;      off = align_up(off + (size_t)(p.cap + 32) * 4, 256);
    p.route_bytes = off;
    p.off_h = off;         off = align_up(off + (size_t)p.cap * D.I * elt, 256);
    p.off_o = off;         off = align_up(off + (size_t)p.cap * D.d * elt, 256);
    p.total_bytes = off;
    return BEAM_OK;
}

int check_routing(const beam_moe_routing *o, Routing &r) {
    if (!o) return fail(BEAM_EINVAL, "routing struct is NULL");
    const void *ptrs[] = {o->gate_logits,  o->mask_logits,    o->topk_ids,     o->topk_weights,
                          o->g_hat,        o->masked_ids,     o->expert_counts, o->expert_offsets,
                          o->sorted_pairs, o->block_expert,   o->active_experts, o->num_active};
    const char *names[] = {"gate_logits",  "mask_logits",  "topk_ids",      "topk_weights",
                           "g_hat",        "masked_ids",   "expert_counts", "expert_offsets",
                           "sorted_pairs", "block_expert", "active_experts", "num_active"};
    for (size_t i = 0; i < sizeof ptrs / sizeof ptrs[0]; ++i)
        if (!aligned(ptrs[i], 4)) return fail(BEAM_EINVAL, "routing.%s is NULL or not 4-byte aligned", names[i]);
    if (!o->mask) return fail(BEAM_EINVAL, "routing.mask is NULL");
    r.gate_logits = o->gate_logits; r.mask_logits = o->mask_logits;
    r.topk_ids = o->topk_ids; r.topk_weights = o->topk_weights; r.mask = o->mask;
    r.g_hat = o->g_hat; r.masked_ids = o->masked_ids;
    r.expert_counts = o->expert_counts; r.expert_offsets = o->expert_offsets;
    r.sorted_pairs = o->sorted_pairs; r.block_expert = o->block_expert;
    r.active_experts = o->active_experts; r.num_active = o->num_active;
    return BEAM_OK;
}

Work carve(const Plan &p, void *ws) {
    char *b = static_cast<char *>(ws);
    Work w;
    w.tile_mask = reinterpret_cast<uint64_t *>(b + p.off_tile_mask);
    w.tile_base = reinterpret_cast<int32_t *>(b + p.off_tile_base);
    w.cnt = reinterpret_cast<int32_t *>(b + p.off_cnt);
    w.pair_pos = reinterpret_cast<int32_t *>(b + p.off_pair_pos);
    w.meta = reinterpret_cast<int32_t *>(b + p.off_meta);
    w.pbt = reinterpret_cast<int32_t *>(b + p.off_pbt);
    w.sorted_tok = reinterpret_cast<int32_t *>(b + p.off_stok);
    w.h = b + p.off_h;
    w.o = b + p.off_o;
    return w;
}

struct Events {
    hipEvent_t *ev;
    hipStream_t s;
    hipError_t mark(int i) const { return ev && ev[i] ? hipEventRecord(ev[i], s) : hipSuccess; }
};

#define BEAM_TRY(expr, stage)                                                             \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess)                                                             \
            return fail(BEAM_EHIP, "%s: %s", stage, hipGetErrorString(e_));               \
    } while (0)

int enqueue_route(const Plan &p, const void *x, const void *Wg, const void *Wm, const Routing &r,
                  const Work &w, hipStream_t s, const Events &ev) {
    BEAM_TRY(ev.mark(BEAM_STAGE_ROUTER), "event");
    BEAM_TRY(launch_route(p, x, Wg, Wm, r, w, s), "routing");
    BEAM_TRY(ev.mark(BEAM_STAGE_SELECT), "event");
    BEAM_TRY(ev.mark(BEAM_STAGE_SCAN), "event");
    BEAM_TRY(ev.mark(BEAM_STAGE_SCATTER), "event");
    BEAM_TRY(launch_scatter(p, r, w, s), "compaction scatter");
    return BEAM_OK;
}

int check_inputs(const void *x, const void *Wg, const void *Wm) {
    if (!aligned(x, 16)) return fail(BEAM_EINVAL, "x is NULL or not 16-byte aligned");
    if (!aligned(Wg, 16)) return fail(BEAM_EINVAL, "W_gate is NULL or not 16-byte aligned");
    if (!aligned(Wm, 16)) return fail(BEAM_EINVAL, "W_mask is NULL or not 16-byte aligned");
    return BEAM_OK;
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// The device address of the current GPU's scratch copy, looked up once per
// device (with that device current) and kept.
int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BEAM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(BEAM_EUNSUPPORTED, "device %d is beyond the %d devices the scratch table holds",
                    dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(BEAM_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BEAM_OK;
}

}  // namespace

extern "C" {

int beam_moe_query(const beam_moe_desc *desc, beam_moe_sizes *out) {
    Plan p;
    int rc = make_plan(desc, p);
    if (rc) return rc;
    if (!out) return fail(BEAM_EINVAL, "sizes output is NULL");
    out->workspace_bytes = p.total_bytes;
    out->route_workspace_bytes = p.route_bytes;
    out->cap = p.cap;
    out->n_blocks_cap = p.n_blocks_cap;
    out->block_m = p.bm;
    out->path = p.path;
    out->mask_backward_workspace_bytes = mask_backward_plan(p).bytes;
    return BEAM_OK;
}

int beam_moe_route(const beam_moe_desc *desc, const void *x, const void *W_gate,
                   const void *W_mask, const beam_moe_routing *out, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
    Plan p;
    int rc = make_plan(desc, p);
    if (rc) return rc;
    if (p.T == 0) return BEAM_OK;
    if ((rc = check_inputs(x, W_gate, W_mask))) return rc;
    Routing r;
    if ((rc = check_routing(out, r))) return rc;
    if (!aligned(ws, 16)) return fail(BEAM_EINVAL, "workspace is NULL or not 16-byte aligned");
    if (ws_bytes < p.route_bytes)
        return fail(BEAM_EWORKSPACE, "workspace has %zu bytes, route needs %zu", ws_bytes, p.route_bytes);
    return enqueue_route(p, x, W_gate, W_mask, r, carve(p, ws), stream, Events{nullptr, stream});
}

int beam_moe_forward_ex(const beam_moe_desc *desc, const void *x, const void *W_gate,
                        const void *W_mask, const void *W_gu, const void *W_dt, void *y,
                        const beam_moe_routing *out, void *ws, size_t ws_bytes,
                        hipStream_t stream, hipEvent_t *stage_events) {
    Plan p;
    int rc = make_plan(desc, p);
    if (rc) return rc;
    if (p.T == 0) return BEAM_OK;
    if ((rc = check_inputs(x, W_gate, W_mask))) return rc;
    if (!aligned(W_gu, 16)) return fail(BEAM_EINVAL, "W_gu is NULL or not 16-byte aligned");
    if (!aligned(W_dt, 16)) return fail(BEAM_EINVAL, "W_dt is NULL or not 16-byte aligned");
    if (!aligned(y, 16)) return fail(BEAM_EINVAL, "y is NULL or not 16-byte aligned");
    Routing r;
    if ((rc = check_routing(out, r))) return rc;
    if (!aligned(ws, 16)) return fail(BEAM_EINVAL, "workspace is NULL or not 16-byte aligned");
    if (ws_bytes < p.total_bytes)
        return fail(BEAM_EWORKSPACE, "workspace has %zu bytes, forward needs %zu", ws_bytes, p.total_bytes);

    const Work w = carve(p, ws);
    const Events ev{stage_events, stream};
    if (p.small) {
        // logits; then routing + up projection; then down projection + combine
        BEAM_TRY(ev.mark(BEAM_STAGE_ROUTER), "event");
        BEAM_TRY(launch_router_logits(p, x, W_gate, W_mask, r, stream), "router logits");
        for (int st = BEAM_STAGE_SELECT; st <= BEAM_STAGE_UP; ++st) BEAM_TRY(ev.mark(st), "event");
        BEAM_TRY(launch_up_small(p, x, W_gu, r, w, stream), "routing and expert up");
        BEAM_TRY(ev.mark(BEAM_STAGE_DOWN), "event");
        BEAM_TRY(launch_down_small(p, W_dt, r, w, y, stream), "expert down and combine");
        BEAM_TRY(ev.mark(BEAM_STAGE_COMBINE), "event");
        BEAM_TRY(ev.mark(BEAM_NUM_STAGES), "event");
        return BEAM_OK;
    }
    if ((rc = enqueue_route(p, x, W_gate, W_mask, r, w, stream, ev))) return rc;
    BEAM_TRY(ev.mark(BEAM_STAGE_UP), "event");
    BEAM_TRY(launch_expert_up(p, x, W_gu, r, w, stream), "expert up");
    BEAM_TRY(ev.mark(BEAM_STAGE_DOWN), "event");
    BEAM_TRY(launch_expert_down(p, W_dt, r, w, stream), "expert down");
    BEAM_TRY(ev.mark(BEAM_STAGE_COMBINE), "event");
    BEAM_TRY(launch_combine(p, r, w, y, stream), "combine");
    BEAM_TRY(ev.mark(BEAM_NUM_STAGES), "event");
    return BEAM_OK;
}

int beam_moe_forward(const beam_moe_desc *desc, const void *x, const void *W_gate,
                     const void *W_mask, const void *W_gu, const void *W_dt, void *y,
                     const beam_moe_routing *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    return beam_moe_forward_ex(desc, x, W_gate, W_mask, W_gu, W_dt, y, out, ws, ws_bytes, stream,
                               nullptr);
}

int beam_moe_forward_noalloc(const beam_moe_desc *desc, const void *x, const void *W_gate,
                             const void *W_mask, const void *W_gu, const void *W_dt, void *y,
                             const beam_moe_routing *out, hipStream_t stream) {
    Plan p;
    int rc = make_plan(desc, p);
    if (rc) return rc;
    if (p.total_bytes > (size_t)BEAM_NOALLOC_SCRATCH_BYTES)
        return fail(BEAM_EWORKSPACE,
                    "this layer call needs %zu bytes of workspace; the allocation-free entry point "
                    "holds %zu (use beam_moe_forward with a workspace)",
                    p.total_bytes, (size_t)BEAM_NOALLOC_SCRATCH_BYTES);
    if (p.T == 0) return BEAM_OK;
    void *ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return beam_moe_forward_ex(desc, x, W_gate, W_mask, W_gu, W_dt, y, out, ws,
                               (size_t)BEAM_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int beam_moe_mask_backward(const beam_moe_desc *desc, const void *x, const void *W_mask,
                           const beam_moe_routing *routing, const float *slot_grad, float beta,
                           float *d_mask_logits, float *dW_mask, float *dx,
                           float *d_gate_logits, void *ws, size_t ws_bytes, hipStream_t stream) {
    Plan p;
    int rc = make_plan(desc, p);
    if (rc) return rc;
    if (p.T == 0) return BEAM_OK;
    if (!aligned(x, 16)) return fail(BEAM_EINVAL, "x is NULL or not 16-byte aligned");
    if (!aligned(W_mask, 16)) return fail(BEAM_EINVAL, "W_mask is NULL or not 16-byte aligned");
    if (!routing) return fail(BEAM_EINVAL, "routing struct is NULL");
    if (!aligned(routing->topk_ids, 4) || !aligned(routing->topk_weights, 4) || !routing->mask ||
        !aligned(routing->mask_logits, 4))
        return fail(BEAM_EINVAL,
                    "routing.topk_ids, topk_weights, mask and mask_logits must be set");
    if (!aligned(slot_grad, 4)) return fail(BEAM_EINVAL, "slot_grad is NULL or misaligned");
    if (!aligned(d_mask_logits, 4)) return fail(BEAM_EINVAL, "d_mask_logits is NULL or misaligned");
    if (dW_mask && !aligned(dW_mask, 16)) return fail(BEAM_EINVAL, "dW_mask is not 16-byte aligned");
    if (dx && !aligned(dx, 16)) return fail(BEAM_EINVAL, "dx is not 16-byte aligned");
    if (d_gate_logits && !aligned(d_gate_logits, 4))
        return fail(BEAM_EINVAL, "d_gate_logits is not 4-byte aligned");
    if (!std::isfinite(beta)) return fail(BEAM_EINVAL, "beta is not finite");
    const BwdPlan b = mask_backward_plan(p);
    // the dW contraction addresses dz transposed with 32-bit byte offsets
    if (p.dtype == 1 && dW_mask && (unsigned long long)b.E_pad * b.T_pad * 2 >= (1ull << 32))
        return fail(BEAM_EUNSUPPORTED, "dW_mask of a bf16 layer needs E * T * 2 < 2^32 (T=%d)", p.T);
    if (b.bytes > 0 && !aligned(ws, 16))
        return fail(BEAM_EINVAL, "workspace is NULL or not 16-byte aligned");
    if (ws_bytes < b.bytes)
        return fail(BEAM_EWORKSPACE, "workspace has %zu bytes, the backward needs %zu", ws_bytes,
                    b.bytes);
    Routing r{};
    r.topk_ids = routing->topk_ids;
    r.topk_weights = routing->topk_weights;
    r.mask = routing->mask;
    r.mask_logits = routing->mask_logits;
    BEAM_TRY(launch_mask_backward(p, b, x, W_mask, r, slot_grad, beta, d_mask_logits, dW_mask, dx,
                                  d_gate_logits, ws, stream),
             "mask backward");
    return BEAM_OK;
}

int beam_moe_stats(const beam_moe_desc *desc, const beam_moe_routing *routing,
                   uint64_t *rank_masked, uint64_t *active_hist, uint64_t *expert_load,
                   hipStream_t stream) {
    Plan p;
    int rc = make_plan(desc, p);
    if (rc) return rc;
    if (!routing) return fail(BEAM_EINVAL, "routing struct is NULL");
    if (!routing->mask) return fail(BEAM_EINVAL, "routing.mask is NULL");
    if (!aligned(routing->masked_ids, 4))
        return fail(BEAM_EINVAL, "routing.masked_ids is NULL or not 4-byte aligned");
    const void *outs[] = {rank_masked, active_hist, expert_load};
    const char *names[] = {"rank_masked", "active_hist", "expert_load"};
    for (int i = 0; i < 3; ++i)
        if (outs[i] && !aligned(outs[i], 8))
            return fail(BEAM_EINVAL, "%s is not 8-byte aligned", names[i]);
    if (p.T == 0 || (!rank_masked && !active_hist && !expert_load)) return BEAM_OK;
    Routing r{};
    r.mask = routing->mask;
    r.masked_ids = routing->masked_ids;
    BEAM_TRY(launch_stats(p, r, rank_masked, active_hist, expert_load, stream), "statistics");
    return BEAM_OK;
}

const char *beam_moe_strerror(int status) {
    switch (status) {
        case BEAM_OK: return "ok";
        case BEAM_EINVAL: return "invalid argument";
        case BEAM_EUNSUPPORTED: return "unsupported configuration";
        case BEAM_EWORKSPACE: return "workspace too small";
        case BEAM_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

const char *beam_moe_last_error(void) { return g_last_error.c_str(); }

const char *beam_moe_version(void) { return "0.1.0"; }

}  // extern "C"
