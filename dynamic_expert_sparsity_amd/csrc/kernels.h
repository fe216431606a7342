// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace beam {

// decode batches of at most this many tokens take the small-batch kernels
// (routing + up projection in one launch, down projection + combine in one)
constexpr int SMALL_DECODE_T = 8;
// slots per token the small-batch down kernel holds in LDS (K + S)
constexpr int SMALL_SLOTS = 32;
// batches of at most this many tokens (one 64-token select tile) are routed
// and grouped by one workgroup (route_small)
constexpr int ROUTE_SMALL_T = 64;
static_assert(ROUTE_SMALL_T <= 64, "route_small holds one 64-token tile");
// larger batches of at most this many select tiles (64 tokens each): the
// pair-scatter workgroups make the per-tile bases themselves
constexpr int SCATTER_SELF_TILES = 32;

// Everything the launchers need, fixed on the host from the descriptor.
struct Plan {
    int T, d, E, K, I;
    int S;              // shared (always-on) experts, numbered E .. E+S-1
    int E2;             // E + S: experts of the grouping and the expert kernels
    int PT;             // T * (K + S): pair ids (routed t*K+k, then shared
                        // T*K + t*S + s); also the pad value of sorted_pairs
    int dtype;          // 0 f32, 1 bf16
    int bm;             // block_m
    int path;           // 0 streaming (decode), 1 tiled (prefill)
    int split;          // INT_MAX: streaming kernels only; 0: tiled kernels only;
                        // else (1) chosen per call on the device: tiled if the
                        // blocks of <= 32 positions number >= 1.25 x the active
                        // experts or one expert has more than 512 pairs (the
                        // per-call record meta)
    float thr;          // mask logit threshold: m = [z >= thr]
    // select / compaction
    int s_ts;           // tokens per select tile (64)
    int n_tiles;        // ceil(T / s_ts)
    int fuse_scatter;   // T <= ROUTE_SMALL_T: the routing workgroup also places the pairs
    int small;          // bf16 decode batch of <= SMALL_DECODE_T tokens: up_small / down_small
    long long cap;          // sorted_pairs capacity
    long long n_blocks_cap; // block_expert capacity
    int max_active;     // host upper bound on experts with >= 1 active pair
    // workspace carve-up (byte offsets) and totals
    size_t off_tile_mask, off_tile_base, off_cnt, off_pair_pos, off_meta, off_pbt, off_stok, off_h,
        off_o;
    size_t route_bytes, total_bytes;
};

struct Routing {
    float *gate_logits, *mask_logits;
    int32_t *topk_ids;
    float *topk_weights;
    uint8_t *mask;
    float *g_hat;
    int32_t *masked_ids;
    int32_t *expert_counts, *expert_offsets, *sorted_pairs, *block_expert;
    int32_t *active_experts, *num_active;
};

struct Work {  // workspace views
    uint64_t *tile_mask;
    int32_t *tile_base;
    int32_t *cnt;        // [E + S] per-expert active-pair counts (batches of > 32 tiles)
    int32_t *pair_pos;   // [T*K] sorted position of each pair, -1 if masked
    int32_t *meta;       // [4] the call's record {mode (1 tiled, 0 streaming),
                         // max count, position blocks, 0}
    int32_t *pbt;        // [pb_cap][4] per block of <= 32 positions of an expert:
                         // {expert, first position, rows, 0}
    int32_t *sorted_tok; // [cap] token of each sorted position (pads: unset)
    void *h;
    void *o;
};

// CUs of the current device (host; 256 when unknown)
int device_cus();
// router logits only (rows a1), and the logits plus select and compaction
hipError_t launch_router_logits(const Plan &p, const void *x, const void *Wg, const void *Wm,
                                const Routing &r, hipStream_t s);
hipError_t launch_route(const Plan &p, const void *x, const void *Wg, const void *Wm,
                        const Routing &r, const Work &w, hipStream_t s);
// batches of more than ROUTE_SMALL_T tokens: per-expert tile bases and
// counts after the select (more than SCATTER_SELF_TILES tiles; else the
// scatter makes them), then offsets and the pair scatter (a no-op for
// smaller batches, whose routing workgroup placed the pairs)
hipError_t launch_bases(const Plan &p, const Work &w, hipStream_t s);
hipError_t launch_scatter(const Plan &p, const Routing &r, const Work &w, hipStream_t s);
// the tiled path (bf16): one launch per projection runs the kernel family
// the compaction picked for the call (streaming, 128-row or 256-row tiles)
hipError_t launch_tiled_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                           const Work &w, hipStream_t s);
hipError_t launch_tiled_down(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                             hipStream_t s);
hipError_t launch_expert_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                            const Work &w, hipStream_t s);
hipError_t launch_expert_down(const Plan &p, const void *W_dt, const Routing &r,
                              const Work &w, hipStream_t s);
hipError_t launch_combine(const Plan &p, const Routing &r, const Work &w, void *y,
                          hipStream_t s);
// small decode batches: routing + expert up projection; down projection +
// combine (Plan::small)
hipError_t launch_up_small(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                           const Work &w, hipStream_t s);
hipError_t launch_down_small(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                             void *y, hipStream_t s);
// mask-router backward: workspace layout and launches
struct BwdPlan {
    int T_pad, E_pad;       // tokens rounded up to the dW stage, experts to 16
    int n_split;            // token ranges of the dW contraction
    int t_per_split;        // tokens per range (a multiple of the stage)
    int dx_tok;             // tokens per dx workgroup (a multiple of 16)
    size_t off_dzT, off_dzk, off_part, bytes;  // workspace carve-up (bf16 layers)
};
BwdPlan mask_backward_plan(const Plan &p);
hipError_t launch_mask_backward(const Plan &p, const BwdPlan &b, const void *x, const void *Wm,
                                const Routing &r, const float *sg, float beta, float *dz,
                                float *dW, float *dx, float *d_gate, void *ws, hipStream_t s);
// routing statistics added to caller-owned 64-bit counters (NULL: skipped)
hipError_t launch_stats(const Plan &p, const Routing &r, uint64_t *rank_masked,
                        uint64_t *active_hist, uint64_t *expert_load, hipStream_t s);

}  // namespace beam
