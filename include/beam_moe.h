/*
 * beam_moe.h -- C-ABI of the BEAM masked-MoE layer forward on MI355X (gfx950).
 *
 * The layer (BEAM paper, "Binary Expert Activation Masking for Dynamic Routing
 * in MoE", section 3.2, Eq. 4-8):
 *   r = x W_gate^T, Top-K of r, g = Softmax over the K kept logits   (Eq. 4)
 *   z = x W_mask^T, m = [sigmoid(z) >= 0.5] = [z >= 0]                (Eq. 5-6)
 *   g_hat = g * m, no renormalisation, no minimum active count        (Eq. 7)
 *   y = sum_k g_hat_k * E_{id_k}(x), E(x) = (SiLU(x Wg) * (x Wu)) Wd  (Eq. 8, Eq. 3)
 * Masked slots carry the expert id -1 and are left out of the per-expert
 * counts, so masked (token, expert) pairs are never scheduled (the vLLM
 * integration described in section 5 of the news article on the paper).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *     16-byte aligned (tensor inputs/outputs) or 4-byte aligned (routing
 *     buffers).  The library never allocates, frees or retains memory, never
 *     synchronises the stream and never reads device memory on the host
 *     (beam_moe_forward_noalloc's static per-GPU workspace aside: it lives
 *     in the library's code object).
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; a return value of 0 means "enqueued".
 *   - Errors are negative and are detected on the host BEFORE anything is
 *     enqueued, except BEAM_EHIP (a launch failed; earlier stages of the same
 *     call may have been enqueued).  beam_moe_last_error() gives the message
 *     for the calling thread.
 *   - T = 0 is a valid call that enqueues nothing.
 *   - The library holds no mutable global state (beyond the static
 *     workspace of beam_moe_forward_noalloc and its per-GPU address table);
 *     calls from several threads are safe as long as they use distinct
 *     output and workspace buffers.
 *
 * Storage layouts (dtype = BEAM_F32: float everywhere; BEAM_BF16: bfloat16):
 *   x       [T, d]
 *   W_gate  [E, d]      one row per expert (the transpose of the paper's
 *   W_mask  [E, d]      R in R^{d x N} and W_m in R^{d_h x N}; nn.Linear layout)
 *   W_gu    [E+S, 2I, d] rows 0..I-1: gate projection (Eq. 3 "W_gate^(i)"),
 *                       rows I..2I-1: up projection; each row is one
 *                       intermediate unit; experts 0..E-1 routed, E..E+S-1
 *                       the S = desc.n_shared shared experts
 *   W_dt    [E+S, d, I] down projection, one row per output channel
 *   y       [T, d]
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BEAM_OK            0
#define BEAM_EINVAL       (-1) /* null/misaligned pointer, bad sizes, K > E ...   */
#define BEAM_EUNSUPPORTED (-2) /* valid but outside kernel coverage: E+S > 256,
                                  K > 16, or (bf16) d % 128, I % 64, I > 2040     */
#define BEAM_EWORKSPACE   (-3) /* workspace too small                              */
#define BEAM_EHIP         (-4) /* a HIP launch failed                              */

/* dtypes */
#define BEAM_F32  0
#define BEAM_BF16 1

/* desc.flags */
#define BEAM_FORCE_DECODE   (1u << 0) /* weight-streaming expert kernels          */
#define BEAM_FORCE_PREFILL  (1u << 1) /* LDS-tiled grouped-GEMM expert kernels;
                                         bf16, d % 256 == 0, I % 128 == 0.
                                         Without a flag, where allowed and
                                         T > 512, the device picks per call from
                                         the routed counts: tiled kernels if the
                                         blocks of <= 32 positions per expert
                                         number >= 1.25 x the active experts, or
                                         one expert has > 512 active pairs, else
                                         the streaming kernels.  Tiled calls use
                                         128-row tiles while those number < 1.3 x
                                         the 256-row tiles, else 256-row tiles */

/* stage ids for the optional per-stage events of beam_moe_forward_ex */
#define BEAM_STAGE_ROUTER   0 /* a1-a4: router logits, top-K, softmax, mask,
                                 g_hat, -1 ids, counts, offsets, lists (batches
                                 of at most 8 tokens: the logits only)            */
#define BEAM_STAGE_SELECT   1 /* (inside BEAM_STAGE_ROUTER: empty)                */
#define BEAM_STAGE_SCAN     2 /* (inside BEAM_STAGE_ROUTER: empty)                */
#define BEAM_STAGE_SCATTER  3 /* a4: pairs into per-expert lists, T > 64 only     */
#define BEAM_STAGE_UP       4 /* a5: expert gate/up projections + SiLU * up       */
#define BEAM_STAGE_DOWN     5 /* a6: expert down projection                       */
#define BEAM_STAGE_COMBINE  6 /* a7: masked weighted sum                          */
#define BEAM_NUM_STAGES     7

typedef struct beam_moe_desc {
    int32_t  T;        /* tokens                                   (>= 0)      */
    int32_t  d;        /* hidden size                              (> 0)       */
    int32_t  E;        /* routed experts, the paper's N            (> 0)       */
    int32_t  K;        /* top-K                                    (1..E)      */
    int32_t  I;        /* expert intermediate size                 (> 0)       */
    int32_t  dtype;    /* BEAM_F32 or BEAM_BF16                                */
    int32_t  block_m;  /* 0 = library picks (16 streaming, 128 tiled); else
                          16, 32, 64, 128 or 256 (the tiled path: 128 only)   */
    uint32_t flags;    /* BEAM_FORCE_*                                         */
    float    tau;      /* mask threshold on sigmoid(z); 0 means 0.5 (Eq. 6).
                          Evaluated exactly as z >= ln(tau / (1 - tau)).       */
    int32_t  n_shared; /* S >= 0 always-on shared experts (E + S <= 256): applied
                          to every token with weight 1, never masked, added
                          to the routed sum; their weights follow the routed
                          experts' in W_gu and W_dt (news article on the
                          paper, sections 5-6: DeepSeek / Qwen1.5-MoE shapes) */
    int32_t  reserved[2]; /* must be 0                                         */
} beam_moe_desc;

/* Routing outputs (all device pointers, caller-owned; sizes from
 * beam_moe_query).  A "pair" is p = t*K + k for the routed slot k of token t,
 * and p = T*K + t*S + s for shared expert E + s (S = desc.n_shared); the
 * grouping fields below cover the E + S experts. */
typedef struct beam_moe_routing {
    float   *gate_logits;    /* [T, E]  r (fp32 accumulate)                      */
    float   *mask_logits;    /* [T, E]  z                                        */
    int32_t *topk_ids;       /* [T, K]  descending r, equal r -> lower id first  */
    float   *topk_weights;   /* [T, K]  g (Eq. 4), before the mask               */
    uint8_t *mask;           /* [T, K]  m in {0, 1} (Eq. 6)                      */
    float   *g_hat;          /* [T, K]  g * m (Eq. 7)                            */
    int32_t *masked_ids;     /* [T, K]  topk_ids, or -1 where m = 0              */
    int32_t *expert_counts;  /* [E+S]   active pairs per expert (shared: T)      */
    int32_t *expert_offsets; /* [E+S+1] exclusive scan of counts rounded up to
                                        block_m                                  */
    int32_t *sorted_pairs;   /* [cap]   per expert: its pair ids ascending, then
                                        the pad value T*(K+S) up to a multiple
                                        of block_m; entries >= num_padded unused */
    int32_t *block_expert;   /* [cap/block_m] expert of each block_m block       */
    int32_t *active_experts; /* [E+S]   experts with count >= 1, ascending;
                                        entries >= n_active_experts unused       */
    int32_t *num_active;     /* [4]     {P = active pairs (shared included),
                                         num_padded, n_active_experts, n_blocks} */
} beam_moe_routing;

/* Sizes for a descriptor (host only, enqueues nothing). */
typedef struct beam_moe_sizes {
    size_t  workspace_bytes;   /* bytes needed by beam_moe_forward              */
    size_t  route_workspace_bytes; /* bytes needed by beam_moe_route            */
    int64_t cap;               /* length of sorted_pairs                        */
    int64_t n_blocks_cap;      /* length of block_expert                        */
    int32_t block_m;           /* block size in effect                          */
    int32_t path;              /* 0 = streaming kernels; 1 = tiled kernels (or,
                                  without BEAM_FORCE_PREFILL, streaming ones
                                  when the device finds few pairs per expert) */
    size_t  mask_backward_workspace_bytes; /* bytes needed by
                                  beam_moe_mask_backward                        */
} beam_moe_sizes;

/* beam_moe_query: validate `desc` and fill `out`.
 * Returns BEAM_OK, BEAM_EINVAL or BEAM_EUNSUPPORTED. */
int beam_moe_query(const beam_moe_desc *desc, beam_moe_sizes *out);

/* beam_moe_route: Eq. 4-7 and the grouping of active pairs (news article,
 * section 5: masked ids -> -1, excluded from the counts).
 * x, W_gate, W_mask: see the layouts above.  Writes every field of `out`.
 * ws: device workspace of at least sizes.route_workspace_bytes bytes. */
int beam_moe_route(const beam_moe_desc *desc, const void *x, const void *W_gate,
                   const void *W_mask, const beam_moe_routing *out, void *ws,
                   size_t ws_bytes, hipStream_t stream);

/* beam_moe_forward: the whole layer, Eq. 3-8.  Writes y [T, d] and every
 * routing field.  ws: at least sizes.workspace_bytes bytes. */
int beam_moe_forward(const beam_moe_desc *desc, const void *x, const void *W_gate,
                     const void *W_mask, const void *W_gu, const void *W_dt, void *y,
                     const beam_moe_routing *out, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* beam_moe_forward_ex: beam_moe_forward plus optional per-stage events.
 * stage_events: NULL, or an array of BEAM_NUM_STAGES + 1 entries, each a
 * caller-created event or NULL (not recorded); event i is recorded on
 * `stream` just before stage i is enqueued and event BEAM_NUM_STAGES after
 * the last stage (a stage that the chosen path fuses into another one, or
 * skips, has equal start and end events).  Decode batches of at most 8
 * tokens (bf16, streaming path, K + n_shared <= 32, T d * 2 and
 * (K + n_shared) I * 2 bytes at most 48 KB each) run three launches: stage ROUTER holds the router
 * logits only, the rest of a1-a4 runs inside stage UP and the combine inside
 * stage DOWN.  Each record is a separate stream command and adds a few
 * microseconds between the stages it separates. */
int beam_moe_forward_ex(const beam_moe_desc *desc, const void *x, const void *W_gate,
                        const void *W_mask, const void *W_gu, const void *W_dt,
                        void *y, const beam_moe_routing *out, void *ws,
                        size_t ws_bytes, hipStream_t stream,
                        hipEvent_t *stage_events);

/* beam_moe_forward_noalloc: beam_moe_forward without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * caller still passes the inputs, y and the routing outputs.  The workspace
 * is a static array of BEAM_NOALLOC_SCRATCH_BYTES in the library's code
 * object: one copy per GPU, allocated when the library's code is loaded on
 * that GPU and held until the process ends.  The call allocates and frees
 * nothing; its first call on a GPU looks up that GPU's copy (the current
 * device must be the stream's device).  Every call on one GPU shares that
 * GPU's copy, which keeps the last call's contents (no part of it needs to
 * start at zero): calls that may overlap on one GPU (different streams, or
 * several threads) race and must be serialised by the caller.
 * Returns BEAM_EWORKSPACE when the call needs more than
 * BEAM_NOALLOC_SCRATCH_BYTES (sizes.workspace_bytes of beam_moe_query); with
 * the Qwen3-30B-A3B-shaped layer (d 2048, I 768, E 128, K 8) that holds
 * batches of up to 512 tokens.  Other errors as for beam_moe_forward. */
#define BEAM_NOALLOC_SCRATCH_BYTES (64u << 20)
int beam_moe_forward_noalloc(const beam_moe_desc *desc, const void *x, const void *W_gate,
                             const void *W_mask, const void *W_gu, const void *W_dt, void *y,
                             const beam_moe_routing *out, hipStream_t stream);

/* beam_moe_mask_backward: gradients of the mask router for one layer call
 * (BEAM paper, section 3.3: straight-through estimation of the binarisation;
 * news article on the paper, section 4: a beta-weighted sparsity term over
 * the Top-K candidates' mask scores).  For token t, slot k (expert id_k,
 * softmax weight g_k, hard mask m_k, mask logit z = z[t, id_k]) and
 * slot_grad[t, k] = dL/dg_hat_k (the dot product of dL/dy_t with expert
 * id_k's output; needed for masked slots too):
 *   d_mask_logits[t, id_k] = (g_k * slot_grad[t,k] + beta) * sig(z)(1 - sig(z)),
 *                            0 at non-candidates       [T, E], required
 *   dW_mask = d_mask_logits^T x                       [E, d] or NULL
 *   dx      = d_mask_logits W_mask (mask router only)  [T, d] or NULL
 *   d_gate_logits[t, id_j] = g_j (m_j s_j - sum_k g_k m_k s_k), s = slot_grad,
 *                            0 off the Top-K           [T, E] or NULL
 * i.e. dL/dm_hat = dL/dm (STE) plus beta from L_sp = beta * sum over tokens
 * and candidates of m_hat.  All outputs float32, overwritten (not added to).
 * Reads routing->topk_ids, topk_weights, mask and mask_logits (of the
 * forward of `desc`, earlier on the same stream).  bf16 layers form dW_mask
 * on the matrix cores from d_mask_logits rounded to bf16 (float32
 * accumulation); dx and the other outputs use float32 arithmetic.
 * ws: at least sizes.mask_backward_workspace_bytes (may be 0 for float32
 * layers).  Errors as for beam_moe_forward; beta must be finite;
 * BEAM_EUNSUPPORTED for dW_mask of a bf16 layer with E * T * 2 >= 2^32
 * (E and T rounded up to 16 and 64). */
int beam_moe_mask_backward(const beam_moe_desc *desc, const void *x, const void *W_mask,
                           const beam_moe_routing *routing, const float *slot_grad, float beta,
                           float *d_mask_logits, float *dW_mask, float *dx,
                           float *d_gate_logits, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* beam_moe_stats: routing statistics, accumulated on the device.  They are
 * the quantities of the paper's analysis of the learned mask (news article on
 * the paper, section 7: how often the expert of each rank is masked, how many
 * experts a token activates, how evenly the experts are loaded).
 * routing: the mask [T, K] and masked_ids [T, K] of a routing of `desc`
 * (written by beam_moe_route or beam_moe_forward, enqueued earlier on the
 * same stream); no other field is read.  ADDS, as 64-bit integers, to:
 *   rank_masked [K]    tokens whose slot k (the k-th largest router logit)
 *                      is masked; rank_masked[k] / T = mask probability
 *   active_hist [K+1]  tokens with exactly j active slots, j = 0..K
 *   expert_load [E]    active pairs of each expert
 * Each output is a caller-owned, 8-byte aligned device array, or NULL (not
 * computed).  Zero them before the first call; the sums are exact and do
 * not depend on the order of the additions.  Returns BEAM_EINVAL for a bad
 * descriptor, a NULL mask or masked_ids or a misaligned output. */
int beam_moe_stats(const beam_moe_desc *desc, const beam_moe_routing *routing,
                   uint64_t *rank_masked, uint64_t *active_hist, uint64_t *expert_load,
                   hipStream_t stream);

/* Text for a status code (static storage). */
const char *beam_moe_strerror(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char *beam_moe_last_error(void);

/* Library version, e.g. "0.1.0". */
const char *beam_moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_MOE_H */
