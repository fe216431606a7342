// a1-a4: router logits (main router and mask router in one pass), then per
// token Top-K, softmax over the kept logits, binary mask, g_hat and -1 ids,
// then the grouping of the active pairs.
//
// BEAM paper, section 3.2: Eq. 4 (r = R(x), Top-K, Softmax over the kept K),
// Eq. 5 (z = x W_m), Eq. 6 (m = [sigmoid(z) >= 0.5], evaluated as z >= 0),
// Eq. 7 (g_hat = g * m, no renormalisation).  Masked slots get the expert id
// -1 and are left out of the per-expert counts (news article on the paper,
// section 5, the two modified kernels).
//
// Kernels: the logits (many workgroups, each a 16-column block), then either
// one workgroup that selects and groups a small batch, or one workgroup per
// quarter of a 64-token tile for the select and one workgroup for the
// grouping.
#include <type_traits>

#include "compact_dev.h"

namespace beam {

// ---------------------------------------------------------------------------
// Router logits block, bf16, MFMA 16x16x32.  The two routers are one GEMM
// with 2E output columns: column n < E is W_gate row n, column E + n is
// W_mask row n.  A workgroup owns 16*NC columns and 16*MT tokens; its NW
// waves split d (every wave requests a batch of its x and weight fragments
// before the MFMAs that use them) and their partial sums meet in LDS, where
// wave c adds them for column block c in wave order and writes the finished
// float32 logits.  A (x rows) and B (weight rows) are both k-contiguous, so
// every lane's 16-byte load lands directly in MFMA layout.  More column
// blocks per workgroup read each x row fewer times (2E / (16 NC) times in
// all); one block gives the most workgroups for small batches.  Out-of-range
// tokens / columns load a clamped row and their results are not stored.
// ---------------------------------------------------------------------------
template <int MT, int NW, int NC>
__global__ __launch_bounds__(NW * 64) void router_logits_bf16(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Wg, const bf16_t *__restrict__ Wm,
    float *__restrict__ gate_logits, float *__restrict__ mask_logits, int T, int d, int E) {
    static_assert(NC <= NW, "one wave per column block in the final sum");
    __shared__ f32x4 red[NW][MT][NC][64];
    const int rtile = blockIdx.x;
    const int cgroup = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int twoE = 2 * E;
    const int kq = (lane >> 4) * 8;
    const int dq = d / NW;
    const int kb = wave * dq + kq;
    const bf16_t *brow[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int n = (cgroup * NC + c) * 16 + (lane & 15);
        const int nc = n < twoE ? n : twoE - 1;
        brow[c] = (nc < E ? Wg + (size_t)nc * d : Wm + (size_t)(nc - E) * d) + kb;
    }
    const int tbase = rtile * 16 * MT;

    const bf16_t *arow[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int t = tbase + m * 16 + (lane & 15);
        t = t < T ? t : T - 1;
        arow[m] = x + (size_t)t * d + kb;
    }
    f32x4 acc[MT][NC];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int CH = NC == 1 ? 8 : 4;  // k-steps requested per batch
    for (int k0 = 0; k0 < dq; k0 += 32 * CH) {
        u32x4 b[CH][NC], a[CH][MT];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int k = k0 + 32 * j;
            if (k < dq) {
#pragma unroll
                for (int c = 0; c < NC; ++c) b[j][c] = ld16(brow[c] + k);
#pragma unroll
                for (int m = 0; m < MT; ++m) a[j][m] = ld16(arow[m] + k);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (k0 + 32 * j < dq)
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int c = 0; c < NC; ++c) acc[m][c] = mfma16x16x32(a[j][m], b[j][c], acc[m][c]);
    }

#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) red[wave][m][c][lane] = acc[m][c];
    __syncthreads();
    if (wave >= NC) return;
    const int c = wave;  // this wave's column block
    const int n = (cgroup * NC + c) * 16 + (lane & 15);
    if (n >= twoE) return;
    float *out = n < E ? gate_logits + n : mask_logits + (n - E);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        f32x4 v = red[0][m][c][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][m][c][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tbase + m * 16 + (lane >> 4) * 4 + i;
            if (t < T) out[(size_t)t * E] = v[i];
        }
    }
}

// Router logits, float32 layer: plain float dot products, one thread per
// (token, column).
template <typename T_>
__global__ __launch_bounds__(256) void router_logits_generic(
    const T_ *__restrict__ x, const T_ *__restrict__ Wg, const T_ *__restrict__ Wm,
    float *__restrict__ gate_logits, float *__restrict__ mask_logits, int T, int d, int E) {
    const int twoE = 2 * E;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * twoE) return;
    const int t = (int)(idx / twoE);
    const int n = (int)(idx % twoE);
    const T_ *w = n < E ? Wg + (size_t)n * d : Wm + (size_t)(n - E) * d;
    const T_ *xr = x + (size_t)t * d;
    float acc = 0.f;
    for (int k = 0; k < d; ++k) acc = fmaf(elem<T_>::load(xr + k), elem<T_>::load(w + k), acc);
    if (n < E) gate_logits[(size_t)t * E + n] = acc;
    else mask_logits[(size_t)t * E + (n - E)] = acc;
}

// ---------------------------------------------------------------------------
// Select (Eq. 4-7 per token).  A token is handled by the 16 lanes of one DPP
// row of a wavefront; lane i of the row holds the gate logits of experts
// i*EJ .. i*EJ+EJ-1, so a wavefront handles 4 consecutive tokens.  K rounds
// of a row-wide arg-max under the key (value desc, expert asc) give the Top-K
// slots in order (Eq. 4); slot k (K <= 16) is kept by lane k.  Softmax over the kept logits shifted by the largest
// (Eq. 4); the winners' mask logits are gathered afterwards and m = z >= thr
// (Eq. 6, thr = 0 for tau = 0.5); g_hat = g * m (Eq. 7); id -1 where masked.
// tmask[e] collects the set of tokens with an active pair for expert e, bit
// t % TB for token t (TB = 64: a 64-token tile in 64-bit words; TB = 16: a
// quarter tile in 32-bit words); s_mid (optional, LDS) receives the masked ids.
//
// The group reductions use DPP lane moves: swap neighbours, swap pairs (a
// quad), then mirror within 8 and within 16 (a row).  Each step combines two
// values that are the same pair for both partners, so every lane of the
// group ends with the same result (also for the float sum).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool beats(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

constexpr int DPP_QUAD_1032 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

constexpr int NO_EXPERT = 0x7fffffff;

template <int CTRL>
__device__ __forceinline__ void argmax_step(float &bv, int &be) {
    const float ov = dpp_f<CTRL>(bv);
    const int oe = dpp_i<CTRL>(be);
    if (oe != NO_EXPERT && (be == NO_EXPERT || beats(ov, oe, bv, be))) {
        bv = ov;
        be = oe;
    }
}

__device__ __forceinline__ void row_argmax(float &bv, int &be) {
    argmax_step<DPP_QUAD_1032>(bv, be);
    argmax_step<DPP_QUAD_2301>(bv, be);
    argmax_step<DPP_ROW_HALF_MIRROR>(bv, be);
    argmax_step<DPP_ROW_MIRROR>(bv, be);
}

__device__ __forceinline__ float row_sum(float v) {
    v += dpp_f<DPP_QUAD_1032>(v);
    v += dpp_f<DPP_QUAD_2301>(v);
    v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_f<DPP_ROW_MIRROR>(v);
    return v;
}

// One wavefront: tokens t_first .. t_first + 3 (all in one tile).
template <int EJ, int TB>
__device__ __forceinline__ void select_group(
    int T, int E, int K, float thr, const Routing &r,
    std::conditional_t<TB == 64, unsigned long long, unsigned> *tmask, int *s_mid, int t_first,
    int lane) {
    using MW = std::conditional_t<TB == 64, unsigned long long, unsigned>;
    static_assert(TB == 64 || TB == 16, "token bits per mask word");
    static_assert(EJ >= 1 && EJ <= 16, "at most 16 experts per lane (E <= 256)");
    const int i = lane & 15;
    const int t = t_first + (lane >> 4);
    const bool valid = t < T;
    const int tc = valid ? t : T - 1;
    const int tl = t & (TB - 1);
    const int e0 = i * EJ;
    // 16-byte loads when every lane's run of EJ logits is 16-byte aligned and whole
    const bool vec = (EJ % 4 == 0) && (E % 4 == 0) && (e0 + EJ <= E);
    const float *gr = r.gate_logits + (size_t)tc * E + e0;

    float rv[EJ];
    if (vec) {
        if constexpr (EJ % 4 == 0) {
#pragma unroll
            for (int j = 0; j < EJ / 4; ++j) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(gr + 4 * j);
#pragma unroll
                for (int u = 0; u < 4; ++u) rv[4 * j + u] = a[u];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < EJ; ++j) rv[j] = e0 + j < E ? gr[j] : 0.f;
    }
    unsigned live = 0;
#pragma unroll
    for (int j = 0; j < EJ; ++j)
        if (e0 + j < E) live |= 1u << j;

    // slot k is kept by lane k
    float v0 = 0.f, myv = 0.f;
    int mye = 0;
    for (int k = 0; k < K; ++k) {
        float bv = 0.f;
        int be = NO_EXPERT;
#pragma unroll
        for (int j = 0; j < EJ; ++j) {  // expert index ascends with j: ties keep the first
            if (((live >> j) & 1u) && (be == NO_EXPERT || rv[j] > bv)) {
                bv = rv[j];
                be = e0 + j;
            }
        }
        row_argmax(bv, be);
        const int jw = be - e0;
        if (jw >= 0 && jw < EJ) live &= ~(1u << jw);
        if (k == 0) v0 = bv;
        if (k == i) {
            myv = bv;
            mye = be;
        }
    }

    const float num = i < K ? expf(myv - v0) : 0.f;
    const float den = row_sum(num);
    if (!valid || i >= K) return;
    const int k = i;
    const float z = r.mask_logits[(size_t)t * E + mye];
    const float g = num / den;
    const bool m = z >= thr;
    const int o = t * K + k;
    r.topk_ids[o] = mye;
    r.topk_weights[o] = g;
    r.mask[o] = m ? 1 : 0;
    r.g_hat[o] = m ? g : 0.f;
    r.masked_ids[o] = m ? mye : -1;
    if (s_mid) s_mid[o] = m ? mye : -1;
    if (m) atomicOr(&tmask[mye], (MW)1 << tl);
}

// The token set of tile `tile` for a shared expert: every valid token.
__device__ __forceinline__ unsigned long long tile_all(int tile, int T) {
    const int n = T - tile * 64;
    return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
}

// One workgroup of four wavefronts per quarter (16 tokens) of a 64-token
// tile, 16 lanes per token: the select, and the quarter's bits of the tile's
// token sets for the E routed and S shared experts ([tile][E + S] 64-bit
// words; bits 16 q .. 16 q + 15 belong to quarter q).  A quarter writes its
// 16 bits of every word with one 16-bit store, so the words need neither
// clearing nor atomics across workgroups.  Quarter-tile workgroups spread a
// batch of a few hundred tokens over four times as many compute units as
// whole-tile ones: the K dependent arg-max rounds are the select's critical
// path.
template <int EJ>
__global__ __launch_bounds__(256) void select_topk_mask(int T, int E, int S, int K, float thr,
                                                        Routing r,
                                                        uint64_t *__restrict__ tile_mask) {
    __shared__ unsigned tmask[256];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) tmask[e] = 0u;
    __syncthreads();
    const int tile = blockIdx.x >> 2, q = blockIdx.x & 3;
    const int t_first = blockIdx.x * 16 + (tid >> 6) * 4;
    if (t_first < T) select_group<EJ, 16>(T, E, K, thr, r, tmask, nullptr, t_first, tid & 63);
    __syncthreads();
    const int E2 = E + S;
    // 16-bit field q of word [tile][e]
    uint16_t *dst = reinterpret_cast<uint16_t *>(tile_mask + (size_t)tile * E2) + q;
    for (int e = tid; e < E2; e += 256)
        dst[4 * e] = (uint16_t)(e < E ? tmask[e] : tile_all(tile, T) >> (16 * q));
}

// The grouping of a batch of tiles by one workgroup (and the pair positions
// when the batch is small).  KEEPW (batches of more than 16 tiles): keep each
// thread's tile words in registers between the two passes; the pairs are
// placed by a separate kernel.  Else (at most 16 tiles, fuse_scatter set):
// the tile words and bases stay in LDS and the pairs are placed here.
template <bool KEEPW>
__global__ __launch_bounds__(1024) void compact_tiles(const uint64_t *__restrict__ tile_mask,
                                                      int n_tiles, int E, int S, int bm, int K,
                                                      int TK, Routing r,
                                                      int32_t *__restrict__ tile_base,
                                                      int32_t *__restrict__ pair_pos,
                                                      int32_t *__restrict__ meta,
                                                      int32_t *__restrict__ sorted_tok,
                                                      int32_t *__restrict__ pbt,
                                                      int fuse_scatter, int split) {
    __shared__ int s_part[1024];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ uint64_t s_words[KEEPW ? 1 : 16 * 256];
    __shared__ int32_t s_tb[KEEPW ? 1 : 16 * 256];
    scan_tiles<KEEPW, !KEEPW>(tile_mask, n_tiles, E, S, bm, K, TK, r, tile_base, pair_pos, meta,
                              sorted_tok, pbt, fuse_scatter != 0, split, threadIdx.x, 1024,
                              s_part, s_cnt, s_off, s_words, s_tb);
}

// A small batch (T <= 64, one tile) in one workgroup: select, counts,
// offsets, lists and pair positions of the E routed and S shared experts;
// the token sets and masked ids stay in LDS.
template <int EJ>
__global__ __launch_bounds__(1024) void route_small(int T, int E, int S, int K, float thr, int bm,
                                                    Routing r, int32_t *__restrict__ pair_pos,
                                                    int32_t *__restrict__ meta,
                                                    int32_t *__restrict__ sorted_tok,
                                                    int32_t *__restrict__ pbt, int split) {
    __shared__ unsigned long long tmask[256];
    __shared__ int s_mid[64 * 16];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    const int tid = threadIdx.x;
    const int E2 = E + S;
    if (tid < E) tmask[tid] = 0ull;
    __syncthreads();
    // 16 waves of 4 tokens: one pass over a 64-token tile
    const int t_first = (tid >> 6) * 4;
    if (t_first < T) select_group<EJ, 64>(T, E, K, thr, r, tmask, s_mid, t_first, tid & 63);
    __syncthreads();
    if (tid < E2) s_cnt[tid] = tid < E ? __popcll(tmask[tid]) : T;
    __syncthreads();
    if (tid < 64) offsets_from_counts(s_cnt, s_off, E2, bm, r, meta, pbt, split, tid);
    __syncthreads();
    const int TK = T * K, PT = TK + T * S;
    blocks_and_pads(s_off, s_cnt, E2, bm, PT, r, sorted_tok, tid, 1024);
    for (int p = tid; p < TK; p += 1024) {
        const int e = s_mid[p];
        if (e < 0) {
            pair_pos[p] = -1;
            continue;
        }
        const int t = p / K;
        place_pair(p, t, s_off[e] + __popcll(tmask[e] & ((1ull << t) - 1ull)), r, pair_pos,
                   sorted_tok);
    }
    for (int q = tid; q < T * S; q += 1024) {  // shared experts: every token, in order
        const int t = q / S, sx = q - t * S;
        place_pair(TK + q, t, s_off[E + sx] + t, r, pair_pos, sorted_tok);
    }
}

// A batch of at most BEAM_SMALL_T tokens (one 64-token tile) is routed by
// one workgroup; a larger one by quarter-tile select workgroups and one
// grouping workgroup.
#ifndef BEAM_SMALL_T
#define BEAM_SMALL_T 64
#endif
static_assert(BEAM_SMALL_T <= 64, "route_small holds one 64-token tile");

template <int EJ>
static void launch_select_t(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    if (p.T <= BEAM_SMALL_T) {
        route_small<EJ><<<1, 1024, 0, s>>>(p.T, p.E, p.S, p.K, p.thr, p.bm, r, w.pair_pos, w.meta,
                                           w.sorted_tok, w.pbt, p.split);
    } else {
        select_topk_mask<EJ><<<p.n_tiles * 4, 256, 0, s>>>(p.T, p.E, p.S, p.K, p.thr, r,
                                                          w.tile_mask);
        if (!p.fuse_scatter)  // more than 16 tiles
            compact_tiles<true><<<1, 1024, 0, s>>>(w.tile_mask, p.n_tiles, p.E, p.S, p.bm, p.K,
                                                   p.T * p.K, r, w.tile_base, w.pair_pos, w.meta,
                                                   w.sorted_tok, w.pbt, p.fuse_scatter, p.split);
        else
            compact_tiles<false><<<1, 1024, 0, s>>>(w.tile_mask, p.n_tiles, p.E, p.S, p.bm, p.K,
                                                    p.T * p.K, r, w.tile_base, w.pair_pos, w.meta,
                                                    w.sorted_tok, w.pbt, p.fuse_scatter, p.split);
    }
}

static void launch_select(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    // experts per select lane (16 lanes per token), rounded up to a power of two
    const int ej = (p.E + 15) / 16;
    if (ej <= 1) launch_select_t<1>(p, r, w, s);
    else if (ej <= 2) launch_select_t<2>(p, r, w, s);
    else if (ej <= 4) launch_select_t<4>(p, r, w, s);
    else if (ej <= 8) launch_select_t<8>(p, r, w, s);
    else launch_select_t<16>(p, r, w, s);
}

#ifndef BEAM_ROUTER_NARROW_T
#define BEAM_ROUTER_NARROW_T 256
#endif
#ifndef BEAM_ROUTER_GEMM_T
#define BEAM_ROUTER_GEMM_T 8192
#endif
#ifndef BEAM_ROUTER_BIG_T
#define BEAM_ROUTER_BIG_T 2048
#endif
#ifndef BEAM_ROUTER_WIDE_T
#define BEAM_ROUTER_WIDE_T 1024
#endif

hipError_t launch_route(const Plan &p, const void *x, const void *Wg, const void *Wm,
                        const Routing &r, const Work &w, hipStream_t s) {
    if (p.dtype == 1 && p.path == 1 && p.T > BEAM_ROUTER_GEMM_T) {
        // large batch: the logits as one dense MFMA GEMM
        hipError_t err = launch_gemm_router(p, x, Wg, Wm, r, s);
        if (err != hipSuccess) return err;
    } else if (p.dtype == 1) {
        // up to a few hundred tokens: 16-token tiles of one column block (the
        // most workgroups, the fewest bytes per workgroup); more: 32-token
        // tiles; large batches: tiles of four column blocks, so x and the
        // weights are each re-read fewer times (32 tokens up to 2048, then 64
        // tokens with four waves per workgroup, two workgroups per CU)
        const int mt = p.T <= BEAM_ROUTER_NARROW_T ? 1
                       : p.T <= BEAM_ROUTER_WIDE_T ? 2 : p.T <= BEAM_ROUTER_BIG_T ? 2 : 4;
        const int ncb = p.T <= BEAM_ROUTER_WIDE_T ? 1 : 4;
        const dim3 grid((p.T + 16 * mt - 1) / (16 * mt), (2 * p.E + 16 * ncb - 1) / (16 * ncb));
#define BEAM_ROUTER(MTV, NWV, NCV)                                                             \
    router_logits_bf16<MTV, NWV, NCV><<<grid, NWV * 64, 0, s>>>(                              \
        (const bf16_t *)x, (const bf16_t *)Wg, (const bf16_t *)Wm, r.gate_logits,            \
        r.mask_logits, p.T, p.d, p.E)
        // eight waves split d in 256-wide parts (d % 256 == 0), four in d / 4
        const bool d256 = p.d % 256 == 0;
        if (mt == 1) {
            if (d256) BEAM_ROUTER(1, 8, 1);
            else BEAM_ROUTER(1, 4, 1);
        } else if (ncb == 1) {
            if (d256) BEAM_ROUTER(2, 8, 1);
            else BEAM_ROUTER(2, 4, 1);
        } else if (mt == 2) {
            if (d256) BEAM_ROUTER(2, 8, 4);
            else BEAM_ROUTER(2, 4, 4);
        } else {
            BEAM_ROUTER(4, 4, 4);
        }
#undef BEAM_ROUTER
    } else {
        const long long n = (long long)p.T * 2 * p.E;
        router_logits_generic<float><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const float *)x, (const float *)Wg, (const float *)Wm, r.gate_logits, r.mask_logits,
            p.T, p.d, p.E);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    launch_select(p, r, w, s);
    return hipGetLastError();
}

}  // namespace beam
