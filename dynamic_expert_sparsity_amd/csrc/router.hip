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
#include <mutex>
#include <type_traits>

#include "compact_dev.h"
#include "gemm_dev.h"

namespace beam {

// ---------------------------------------------------------------------------
// Router logits block, bf16, MFMA 16x16x32.  The two routers are one GEMM with
// 2E output columns: column n < E is W_gate row n, column E + n is W_mask row
// n.  A workgroup owns 16*MT tokens and 16*NC columns of one of the two routers
// (each router's columns are tiled on their own, so a workgroup's weight rows
// all lie in one matrix and one buffer resource covers them).  Its NW waves
// split d into contiguous runs of 64-wide k-chunks, and every wave streams its
// run through a private ring of DEPTH LDS buffers: a chunk is the tile's x
// rows and weight rows, 128 bytes (one cache line) of each, moved by
// global_load_lds where every group of four lanes fetches one aligned 64-byte
// piece.  (Loading MFMA fragments straight into registers puts sixteen
// different rows in each load instruction, four lines per group of four lanes,
// and the address unit then needs about four times as many cycles for the same
// bytes.)  16-byte piece c of buffer row r sits at slot c ^ f(r) (f as in the
// GEMM), so the sixteen rows of a fragment read fall in distinct banks.  A wave's chunks land in
// order and it waits for each with an explicit vmcnt (the loads into its own
// ring are its only vector memory operations), so no barrier is needed until
// the partial sums meet in LDS, where wave c adds them for column blocks c, c
// + NW, ... in wave order and writes the float32 logits.  More column blocks
// per workgroup read each x row fewer times (2 ceil(E / 16 NC) times in all);
// one block gives the most workgroups for small batches.  Out-of-range tokens /
// columns load a clamped row and their results are not stored.
// ---------------------------------------------------------------------------
template <int MT, int NW, int NC, int DEPTH>
struct RouterCfg {
    static constexpr int ROWS = (MT + NC) * 16;  // buffer rows: x rows, then weight rows
    static constexpr int BUF = ROWS * G_ROWB;    // one 64-wide k-chunk of them
    static constexpr int LOADS = ROWS / G_RPI;   // 1 KB wave loads per chunk
    static constexpr int WREG = DEPTH * BUF;     // a wave's ring
    static constexpr int PART = MT * NC * 1024;  // a wave's partial sums
    // partials in the wave's own ring when they fit (no barrier first), else
    // in a region of their own after every wave is done with its ring
    static constexpr bool OWN = PART <= WREG;
    static constexpr int PSTRIDE = OWN ? WREG : PART;
    static constexpr int LDS = NW * (OWN ? WREG : PART);
    static_assert(OWN || PART >= WREG, "one layout for the LDS");
    static_assert((DEPTH - 1) * LOADS < 64, "vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// wait until at most `ahead` chunks of STEP loads each are in flight
// (ahead <= N, wave-uniform)
template <int N, int STEP>
__device__ __forceinline__ void router_wait_chunks(int ahead) {
    if constexpr (N == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= N) wait_vmcnt<N * STEP>();
        else router_wait_chunks<N - 1, STEP>(ahead);
    }
}

template <int MT, int NW, int NC, int DEPTH>
__global__ __launch_bounds__(NW * 64) void router_logits_bf16(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Wg, const bf16_t *__restrict__ Wm,
    float *__restrict__ gate_logits, float *__restrict__ mask_logits, int T, int d, int E) {
    using C = RouterCfg<MT, NW, NC, DEPTH>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ncg = (E + 16 * NC - 1) / (16 * NC);  // column groups per router
    const bool mask_half = (int)blockIdx.y >= ncg;
    const int c0 = ((int)blockIdx.y - (mask_half ? ncg : 0)) * 16 * NC;  // first weight row
    const int tbase = blockIdx.x * 16 * MT;
    const int xrows = min(16 * MT, T - tbase);
    const int wrows = min(16 * NC, E - c0);
    const rsrc_t rx = make_rsrc(x + (size_t)tbase * d, (uint32_t)((size_t)xrows * d * 2));
    const rsrc_t rw = make_rsrc((mask_half ? Wm : Wg) + (size_t)c0 * d,
                                (uint32_t)((size_t)wrows * d * 2));

    // load i of a chunk fills buffer rows 8i .. 8i + 7 (all x rows or all
    // weight rows: 16 MT is a multiple of 8); lane l writes slot l % 8 of row
    // 8i + l / 8, so it fetches piece (l % 8) ^ f(row) of that row
    uint32_t off[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int piece = (lane & 7) ^ swz_f(r);
        const int row = r < 16 * MT ? min(r, xrows - 1) : min(r - 16 * MT, wrows - 1);
        off[i] = (uint32_t)row * (uint32_t)d * 2u + (uint32_t)piece * 16u;
    }
    // this wave's run of chunks: [kbeg, kbeg + nk)
    const int nkc = d >> 6;
    const int q = nkc / NW, rm = nkc % NW;
    const int kbeg = wave * q + min(wave, rm);
    const int nk = q + (wave < rm ? 1 : 0);
    unsigned char *ring = lds + wave * C::WREG;

    auto issue = [&](int j) {  // chunk j of the run into buffer j % DEPTH
        unsigned char *buf = ring + (j % DEPTH) * C::BUF;
        const uint32_t soff = (uint32_t)(kbeg + j) * G_ROWB;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
            lds_dma16_buf<0>(8 * i < 16 * MT ? rx : rw, off[i], soff, buf + i * 1024);
    };

    f32x4 acc[MT][NC];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int npro = min(DEPTH, nk);
    for (int j = 0; j < npro; ++j) issue(j);
    const int fr = lane & 15;
    for (int j = 0; j < nk; ++j) {
        router_wait_chunks<DEPTH - 1, C::LOADS>(min(DEPTH - 1, nk - 1 - j));
        const unsigned char *buf = ring + (j % DEPTH) * C::BUF;
#pragma unroll
        for (int st = 0; st < 2; ++st) {  // two 32-wide k-steps per chunk
            const int pc = 4 * st + (lane >> 4);
            u32x4 a[MT], b[NC];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                a[m] = *reinterpret_cast<const u32x4 *>(buf + swz(16 * m + fr, pc));
#pragma unroll
            for (int c = 0; c < NC; ++c)
                b[c] = *reinterpret_cast<const u32x4 *>(buf + swz(16 * (MT + c) + fr, pc));
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[m][c] = mfma16x16x32(a[m], b[c], acc[m][c]);
        }
        // the reads above fed the MFMAs, so the buffer is free again
        if (j + DEPTH < nk) issue(j + DEPTH);
    }

    // partial sums into this wave's own ring (all of its loads have landed),
    // or, when they do not fit there, into slot `wave` of a layout of their
    // own once every wave is done with its ring
    if constexpr (!C::OWN) __syncthreads();
    f32x4 *part = reinterpret_cast<f32x4 *>(lds + wave * C::PSTRIDE);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) part[(m * NC + c) * 64 + lane] = acc[m][c];
    __syncthreads();
    for (int c = wave; c < NC; c += NW) {  // wave w sums column blocks w, w + NW, ...
        const int n = c0 + c * 16 + fr;
        if (n >= E) continue;
        float *out = (mask_half ? mask_logits : gate_logits) + n;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int slot = (m * NC + c) * 64 + lane;
            f32x4 v = reinterpret_cast<const f32x4 *>(lds)[slot];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                v += reinterpret_cast<const f32x4 *>(lds + w * C::PSTRIDE)[slot];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tbase + m * 16 + (lane >> 4) * 4 + i;
                if (t < T) out[(size_t)t * E] = v[i];
            }
        }
    }
}

// Router logits of a decode batch of at most SMALL_DECODE_T tokens (bf16):
// one workgroup per logit column (row n of W_gate, or of W_mask for n >= E),
// its four waves splitting the row (thread i reads 16-byte chunks i, i + 256,
// ...), all of its weight chunks and the batch's x chunks requested at once,
// bf16 dot products with float32 accumulation, each wave's lanes summed in a
// fixed order and then the four waves in order.  Every column's bytes are
// read in one round trip, where the MFMA kernel's 16-column blocks leave
// most CUs idle for a batch this small; a column per workgroup (2E of them)
// rather than per wave spreads the x reads over all CUs (33.5 against 34.5 us
// per layer call at 8 tokens, 13.3 against 13.5 at one).
__global__ __launch_bounds__(256) void router_logits_small(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Wg, const bf16_t *__restrict__ Wm,
    float *__restrict__ gate_logits, float *__restrict__ mask_logits, int T, int d, int E) {
    __shared__ float s_part[4][SMALL_DECODE_T];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x;
    const bf16_t *w = n < E ? Wg + (size_t)n * d : Wm + (size_t)(n - E) * d;
    const int nch = d >> 3;
    float acc[SMALL_DECODE_T];
#pragma unroll
    for (int t = 0; t < SMALL_DECODE_T; ++t) acc[t] = 0.f;
    // thread i takes chunks i, i + 256, ...; Q of them requested at a time
    auto pass = [&](auto QC) {
        constexpr int Q = decltype(QC)::value;
        for (int c0 = 0; c0 < nch; c0 += 256 * Q) {
            u32x4 wv[Q], xv[SMALL_DECODE_T][Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int ch = c0 + tid + 256 * q;
                const int chc = ch < nch ? ch : 0;
                wv[q] = ld16(w + (size_t)chc * 8);
#pragma unroll
                for (int t = 0; t < SMALL_DECODE_T; ++t)
                    if (t < T) xv[t][q] = ld16(x + (size_t)t * d + (size_t)chc * 8);
            }
#pragma unroll
            for (int t = 0; t < SMALL_DECODE_T; ++t) {
                if (t >= T) break;
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    if (c0 + tid + 256 * q < nch) acc[t] = dot8_bf16(wv[q], xv[t][q], acc[t]);
            }
        }
    };
    if (nch <= 256) pass(std::integral_constant<int, 1>{});
    else pass(std::integral_constant<int, 2>{});
#pragma unroll
    for (int t = 0; t < SMALL_DECODE_T; ++t) {
        if (t >= T) break;
        const float v = wave_sum(acc[t]);
        if (lane == 0) s_part[wave][t] = v;
    }
    __syncthreads();
    if (tid < T) {
        float *out = n < E ? gate_logits + n : mask_logits + (n - E);
        out[(size_t)tid * E] = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
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
// i*EJ .. i*EJ+EJ-1, so a wavefront handles 4 consecutive tokens.  Each lane
// sorts its EJ candidates once; then K rounds take the row-wide maximum of the
// lanes' best remaining candidates under the order (value desc, expert asc),
// which gives the Top-K slots in order (Eq. 4); slot k (K <= 16) is kept by
// lane k.  Softmax over the kept logits shifted by the largest
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

// Selection keys: 64-bit words that order like (value desc, expert asc).
// High word: the logit's bits mapped to an unsigned order (negative values
// inverted, positive ones with the sign bit set; -0 folded into +0 first, so
// the two zeros tie as they compare equal); low word: ~expert.  The Top-K
// rounds then take plain maxima of keys, which compile to compares and
// selects (a value-and-index form with branches took ~0.5 us per round in
// the single-wave select of a small batch).
__device__ __forceinline__ unsigned long long sel_key(float v, int e) {
    const unsigned b = __float_as_uint(v + 0.f);
    const unsigned o = b ^ ((unsigned)((int)b >> 31) | 0x80000000u);
    return ((unsigned long long)o << 32) | (unsigned)~e;
}
__device__ __forceinline__ float key_value(unsigned long long key) {
    const unsigned o = (unsigned)(key >> 32);
    return __uint_as_float(o ^ (((o >> 31) - 1u) | 0x80000000u));
}
__device__ __forceinline__ int key_expert(unsigned long long key) { return (int)~(unsigned)key; }

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_key(unsigned long long v) {
    const unsigned lo = (unsigned)dpp_i<CTRL>((int)(unsigned)v);
    const unsigned hi = (unsigned)dpp_i<CTRL>((int)(unsigned)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}
template <int CTRL>
__device__ __forceinline__ unsigned long long key_max_step(unsigned long long v) {
    const unsigned long long o = dpp_key<CTRL>(v);
    return o > v ? o : v;
}
// largest key of a row of 16 lanes, in every lane of the row
__device__ __forceinline__ unsigned long long row_max_key(unsigned long long v) {
    v = key_max_step<DPP_QUAD_1032>(v);
    v = key_max_step<DPP_QUAD_2301>(v);
    v = key_max_step<DPP_ROW_HALF_MIRROR>(v);
    return key_max_step<DPP_ROW_MIRROR>(v);
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
    int lane, bool write = true) {
    using MW = std::conditional_t<TB == 64, unsigned long long, unsigned>;
    static_assert(TB == 64 || TB == 16, "token bits per mask word");
    static_assert(EJ >= 1 && EJ <= 16 && (EJ & (EJ - 1)) == 0,
                  "a power of two, at most 16 experts per lane (E <= 256)");
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
    // candidate keys (0 below every key: no expert, or already taken)
    unsigned long long key[EJ];
#pragma unroll
    for (int j = 0; j < EJ; ++j) key[j] = e0 + j < E ? sel_key(rv[j], e0 + j) : 0ull;

    // each lane's keys in descending order (a bitonic network, EJ a power of
    // two), so a lane's best remaining candidate is always key[0]
#pragma unroll
    for (int w = 2; w <= EJ; w <<= 1)
#pragma unroll
        for (int h = w >> 1; h > 0; h >>= 1)
#pragma unroll
            for (int a = 0; a < EJ; ++a) {
                const int c = a ^ h;
                if (c > a) {
                    const unsigned long long hi = key[a] > key[c] ? key[a] : key[c];
                    const unsigned long long lo = key[a] > key[c] ? key[c] : key[a];
                    const bool desc = (a & w) == 0;
                    key[a] = desc ? hi : lo;
                    key[c] = desc ? lo : hi;
                }
            }
    // round k takes the row's largest head; the lane that held it moves its
    // list up by one.  Slot k is kept by lane k.
    unsigned long long top = 0ull, kept = 0ull;
    for (int k = 0; k < K; ++k) {
        const unsigned long long b = row_max_key(key[0]);
        // all ones in the lane that held the head, whose list then moves up
        // by a select per word (written with masks: the compiler turned the
        // plain conditional copies into a chain of index compares)
        const unsigned long long m = 0ull - (unsigned long long)(key[0] == b);
#pragma unroll
        for (int j = 0; j + 1 < EJ; ++j) key[j] = (key[j + 1] & m) | (key[j] & ~m);
        key[EJ - 1] &= ~m;
        top = k == 0 ? b : top;
        kept = k == i ? b : kept;
    }
    const float v0 = key_value(top), myv = key_value(kept);
    const int mye = key_expert(kept);

    const float num = i < K ? expf(myv - v0) : 0.f;
    const float den = row_sum(num);
    if (!valid || i >= K) return;
    const int k = i;
    const float z = r.mask_logits[(size_t)t * E + mye];
    const float g = num / den;
    const bool m = z >= thr;
    const int o = t * K + k;
    if (write) {
        r.topk_ids[o] = mye;
        r.topk_weights[o] = g;
        r.mask[o] = m ? 1 : 0;
        r.g_hat[o] = m ? g : 0.f;
        r.masked_ids[o] = m ? mye : -1;
    }
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

// The routing of a small batch (T <= 64, one tile) by one workgroup of
// nthreads threads (>= 256, a multiple of 64): select, counts, offsets,
// lists and pair positions of the E routed and S shared experts; the token
// sets and masked ids stay in LDS.  write = false keeps every result in LDS
// (token sets, masked ids, counts, offsets and, if given, the ascending
// active-expert list) and writes nothing to global memory.
template <int EJ>
__device__ __forceinline__ void route_small_body(
    int T, int E, int S, int K, float thr, int bm, const Routing &r, int32_t *pair_pos,
    int32_t *meta, int32_t *sorted_tok, int32_t *pbt, int split, bool write, int tid, int nthreads,
    unsigned long long *tmask, int *s_mid, int *s_cnt, int *s_off, int *s_act, int *s_nact) {
    const int E2 = E + S;
    if (tid < E) tmask[tid] = 0ull;
    __syncthreads();
    // four tokens per wave
    for (int t_first = (tid >> 6) * 4; t_first < T; t_first += (nthreads >> 6) * 4)
        select_group<EJ, 64>(T, E, K, thr, r, tmask, s_mid, t_first, tid & 63, write);
    __syncthreads();
    if (tid < E2) s_cnt[tid] = tid < E ? __popcll(tmask[tid]) : T;
    __syncthreads();
    if (tid < 64)
        offsets_from_counts(s_cnt, s_off, E2, bm, r, meta, pbt, split, tid, write, s_act, s_nact);
    __syncthreads();
    if (!write) return;
    const int TK = T * K, PT = TK + T * S;
    blocks_and_pads(s_off, s_cnt, E2, bm, PT, r, sorted_tok, tid, nthreads);
    for (int p = tid; p < TK; p += nthreads) {
        const int e = s_mid[p];
        if (e < 0) {
            pair_pos[p] = -1;
            continue;
        }
        const int t = p / K;
        place_pair(p, t, s_off[e] + __popcll(tmask[e] & ((1ull << t) - 1ull)), r, pair_pos,
                   sorted_tok);
    }
    for (int q = tid; q < T * S; q += nthreads) {  // shared experts: every token, in order
        const int t = q / S, sx = q - t * S;
        place_pair(TK + q, t, s_off[E + sx] + t, r, pair_pos, sorted_tok);
    }
}

// The part of route_small_body that the expert items of a small batch need,
// in LDS only: the token sets tmask[e] (routed experts), the block-padded
// list offsets s_off[e] (the same formula as offsets_from_counts, so the
// positions equal the ones the routing outputs describe) and the ascending
// list of active experts (routed experts with a pair, then every shared
// expert) with its length.
template <int EJ>
__device__ __forceinline__ void route_small_active(int T, int E, int S, int K, float thr, int bm,
                                                   const Routing &r, int tid,
                                                   unsigned long long *tmask, int *s_off,
                                                   int *s_act, int *s_nact) {
    if (tid < E) tmask[tid] = 0ull;
    __syncthreads();
    if ((tid >> 6) * 4 < T)  // four tokens per wave
        select_group<EJ, 64>(T, E, K, thr, r, tmask, nullptr, (tid >> 6) * 4, tid & 63, false);
    __syncthreads();
    if (tid < 64) {
        // four experts per lane, in expert order
        const int E2 = E + S;
        int act[4], pad[4], sa = 0, sp = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ex = tid * 4 + j;
            const int c = ex < E ? __popcll(tmask[ex]) : (ex < E2 ? T : 0);
            act[j] = c > 0 ? 1 : 0;
            pad[j] = (c + bm - 1) / bm * bm;
            sa += act[j];
            sp += pad[j];
        }
        const int ia = wave_incl_scan(sa, tid);
        const int ip = wave_incl_scan(sp, tid);
        int oa = ia - sa, op = ip - sp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ex = tid * 4 + j;
            if (ex < E2) s_off[ex] = op;
            if (act[j]) s_act[oa] = ex;
            oa += act[j];
            op += pad[j];
        }
        if (tid == 63) *s_nact = ia;
    }
    __syncthreads();
}

// A small batch (T <= 64, one tile) in one workgroup.
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
    route_small_body<EJ>(T, E, S, K, thr, bm, r, pair_pos, meta, sorted_tok, pbt, split, true,
                         threadIdx.x, 1024, tmask, s_mid, s_cnt, s_off, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// A decode batch of at most SMALL_DECODE_T tokens: the routing (rows a2-a4)
// and the expert up projection (row a5) in one launch after the logits.
// Every workgroup routes the batch itself from the logits (Top-K, mask,
// counts, offsets and the active-expert list in LDS); workgroup 0 also
// writes every routing output exactly as route_small does.  Then each wave
// takes (active expert, intermediate unit j) items: it streams the gate row j
// and the up row I + j of the expert (16-byte loads, lane l reading chunks
// l, l + 64, ...), dots them with the x rows of the expert's tokens (staged
// in LDS; bf16 pairs, float32 accumulation), sums the lanes in a fixed order
// and writes h = SiLU(a) * u for each token at its sorted position.  With a
// few tokens per expert the work is reading the active experts' rows, and
// one item per wave at a time keeps every CU streaming (a projection of a
// single token has 1536 such rows per expert).
// ---------------------------------------------------------------------------
template <int EJ>
__global__ __launch_bounds__(512) void up_small(int T, int E, int S, int K, float thr, int bm,
                                                int d, int I, Routing r,
                                                int32_t *__restrict__ pair_pos,
                                                int32_t *__restrict__ meta,
                                                int32_t *__restrict__ sorted_tok,
                                                int32_t *__restrict__ pbt, int split,
                                                const bf16_t *__restrict__ x,
                                                const bf16_t *__restrict__ Wgu,
                                                bf16_t *__restrict__ h) {
    __shared__ unsigned long long tmask[256];
    __shared__ int s_mid[SMALL_DECODE_T * 16];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int s_act[256];
    __shared__ int s_nact;
    extern __shared__ __align__(16) unsigned char xs_raw[];  // [T][d] bf16
    u32x4 *xs = reinterpret_cast<u32x4 *>(xs_raw);
    const int tid = threadIdx.x;
    const int nch = d >> 3;  // 16-byte chunks per row
    // the batch's x rows: requested before the routing, stored to LDS after
    // it (T * d * 2 <= 48 KB: at most 6 chunks per thread).  Every load is
    // issued (past the end: chunk 0 again), so none is waited for before the
    // routing.
    constexpr int XR = 6;
    u32x4 xr[XR];
#pragma unroll
    for (int k = 0; k < XR; ++k) {
        const int i = tid + 512 * k;
        xr[k] = ld16(x + (size_t)(i < T * nch ? i : 0) * 8);
    }
    // workgroup 0 writes every routing output; the others only need the
    // token sets and the active-expert list
    if (blockIdx.x == 0)
        route_small_body<EJ>(T, E, S, K, thr, bm, r, pair_pos, meta, sorted_tok, pbt, split,
                             true, tid, 512, tmask, s_mid, s_cnt, s_off, s_act, &s_nact);
    else
        route_small_active<EJ>(T, E, S, K, thr, bm, r, tid, tmask, s_off, s_act, &s_nact);
#pragma unroll
    for (int k = 0; k < XR; ++k) {
        const int i = tid + 512 * k;
        if (i < T * nch) xs[i] = xr[k];
    }
    __syncthreads();
    const int lane = tid & 63;
    const int n_items = s_nact * I;
    // workgroup 0 writes the routing outputs; the others take the items, so
    // its writes overlap their streaming (with one workgroup it takes them)
    const int g0 = gridDim.x > 1 ? 1 : 0;
    if (blockIdx.x < g0) return;
    const int nwg = gridDim.x - g0, waves = nwg * 8;
    // U items per wave at a time, all their row pieces requested before any
    // arithmetic: two, or one when every wave has at most one (then a wave
    // issues no loads for a missing second item, and consecutive items go to
    // consecutive workgroups, so a few items spread over every CU; with more,
    // a workgroup's waves take consecutive rows, 0.6 us faster at 8 tokens).
    auto items = [&](auto UC) {
        constexpr int U = decltype(UC)::value;
        const int first = U == 1 ? (int)(blockIdx.x - g0) + (tid >> 6) * nwg
                                 : (int)(blockIdx.x - g0) * 8 + (tid >> 6);
        for (int it0 = first; it0 < n_items; it0 += U * waves) {
            int e2[U], j2[U];
            unsigned tm2[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int it = it0 + u * waves;
                const bool ok = it < n_items;
                const int itc = ok ? it : it0;
                const int a = itc / I;
                j2[u] = itc - a * I;
                e2[u] = s_act[a];
                // tokens of this expert's active pairs (shared experts: every token)
                tm2[u] = ok ? (e2[u] < E ? (unsigned)tmask[e2[u]] : (1u << T) - 1u) : 0u;
            }
            float ga[U][SMALL_DECODE_T], ua[U][SMALL_DECODE_T];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int t = 0; t < SMALL_DECODE_T; ++t) ga[u][t] = ua[u][t] = 0.f;
            for (int c0 = 0; c0 < nch; c0 += 256) {
                // every load is issued (past the row end: the row's first chunk
                // again, in bounds and unused), so all of them stay in flight
                u32x4 wgv[U][4], wuv[U][4];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bf16_t *wg = Wgu + ((size_t)e2[u] * 2 * I + j2[u]) * d;
                    const bf16_t *wu = wg + (size_t)I * d;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int ch = c0 + lane + 64 * q;
                        const int chc = ch < nch ? ch : 0;
                        wgv[u][q] = ld16_stream(wg + (size_t)chc * 8);
                        wuv[u][q] = ld16_stream(wu + (size_t)chc * 8);
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int t = 0; t < SMALL_DECODE_T; ++t) {
                        if (!((tm2[u] >> t) & 1u)) continue;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int ch = c0 + lane + 64 * q;
                            if (ch < nch) {
                                const u32x4 xv = xs[t * nch + ch];
                                ga[u][t] = dot8_bf16(wgv[u][q], xv, ga[u][t]);
                                ua[u][t] = dot8_bf16(wuv[u][q], xv, ua[u][t]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int t = 0; t < SMALL_DECODE_T; ++t) {
                    if (!((tm2[u] >> t) & 1u)) continue;
                    const float av = wave_sum(ga[u][t]);
                    const float uv = wave_sum(ua[u][t]);
                    if (lane == 0) {
                        const int e = e2[u];
                        const int pos = s_off[e] + (e < E ? __popc(tm2[u] & ((1u << t) - 1u)) : t);
                        h[(size_t)pos * I + j2[u]] = f32_to_bf16(silu_fast(av) * uv);
                    }
                }
            }
        }
    };
    if (n_items <= waves)
        items(std::integral_constant<int, 1>{});
    else
        items(std::integral_constant<int, 2>{});
}

hipError_t launch_up_small(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                           const Work &w, hipStream_t s) {
    const int ej = (p.E + 15) / 16;
    const size_t lds = (size_t)p.T * p.d * 2;
    const int grid = device_cus();
#define BEAM_UP_SMALL(EJV)                                                                     \
    up_small<EJV><<<grid, 512, lds, s>>>(p.T, p.E, p.S, p.K, p.thr, p.bm, p.d, p.I, r,        \
                                         w.pair_pos, w.meta, w.sorted_tok, w.pbt, p.split,   \
                                         (const bf16_t *)x, (const bf16_t *)W_gu, (bf16_t *)w.h)
    if (ej <= 1) BEAM_UP_SMALL(1);
    else if (ej <= 2) BEAM_UP_SMALL(2);
    else if (ej <= 4) BEAM_UP_SMALL(4);
    else if (ej <= 8) BEAM_UP_SMALL(8);
    else BEAM_UP_SMALL(16);
#undef BEAM_UP_SMALL
    return hipGetLastError();
}

// A batch of at most ROUTE_SMALL_T tokens (one 64-token tile) is routed by
// one workgroup; a larger one by quarter-tile select workgroups, then (more
// than SCATTER_SELF_TILES tiles) compact_bases, then the pair-scatter
// workgroups.  (One grouping workgroup for up to 16 tiles was 2-8 us slower
// per layer call at 128-1024 tokens than the scatter workgroups making the
// bases themselves.)

template <int EJ>
static void launch_select_t(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    if (p.T <= ROUTE_SMALL_T) {
        route_small<EJ><<<1, 1024, 0, s>>>(p.T, p.E, p.S, p.K, p.thr, p.bm, r, w.pair_pos, w.meta,
                                           w.sorted_tok, w.pbt, p.split);
    } else {
        select_topk_mask<EJ><<<p.n_tiles * 4, 256, 0, s>>>(p.T, p.E, p.S, p.K, p.thr, r,
                                                          w.tile_mask);
        launch_bases(p, w, s);  // (a no-op up to SCATTER_SELF_TILES tiles)
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
#ifndef BEAM_ROUTER_PAIR_T
#define BEAM_ROUTER_PAIR_T 4096
#endif
#ifndef BEAM_ROUTER_BIG_T
#define BEAM_ROUTER_BIG_T 2048
#endif
#ifndef BEAM_ROUTER_WIDE_T
#define BEAM_ROUTER_WIDE_T 1024
#endif

template <int MT, int NW, int NC, int DEPTH>
static hipError_t launch_router_t(const Plan &p, const void *x, const void *Wg, const void *Wm,
                                  const Routing &r, hipStream_t s) {
    using C = RouterCfg<MT, NW, NC, DEPTH>;
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [] {
        attr_err = hipFuncSetAttribute((const void *)router_logits_bf16<MT, NW, NC, DEPTH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    });
    if (attr_err != hipSuccess) return attr_err;
    // token tiles x (column groups of W_gate, then of W_mask)
    const dim3 grid((p.T + 16 * MT - 1) / (16 * MT), 2 * ((p.E + 16 * NC - 1) / (16 * NC)));
    router_logits_bf16<MT, NW, NC, DEPTH><<<grid, NW * 64, C::LDS, s>>>(
        (const bf16_t *)x, (const bf16_t *)Wg, (const bf16_t *)Wm, r.gate_logits, r.mask_logits,
        p.T, p.d, p.E);
    return hipGetLastError();
}

hipError_t launch_router_logits(const Plan &p, const void *x, const void *Wg, const void *Wm,
                                const Routing &r, hipStream_t s) {
    if (p.small) {
        router_logits_small<<<2 * p.E, 256, 0, s>>>(
            (const bf16_t *)x, (const bf16_t *)Wg, (const bf16_t *)Wm, r.gate_logits,
            r.mask_logits, p.T, p.d, p.E);
    } else if (p.dtype == 1) {
        // up to a few hundred tokens: 16-token tiles of one column block (the
        // most workgroups, the fewest bytes per workgroup); more: 32-token
        // tiles; large batches: tiles of four column blocks, so x and the
        // weights are each re-read fewer times (32 tokens up to 2048, then 64
        // tokens with four waves per workgroup).  Up to 4096 tokens the rings
        // fill 96-128 KB of LDS (one workgroup per CU, each wave two chunks
        // deep where that fits); above, single-chunk rings of 64 KB let two
        // workgroups share a CU (at 8192 tokens 36.6 against 39.8 us for the
        // whole routing call; with fewer than two workgroups per CU the pairs
        // leave CUs idle instead)
        hipError_t err;
        if (p.T <= BEAM_ROUTER_NARROW_T) err = launch_router_t<1, 8, 1, 4>(p, x, Wg, Wm, r, s);
        else if (p.T <= BEAM_ROUTER_WIDE_T) err = launch_router_t<2, 8, 1, 2>(p, x, Wg, Wm, r, s);
        else if (p.T <= BEAM_ROUTER_BIG_T) err = launch_router_t<2, 8, 4, 1>(p, x, Wg, Wm, r, s);
        else if (p.T <= BEAM_ROUTER_PAIR_T) err = launch_router_t<4, 4, 4, 2>(p, x, Wg, Wm, r, s);
        else err = launch_router_t<4, 4, 4, 1>(p, x, Wg, Wm, r, s);
        if (err != hipSuccess) return err;
    } else {
        const long long n = (long long)p.T * 2 * p.E;
        router_logits_generic<float><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const float *)x, (const float *)Wg, (const float *)Wm, r.gate_logits, r.mask_logits,
            p.T, p.d, p.E);
    }
    return hipGetLastError();
}

hipError_t launch_route(const Plan &p, const void *x, const void *Wg, const void *Wm,
                        const Routing &r, const Work &w, hipStream_t s) {
    const hipError_t err = launch_router_logits(p, x, Wg, Wm, r, s);
    if (err != hipSuccess) return err;
    launch_select(p, r, w, s);
    return hipGetLastError();
}

}  // namespace beam
