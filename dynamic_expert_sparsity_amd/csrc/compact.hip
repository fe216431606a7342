// a4 for batches of more than one select tile (64 tokens): the grouping in
// one or two launches of many workgroups (see compact_dev.h for the
// arithmetic).
//   compact_bases:   per expert, the running count of its tokens over the
//                    tiles (tile_base[tile][e]) and its total (cnt[e]);
//   compact_scatter: every workgroup turns the totals into the block-padded
//                    offsets itself (one wave, LDS; workgroup 0 also writes
//                    the routing records and the call's kernel record), then
//                    takes its share of the block -> expert map and the pad
//                    entries, and places its pairs.
// Up to SCATTER_SELF_TILES tiles compact_bases does not run: every scatter
// workgroup makes the bases it needs itself.  A single workgroup did the
// first step and the offsets, block map and pads (9.4 us at 8192 tokens, its
// steps one after another); spread out, the serial part left is one wave's
// prefix sums per workgroup.
#include "compact_dev.h"

namespace beam {

// One wave per expert: lane l sums a contiguous run of tiles, a wave prefix
// sum turns the runs into bases.  Up to KEEP tiles per lane stay in
// registers between the two passes; longer runs read their words again.
__global__ __launch_bounds__(256) void compact_bases(const uint64_t *__restrict__ tile_mask,
                                                    int n_tiles, int E2,
                                                    int32_t *__restrict__ tile_base,
                                                    int32_t *__restrict__ cnt) {
    constexpr int KEEP = 8;
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E2) return;
    const int per = (n_tiles + 63) / 64;
    const int t0 = min(n_tiles, lane * per), t1 = min(n_tiles, t0 + per);
    int local = 0;
    uint64_t wv[KEEP];
    if (per <= KEEP) {
#pragma unroll
        for (int i = 0; i < KEEP; ++i) {
            wv[i] = t0 + i < t1 ? tile_mask[(size_t)(t0 + i) * E2 + e] : 0ull;
            local += __popcll(wv[i]);
        }
    } else {
        for (int t = t0; t < t1; ++t) local += __popcll(tile_mask[(size_t)t * E2 + e]);
    }
    const int incl = wave_incl_scan(local, lane);
    int base = incl - local;
    if (per <= KEEP) {
#pragma unroll
        for (int i = 0; i < KEEP; ++i) {
            if (t0 + i < t1) {
                tile_base[(size_t)(t0 + i) * E2 + e] = base;
                base += __popcll(wv[i]);
            }
        }
    } else {
        for (int t = t0; t < t1; ++t) {
            tile_base[(size_t)t * E2 + e] = base;
            base += __popcll(tile_mask[(size_t)t * E2 + e]);
        }
    }
    if (lane == 63) cnt[e] = incl;
}

// One thread per pair, after the offsets (recomputed in every workgroup from
// the counts; only workgroup 0 writes them out, so no workgroup reads
// another's writes).  SELF (at most SCATTER_SELF_TILES tiles): every
// workgroup also makes the counts and the per-tile bases itself, in LDS,
// from the tile words (thread e reads expert e's word of every tile at
// once), so compact_bases does not run; at 2048 tokens that launch cost
// more than the 32 words per expert it spares each workgroup.
template <bool SELF>
__global__ __launch_bounds__(256) void compact_scatter(
    Routing r, const int32_t *__restrict__ cnt, int bm, int split, int32_t *__restrict__ meta,
    int32_t *__restrict__ pbt, const int32_t *__restrict__ tile_base,
    const uint64_t *__restrict__ tile_mask, int n_tiles, int PT, int TK, int K, int E, int S,
    int32_t *__restrict__ pair_pos, int32_t *__restrict__ sorted_tok) {
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int32_t s_tb[SELF ? SCATTER_SELF_TILES * 256 : 1];
    const int E2 = E + S;
    const int tid = threadIdx.x;
    const int p = blockIdx.x * 256 + tid;
    // the pair's masked id is requested before the offsets are made
    const int mid = p < TK ? r.masked_ids[p] : -1;
    if (SELF) {
        if (tid < E2) {
            uint64_t wv[SCATTER_SELF_TILES];
#pragma unroll
            for (int t = 0; t < SCATTER_SELF_TILES; ++t)  // past n_tiles: tile 0 again, unused
                wv[t] = tile_mask[(size_t)(t < n_tiles ? t : 0) * E2 + tid];
            int base = 0;
#pragma unroll
            for (int t = 0; t < SCATTER_SELF_TILES; ++t) {
                if (t < n_tiles) {
                    s_tb[t * E2 + tid] = base;
                    base += __popcll(wv[t]);
                }
            }
            s_cnt[tid] = base;
        }
    } else {
        if (tid < E2) s_cnt[tid] = cnt[tid];
    }
    __syncthreads();
    if (tid < 64)
        offsets_from_counts(s_cnt, s_off, E2, bm, r, meta, pbt, split, tid, blockIdx.x == 0);
    __syncthreads();
    blocks_and_pads(s_off, s_cnt, E2, bm, PT, r, sorted_tok, p, gridDim.x * 256);
    if (p < PT)
        scatter_pair(p, mid, K, TK, E, S, r, s_off, SELF ? s_tb : tile_base, tile_mask, pair_pos,
                     sorted_tok);
}

hipError_t launch_scatter(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    if (p.fuse_scatter) return hipSuccess;
    if (p.n_tiles <= SCATTER_SELF_TILES)
        compact_scatter<true><<<(p.PT + 255) / 256, 256, 0, s>>>(
            r, w.cnt, p.bm, p.split, w.meta, w.pbt, w.tile_base, w.tile_mask, p.n_tiles, p.PT,
            p.T * p.K, p.K, p.E, p.S, w.pair_pos, w.sorted_tok);
    else
        compact_scatter<false><<<(p.PT + 255) / 256, 256, 0, s>>>(
            r, w.cnt, p.bm, p.split, w.meta, w.pbt, w.tile_base, w.tile_mask, p.n_tiles, p.PT,
            p.T * p.K, p.K, p.E, p.S, w.pair_pos, w.sorted_tok);
    return hipGetLastError();
}

hipError_t launch_bases(const Plan &p, const Work &w, hipStream_t s) {
    if (p.n_tiles <= SCATTER_SELF_TILES) return hipSuccess;  // the scatter makes them
    compact_bases<<<(p.E2 + 3) / 4, 256, 0, s>>>(w.tile_mask, p.n_tiles, p.E2, w.tile_base,
                                                 w.cnt);
    return hipGetLastError();
}

}  // namespace beam
