// a4: grouping of the active (token, expert) pairs into per-expert lists.
// Masked slots (id -1) are left out of the per-expert counts, so masked pairs
// are never scheduled (news article on the BEAM paper, section 5, the
// modified expert/token grouping kernel).
//
// Input: per select tile (64 tokens) and expert, the 64-bit set of tile
// tokens that have an active pair for that expert (built by the select
// kernel; an expert appears at most once among a token's K slots).
//   count(tile, e)        = popcount(set)
//   rank of token tl      = popcount(set & ((1 << tl) - 1))
// so a pair's position in its expert's list is
//   offsets[e] + (pairs of e in earlier tiles) + rank,
// which lists each expert's pairs in ascending pair id with no atomics.
#include "compact_dev.h"

namespace beam {

__device__ __forceinline__ void scatter_pair(int p, int K, int E, const Routing &r,
                                             const int *off, const int32_t *tile_base,
                                             const uint64_t *tile_mask, int32_t *pair_pos,
                                             int32_t *sorted_tok) {
    const int e = r.masked_ids[p];
    if (e < 0) {
        pair_pos[p] = -1;
        return;
    }
    const int t = p / K;
    const size_t q = (size_t)(t >> 6) * E + e;
    const int rank = __popcll(tile_mask[q] & ((1ull << (t & 63)) - 1ull));
    place_pair(p, e, off[e] + tile_base[q] + rank, K, r, pair_pos, sorted_tok);
}

// One workgroup of 1024 threads.  Thread (g, e) with g = tid / E sums the
// popcounts of a contiguous range of tiles for expert e; group partials give
// every (tile, expert) its base; wave 0 scans the experts into block-padded
// offsets.  With fuse_scatter the same workgroup then places every pair.
__global__ __launch_bounds__(1024) void compact_scan(const uint64_t *__restrict__ tile_mask,
                                                     int n_tiles, int E, int bm, int K, int TK,
                                                     Routing r, int32_t *__restrict__ tile_base,
                                                     int32_t *__restrict__ pair_pos,
                                                     int32_t *__restrict__ meta,
                                                     int32_t *__restrict__ sorted_tok,
                                                     int fuse_scatter) {
    __shared__ int s_part[1024];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    const int tid = threadIdx.x;
    const int NG = 1024 / E;                 // >= 4 because E <= 256
    const int g = tid / E;
    const int e = tid - g * E;
    const bool on = g < NG;
    const int chunk = (n_tiles + NG - 1) / NG;
    const int tb = g * chunk;
    const int te = min(n_tiles, tb + chunk);

    int local = 0;
    if (on)
        for (int t = tb; t < te; ++t) local += __popcll(tile_mask[(size_t)t * E + e]);
    s_part[tid] = local;
    __syncthreads();

    if (on) {
        int base = 0, total = 0;
        for (int q = 0; q < NG; ++q) {
            const int v = s_part[q * E + e];
            if (q < g) base += v;
            total += v;
        }
        for (int t = tb; t < te; ++t) {
            tile_base[(size_t)t * E + e] = base;
            base += __popcll(tile_mask[(size_t)t * E + e]);
        }
        if (g == 0) s_cnt[e] = total;
    }
    __syncthreads();
    if (tid < 64) offsets_from_counts(s_cnt, s_off, E, bm, r, meta, tid);
    __syncthreads();
    blocks_and_pads(s_off, s_cnt, E, bm, TK, r, tid, 1024);
    if (fuse_scatter)
        for (int p = tid; p < TK; p += 1024)
            scatter_pair(p, K, E, r, s_off, tile_base, tile_mask, pair_pos, sorted_tok);
}

__global__ __launch_bounds__(256) void compact_scatter(Routing r,
                                                      const int32_t *__restrict__ tile_base,
                                                      const uint64_t *__restrict__ tile_mask,
                                                      int TK, int K, int E,
                                                      int32_t *__restrict__ pair_pos,
                                                      int32_t *__restrict__ sorted_tok) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= TK) return;
    scatter_pair(p, K, E, r, r.expert_offsets, tile_base, tile_mask, pair_pos, sorted_tok);
}

hipError_t launch_scan(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    compact_scan<<<1, 1024, 0, s>>>(w.tile_mask, p.n_tiles, p.E, p.bm, p.K, p.T * p.K, r,
                                    w.tile_base, w.pair_pos, w.meta, w.sorted_tok,
                                    p.fuse_scatter);
    return hipGetLastError();
}

hipError_t launch_scatter(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    if (p.fuse_scatter) return hipSuccess;
    const int TK = p.T * p.K;
    compact_scatter<<<(TK + 255) / 256, 256, 0, s>>>(r, w.tile_base, w.tile_mask, TK, p.K, p.E,
                                                     w.pair_pos, w.sorted_tok);
    return hipGetLastError();
}

}  // namespace beam
