// a4: grouping of the active (token, expert) pairs.  Masked slots (id -1)
// are left out of the per-expert counts, so masked pairs are never scheduled
// (news article on the BEAM paper, section 5, the modified expert/token
// grouping kernel).
//
// Input: per select tile (64 tokens) and expert, the 64-bit set of tile
// tokens that have an active pair for that expert (built by the select
// kernel; an expert appears at most once among a token's K slots).
//   count(tile, e)        = popcount(set)
//   rank of token tl      = popcount(set & ((1 << tl) - 1))
// so a pair's position in its expert's list is
//   offsets[e] + (pairs of e in earlier tiles) + rank,
// which lists each expert's pairs in ascending pair id with no atomics.
#include "common.h"
#include "kernels.h"

namespace beam {

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off);
        if (lane >= off) v += y;
    }
    return v;
}

// One workgroup of 1024 threads.  Thread (g, e) with g = tid / E sums the
// popcounts of a contiguous range of tiles for expert e; group partials are
// scanned to give every (tile, expert) its base, then wave 0 scans the
// experts (4 per lane, E <= 256) into block-padded offsets.
__global__ __launch_bounds__(1024) void compact_scan(const uint64_t *__restrict__ tile_mask,
                                                     int n_tiles, int E, int bm, int TK,
                                                     Routing r, int32_t *__restrict__ tile_base) {
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
        if (g == 0) {
            s_cnt[e] = total;
            r.expert_counts[e] = total;
        }
    }
    __syncthreads();

    if (tid < 64) {
        const int lane = tid;
        int c[4], pad[4], act[4];
        int sc = 0, sp = 0, sa = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ex = lane * 4 + j;
            c[j] = ex < E ? s_cnt[ex] : 0;
            pad[j] = (c[j] + bm - 1) / bm * bm;
            act[j] = c[j] > 0 ? 1 : 0;
            sc += c[j];
            sp += pad[j];
            sa += act[j];
        }
        const int ic = wave_incl_scan(sc, lane);
        const int ip = wave_incl_scan(sp, lane);
        const int ia = wave_incl_scan(sa, lane);
        int op = ip - sp, oa = ia - sa;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ex = lane * 4 + j;
            if (ex < E) {
                s_off[ex] = op;
                r.expert_offsets[ex] = op;
                if (act[j]) r.active_experts[oa] = ex;
            }
            op += pad[j];
            oa += act[j];
        }
        if (lane == 63) {
            s_off[E] = ip;
            r.expert_offsets[E] = ip;
            r.num_active[0] = ic;
            r.num_active[1] = ip;
            r.num_active[2] = ia;
            r.num_active[3] = ip / bm;
        }
    }
    __syncthreads();

    // block -> expert map and pad entries, one thread per block of bm slots
    const int n_blocks = s_off[E] / bm;
    for (int b = tid; b < n_blocks; b += 1024) {
        const int pos = b * bm;
        int lo = 0, hi = E - 1;  // last expert with s_off[ex] <= pos
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        // skip experts with empty segments that share the same offset
        while (lo + 1 < E && s_off[lo + 1] <= pos) ++lo;
        r.block_expert[b] = lo;
        const int end_valid = s_off[lo] + s_cnt[lo];
        for (int q = max(pos, end_valid); q < pos + bm; ++q) r.sorted_pairs[q] = TK;
    }
}

__global__ __launch_bounds__(256) void compact_scatter(
    const int32_t *__restrict__ masked_ids, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ tile_base, const uint64_t *__restrict__ tile_mask, int TK,
    int K, int E, int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ pair_pos) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= TK) return;
    const int e = masked_ids[p];
    if (e < 0) {
        pair_pos[p] = -1;
        return;
    }
    const int t = p / K;
    const int tile = t >> 6;
    const int tl = t & 63;
    const size_t q = (size_t)tile * E + e;
    const int rank = __popcll(tile_mask[q] & ((1ull << tl) - 1ull));
    const int pos = offsets[e] + tile_base[q] + rank;
    sorted_pairs[pos] = p;
    pair_pos[p] = pos;
}

hipError_t launch_scan(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    compact_scan<<<1, 1024, 0, s>>>(w.tile_mask, p.n_tiles, p.E, p.bm, p.T * p.K, r,
                                    w.tile_base);
    return hipGetLastError();
}

hipError_t launch_scatter(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    const int TK = p.T * p.K;
    compact_scatter<<<(TK + 255) / 256, 256, 0, s>>>(r.masked_ids, r.expert_offsets,
                                                     w.tile_base, w.tile_mask, TK, p.K, p.E,
                                                     r.sorted_pairs, w.pair_pos);
    return hipGetLastError();
}

}  // namespace beam
