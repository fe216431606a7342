// Device-side pieces of the grouping of active pairs, shared by the
// multi-tile compaction kernels and the single-workgroup small-batch routing
// kernel.  Masked slots (id -1) are left out of every count, so masked pairs
// are never scheduled (news article on the BEAM paper, section 5).
#pragma once
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

// Wave 0 only (lane = threadIdx.x < 64): from per-expert counts s_cnt[E]
// (E <= 256, four experts per lane) write block-padded exclusive offsets to
// s_off[0..E] and r.expert_offsets, the ascending active-expert list and
// r.num_active = {P, num_padded, n_active_experts, n_blocks}, and the E
// records meta[i] = {expert, offset, count, 0} of the active experts in
// ascending order followed by zero records, which the expert kernels start
// from (count 0: nothing to do).
__device__ __forceinline__ void offsets_from_counts(const int *s_cnt, int *s_off, int E, int bm,
                                                    const Routing &r, int32_t *meta, int lane) {
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
            r.expert_counts[ex] = c[j];
            if (act[j]) {
                r.active_experts[oa] = ex;
                *reinterpret_cast<int4 *>(meta + 4 * oa) = make_int4(ex, op, c[j], 0);
            }
        }
        op += pad[j];
        oa += act[j];
    }
    // slots past the active count get count 0, the expert kernels' exit test
    const int n_act = __shfl(ia, 63);
    for (int q = n_act + lane; q < E; q += 64)
        *reinterpret_cast<int4 *>(meta + 4 * q) = make_int4(0, 0, 0, 0);
    if (lane == 63) {
        s_off[E] = ip;
        r.expert_offsets[E] = ip;
        r.num_active[0] = ic;
        r.num_active[1] = ip;
        r.num_active[2] = ia;
        r.num_active[3] = ip / bm;
    }
}

// All threads: block -> expert map and the pad entries (value TK) of every
// expert's segment, one thread per block of bm slots.
__device__ __forceinline__ void blocks_and_pads(const int *s_off, const int *s_cnt, int E, int bm,
                                                int TK, const Routing &r, int tid, int nthreads) {
    const int n_blocks = s_off[E] / bm;
    for (int b = tid; b < n_blocks; b += nthreads) {
        const int pos = b * bm;
        int lo = 0, hi = E - 1;  // last expert whose segment starts at or before pos
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        r.block_expert[b] = lo;
        const int end_valid = s_off[lo] + s_cnt[lo];
        for (int q = max(pos, end_valid); q < pos + bm; ++q) r.sorted_pairs[q] = TK;
    }
}

// Place one pair: its position in its expert's list, and the inverse maps.
__device__ __forceinline__ void place_pair(int p, int e, int pos, int K, const Routing &r,
                                           int32_t *pair_pos, int32_t *sorted_tok) {
    r.sorted_pairs[pos] = p;
    sorted_tok[pos] = p / K;
    pair_pos[p] = pos;
}

}  // namespace beam
