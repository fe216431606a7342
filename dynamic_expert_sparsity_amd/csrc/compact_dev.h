// Device-side grouping of the active (token, expert) pairs into per-expert
// lists.  Masked slots (id -1) are left out of every count, so masked pairs
// are never scheduled (news article on the BEAM paper, section 5, the
// modified expert/token grouping kernel).
//
// Input: per select tile (64 tokens) and expert, the 64-bit set of tile
// tokens that have an active pair for that expert (an expert appears at most
// once among a token's K slots).
//   count(tile, e)        = popcount(set)
//   rank of token tl      = popcount(set & ((1 << tl) - 1))
// so a pair's position in its expert's list is
//   offsets[e] + (pairs of e in earlier tiles) + rank,
// which lists each expert's pairs in ascending pair id with no atomics.
#pragma once
#include <climits>

#include "common.h"
#include "kernels.h"

namespace beam {

// 128-row tiles while they number fewer than BEAM_TILE128_X10 / 10 times the
// 256-row tiles
#ifndef BEAM_TILE128_X10
#define BEAM_TILE128_X10 13
#endif

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round
// trips): shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes without a
// source add 0), then row 15's total added to rows 1 and 3 and lane 31's to
// rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
    v = dpp_add<0x111, 0xF>(v);  // row_shr:1
    v = dpp_add<0x112, 0xF>(v);  // row_shr:2
    v = dpp_add<0x114, 0xF>(v);  // row_shr:4
    v = dpp_add<0x118, 0xF>(v);  // row_shr:8
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return v;
}

// Wave 0 only (lane = threadIdx.x < 64): from per-expert counts s_cnt[E]
// (E <= 256, four experts per lane) write block-padded exclusive offsets to
// s_off[0..E] and r.expert_offsets, the ascending active-expert list and
// r.num_active = {P, num_padded, n_active_experts, n_blocks}, the call's
// record meta = {kernel family, max count, records, layout} and the work records
// of the family (pbt, in expert order): the streaming kernels (family 0) get
// one record {expert, first position, rows, 0} per block of up to 32
// consecutive positions of an expert; the 256-row tiled kernels (family 2)
// one record {expert, first position, segment rows, valid rows} per 256-row
// tile of an expert's 128-padded segment (the last may hold 128 rows); the
// 128-row tiled kernels (family 1) walk the block map.
// write = false: only s_off (and, when given, the active-expert list s_act
// and its length *s_nact) in LDS; nothing in global memory.
__device__ __forceinline__ void offsets_from_counts(const int *s_cnt, int *s_off, int E, int bm,
                                                    const Routing &r, int32_t *meta,
                                                    int32_t *pbt, int split, int lane,
                                                    bool write = true, int *s_act = nullptr,
                                                    int *s_nact = nullptr) {
    int c[4], pad[4], act[4], npb[4], nq[4];
    int sc = 0, sp = 0, sa = 0, mx = 0, sb = 0, sq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ex = lane * 4 + j;
        c[j] = ex < E ? s_cnt[ex] : 0;
        pad[j] = (c[j] + bm - 1) / bm * bm;
        act[j] = c[j] > 0 ? 1 : 0;
        npb[j] = (c[j] + 31) >> 5;
        nq[j] = (c[j] + 255) >> 8;
        sq += nq[j];
        sc += c[j];
        sp += pad[j];
        sa += act[j];
        sb += npb[j];
        mx = max(mx, c[j]);
    }
    // largest count: within each row of 16 by DPP, then the four rows' maxima
    mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0x141, 0xF, 0xF, false));  // row_half_mirror
    mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0x140, 0xF, 0xF, false));  // row_mirror
    mx = max(max(__builtin_amdgcn_readlane(mx, 0), __builtin_amdgcn_readlane(mx, 16)),
             max(__builtin_amdgcn_readlane(mx, 32), __builtin_amdgcn_readlane(mx, 48)));
    const int ic = wave_incl_scan(sc, lane);
    const int ip = wave_incl_scan(sp, lane);
    const int ia = wave_incl_scan(sa, lane);
    const int ib = wave_incl_scan(sb, lane);
    const int iq = wave_incl_scan(sq, lane);
    int op = ip - sp, oa = ia - sa, ob = ib - sb, oq = iq - sq;
    // expert kernels for this call (Plan::split).  The streaming kernels
    // stream an expert's weights once per block of 32 positions: the tiled
    // kernels take the call once those re-reads reach a quarter of the
    // active experts' weights, or one expert has more than 512 pairs
    // (measured on the Qwen3-shaped layer at 1024-2048 tokens: the streaming
    // kernels' time grows with the blocks per active expert, ~264 us per
    // layer at 1.0, while the tiled kernels' stays near 320 us; they cross
    // near 1.2).  A tiled tile
    // reads its expert's weight slice once and computes all its rows: 128-row
    // tiles waste fewer rows on sparse experts, 256-row tiles read the weights
    // of a dense expert half as often; 128-row tiles are taken while their
    // count stays under 1.3 x the 256-row tiles' (measured on the Qwen3-shaped
    // layer: 128-row tiles are 13-15% faster at ratios near 1, 256-row tiles
    // about 4% faster at ratios near 1.5)
    const int tot_b = __builtin_amdgcn_readlane(ib, 63), tot_a = __builtin_amdgcn_readlane(ia, 63),
              tot_q = __builtin_amdgcn_readlane(iq, 63);
    const bool tiled = split == 0 || (split != INT_MAX && (4 * tot_b >= 5 * tot_a || mx > 512));
    const int n_bm = __builtin_amdgcn_readlane(ip, 63) / bm;
    const int mode = !tiled ? 0 : (10 * n_bm < BEAM_TILE128_X10 * tot_q ? 1 : 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ex = lane * 4 + j;
        if (ex < E) {
            s_off[ex] = op;
            if (s_act && act[j]) s_act[oa] = ex;
        }
        if (ex < E && write) {
            r.expert_offsets[ex] = op;
            r.expert_counts[ex] = c[j];
            if (act[j]) r.active_experts[oa] = ex;
            if (mode == 0)
                for (int q = 0; q < npb[j]; ++q)
                    *reinterpret_cast<int4 *>(pbt + 4 * (ob + q)) =
                        make_int4(ex, op + 32 * q, min(32, c[j] - 32 * q), 0);
            else if (mode == 2)
                for (int q = 0; q < nq[j]; ++q)
                    *reinterpret_cast<int4 *>(pbt + 4 * (oq + q)) =
                        make_int4(ex, op + 256 * q, min(256, pad[j] - 256 * q),
                                  min(256, c[j] - 256 * q));
        }
        op += pad[j];
        oa += act[j];
        ob += npb[j];
        oq += nq[j];
    }
    if (lane == 63) {
        s_off[E] = ip;
        if (s_nact) *s_nact = ia;
    }
    if (lane == 63 && write) {
        r.expert_offsets[E] = ip;
        r.num_active[0] = ic;
        r.num_active[1] = ip;
        r.num_active[2] = ia;
        r.num_active[3] = ip / bm;
        // streaming kernels' layout: two column groups per unit once the
        // blocks of 32 positions hold 6 routed pairs or more on average (their
        // x rows then cost about as much as the weights; measured on the
        // Qwen3-shaped layer: one group is faster at ~2.6 and ~4.8 pairs per
        // block, two at ~7 and above)
        const int wide = ic >= 6 * ib ? 1 : 0;
        *reinterpret_cast<int4 *>(meta) = make_int4(mode, mx, mode == 2 ? iq : ib, wide);
    }
}

// All threads: block -> expert map (one thread per block) and the pad entries
// of every expert's segment (sorted pair `pad`, token 0; one wave per expert,
// its lanes over the pad slots, so the stores coalesce).
__device__ __forceinline__ void blocks_and_pads(const int *s_off, const int *s_cnt, int E, int bm,
                                                int pad, const Routing &r, int32_t *sorted_tok,
                                                int tid, int nthreads) {
    const int n_blocks = s_off[E] / bm;
    for (int b = tid; b < n_blocks; b += nthreads) {
        const int pos = b * bm;
        int lo = 0, hi = E - 1;  // last expert whose segment starts at or before pos
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        r.block_expert[b] = lo;
    }
    const int lane = tid & 63, nw = nthreads >> 6;
    for (int e = tid >> 6; e < E; e += nw) {
        const int end = s_off[e + 1];
        for (int q = s_off[e] + s_cnt[e] + lane; q < end; q += 64) {
            r.sorted_pairs[q] = pad;
            sorted_tok[q] = 0;
        }
    }
}

// Place one pair of token t: its position in its expert's list, and the
// inverse maps.
__device__ __forceinline__ void place_pair(int p, int t, int pos, const Routing &r,
                                           int32_t *pair_pos, int32_t *sorted_tok) {
    r.sorted_pairs[pos] = p;
    sorted_tok[pos] = t;
    pair_pos[p] = pos;
}

// Pair p < T*K is routed slot (t, k) = (p / K, p % K); p >= T*K is shared
// expert E + s of token t, p = T*K + t*S + s.  Tile token sets and bases are
// [tile][E + S].
// mid: the masked id of a routed pair (ignored for shared ones).  The token
// sets and bases may sit in global memory or in LDS.
__device__ __forceinline__ void scatter_pair(int p, int mid, int K, int TK, int E, int S,
                                             const Routing &r, const int *off,
                                             const int32_t *tile_base, const uint64_t *tile_mask,
                                             int32_t *pair_pos, int32_t *sorted_tok) {
    int e, t;
    if (p < TK) {
        e = mid;
        if (e < 0) {
            pair_pos[p] = -1;
            return;
        }
        t = p / K;
    } else {
        const int q = p - TK;
        t = q / S;
        e = E + (q - t * S);
    }
    const size_t qi = (size_t)(t >> 6) * (E + S) + e;
    const int rank = __popcll(tile_mask[qi] & ((1ull << (t & 63)) - 1ull));
    place_pair(p, t, off[e] + tile_base[qi] + rank, r, pair_pos, sorted_tok);
}

}  // namespace beam
