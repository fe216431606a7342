// a5-a7: SwiGLU experts on the active pairs only, then the masked weighted
// sum.  BEAM paper, section 3.1 Eq. 3 (E(x) = (SiLU(x Wg) * (x Wu)) Wd) and
// section 3.2 Eq. 8 (y = sum_i g_hat_i E_i(x)).  Only experts with at least
// one active pair are visited, so masked pairs cost neither FLOPs nor weight
// bytes (the point of the binary mask, paper section 3.2 and the news
// article's section 5).
//
// Buffers (workspace):
//   h [cap, I]  SiLU(x Wg) * (x Wu) per sorted position (bf16 for the bf16
//               layer, rounded to nearest even; float for the float layer)
//   o [cap, d]  expert output per sorted position (same element type)
// and the combine reads o through pair_pos[t*K + k] (-1 when masked).
#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// Weight-streaming path (decode, bf16).  A unit is (active expert, 16
// intermediate units): 16 gate rows + 16 up rows of W_gu, streamed once.
// The expert's tokens (at most 16 per MFMA row block; more are looped) form
// the MFMA A operand straight from x; the four waves split d and their
// partial sums meet in LDS.  Grid: max_active * (I / 16) workgroups; units
// past the device-side active-expert count exit at once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void up_stream_bf16(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Wgu,
    const int32_t *__restrict__ active, const int32_t *__restrict__ num_active,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_pairs, bf16_t *__restrict__ h, int d, int I, int K) {
    const int ncg = I >> 4;
    const int ai = blockIdx.x / ncg;
    const int cg = blockIdx.x - ai * ncg;
    if (ai >= num_active[2]) return;
    const int e = active[ai];
    const int off = offsets[e];
    const int cnt = counts[e];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = (lane >> 4) * 8;
    const int dq = d >> 2;
    const int kb = wave * dq;
    const bf16_t *bg = Wgu + ((size_t)e * 2 * I + cg * 16 + (lane & 15)) * d + kb + kq;
    const bf16_t *bu = bg + (size_t)I * d;
    __shared__ f32x4 red[4][2][64];

    for (int pc = 0; pc < cnt; pc += 16) {
        const int i = pc + (lane & 15);
        const int tok = i < cnt ? sorted_pairs[off + i] / K : 0;
        const bf16_t *xa = x + (size_t)tok * d + kb + kq;
        f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k = 0; k < dq; k += 32) {
            const u32x4 a = ld16(xa + k);
            const u32x4 wgv = ld16_stream(bg + k);
            const u32x4 wuv = ld16_stream(bu + k);
            ag = mfma16x16x32(a, wgv, ag);
            au = mfma16x16x32(a, wuv, au);
        }
        red[wave][0][lane] = ag;
        red[wave][1][lane] = au;
        __syncthreads();
        if (wave == 0) {
            f32x4 sg = red[0][0][lane], su = red[0][1][lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                sg += red[w][0][lane];
                su += red[w][1][lane];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = pc + (lane >> 4) * 4 + q;
                if (row < cnt)
                    h[(size_t)(off + row) * I + cg * 16 + (lane & 15)] =
                        f32_to_bf16(silu<false>(sg[q]) * su[q]);
            }
        }
        __syncthreads();
    }
}

// Down projection, streaming: a unit is (active expert, 64 output channels);
// each wave owns 16 channels (16 rows of W_dt[e], each I long) over all of I.
__global__ __launch_bounds__(256) void down_stream_bf16(
    const bf16_t *__restrict__ Wdt, const bf16_t *__restrict__ h,
    const int32_t *__restrict__ active, const int32_t *__restrict__ num_active,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    bf16_t *__restrict__ o, int d, int I) {
    const int ncg = d >> 6;
    const int ai = blockIdx.x / ncg;
    const int cg = blockIdx.x - ai * ncg;
    if (ai >= num_active[2]) return;
    const int e = active[ai];
    const int off = offsets[e];
    const int cnt = counts[e];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = (lane >> 4) * 8;
    const int c = cg * 64 + wave * 16 + (lane & 15);
    const bf16_t *brow = Wdt + ((size_t)e * d + c) * I + kq;

    for (int pc = 0; pc < cnt; pc += 16) {
        // rows past cnt read h rows of the padded segment (inside the buffer);
        // their results land in D rows that are not stored
        const bf16_t *arow = h + (size_t)(off + pc + (lane & 15)) * I + kq;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k = 0; k < I; k += 32) acc = mfma16x16x32(ld16(arow + k), ld16_stream(brow + k), acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = pc + (lane >> 4) * 4 + q;
            if (row < cnt) o[(size_t)(off + row) * d + c] = f32_to_bf16(acc[q]);
        }
    }
}

// ---------------------------------------------------------------------------
// Generic path (float32 layer): one workgroup per block of bm sorted
// positions, one thread per output column; plain fp32 FMAs.
// ---------------------------------------------------------------------------
template <typename T_>
__global__ __launch_bounds__(256) void up_generic(
    const T_ *__restrict__ x, const T_ *__restrict__ Wgu, const int32_t *__restrict__ block_expert,
    const int32_t *__restrict__ num_active, const int32_t *__restrict__ sorted_pairs,
    T_ *__restrict__ h, int d, int I, int K, int TK, int bm) {
    const int b = blockIdx.x;
    if (b >= num_active[3]) return;
    const int j = blockIdx.y * 256 + threadIdx.x;
    if (j >= I) return;
    const int e = block_expert[b];
    const T_ *wg = Wgu + ((size_t)e * 2 * I + j) * d;
    const T_ *wu = wg + (size_t)I * d;
    for (int i = 0; i < bm; ++i) {
        const int pos = b * bm + i;
        const int pr = sorted_pairs[pos];
        if (pr >= TK) break;  // pads only follow the valid entries
        const T_ *xr = x + (size_t)(pr / K) * d;
        float a = 0.f, u = 0.f;
        for (int k = 0; k < d; ++k) {
            const float xv = elem<T_>::load(xr + k);
            a = fmaf(xv, elem<T_>::load(wg + k), a);
            u = fmaf(xv, elem<T_>::load(wu + k), u);
        }
        elem<T_>::store(h + (size_t)pos * I + j, silu<true>(a) * u);
    }
}

template <typename T_>
__global__ __launch_bounds__(256) void down_generic(
    const T_ *__restrict__ Wdt, const T_ *__restrict__ h,
    const int32_t *__restrict__ block_expert, const int32_t *__restrict__ num_active,
    const int32_t *__restrict__ sorted_pairs, T_ *__restrict__ o, int d, int I, int TK, int bm) {
    const int b = blockIdx.x;
    if (b >= num_active[3]) return;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= d) return;
    const int e = block_expert[b];
    const T_ *w = Wdt + ((size_t)e * d + c) * I;
    for (int i = 0; i < bm; ++i) {
        const int pos = b * bm + i;
        if (sorted_pairs[pos] >= TK) break;
        const T_ *hr = h + (size_t)pos * I;
        float acc = 0.f;
        for (int k = 0; k < I; ++k) acc = fmaf(elem<T_>::load(hr + k), elem<T_>::load(w + k), acc);
        elem<T_>::store(o + (size_t)pos * d + c, acc);
    }
}

// ---------------------------------------------------------------------------
// Combine (Eq. 8): y_t = sum over k of g_hat[t,k] * o[pair_pos[t*K+k]], in
// slot order, float accumulate; masked slots (pair_pos -1) are skipped, so a
// token with no active slot gets exactly 0.
// ---------------------------------------------------------------------------
template <typename T_>
__global__ __launch_bounds__(256) void combine_generic(const T_ *__restrict__ o,
                                                       const int32_t *__restrict__ pair_pos,
                                                       const float *__restrict__ g_hat,
                                                       T_ *__restrict__ y, int d, int K) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < d; c += 256) {
        float acc = 0.f;
        for (int k = 0; k < K; ++k) {
            const int pp = pair_pos[(size_t)t * K + k];
            if (pp >= 0) acc = fmaf(g_hat[(size_t)t * K + k], elem<T_>::load(o + (size_t)pp * d + c), acc);
        }
        elem<T_>::store(y + (size_t)t * d + c, acc);
    }
}

// bf16, 8 channels per thread with 16-byte loads and stores.
__global__ __launch_bounds__(256) void combine_bf16(const bf16_t *__restrict__ o,
                                                    const int32_t *__restrict__ pair_pos,
                                                    const float *__restrict__ g_hat,
                                                    bf16_t *__restrict__ y, int d, int K) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        for (int k = 0; k < K; ++k) {
            const int pp = pair_pos[(size_t)t * K + k];
            if (pp < 0) continue;
            const float gk = g_hat[(size_t)t * K + k];
            const u32x4 v = ld16(o + (size_t)pp * d + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(gk, __uint_as_float(v[q] << 16), acc[2 * q]);
                acc[2 * q + 1] = fmaf(gk, __uint_as_float(v[q] & 0xffff0000u), acc[2 * q + 1]);
            }
        }
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            out[q] = (uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16);
        *reinterpret_cast<u32x4 *>(y + (size_t)t * d + c) = out;
    }
}

hipError_t launch_expert_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                            const Work &w, hipStream_t s) {
    if (p.dtype == 1) {
        const unsigned grid = (unsigned)p.max_active * (unsigned)(p.I / 16);
        up_stream_bf16<<<grid, 256, 0, s>>>((const bf16_t *)x, (const bf16_t *)W_gu,
                                            r.active_experts, r.num_active, r.expert_counts,
                                            r.expert_offsets, r.sorted_pairs, (bf16_t *)w.h, p.d,
                                            p.I, p.K);
    } else {
        const dim3 grid((unsigned)p.n_blocks_cap, (p.I + 255) / 256);
        up_generic<float><<<grid, 256, 0, s>>>((const float *)x, (const float *)W_gu,
                                               r.block_expert, r.num_active, r.sorted_pairs,
                                               (float *)w.h, p.d, p.I, p.K, p.T * p.K, p.bm);
    }
    return hipGetLastError();
}

hipError_t launch_expert_down(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                              hipStream_t s) {
    if (p.dtype == 1) {
        const unsigned grid = (unsigned)p.max_active * (unsigned)(p.d / 64);
        down_stream_bf16<<<grid, 256, 0, s>>>((const bf16_t *)W_dt, (const bf16_t *)w.h,
                                              r.active_experts, r.num_active, r.expert_counts,
                                              r.expert_offsets, (bf16_t *)w.o, p.d, p.I);
    } else {
        const dim3 grid((unsigned)p.n_blocks_cap, (p.d + 255) / 256);
        down_generic<float><<<grid, 256, 0, s>>>((const float *)W_dt, (const float *)w.h,
                                                 r.block_expert, r.num_active, r.sorted_pairs,
                                                 (float *)w.o, p.d, p.I, p.T * p.K, p.bm);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const Plan &p, const Routing &r, const Work &w, void *y,
                          hipStream_t s) {
    if (p.dtype == 1)
        combine_bf16<<<p.T, 256, 0, s>>>((const bf16_t *)w.o, w.pair_pos, r.g_hat, (bf16_t *)y,
                                         p.d, p.K);
    else
        combine_generic<float><<<p.T, 256, 0, s>>>((const float *)w.o, w.pair_pos, r.g_hat,
                                                   (float *)y, p.d, p.K);
    return hipGetLastError();
}

}  // namespace beam
