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
// Weight-streaming path (decode, bf16).
//
// The k-loop of a wave streams NK steps of 32 elements; every step is one
// 16-byte load per lane per operand row (the MFMA 16x16x32 operand layout),
// and the loads run PF steps ahead of the MFMAs in a ring of register slots.
// With NK a compile-time constant the loop is fully unrolled, so the ring
// needs no register copies and the wait counts stay exact; NK = 0 selects a
// runtime-count loop for other sizes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stream_k2_rt(const bf16_t *__restrict__ b0,
                                             const bf16_t *__restrict__ b1,
                                             const bf16_t *__restrict__ a, int nk, f32x4 &acc0,
                                             f32x4 &acc1) {
    for (int k = 0; k < nk; ++k) {
        const u32x4 av = ld16(a + 32 * k);
        acc0 = mfma16x16x32(av, ld16(b0 + 32 * k), acc0);
        acc1 = mfma16x16x32(av, ld16(b1 + 32 * k), acc1);
    }
}

template <int NK, int PF>
__device__ __forceinline__ void stream_k1_lds(const bf16_t *__restrict__ b,
                                              const bf16_t *__restrict__ a_lds, f32x4 &acc) {
    // acc += A * B over NK k-steps; A from LDS
    u32x4 rb[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < NK) rb[p] = ld16(b + 32 * p);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int sl = k % PF;
        const u32x4 w = rb[sl];
        if (k + PF < NK) rb[sl] = ld16(b + 32 * (k + PF));
        const u32x4 av = *reinterpret_cast<const u32x4 *>(a_lds + 32 * k);
        acc = mfma16x16x32(av, w, acc);
    }
}

__device__ __forceinline__ void stream_k1_lds_rt(const bf16_t *__restrict__ b,
                                                 const bf16_t *__restrict__ a_lds, int nk,
                                                 f32x4 &acc) {
    for (int k = 0; k < nk; ++k)
        acc = mfma16x16x32(*reinterpret_cast<const u32x4 *>(a_lds + 32 * k),
                           ld16(b + 32 * k), acc);
}

// Up projection, streaming.  A unit is (active expert, 16 intermediate
// units): 16 gate rows + 16 up rows of W_gu, streamed once.  The expert's
// tokens (16 per MFMA row block; more are looped) form the A operand straight
// from x; the NW waves split d (NK k-steps each) and their partial sums meet
// in LDS.  Latency chain per unit: the expert's record {e, offset, count}
// (scalar load) -> every weight fragment of the wave is requested at once ->
// the block's 16 token ids (scalar loads, so they do not queue behind the
// weights) -> the x fragments.  Scheduling barriers keep the compiler from
// spreading the loads over the MFMAs; the weights stay in registers across
// further 16-token blocks.  Grid: max_active * (I / 16); units past the
// device-side active-expert count exit at once.
template <int NW, int NK>
__global__ __launch_bounds__(NW * 64) void up_stream_bf16(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Wgu,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ num_active,
    const int32_t *__restrict__ sorted_tok, bf16_t *__restrict__ h, int d, int I,
    const int32_t *__restrict__ mode) {
    // mode: NULL, or the per-call choice (1: this call's experts take the tiled kernels)
    if (mode != nullptr && *mode == 1) return;
    const int ncg = I >> 4;
    const int ai = blockIdx.x / ncg;
    const int cg = blockIdx.x - ai * ncg;
    // ai < max_active <= E: the record exists; count 0 marks an inactive slot
    const i32x4 mt = sload16(meta + 4 * ai);
    if (mt[2] == 0) return;
    const int e = mt[0], off = mt[1], cnt = mt[2];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int dq = d / NW;
    const int kb = wave * dq;
    const bf16_t *bg = Wgu + ((size_t)e * 2 * I + cg * 16 + li) * d + kb + kq;
    const bf16_t *bu = bg + (size_t)I * d;
    __shared__ f32x4 red[NW][2][64];

    u32x4 rg[NK > 0 ? NK : 1], ru[NK > 0 ? NK : 1], rx[NK > 0 ? NK : 1];
    if constexpr (NK > 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            rg[k] = ld16(bg + 32 * k);
            ru[k] = ld16(bu + 32 * k);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int pc = 0; pc < cnt; pc += 16) {
        // token ids of the block's 16 positions (inside the padded segment)
        const int *st = sorted_tok + off + pc;
        int tok = st[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) {
            const int v = st[j];
            tok = li == j ? v : tok;
        }
        tok = pc + li < cnt ? tok : 0;
        const bf16_t *xa = x + (size_t)tok * d + kb + kq;
        f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NK > 0) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NK; ++k) rx[k] = ld16(xa + 32 * k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                ag = mfma16x16x32(rx[k], rg[k], ag);
                au = mfma16x16x32(rx[k], ru[k], au);
            }
        } else {
            stream_k2_rt(bg, bu, xa, dq >> 5, ag, au);
        }
        red[wave][0][lane] = ag;
        red[wave][1][lane] = au;
        __syncthreads();
        if (wave == 0) {
            f32x4 sg = red[0][0][lane], su = red[0][1][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                sg += red[w][0][lane];
                su += red[w][1][lane];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = pc + (lane >> 4) * 4 + q;
                if (row < cnt)
                    h[(size_t)(off + row) * I + cg * 16 + li] =
                        f32_to_bf16(silu<false>(sg[q]) * su[q]);
            }
        }
        __syncthreads();
    }
}

// Down projection, streaming: a unit is (active expert, 64 output channels);
// each wave owns 16 channels (16 rows of W_dt[e], each I long) over all of I
// (NK = I / 32 k-steps).  The 16 h rows of the current position block are
// staged in LDS once per workgroup (row pitch I + 8 elements keeps the MFMA
// reads conflict-free).
template <int NK>
__global__ __launch_bounds__(256) void down_stream_bf16(
    const bf16_t *__restrict__ Wdt, const bf16_t *__restrict__ h,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ num_active,
    bf16_t *__restrict__ o, int d, int I, const int32_t *__restrict__ mode) {
    if (mode != nullptr && *mode == 1) return;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    bf16_t *hs = reinterpret_cast<bf16_t *>(lds_raw);
    const int pitch = I + 8;
    const int ncg = d >> 6;
    const int ai = blockIdx.x / ncg;
    const int cg = blockIdx.x - ai * ncg;
    // ai < max_active <= E: the record exists; count 0 marks an inactive slot
    const i32x4 mt = sload16(meta + 4 * ai);
    if (mt[2] == 0) return;
    const int e = mt[0], off = mt[1], cnt = mt[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kq = (lane >> 4) * 8;
    const int c = cg * 64 + wave * 16 + (lane & 15);
    const bf16_t *brow = Wdt + ((size_t)e * d + c) * I + kq;
    const bf16_t *arow = hs + (lane & 15) * pitch + kq;
    const int chunks = I >> 3;  // 16-byte chunks per row

    for (int pc = 0; pc < cnt; pc += 16) {
        // rows past cnt are the padded segment's rows (inside the buffer);
        // their results land in D rows that are not stored
        for (int q = tid; q < 16 * chunks; q += 256) {
            const int row = q / chunks, ch = q - row * chunks;
            *reinterpret_cast<u32x4 *>(hs + row * pitch + ch * 8) =
                ld16(h + (size_t)(off + pc + row) * I + ch * 8);
        }
        __syncthreads();
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NK > 0) stream_k1_lds<NK, (NK < 8 ? NK : 8)>(brow, arow, acc);
        else stream_k1_lds_rt(brow, arow, I >> 5, acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = pc + (lane >> 4) * 4 + q;
            if (row < cnt) o[(size_t)(off + row) * d + c] = f32_to_bf16(acc[q]);
        }
        __syncthreads();
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
    if (p.path == 1) {
        // tiled GEMM, then the streaming kernels; the per-call mode record
        // lets exactly one of them work (only the GEMM when split == 0)
        const hipError_t e = launch_gemm_up(p, x, W_gu, r, w, s);
        if (e != hipSuccess || p.split == 0) return e;
    }
    if (p.dtype == 1) {
        const unsigned grid = (unsigned)p.max_active * (unsigned)(p.I / 16);
#define BEAM_UP(NWV, NKV)                                                                     \
    up_stream_bf16<NWV, NKV><<<grid, NWV * 64, 0, s>>>(                                      \
        (const bf16_t *)x, (const bf16_t *)W_gu, w.meta, r.num_active, w.sorted_tok,          \
        (bf16_t *)w.h, p.d, p.I, p.path == 1 ? w.meta + 4 * p.E : nullptr)
        if (p.d % 256 == 0) {  // eight waves split d, d / 256 k-steps each
            switch (p.d / 256) {
                case 1: BEAM_UP(8, 1); break;
                case 2: BEAM_UP(8, 2); break;
                case 4: BEAM_UP(8, 4); break;
                case 8: BEAM_UP(8, 8); break;
                case 12: BEAM_UP(8, 12); break;
                case 16: BEAM_UP(8, 16); break;
                default: BEAM_UP(8, 0); break;
            }
        } else {               // four waves, d / 128 k-steps each
            BEAM_UP(4, 0);
        }
#undef BEAM_UP
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
    if (p.path == 1) {
        const hipError_t e = launch_gemm_down(p, W_dt, r, w, s);
        if (e != hipSuccess || p.split == 0) return e;
    }
    if (p.dtype == 1) {
        const unsigned grid = (unsigned)p.max_active * (unsigned)(p.d / 64);
        const size_t lds = (size_t)16 * (p.I + 8) * sizeof(bf16_t);
#define BEAM_DOWN(NKV)                                                                        \
    down_stream_bf16<NKV><<<grid, 256, lds, s>>>((const bf16_t *)W_dt, (const bf16_t *)w.h,   \
                                                 w.meta, r.num_active, (bf16_t *)w.o, p.d,    \
                                                 p.I, p.path == 1 ? w.meta + 4 * p.E : nullptr)
        switch (p.I / 32) {  // k-steps per wave
            case 2: BEAM_DOWN(2); break;
            case 4: BEAM_DOWN(4); break;
            case 8: BEAM_DOWN(8); break;
            case 12: BEAM_DOWN(12); break;
            case 16: BEAM_DOWN(16); break;
            case 24: BEAM_DOWN(24); break;
            case 32: BEAM_DOWN(32); break;
            case 48: BEAM_DOWN(48); break;
            default: BEAM_DOWN(0); break;
        }
#undef BEAM_DOWN
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
