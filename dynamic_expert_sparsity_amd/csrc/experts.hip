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
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "ring_dev.h"

namespace beam {

// ---------------------------------------------------------------------------
// Generic path (float32 layer): one workgroup per block of bm sorted
// positions, one thread per output column; plain fp32 FMAs.
// ---------------------------------------------------------------------------
template <typename T_>
__global__ __launch_bounds__(256) void up_generic(
    const T_ *__restrict__ x, const T_ *__restrict__ Wgu, const int32_t *__restrict__ block_expert,
    const int32_t *__restrict__ num_active, const int32_t *__restrict__ sorted_pairs,
    const int32_t *__restrict__ sorted_tok, T_ *__restrict__ h, int d, int I, int PT, int bm) {
    const int b = blockIdx.x;
    if (b >= num_active[3]) return;
    const int j = blockIdx.y * 256 + threadIdx.x;
    if (j >= I) return;
    const int e = block_expert[b];
    const T_ *wg = Wgu + ((size_t)e * 2 * I + j) * d;
    const T_ *wu = wg + (size_t)I * d;
    for (int i = 0; i < bm; ++i) {
        const int pos = b * bm + i;
        if (sorted_pairs[pos] >= PT) break;  // pads only follow the valid entries
        const T_ *xr = x + (size_t)sorted_tok[pos] * d;
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
    const int32_t *__restrict__ sorted_pairs, T_ *__restrict__ o, int d, int I, int PT, int bm) {
    const int b = blockIdx.x;
    if (b >= num_active[3]) return;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= d) return;
    const int e = block_expert[b];
    const T_ *w = Wdt + ((size_t)e * d + c) * I;
    for (int i = 0; i < bm; ++i) {
        const int pos = b * bm + i;
        if (sorted_pairs[pos] >= PT) break;
        const T_ *hr = h + (size_t)pos * I;
        float acc = 0.f;
        for (int k = 0; k < I; ++k) acc = fmaf(elem<T_>::load(hr + k), elem<T_>::load(w + k), acc);
        elem<T_>::store(o + (size_t)pos * d + c, acc);
    }
}

// ---------------------------------------------------------------------------
// Combine (Eq. 8): y_t = the S shared experts' rows o[pair_pos[T*K + t*S + s]]
// (weight 1), then sum over k of g_hat[t,k] * o[pair_pos[t*K+k]] in slot
// order, float accumulate; masked slots (pair_pos -1) are skipped, so
// without shared experts a token with no active slot gets exactly 0.
// ---------------------------------------------------------------------------
template <typename T_>
__global__ __launch_bounds__(256) void combine_generic(const T_ *__restrict__ o,
                                                       const int32_t *__restrict__ pair_pos,
                                                       const float *__restrict__ g_hat,
                                                       T_ *__restrict__ y, int d, int K, int TK,
                                                       int S) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < d; c += 256) {
        float acc = 0.f;
        for (int q = 0; q < S; ++q)
            acc += elem<T_>::load(o + (size_t)pair_pos[TK + t * S + q] * d + c);
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
                                                    bf16_t *__restrict__ y, int d, int K, int TK,
                                                    int S) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        for (int sx = 0; sx < S; ++sx) {
            const int pp = pair_pos[TK + t * S + sx];
            const u32x4 v = ld16(o + (size_t)pp * d + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
            }
        }
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

// The streaming kernel: the per-call record's layout flag (mrec[3], set by
// the compaction when the routed pairs number at least 6 per block of 32
// positions) picks two column groups per unit, else one.
template <bool DOWN, bool TAIL>
__global__ __launch_bounds__(512, 1) void ring_bf16(
    const bf16_t *__restrict__ A, const bf16_t *__restrict__ W,
    const int32_t *__restrict__ pbt, const int32_t *__restrict__ mrec,
    const int32_t *__restrict__ sorted_tok, bf16_t *__restrict__ out, int klen, int ncols,
    int check_mode) {
    if (mrec[3])
        ring2_body<DOWN, TAIL>(A, W, pbt, mrec, sorted_tok, out, klen, ncols, check_mode);
    else
        ring1_body<DOWN, TAIL>(A, W, pbt, mrec, sorted_tok, out, klen, ncols, check_mode);
}

// The ring kernels need a k length (d for up, I for down) that is a multiple
// of 64 and whole units (I % 32 for up, d % 64 for down, as the
// two-column-group layout needs): the descriptor checks of a bf16 layer (d % 128 == 0, I % 64 == 0)
// imply both.
static int ring_grid() {
    static int n = 0;
    static std::once_flag once;
    std::call_once(once, [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            n = cus;
        if (n <= 0) n = 256;
    });
    return n;
}
// up to 160 KB of dynamic LDS: allowed once per kernel (the attribute is per function)
static hipError_t ring_attr(const void *fn, int bytes) {
    static std::mutex mu;
    static const void *done[16] = {};
    std::lock_guard<std::mutex> lk(mu);
    for (const void *f : done)
        if (f == fn) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    for (const void *&f : done)
        if (!f) { f = fn; break; }
    return hipSuccess;
}

// one ring launch; TAIL: the k length ends in a short chunk
template <bool DOWN, bool TAIL>
static hipError_t launch_ring_t(const void *A, const void *W, const Plan &p, const Work &w, void *out,
                                int klen, int ncols, hipStream_t s) {
    static_assert(RING2_LDS <= RING_LDS, "one LDS size for both layouts");
    const hipError_t e = ring_attr((const void *)ring_bf16<DOWN, TAIL>, RING_LDS);
    if (e != hipSuccess) return e;
    ring_bf16<DOWN, TAIL><<<ring_grid(), 512, RING_LDS, s>>>(
        (const bf16_t *)A, (const bf16_t *)W, w.pbt, w.meta, w.sorted_tok, (bf16_t *)out, klen, ncols,
        p.path == 1 ? 1 : 0);
    return hipGetLastError();
}
template <bool DOWN>
static hipError_t launch_ring(const void *A, const void *W, const Plan &p, const Work &w, void *out,
                              int klen, int ncols, hipStream_t s) {
    return klen % 256 == 0 ? launch_ring_t<DOWN, false>(A, W, p, w, out, klen, ncols, s)
                           : launch_ring_t<DOWN, true>(A, W, p, w, out, klen, ncols, s);
}

hipError_t launch_expert_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                            const Work &w, hipStream_t s) {
    if (p.path == 1) return launch_tiled_up(p, x, W_gu, r, w, s);
    if (p.dtype == 1) {
        const hipError_t e = launch_ring<false>(x, W_gu, p, w, w.h, p.d, p.I, s);
        if (e != hipSuccess) return e;
    } else {
        const dim3 grid((unsigned)p.n_blocks_cap, (p.I + 255) / 256);
        up_generic<float><<<grid, 256, 0, s>>>((const float *)x, (const float *)W_gu,
                                               r.block_expert, r.num_active, r.sorted_pairs,
                                               w.sorted_tok, (float *)w.h, p.d, p.I, p.PT, p.bm);
    }
    return hipGetLastError();
}

hipError_t launch_expert_down(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                              hipStream_t s) {
    if (p.path == 1) return launch_tiled_down(p, W_dt, r, w, s);
    if (p.dtype == 1) {
        const hipError_t e = launch_ring<true>(w.h, W_dt, p, w, w.o, p.I, p.d, s);
        if (e != hipSuccess) return e;
    } else {
        const dim3 grid((unsigned)p.n_blocks_cap, (p.d + 255) / 256);
        down_generic<float><<<grid, 256, 0, s>>>((const float *)W_dt, (const float *)w.h,
                                                 r.block_expert, r.num_active, r.sorted_pairs,
                                                 (float *)w.o, p.d, p.I, p.PT, p.bm);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const Plan &p, const Routing &r, const Work &w, void *y,
                          hipStream_t s) {
    if (p.dtype == 1)
        combine_bf16<<<p.T, 256, 0, s>>>((const bf16_t *)w.o, w.pair_pos, r.g_hat, (bf16_t *)y,
                                         p.d, p.K, p.T * p.K, p.S);
    else
        combine_generic<float><<<p.T, 256, 0, s>>>((const float *)w.o, w.pair_pos, r.g_hat,
                                                   (float *)y, p.d, p.K, p.T * p.K, p.S);
    return hipGetLastError();
}

}  // namespace beam
