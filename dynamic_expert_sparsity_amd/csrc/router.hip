// a1-a3: router logits (main router and mask router in one pass), then per
// token Top-K, softmax over the kept logits, binary mask, g_hat and -1 ids.
//
// BEAM paper, section 3.2: Eq. 4 (r = R(x), Top-K, Softmax over the kept K),
// Eq. 5 (z = x W_m), Eq. 6 (m = [sigmoid(z) >= 0.5], evaluated as z >= 0),
// Eq. 7 (g_hat = g * m, no renormalisation).  Masked slots get the expert id
// -1 (news article on the paper, section 5, the modified routing kernel).
#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// Router logits, bf16, MFMA 16x16x32.  The two routers are one GEMM with
// 2E output columns: column n < E is W_gate row n, column E + n is W_mask
// row n.  Grid: (token tiles of 16*MT, column tiles of 64, splits of d).
// Each wave owns 16 columns; A (x rows) and B (weight rows) are both
// k-contiguous, so every lane's 16-byte load lands directly in MFMA layout.
// Out-of-range tokens / columns load a clamped row and their results are
// not stored.  partial[s][t][n] holds the split-s partial sums.
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(256) void router_logits_bf16(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Wg,
    const bf16_t *__restrict__ Wm, float *__restrict__ partial, int T, int d, int E,
    int dchunk) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int twoE = 2 * E;
    const int n = blockIdx.y * 64 + wave * 16 + (lane & 15);
    const int nc = n < twoE ? n : twoE - 1;
    const bf16_t *brow = nc < E ? Wg + (size_t)nc * d : Wm + (size_t)(nc - E) * d;
    const int kq = (lane >> 4) * 8;
    const int tbase = blockIdx.x * 16 * MT;

    const bf16_t *arow[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int t = tbase + m * 16 + (lane & 15);
        t = t < T ? t : T - 1;
        arow[m] = x + (size_t)t * d + kq;
    }
    brow += kq;

    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int k0 = blockIdx.z * dchunk;
    const int k1 = min(d, k0 + dchunk);
#pragma unroll 4
    for (int k = k0; k < k1; k += 32) {
        const u32x4 b = ld16(brow + k);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = mfma16x16x32(ld16(arow[m] + k), b, acc[m]);
    }

    if (n >= twoE) return;
    float *out = partial + (size_t)blockIdx.z * T * twoE + n;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tbase + m * 16 + (lane >> 4) * 4 + i;
            if (t < T) out[(size_t)t * twoE] = acc[m][i];
        }
    }
}

// Router logits, any element type, plain float dot products (used for the
// float32 layer).  One thread per (token, column).
template <typename T_>
__global__ __launch_bounds__(256) void router_logits_generic(
    const T_ *__restrict__ x, const T_ *__restrict__ Wg, const T_ *__restrict__ Wm,
    float *__restrict__ partial, int T, int d, int E) {
    const int twoE = 2 * E;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * twoE) return;
    const int t = (int)(idx / twoE);
    const int n = (int)(idx % twoE);
    const T_ *w = n < E ? Wg + (size_t)n * d : Wm + (size_t)(n - E) * d;
    const T_ *xr = x + (size_t)t * d;
    float acc = 0.f;
    for (int k = 0; k < d; ++k) acc = fmaf(elem<T_>::load(xr + k), elem<T_>::load(w + k), acc);
    partial[idx] = acc;
}

// ---------------------------------------------------------------------------
// Select: one wavefront per token, a workgroup per tile of `TS` (= 64) tokens.
// Lane l holds the logits of experts l, l+64, l+128, l+192.  K rounds of a
// wave-wide arg-max under the key (value desc, expert asc) give the Top-K
// slots in order; lane k keeps slot k.  Also builds, per tile and expert, the
// 64-bit set of tile tokens with an active pair for that expert; the
// compaction turns these into counts and stable ranks with popcounts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool beats(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

__global__ __launch_bounds__(256) void select_topk_mask(
    const float *__restrict__ partial, int splits, int T, int E, int K, float thr,
    Routing r, uint64_t *__restrict__ tile_mask) {
    __shared__ unsigned long long tmask[256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int e = tid; e < E; e += 256) tmask[e] = 0ull;
    __syncthreads();

    const int twoE = 2 * E;
    const int t0 = blockIdx.x * 64;
    for (int tl = wave; tl < 64; tl += 4) {
        const int t = t0 + tl;
        if (t >= T) break;
        float rv[4], zv[4];
        bool live[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            live[j] = e < E;
            rv[j] = 0.f;
            zv[j] = 0.f;
            if (live[j]) {
                for (int s = 0; s < splits; ++s) {
                    const float *ps = partial + ((size_t)s * T + t) * twoE;
                    rv[j] += ps[e];
                    zv[j] += ps[E + e];
                }
                r.gate_logits[(size_t)t * E + e] = rv[j];
                r.mask_logits[(size_t)t * E + e] = zv[j];
            }
        }

        float v0 = 0.f, myv = 0.f;
        int mye = 0;
        for (int k = 0; k < K; ++k) {
            float bv = 0.f;
            int be = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                if (live[j] && (be == 0x7fffffff || rv[j] > bv)) {  // e ascending in j
                    bv = rv[j];
                    be = e;
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oe = __shfl_xor(be, off);
                if (oe != 0x7fffffff && (be == 0x7fffffff || beats(ov, oe, bv, be))) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be & 63) == lane) live[be >> 6] = false;
            if (k == 0) v0 = bv;
            if (lane == k) {
                myv = bv;
                mye = be;
            }
        }

        // Softmax over the K kept logits, shifted by the largest one.
        const float num = lane < K ? expf(myv - v0) : 0.f;
        float den = num;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);

        // z of this lane's slot expert lives in lane (mye & 63), register mye >> 6.
        float zk = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float zz = __shfl(zv[j], mye & 63);
            if ((mye >> 6) == j) zk = zz;
        }
        if (lane < K) {
            const float g = num / den;
            const bool m = zk >= thr;
            const size_t q = (size_t)t * K + lane;
            r.topk_ids[q] = mye;
            r.topk_weights[q] = g;
            r.mask[q] = m ? 1 : 0;
            r.g_hat[q] = m ? g : 0.f;
            r.masked_ids[q] = m ? mye : -1;
            if (m) atomicOr(&tmask[mye], 1ull << tl);
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) tile_mask[(size_t)blockIdx.x * E + e] = tmask[e];
}

hipError_t launch_router_logits(const Plan &p, const void *x, const void *Wg, const void *Wm,
                                const Work &w, hipStream_t s) {
    if (p.dtype == 1) {
        const dim3 grid((p.T + p.r_tt - 1) / p.r_tt, (2 * p.E + 63) / 64, p.r_splits);
        if (p.r_tt == 16)
            router_logits_bf16<1><<<grid, 256, 0, s>>>((const bf16_t *)x, (const bf16_t *)Wg,
                                                       (const bf16_t *)Wm, w.partial, p.T, p.d,
                                                       p.E, p.r_dchunk);
        else
            router_logits_bf16<4><<<grid, 256, 0, s>>>((const bf16_t *)x, (const bf16_t *)Wg,
                                                       (const bf16_t *)Wm, w.partial, p.T, p.d,
                                                       p.E, p.r_dchunk);
    } else {
        const long long n = (long long)p.T * 2 * p.E;
        router_logits_generic<float><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const float *)x, (const float *)Wg, (const float *)Wm, w.partial, p.T, p.d, p.E);
    }
    return hipGetLastError();
}

hipError_t launch_select(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    select_topk_mask<<<p.n_tiles, 256, 0, s>>>(w.partial, p.r_splits, p.T, p.E, p.K, p.thr, r,
                                               w.tile_mask);
    return hipGetLastError();
}

}  // namespace beam
