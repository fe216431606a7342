// Mask-router backward: the straight-through estimator of the binarisation
// and the gradient of the sparsity term (BEAM paper, section 3.3; news
// article on the paper, section 4: the hard 0/1 decision is used forward and
// passed straight through backward; a beta-weighted sum of the Top-K
// candidates' mask scores pushes towards fewer experts).
//
// For token t, candidate slot k (expert id_k, weight g_k, hard mask m_k) and
// the upstream slot gradient s_k = dL/dg_hat_k:
//   dL/dm_hat_k = g_k s_k + beta                     (STE: dL/dm_hat = dL/dm)
//   dz[t, id_k] = dL/dm_hat_k * sig(z) (1 - sig(z))  (m_hat = sigmoid(z), Eq. 5)
//   dW_mask     = dz^T x,   dx = dz W_mask           (z = x W_mask^T)
//   d_gate[t, id_j] = g_j (m_j s_j - sum_k g_k m_k s_k)   (softmax over the
//                     kept logits, Eq. 4, with g_hat = g * m, Eq. 7)
//
// Kernels: one wave per token for the slot terms (dz, d_gate, and dz
// transposed in bf16 for the matrix cores, staged through LDS); dx as K weighted rows of W_mask
// per token (the K-sparse form of dz W_mask); dW_mask = dz^T x as a bf16 MFMA
// contraction over the tokens, split over token ranges whose float32
// partials are then added in a fixed order.
#include "common.h"
#include "kernels.h"

namespace beam {

namespace {

constexpr int BW_CHUNK = 128;   // tokens per dW k-chunk
constexpr int BW_LDT = BW_CHUNK + 8;  // LDS row pitch (bf16) of the transposed x chunk

constexpr int BS_T = 16;             // tokens per slot-term workgroup (one per wave)
constexpr int BS_LD = BS_T + 8;      // LDS row pitch (bf16) of the transposed dz group

// A workgroup of 16 waves takes BS_T consecutive tokens, one per wave; lane
// l owns experts l, l + 64, l + 128, l + 192.  dz and d_gate rows are written
// as they are made (consecutive lanes, consecutive experts); dz transposed
// (bf16, for the matrix cores) is collected in LDS as [expert][token of the
// group] and written out as 32-byte row pieces (two 16-byte stores) instead
// of one 2-byte store per expert and token.  Tokens t >= T (up to T_pad) only
// zero their dzT column.
__global__ __launch_bounds__(1024) void mask_bwd_slots(
    const int32_t *__restrict__ ids, const float *__restrict__ g, const uint8_t *__restrict__ m,
    const float *__restrict__ z, const float *__restrict__ sg, float beta, int T, int T_pad,
    int E, int E_pad, int K, float *__restrict__ dz, float *__restrict__ d_gate,
    bf16_t *__restrict__ dzT) {
    __shared__ __align__(16) bf16_t tS[256 * BS_LD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * BS_T;
    {
        const int tl = wave;
        const int t = t0 + tl;
        float dzv[4] = {0.f, 0.f, 0.f, 0.f}, dgv[4] = {0.f, 0.f, 0.f, 0.f};
        if (t < T) {
            const size_t rk = (size_t)t * K;
            float inner = 0.f;
            for (int k = 0; k < K; ++k) inner += g[rk + k] * (m[rk + k] ? sg[rk + k] : 0.f);
            for (int k = 0; k < K; ++k) {
                const int e = ids[rk + k];
                const float gk = g[rk + k], sk = sg[rk + k];
                const float dg = m[rk + k] ? sk : 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (lane + 64 * j == e) {
                        const float sgm = 1.f / (1.f + expf(-z[(size_t)t * E + e]));
                        dzv[j] = (gk * sk + beta) * sgm * (1.f - sgm);
                        dgv[j] = gk * (dg - inner);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                if (e < E) {
                    dz[(size_t)t * E + e] = dzv[j];
                    if (d_gate) d_gate[(size_t)t * E + e] = dgv[j];
                }
            }
        }
        if (dzT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                if (e < E_pad) tS[e * BS_LD + tl] = f32_to_bf16(dzv[j]);
            }
        }
    }
    if (!dzT) return;
    __syncthreads();
    // row e of the group: BS_T tokens = 2 pieces of 16 bytes (t0 + BS_T <= T_pad)
    for (int q = threadIdx.x; q < E_pad * (BS_T / 8); q += 1024) {
        const int e = q / (BS_T / 8), c = q - e * (BS_T / 8);
        *reinterpret_cast<u32x4 *>(dzT + (size_t)e * T_pad + t0 + c * 8) =
            *reinterpret_cast<const u32x4 *>(&tS[e * BS_LD + c * 8]);
    }
}

// dx[t, :] = sum_k dz[t, id_k] W_mask[id_k, :], k ascending; one workgroup per
// token, 8 channels per thread (bf16 weights) or 1 (float32).
__global__ __launch_bounds__(256) void mask_bwd_dx_bf16(const int32_t *__restrict__ ids,
                                                        const float *__restrict__ dz,
                                                        const bf16_t *__restrict__ Wm, int E,
                                                        int K, int d, float *__restrict__ dx) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < K; ++k) {
            const int e = ids[(size_t)t * K + k];
            const float w = dz[(size_t)t * E + e];
            const u32x4 v = ld16(Wm + (size_t)e * d + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(w, __uint_as_float(v[q] << 16), acc[2 * q]);
                acc[2 * q + 1] = fmaf(w, __uint_as_float(v[q] & 0xffff0000u), acc[2 * q + 1]);
            }
        }
        float *o = dx + (size_t)t * d + c;
        *reinterpret_cast<f32x4 *>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4 *>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
}

__global__ __launch_bounds__(256) void mask_bwd_dx_f32(const int32_t *__restrict__ ids,
                                                       const float *__restrict__ dz,
                                                       const float *__restrict__ Wm, int E, int K,
                                                       int d, float *__restrict__ dx) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < d; c += 256) {
        float acc = 0.f;
        for (int k = 0; k < K; ++k) {
            const int e = ids[(size_t)t * K + k];
            acc = fmaf(dz[(size_t)t * E + e], Wm[(size_t)e * d + c], acc);
        }
        dx[(size_t)t * d + c] = acc;
    }
}

// Partial dW_mask over one token range: rows = all E_pad = 16*MT experts,
// 64 channels per workgroup, four waves of 16 channels each.  A chunk of
// BW_CHUNK tokens x 64 channels of x is staged in LDS transposed (channel
// rows, token columns) so that an MFMA B fragment (8 consecutive tokens of
// one channel) is one 16-byte LDS read; A fragments (8 consecutive tokens of
// one expert) are 16-byte loads of dzT.  out: the split's [E, d] float32 slab.
template <int MT>
__global__ __launch_bounds__(256) void mask_bwd_dw(const bf16_t *__restrict__ dzT, int T_pad,
                                                   const bf16_t *__restrict__ x, int T, int d,
                                                   int E, int t_per_split,
                                                   float *__restrict__ out) {
    __shared__ __align__(16) bf16_t xs[64 * BW_LDT];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c0 = blockIdx.x * 64;
    const int t_begin = blockIdx.y * t_per_split;
    const int t_end = min(T_pad, t_begin + t_per_split);
    f32x4 acc[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = t_begin; t0 < t_end; t0 += BW_CHUNK) {
        // the chunk's A fragments (dz transposed: 8 consecutive tokens of one
        // expert per lane) are requested first, so they arrive while x is
        // staged
        u32x4 afr[BW_CHUNK / 32][MT];
#pragma unroll
        for (int ks = 0; ks < BW_CHUNK / 32; ++ks)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
                afr[ks][mb] = ld16(dzT + (size_t)(16 * mb + (lane & 15)) * T_pad + t0 + ks * 32 +
                                   8 * (lane >> 4));
        // stage x[t0 .. t0+127][c0 .. c0+63]: 4 rows of 8 channels per thread
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int tl = q * 32 + (tid >> 3);
            const int cl = (tid & 7) * 8;
            const int t = t0 + tl;
            const u32x4 v = t < T ? ld16(x + (size_t)t * d + c0 + cl) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[(cl + 2 * i) * BW_LDT + tl] = (bf16_t)(v[i] & 0xffffu);
                xs[(cl + 2 * i + 1) * BW_LDT + tl] = (bf16_t)(v[i] >> 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BW_CHUNK / 32; ++ks) {
            const int tk = ks * 32 + 8 * (lane >> 4);
            const u32x4 b = *reinterpret_cast<const u32x4 *>(
                &xs[(16 * wave + (lane & 15)) * BW_LDT + tk]);
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) acc[mb] = mfma16x16x32(afr[ks][mb], b, acc[mb]);
        }
        __syncthreads();
    }
    float *o = out + (size_t)blockIdx.y * E * d;
    const int c = c0 + 16 * wave + (lane & 15);
#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 16 * mb + 4 * (lane >> 4) + i;
            if (e < E) o[(size_t)e * d + c] = acc[mb][i];
        }
}

// dW = sum over splits of the partial slabs, split order.
__global__ __launch_bounds__(256) void mask_bwd_dw_reduce(const float *__restrict__ part,
                                                          int n_split, size_t n,
                                                          float *__restrict__ dW) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int q = 0; q < n_split; ++q) s += part[(size_t)q * n + i];
    dW[i] = s;
}

// float32 layer: dW[e, c] = sum_t dz[t, e] x[t, c], one thread per output.
__global__ __launch_bounds__(256) void mask_bwd_dw_f32(const float *__restrict__ dz,
                                                       const float *__restrict__ x, int T, int d,
                                                       int E, float *__restrict__ dW) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)E * d) return;
    const int e = (int)(i / d), c = (int)(i % d);
    float acc = 0.f;
    for (int t = 0; t < T; ++t) acc = fmaf(dz[(size_t)t * E + e], x[(size_t)t * d + c], acc);
    dW[i] = acc;
}

}  // namespace

BwdPlan mask_backward_plan(const Plan &p) {
    BwdPlan b{};
    b.T_pad = (p.T + BW_CHUNK - 1) / BW_CHUNK * BW_CHUNK;
    b.E_pad = (p.E + 15) / 16 * 16;
    const int n_chunks = b.T_pad / BW_CHUNK;
    const int n_ctiles = p.d / 64;
    int sk = n_chunks < 1 ? 1 : n_chunks;
    const int want = 512 / (n_ctiles > 0 ? n_ctiles : 1);  // ~2 workgroups per CU
    if (sk > want) sk = want > 1 ? want : 1;
    const int per = (n_chunks + sk - 1) / sk;
    b.n_split = per > 0 ? (n_chunks + per - 1) / per : 1;
    b.t_per_split = per * BW_CHUNK;
    size_t off = 0;
    b.off_dzT = off;
    if (p.dtype == 1) {
        off += (size_t)b.E_pad * b.T_pad * 2;
        off = (off + 255) / 256 * 256;
        b.off_part = off;
        if (b.n_split > 1) off += (size_t)b.n_split * p.E * p.d * 4;
    }
    b.bytes = (off + 255) / 256 * 256;
    return b;
}

hipError_t launch_mask_backward(const Plan &p, const BwdPlan &b, const void *x, const void *Wm,
                                const Routing &r, const float *sg, float beta, float *dz,
                                float *dW, float *dx, float *d_gate, void *ws, hipStream_t s) {
    char *wsb = static_cast<char *>(ws);
    bf16_t *dzT = (p.dtype == 1 && dW) ? reinterpret_cast<bf16_t *>(wsb + b.off_dzT) : nullptr;
    const int t_rows = dzT ? b.T_pad : p.T;
    // with dzT, t_rows = T_pad is a multiple of BW_CHUNK (so of BS_T)
    static_assert(BW_CHUNK % BS_T == 0, "whole slot groups per dW chunk");
    mask_bwd_slots<<<(t_rows + BS_T - 1) / BS_T, 1024, 0, s>>>(r.topk_ids, r.topk_weights, r.mask,
                                                    r.mask_logits, sg, beta, p.T, t_rows, p.E,
                                                    b.E_pad, p.K, dz, d_gate, dzT);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (dx) {
        if (p.dtype == 1)
            mask_bwd_dx_bf16<<<p.T, 256, 0, s>>>(r.topk_ids, dz, (const bf16_t *)Wm, p.E, p.K, p.d,
                                                 dx);
        else
            mask_bwd_dx_f32<<<p.T, 256, 0, s>>>(r.topk_ids, dz, (const float *)Wm, p.E, p.K, p.d,
                                                dx);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (dW) {
        if (p.dtype == 1) {
            float *out = b.n_split > 1 ? reinterpret_cast<float *>(wsb + b.off_part) : dW;
            const dim3 grid(p.d / 64, b.n_split);
#define BEAM_DW(MTV)                                                                         \
    mask_bwd_dw<MTV><<<grid, 256, 0, s>>>(dzT, b.T_pad, (const bf16_t *)x, p.T, p.d, p.E,     \
                                          b.t_per_split, out)
            switch (b.E_pad / 16) {
                case 1: BEAM_DW(1); break;
                case 2: BEAM_DW(2); break;
                case 3: BEAM_DW(3); break;
                case 4: BEAM_DW(4); break;
                case 5: BEAM_DW(5); break;
                case 6: BEAM_DW(6); break;
                case 7: BEAM_DW(7); break;
                case 8: BEAM_DW(8); break;
                case 9: BEAM_DW(9); break;
                case 10: BEAM_DW(10); break;
                case 11: BEAM_DW(11); break;
                case 12: BEAM_DW(12); break;
                case 13: BEAM_DW(13); break;
                case 14: BEAM_DW(14); break;
                case 15: BEAM_DW(15); break;
                default: BEAM_DW(16); break;
            }
#undef BEAM_DW
            if ((err = hipGetLastError()) != hipSuccess) return err;
            if (b.n_split > 1) {
                const size_t n = (size_t)p.E * p.d;
                mask_bwd_dw_reduce<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(out, b.n_split, n,
                                                                               dW);
            }
        } else {
            const size_t n = (size_t)p.E * p.d;
            mask_bwd_dw_f32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dz, (const float *)x,
                                                                        p.T, p.d, p.E, dW);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace beam
