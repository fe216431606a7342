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
// Kernels (bf16 layers): the slot terms (16 lanes per token, one per slot:
// dz and d_gate rows, the compact [T, K] list of dz values, and dz
// transposed in bf16 for the matrix cores); dx as K weighted rows of W_mask
// per token (the K-sparse form of dz W_mask, float32 FMAs) from a slice of
// W_mask staged in LDS; dW_mask = dz^T x as a bf16 MFMA contraction over
// the tokens, both operands streamed into LDS in whole lines, split over
// token ranges whose float32 partials the dx launch (which runs after it)
// adds in a fixed order.
#include <mutex>

#include "common.h"
#include "gemm_dev.h"
#include "kernels.h"

namespace beam {

namespace {

constexpr int BS_T = 16;          // tokens per slot-term workgroup (waves of four tokens)
constexpr int BS_THREADS = BS_T * 16;
constexpr int BS_LD = BS_T + 8;   // LDS row pitch (bf16) of the transposed dz group
constexpr int DW_KT = 64;         // tokens per dW stage (one 128-byte line of a dz^T row)
constexpr int DW_CH = 128;        // channels per dW workgroup (four waves of 32)
constexpr int DX_WG = 256;        // dx workgroups aimed at (one per CU)

// channels per lane of the dx kernel: four (slices of 256) when d allows and
// E float32 rows of 1 KB fit in 128 KB of LDS, else two
inline int dx_cpl(const Plan &p) { return p.d % 256 == 0 && p.E <= 128 ? 4 : 2; }

// Slot terms.  A workgroup takes BS_T consecutive tokens, a wave four of
// them: the 16 lanes of a token hold its slots (lane i: slot i < K), so a
// token's loads go out together (ids, weights, mask and slot gradients,
// then the mask logits of its candidates) and the inner sum of d_gate is a
// 16-lane butterfly (fixed order, the same value in every lane).  The dense
// dz rows, then the d_gate rows, are assembled in LDS (zeros, then the K
// candidates) and stored as 16-byte pieces (4-byte ones when E % 4 != 0 or
// an output is not 16-byte aligned).  dzk: the [T, K] list of dz values (NULL: not written).
// dzT: dz transposed in bf16, [E_pad][T_pad] (NULL: not written); tokens t >= T
// (up to T_rows) only zero their column.
__global__ __launch_bounds__(BS_THREADS) void mask_bwd_slots(
    const int32_t *__restrict__ ids, const float *__restrict__ g, const uint8_t *__restrict__ m,
    const float *__restrict__ z, const float *__restrict__ sg, float beta, int T, int E,
    int E_pad, int K, int vec, float *__restrict__ dz, float *__restrict__ d_gate,
    float *__restrict__ dzk, bf16_t *__restrict__ dzT, int T_pad) {
    __shared__ __align__(16) float rows[BS_T][256];
    __shared__ __align__(16) bf16_t tS[256 * BS_LD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tl = wave * 4 + (lane >> 4);  // the group's token this lane works for
    const int i = lane & 15;                // its slot
    const int t = blockIdx.x * BS_T + tl;
    const bool tv = t < T, sv = tv && i < K;
    // lanes without a slot read slot 0 of token 0 (T >= 1) and use nothing
    const size_t o = sv ? (size_t)t * K + i : 0;
    const int id = ids[o];
    const float gk = g[o], sk = sg[o];
    const bool mk = m[o] != 0;
    const bool ok = sv && id >= 0 && id < E;
    const float zk = z[ok ? (size_t)t * E + id : 0];
    const float ms = sv && mk ? sk : 0.f;  // m_k s_k
    float inner = sv ? gk * ms : 0.f;
    inner += __shfl_xor(inner, 1, 16);
    inner += __shfl_xor(inner, 2, 16);
    inner += __shfl_xor(inner, 4, 16);
    inner += __shfl_xor(inner, 8, 16);
    const float sgm = 1.f / (1.f + expf(-zk));
    const float dzv = (gk * sk + beta) * sgm * (1.f - sgm);
    const float dgv = gk * (ms - inner);
    if (sv && dzk) dzk[o] = ok ? dzv : 0.f;

    float *row = rows[tl];
    // one dense row of the token per pass: pass 0 dz (kept in LDS for dzT),
    // pass 1 d_gate
    for (int pass = 0; pass < (d_gate ? 2 : 1); ++pass) {
        if (pass == 1) __syncthreads();  // every lane is done reading the dz rows
        for (int e = i; e < E_pad; e += 16) row[e] = 0.f;
        __syncthreads();
        if (ok) row[id] = pass == 0 ? dzv : dgv;
        __syncthreads();
        if (tv) {
            float *dst = (pass == 0 ? dz : d_gate) + (size_t)t * E;
            if (vec) {  // outputs only: non-temporal, like dx
                for (int c = i; c < E / 4; c += 16)
                    __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(row + 4 * c),
                                                reinterpret_cast<f32x4 *>(dst + 4 * c));
            } else {
                for (int e = i; e < E; e += 16) dst[e] = row[e];
            }
        }
        if (pass == 0 && dzT) {
            for (int e = i; e < E_pad; e += 16) tS[e * BS_LD + tl] = f32_to_bf16(row[e]);
        }
    }
    if (!dzT) return;
    __syncthreads();
    // row e of the group: BS_T tokens = BS_T / 8 pieces of 16 bytes
    for (int q = threadIdx.x; q < E_pad * (BS_T / 8); q += BS_THREADS) {
        const int e = q / (BS_T / 8), c = q - e * (BS_T / 8);
        *reinterpret_cast<u32x4 *>(dzT + (size_t)e * T_pad + blockIdx.x * BS_T + c * 8) =
            *reinterpret_cast<const u32x4 *>(&tS[e * BS_LD + c * 8]);
    }
}

// dx[t, :] = sum_k dz[t, id_k] W_mask[id_k, :], k ascending (float32 FMAs on
// the bf16 weights).  A workgroup of 16 waves takes a slice of 64 CPL
// channels and a range of tokens: the slice of every W_mask row is staged in
// LDS first, converted to float32 once (so the FMAs read their operands
// without a conversion each), then a wave takes groups of four tokens, lane
// 16 j + k holding slot k of the group's token j (its expert and dz from the
// compact list, loaded one group ahead); slot k of the four tokens is
// broadcast (readlane) and every lane adds its CPL channels of the four
// experts' rows (four independent LDS reads in flight).  Tokens of the group
// past the range take weight 0 and are not stored.
//
// The same launch adds the dW split partials (part, n_split slabs of n4
// 16-byte pieces; none when n_split <= 1) into dW, a contiguous share per
// workgroup, split order: those loads go out together with the W_mask slice.
constexpr int DX_THREADS = 1024;
template <int CPL>
__global__ __launch_bounds__(DX_THREADS) void mask_bwd_dx_bf16(
    const int32_t *__restrict__ ids, const float *__restrict__ dzk, const bf16_t *__restrict__ Wm,
    int T, int E, int K, int d, int tok_per_wg, float *__restrict__ dx,
    const float *__restrict__ part, int n_split, long long n4, float *__restrict__ dW) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int ROWF = 64 * CPL;         // float32 values of a row slice
    constexpr int PPR = ROWF / 8;          // 8-channel pieces per row slice
    constexpr int NW = DX_THREADS / 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = blockIdx.x * ROWF;
    const int t_begin = blockIdx.y * tok_per_wg;
    const int t_end = min(T, t_begin + tok_per_wg);
    float *Ws = reinterpret_cast<float *>(lds);  // [E][ROWF]

    // the slice: piece q = (row, 8 channels), eight requested at a time
    const int npc = E * PPR;
    for (int q0 = threadIdx.x; q0 < npc; q0 += 8 * DX_THREADS) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = min(q0 + j * DX_THREADS, npc - 1);
            const int row = q / PPR, pc = q - row * PPR;
            v[j] = ld16(Wm + (size_t)row * d + c0 + pc * 8);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = q0 + j * DX_THREADS;
            if (q < npc) {
                float *dst = Ws + (size_t)q * 8;  // row * ROWF + pc * 8
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *reinterpret_cast<f32x4 *>(dst + 4 * h) =
                        f32x4{__uint_as_float(v[j][2 * h] << 16),
                              __uint_as_float(v[j][2 * h] & 0xffff0000u),
                              __uint_as_float(v[j][2 * h + 1] << 16),
                              __uint_as_float(v[j][2 * h + 1] & 0xffff0000u)};
            }
        }
    }
    if (n_split > 1) {
        const long long nwg = (long long)gridDim.x * gridDim.y;
        const long long wg = (long long)blockIdx.y * gridDim.x + blockIdx.x;
        const long long share = (n4 + nwg - 1) / nwg;
        const long long i_end = min(n4, (wg + 1) * share);
        const f32x4 *pp = reinterpret_cast<const f32x4 *>(part);
        for (long long i = wg * share + threadIdx.x; i < i_end; i += DX_THREADS) {
            // eight partials requested at a time, then added in split order
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int q0 = 0; q0 < n_split; q0 += 8) {
                f32x4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[j] = pp[(size_t)min(q0 + j, n_split - 1) * n4 + i];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (q0 + j < n_split) acc = q0 + j == 0 ? v[j] : acc + v[j];
            }
            reinterpret_cast<f32x4 *>(dW)[i] = acc;
        }
    }
    __syncthreads();

    // a group's (expert, dz) pairs, loaded one group ahead of their use (both
    // loads unconditional, from a clamped index; invalid slots become weight
    // 0 on expert 0 by selects, so no branch holds the loads back)
    auto pair_index = [&](int q0) -> size_t {
        const int t = q0 + (lane >> 4), k = lane & 15;
        return t < t_end && k < K ? (size_t)t * K + k : 0;
    };
    int e_nx = 0;
    float w_nx = 0.f;
    if (t_begin + 4 * wave < t_end) {
        const size_t o = pair_index(t_begin + 4 * wave);
        e_nx = ids[o];
        w_nx = dzk[o];
    }
    for (int q0 = t_begin + 4 * wave; q0 < t_end; q0 += 4 * NW) {
        const bool v = q0 + (lane >> 4) < t_end && (lane & 15) < K;
        const bool ok = v && e_nx >= 0 && e_nx < E;
        const int e = ok ? e_nx : 0;
        const float w = ok ? w_nx : 0.f;
        if (q0 + 4 * NW < t_end) {
            const size_t o = pair_index(q0 + 4 * NW);
            e_nx = ids[o];
            w_nx = dzk[o];
        }
        float acc[4][CPL];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[j][c] = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            float wv[4][CPL];
            float wk[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ek = __builtin_amdgcn_readlane(e, 16 * j + kk);
                wk[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), 16 * j + kk));
                const float *row = Ws + ek * ROWF + lane * CPL;
                if constexpr (CPL == 4) {
                    const f32x4 r4 = *reinterpret_cast<const f32x4 *>(row);
#pragma unroll
                    for (int c = 0; c < 4; ++c) wv[j][c] = r4[c];
                } else {
                    const float2 r2 = *reinterpret_cast<const float2 *>(row);
                    wv[j][0] = r2.x;
                    wv[j][1] = r2.y;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[j][c] = fmaf(wk[j], wv[j][c], acc[j][c]);
        }
        const int nj = min(4, t_end - q0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= nj) break;
            // dx is read by nothing here: non-temporal stores keep its 4 T d
            // bytes from displacing the slice and pairs in the L2 (T = 2048:
            // 25.5 -> 24.4 us per call; 8192: 41.1 -> 40.4)
            float *out = dx + (size_t)(q0 + j) * d + c0 + lane * CPL;
            if constexpr (CPL == 4)
                __builtin_nontemporal_store(f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]},
                                            reinterpret_cast<f32x4 *>(out));
            else
                __builtin_nontemporal_store(f32x2{acc[j][0], acc[j][1]},
                                            reinterpret_cast<f32x2 *>(out));
        }
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

// Partial dW_mask over one token range: all 16 MT expert rows (E rounded up
// to 32) x DW_CH channels per workgroup, four waves of 32 channels each.  The
// range streams through a ring of NS = 3 LDS stages of DW_KT tokens (one in
// flight behind the one being read and the one being refilled; deeper rings
// measured slower, 15.5 against 14.1 us at 8192 tokens): dz^T
// rows (128 bytes each, 16-byte piece c of row r at slot c ^ f(r)) and x rows
// (DW_CH channels = 256 bytes; piece c of token row r at slot c ^ 2((r / 8)
// % 4)), both fetched as whole lines by global_load_lds and waited for with
// explicit vmcnt counts.  An MFMA A fragment (8 tokens of one expert) is one
// 16-byte LDS read; a B fragment (8 tokens of one channel) is 8 two-byte
// reads of a column of the x rows, which the slot rotation spreads over the
// banks.  Expert rows past the dz^T rows and token rows past T lie outside
// their buffer resources and read as zero.  out: the split's [E, d] float32
// slab.
template <int MT>
struct DwCfg {
    static constexpr int A_BYTES = MT * 16 * DW_KT * 2;
    static constexpr int B_BYTES = DW_KT * DW_CH * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int NS = 3;
    static constexpr int LDS = NS * STAGE;
    static constexpr int L = (A_BYTES + B_BYTES) / 4096;  // 1 KB wave loads per wave per stage
    static_assert(NS >= 3 && NS * STAGE <= 160 * 1024, "a ring of at least three stages");
    static_assert((NS - 2) * L < 64, "vmcnt range");
};

// wait until at most `ahead` stages of STEP loads each are in flight
// (ahead <= N, wave-uniform)
template <int N, int STEP>
__device__ __forceinline__ void dw_wait_stages(int ahead) {
    if constexpr (N == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= N) wait_vmcnt<N * STEP>();
        else dw_wait_stages<N - 1, STEP>(ahead);
    }
}

template <int MT>
__global__ __launch_bounds__(256) void mask_bwd_dw(const bf16_t *__restrict__ dzT, int T_pad,
                                                   int E_pad, const bf16_t *__restrict__ x, int T,
                                                   int d, int E, int t_per_split,
                                                   float *__restrict__ out) {
    static_assert(MT % 2 == 0 && MT <= 16, "expert rows in whole 32-row groups");
    using C = DwCfg<MT>;
    constexpr int A_BYTES = C::A_BYTES;
    constexpr int STAGE = C::STAGE;
    constexpr int NS = C::NS;
    constexpr int LA = A_BYTES / 4096;  // 1 KB wave loads of A per wave per stage
    constexpr int LB = C::B_BYTES / 4096;
    constexpr int L = LA + LB;
    extern __shared__ __align__(16) unsigned char lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = blockIdx.x * DW_CH;
    const int t_begin = blockIdx.y * t_per_split;
    const int t_end = min(T_pad, t_begin + t_per_split);
    const int nst = (t_end - t_begin) / DW_KT;
    const rsrc_t ra =
        make_rsrc(dzT + t_begin, (uint32_t)((size_t)E_pad * T_pad * 2 - (size_t)t_begin * 2));
    const int xrows = max(0, min(T, t_end) - t_begin);
    const rsrc_t rx = make_rsrc(x + (size_t)t_begin * d, (uint32_t)((size_t)xrows * d * 2));

    // A load u = wave + 4 i: rows 8 u .. 8 u + 7, lane l fetching piece
    // (l % 8) ^ f(row) of row 8 u + l / 8; B load u: token rows 4 u .. 4 u + 3,
    // lane l fetching piece (l % 16) ^ 2((row / 8) % 4) of row 4 u + l / 16
    uint32_t offA[LA], offB[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int r = 8 * (wave + 4 * i) + (lane >> 3);
        offA[i] = (uint32_t)r * (uint32_t)T_pad * 2u + (uint32_t)(((lane & 7) ^ swz_f(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int r = 4 * (wave + 4 * i) + (lane >> 4);
        offB[i] = (uint32_t)r * (uint32_t)d * 2u + (uint32_t)(c0 * 2) +
                  (uint32_t)(((lane & 15) ^ (2 * ((r >> 3) & 3))) * 16);
    }
    auto issue = [&](int ts) {
        unsigned char *sa = lds + (ts % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            lds_dma16_buf<0>(ra, offA[i], (uint32_t)(ts * DW_KT * 2), sa + (wave + 4 * i) * 1024);
#pragma unroll
        for (int i = 0; i < LB; ++i)
            lds_dma16_buf<0>(rx, offB[i], (uint32_t)ts * (uint32_t)(DW_KT * d * 2),
                             sa + A_BYTES + (wave + 4 * i) * 1024);
    };

    f32x4 acc[MT][2];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this lane's B column: channel cl of the workgroup's slice; its rows of a
    // fragment all lie in one 8-row group (g = lane / 16), so one slot offset
    const int grp = lane >> 4;
    int boff[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int cl = 32 * wave + 16 * nb + (lane & 15);
        boff[nb] = (((cl >> 3) ^ (2 * grp)) << 4) + (cl & 7) * 2;
    }

    const int npro = min(NS - 1, nst);
    for (int ts = 0; ts < npro; ++ts) issue(ts);
    for (int ts = 0; ts < nst; ++ts) {
        dw_wait_stages<NS - 2, L>(min(NS - 2, nst - 1 - ts));
        // every wave's loads of stage ts have landed, and every wave is done
        // reading stage ts - 1, whose buffers the loads of ts + NS - 1 reuse
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ts + NS - 1 < nst) issue(ts + NS - 1);
        const unsigned char *sa = lds + (ts % NS) * STAGE;
        const unsigned char *sb = sa + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < DW_KT / 32; ++ks) {
            const int pc = 4 * ks + grp;
            u32x4 a[MT], b[2];
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
                a[mb] = *reinterpret_cast<const u32x4 *>(sa + swz(16 * mb + (lane & 15), pc));
            const unsigned char *rb = sb + (32 * ks + 8 * grp) * (DW_CH * 2);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                uint32_t hv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    hv[j] = *reinterpret_cast<const uint16_t *>(rb + j * (DW_CH * 2) + boff[nb]);
                b[nb] = u32x4{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                              hv[6] | (hv[7] << 16)};
            }
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma16x16x32(a[mb], b[nb], acc[mb][nb]);
        }
    }
    float *o = out + (size_t)blockIdx.y * E * d;
#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int c = c0 + 32 * wave + 16 * nb + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 16 * mb + 4 * grp + i;
                if (e < E) o[(size_t)e * d + c] = acc[mb][nb][i];
            }
        }
}

// dW = sum over splits of the partial slabs, split order (16 bytes per
// thread): for calls that ask for dW but not dx (else the dx launch adds them).
__global__ __launch_bounds__(256) void mask_bwd_dw_reduce(const float *__restrict__ part,
                                                          int n_split, size_t n4,
                                                          float *__restrict__ dW) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(part);
    f32x4 s = p[i];
    for (int q = 1; q < n_split; ++q) s += p[(size_t)q * n4 + i];
    reinterpret_cast<f32x4 *>(dW)[i] = s;
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

template <typename K_>
static hipError_t set_lds(K_ kernel, int bytes, std::once_flag &once, hipError_t &err) {
    std::call_once(once, [&] {
        err = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  bytes);
    });
    return err;
}

template <int CPL>
hipError_t launch_dx(const Plan &p, const BwdPlan &b, const Routing &r, const float *dzk,
                     const void *Wm, float *dx, const float *part, int n_split, float *dW,
                     hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    // the float32 slice of every W_mask row: at most 128 KB (the caller picks CPL)
    if (set_lds(mask_bwd_dx_bf16<CPL>, 128 * 1024, once, attr) != hipSuccess) return attr;
    const int lds = p.E * 64 * CPL * 4;
    const dim3 grid(p.d / (64 * CPL), (p.T + b.dx_tok - 1) / b.dx_tok);
    mask_bwd_dx_bf16<CPL><<<grid, DX_THREADS, lds, s>>>(r.topk_ids, dzk, (const bf16_t *)Wm, p.T,
                                                        p.E, p.K, p.d, b.dx_tok, dx, part,
                                                        n_split, (long long)p.E * p.d / 4, dW);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_dw(const Plan &p, const BwdPlan &b, const bf16_t *dzT, const void *x,
                     float *out, hipStream_t s) {
    constexpr int lds = DwCfg<MT>::LDS;
    static_assert(lds <= 160 * 1024, "LDS budget");
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    if (set_lds(mask_bwd_dw<MT>, lds, once, attr) != hipSuccess) return attr;
    const dim3 grid(p.d / DW_CH, b.n_split);
    mask_bwd_dw<MT><<<grid, 256, lds, s>>>(dzT, b.T_pad, b.E_pad, (const bf16_t *)x, p.T, p.d,
                                           p.E, b.t_per_split, out);
    return hipGetLastError();
}

}  // namespace

BwdPlan mask_backward_plan(const Plan &p) {
    BwdPlan b{};
    b.T_pad = (p.T + DW_KT - 1) / DW_KT * DW_KT;
    b.E_pad = (p.E + 15) / 16 * 16;
    // dW: token ranges of at least four stages, at most 16 of them (16
    // channel slices of 128 at d = 2048: up to 256 workgroups); a range's
    // x rows stay below 2^31 bytes (32-bit buffer offsets)
    const int n_chunks = b.T_pad / DW_KT;
    int sk = n_chunks / 4;
    sk = sk < 1 ? 1 : sk > 16 ? 16 : sk;
    int per = (n_chunks + sk - 1) / sk;
    const long long max_per = (1ll << 31) / ((long long)DW_KT * p.d * 2);
    if (per > max_per) per = (int)(max_per > 0 ? max_per : 1);
    b.n_split = per > 0 ? (n_chunks + per - 1) / per : 1;
    b.t_per_split = per * DW_KT;
    // dx: token ranges (multiples of 16) giving about DX_WG workgroups
    const int slices = p.d / (64 * dx_cpl(p));
    long long tok = ((long long)p.T * (slices > 0 ? slices : 1) + DX_WG - 1) / DX_WG;
    tok = (tok + 15) / 16 * 16;
    b.dx_tok = (int)(tok < 16 ? 16 : tok);
    size_t off = 0;
    if (p.dtype == 1) {
        b.off_dzT = off;
        off += (size_t)b.E_pad * b.T_pad * 2;
        off = (off + 255) / 256 * 256;
        b.off_dzk = off;
        off += (size_t)p.T * p.K * 4;
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
    const bool bf16 = p.dtype == 1;
    bf16_t *dzT = (bf16 && dW) ? reinterpret_cast<bf16_t *>(wsb + b.off_dzT) : nullptr;
    float *dzk = (bf16 && dx) ? reinterpret_cast<float *>(wsb + b.off_dzk) : nullptr;
    // with dzT every token column up to T_pad (a multiple of BS_T) is written
    static_assert(DW_KT % BS_T == 0, "whole slot groups per dW stage");
    const int t_rows = dzT ? b.T_pad : p.T;
    const bool al16 = ((uintptr_t)dz % 16 == 0) && (!d_gate || (uintptr_t)d_gate % 16 == 0);
    const int vec = (p.E % 4 == 0) && al16 ? 1 : 0;
    mask_bwd_slots<<<(t_rows + BS_T - 1) / BS_T, BS_THREADS, 0, s>>>(
        r.topk_ids, r.topk_weights, r.mask, r.mask_logits, sg, beta, p.T, p.E, b.E_pad, p.K, vec,
        dz, d_gate, dzk, dzT, b.T_pad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // bf16: dW (its split partials) first, then dx, whose launch also adds the partials
    const float *part = nullptr;
    int n_split = 0;
    if (dW) {
        if (bf16) {
            float *out = b.n_split > 1 ? reinterpret_cast<float *>(wsb + b.off_part) : dW;
            switch ((p.E + 31) / 32) {
                case 1: err = launch_dw<2>(p, b, dzT, x, out, s); break;
                case 2: err = launch_dw<4>(p, b, dzT, x, out, s); break;
                case 3: err = launch_dw<6>(p, b, dzT, x, out, s); break;
                case 4: err = launch_dw<8>(p, b, dzT, x, out, s); break;
                case 5: err = launch_dw<10>(p, b, dzT, x, out, s); break;
                case 6: err = launch_dw<12>(p, b, dzT, x, out, s); break;
                case 7: err = launch_dw<14>(p, b, dzT, x, out, s); break;
                default: err = launch_dw<16>(p, b, dzT, x, out, s); break;
            }
            if (err != hipSuccess) return err;
            if (b.n_split > 1) {
                part = out;
                n_split = b.n_split;
                if (!dx) {
                    const size_t n4 = (size_t)p.E * p.d / 4;
                    mask_bwd_dw_reduce<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(
                        part, n_split, n4, dW);
                }
            }
        } else {
            const size_t n = (size_t)p.E * p.d;
            mask_bwd_dw_f32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dz, (const float *)x,
                                                                        p.T, p.d, p.E, dW);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (dx) {
        if (bf16)
            err = dx_cpl(p) == 4 ? launch_dx<4>(p, b, r, dzk, Wm, dx, part, n_split, dW, s)
                                 : launch_dx<2>(p, b, r, dzk, Wm, dx, part, n_split, dW, s);
        else
            mask_bwd_dx_f32<<<p.T, 256, 0, s>>>(r.topk_ids, dz, (const float *)Wm, p.E, p.K, p.d,
                                                dx);
        if (err != hipSuccess || (err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace beam
