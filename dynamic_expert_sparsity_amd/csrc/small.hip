// The down projection and combine of a decode batch of at most
// SMALL_DECODE_T tokens (its up projection runs with the routing, in
// router.hip).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// Down projection and combine of a decode batch of at most SMALL_DECODE_T
// tokens (Eq. 3 and Eq. 8), token-major: each workgroup owns one token t and
// a range of C output channels.  With one token every workgroup takes it;
// with more, the G workgroups are dealt out in proportion to the tokens' slot
// counts n_t (the S shared experts plus the active routed slots): token t
// gets 1 + floor((G - T) n_t / W) of them, W the sum of the n_t, so a token
// with many active slots does not hold up the launch (with an equal share
// per token its workgroups took several times as long as the others').  The
// token's slots (its S shared experts with weight 1, then its active routed
// slots k in order with weight g_hat) and their h rows are staged in LDS.
// The items (slot q, channel c) are spread over the waves, eight at a time
// per wave with every row piece requested before any arithmetic: each
// streams row c of the slot's W_dt (16-byte loads), dots it with the slot's
// h row and sums the lanes in a fixed order into o[q][c] in LDS.  Then each
// channel adds its slots in slot order (float32, no atomics) and writes
// y[t][c].  With a few tokens the experts' rows are read once per token that
// uses them, about once per active expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void down_small(int T, int K, int S, int E, int d, int I,
                                                  const int32_t *__restrict__ masked_ids,
                                                  const float *__restrict__ g_hat,
                                                  const int32_t *__restrict__ pair_pos,
                                                  const bf16_t *__restrict__ h,
                                                  const bf16_t *__restrict__ Wdt,
                                                  bf16_t *__restrict__ y) {
    __shared__ int s_e[SMALL_SLOTS], s_pos[SMALL_SLOTS];
    __shared__ float s_w[SMALL_SLOTS];
    __shared__ int s_n, s_t, s_grp, s_ng;
    // [slots][I] bf16 h rows, then [slots][per] float slot outputs
    extern __shared__ __align__(16) unsigned char dyn[];
    u32x4 *hs = reinterpret_cast<u32x4 *>(dyn);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x;
    int t = 0, grp = blockIdx.x, ng = G;
    if (T > 1) {
        if (tid < 64) {
            // lane u < T: the active routed slots of token u (T * K <= 128)
            int cnt = 0;
            for (int c0 = 0; c0 < T * K; c0 += 64) {
                const int l = c0 + lane;
                const unsigned long long bal = __ballot(l < T * K && masked_ids[l] >= 0);
                const int lo = max(lane * K - c0, 0), hi = min(lane * K + K - c0, 64);
                if (lane < T && hi > lo)
                    cnt += __popcll((bal >> lo) &
                                    (hi - lo >= 64 ? ~0ull : (1ull << (hi - lo)) - 1ull));
            }
            int W = 0;
            for (int u = 0; u < T; ++u) W += S + __builtin_amdgcn_readlane(cnt, u);
            int first = 0, tt = -1, gg = 0, nn = 0;
            for (int u = 0; u < T; ++u) {
                const int n = S + __builtin_amdgcn_readlane(cnt, u);
                const int g = 1 + (W > 0 ? (int)((long long)(G - T) * n / W) : 0);
                if (tt < 0 && (int)blockIdx.x < first + g) {
                    tt = u;
                    gg = (int)blockIdx.x - first;
                    nn = g;
                }
                first += g;
            }
            if (lane == 0) {
                s_t = tt;
                s_grp = gg;
                s_ng = nn;
            }
        }
        __syncthreads();
        t = s_t;
        grp = s_grp;
        ng = s_ng;
        if (t < 0) return;  // beyond the dealt workgroups (the whole workgroup)
    }
    const int per = (d + ng - 1) / ng;
    float *so = reinterpret_cast<float *>(dyn + (size_t)(K + S) * I * 2);
    if (tid < 64) {
        // lane l < S: shared expert l (weight 1); S <= l < S + K: routed slot
        // l - S (its expert id, or -1 if masked); every lane loads its own
        // slot at once, and the active ones are packed in slot order
        int e = -1, pos = 0;
        float wgt = 1.f;
        if (lane < S) {
            e = E + lane;
            pos = pair_pos[T * K + t * S + lane];
        } else if (lane < S + K) {
            const int k = lane - S;
            e = masked_ids[t * K + k];
            if (e >= 0) {
                pos = pair_pos[t * K + k];
                wgt = g_hat[t * K + k];
            }
        }
        const unsigned long long act = __ballot(e >= 0);
        if (e >= 0) {
            const int idx = __popcll(act & ((1ull << lane) - 1ull));
            s_e[idx] = e;
            s_pos[idx] = pos;
            s_w[idx] = wgt;
        }
        if (lane == 0) s_n = __popcll(act);
    }
    __syncthreads();
    const int n = s_n;
    const int nch = I >> 3;  // 16-byte chunks per row
    const int c_begin = grp * per, c_end = min(d, c_begin + per);
    const int C = c_end > c_begin ? c_end - c_begin : 0;
    const int n_items = n * C;
    // IU items per wave at a time, every row piece requested before any
    // arithmetic; a batch's rows are requested before the previous batch's
    // arithmetic (the first batch before the h rows are staged).  Many items:
    // IU = 8 consecutive ones per wave (items i0 + u, i0 = 8 w + 64 j).  At
    // most 16 (a token's few slots over a short channel range): IU = 2 dealt
    // to the waves in turn (items i0 + 8 u, i0 = w + 16 j), so a wave issues
    // row pieces for at most one missing item.  Every load is issued (past
    // the end: item i0 / the row's first chunk again, in bounds and unused),
    // so the compiler keeps all of them in flight.
    const int ch0 = lane < nch ? lane : 0;
    const int ch1 = lane + 64 < nch ? lane + 64 : 0;
    auto run = [&](auto IUC, auto STC) {
        constexpr int IU = decltype(IUC)::value, ST = decltype(STC)::value;
        u32x4 wv[IU][2];
        int qv[IU], cv[IU];
        auto request = [&](int i0) {
#pragma unroll
            for (int u = 0; u < IU; ++u) {
                const int it = i0 + ST * u < n_items ? i0 + ST * u : i0;
                qv[u] = it / C;
                cv[u] = c_begin + (it - qv[u] * C);
                const bf16_t *wr = Wdt + ((size_t)s_e[qv[u]] * d + cv[u]) * I;
                wv[u][0] = ld16_stream(wr + (size_t)ch0 * 8);
                wv[u][1] = ld16_stream(wr + (size_t)ch1 * 8);
            }
        };
        int i0 = ST == 1 ? wave * IU : wave;
        if (i0 < n_items) request(i0);
        for (int i = tid; i < n * nch; i += 512) {
            const int q = i / nch, ch = i - q * nch;
            hs[i] = ld16(h + (size_t)s_pos[q] * I + (size_t)ch * 8);
        }
        __syncthreads();
        for (; i0 < n_items; i0 += 8 * IU) {
            u32x4 cur[IU][2];
            int qc[IU], cc_[IU];
#pragma unroll
            for (int u = 0; u < IU; ++u) {
                cur[u][0] = wv[u][0];
                cur[u][1] = wv[u][1];
                qc[u] = qv[u];
                cc_[u] = cv[u];
            }
            if (i0 + 8 * IU < n_items) request(i0 + 8 * IU);
#pragma unroll
            for (int u = 0; u < IU; ++u) {
                const int q = qc[u], c = cc_[u];
                float part = 0.f;
                if (lane < nch) part = dot8_bf16(cur[u][0], hs[q * nch + lane], part);
                if (lane + 64 < nch) part = dot8_bf16(cur[u][1], hs[q * nch + lane + 64], part);
                // a row longer than 128 chunks: the rest, one piece at a time
                const bf16_t *wr = Wdt + ((size_t)s_e[q] * d + c) * I;
                for (int ch = lane + 128; ch < nch; ch += 64)
                    part = dot8_bf16(ld16_stream(wr + (size_t)ch * 8), hs[q * nch + ch], part);
                const float o = wave_sum(part);
                if (lane == 0 && i0 + ST * u < n_items) so[q * per + (c - c_begin)] = o;
            }
        }
    };
    if (n_items <= 16)
        run(std::integral_constant<int, 2>{}, std::integral_constant<int, 8>{});
    else
        run(std::integral_constant<int, 8>{}, std::integral_constant<int, 1>{});
    __syncthreads();
    for (int cc = tid; cc < C; cc += 512) {
        float acc = 0.f;
        for (int q = 0; q < n; ++q) {
            const float o = so[q * per + cc];
            acc = q < S ? acc + o : fmaf(s_w[q], o, acc);
        }
        y[(size_t)t * d + c_begin + cc] = f32_to_bf16(acc);
    }
}

// LDS of down_small: the slots' h rows, and the slot outputs n_t x per_t.
// One token: per = ceil(d / G).  More: n_t ceil(d / g_t) with
// g_t = 1 + floor((G - T) n_t / W) > (G - T) n_t / W is below
// d W / (G - T) + n_t <= d T (K + S) / (G - T) + K + S.
static size_t down_small_lds(const Plan &p, int G) {
    const long long slots = p.K + p.S;
    const long long so = p.T == 1 ? slots * ((p.d + G - 1) / G)
                                  : (long long)p.d * p.T * slots / (G - p.T) + slots + 1;
    return (size_t)slots * p.I * 2 + (size_t)so * 4;
}

hipError_t launch_down_small(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                             void *y, hipStream_t s) {
    // about one workgroup per CU in all (two per CU measured 1-4 us slower
    // at 1-2 tokens); at least two per token
    const int G = std::max(device_cus(), 2 * p.T);
    const size_t lds = down_small_lds(p, G);
    if (lds > 64 * 1024) {
        static std::once_flag once;
        static hipError_t attr_err = hipSuccess;
        std::call_once(once, [] {
            attr_err = hipFuncSetAttribute((const void *)down_small,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        });
        if (attr_err != hipSuccess) return attr_err;
    }
    down_small<<<G, 512, lds, s>>>(p.T, p.K, p.S, p.E, p.d, p.I, r.masked_ids, r.g_hat,
                                   w.pair_pos, (const bf16_t *)w.h, (const bf16_t *)W_dt,
                                   (bf16_t *)y);
    return hipGetLastError();
}

}  // namespace beam
