// Routing statistics on the device: per rank (slot k = k-th largest router
// logit) the tokens whose slot is masked, the histogram of active slots per
// token, and the active pairs of each expert.  These are the quantities the
// paper's analysis of the learned mask reports (news article on the paper,
// section 7: mask probability by expert rank, activated experts per token,
// expert load), accumulated over any number of calls.
#include "kernels.h"

namespace beam {

namespace {

// Grid-stride over tokens; each workgroup counts into LDS, then adds its
// non-zero bins to the caller's 64-bit counters.
__global__ __launch_bounds__(256) void routing_stats(const uint8_t *__restrict__ mask,
                                                     const int32_t *__restrict__ masked_ids,
                                                     int T, int K, int E,
                                                     unsigned long long *__restrict__ rank_masked,
                                                     unsigned long long *__restrict__ active_hist,
                                                     unsigned long long *__restrict__ expert_load) {
    __shared__ unsigned s_rank[16];
    __shared__ unsigned s_hist[17];
    __shared__ unsigned s_load[256];
    const int tid = threadIdx.x;
    if (tid < 16) s_rank[tid] = 0u;
    if (tid < 17) s_hist[tid] = 0u;
    s_load[tid] = 0u;
    __syncthreads();
    for (int t = blockIdx.x * 256 + tid; t < T; t += gridDim.x * 256) {
        int n_active = 0;
        for (int k = 0; k < K; ++k) {
            const int p = t * K + k;
            if (mask[p]) {
                ++n_active;
                const int e = masked_ids[p];
                if ((unsigned)e < (unsigned)E) atomicAdd(&s_load[e], 1u);
            } else {
                atomicAdd(&s_rank[k], 1u);
            }
        }
        atomicAdd(&s_hist[n_active], 1u);
    }
    __syncthreads();
    if (rank_masked && tid < K && s_rank[tid]) atomicAdd(&rank_masked[tid], (unsigned long long)s_rank[tid]);
    if (active_hist && tid <= K && s_hist[tid]) atomicAdd(&active_hist[tid], (unsigned long long)s_hist[tid]);
    if (expert_load && tid < E && s_load[tid]) atomicAdd(&expert_load[tid], (unsigned long long)s_load[tid]);
}

}  // namespace

hipError_t launch_stats(const Plan &p, const Routing &r, uint64_t *rank_masked,
                        uint64_t *active_hist, uint64_t *expert_load, hipStream_t s) {
    int blocks = (p.T + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    routing_stats<<<blocks, 256, 0, s>>>(r.mask, r.masked_ids, p.T, p.K, p.E,
                                         (unsigned long long *)rank_masked,
                                         (unsigned long long *)active_hist,
                                         (unsigned long long *)expert_load);
    return hipGetLastError();
}

}  // namespace beam
