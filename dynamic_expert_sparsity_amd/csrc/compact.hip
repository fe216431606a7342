// a4: the pair scatter for large batches (the block-padded offsets and
// per-tile bases come from the routing kernel's compaction; see
// compact_dev.h).  One thread per pair.
#include "compact_dev.h"

namespace beam {

__global__ __launch_bounds__(256) void compact_scatter(Routing r,
                                                      const int32_t *__restrict__ tile_base,
                                                      const uint64_t *__restrict__ tile_mask,
                                                      int PT, int TK, int K, int E, int S,
                                                      int32_t *__restrict__ pair_pos,
                                                      int32_t *__restrict__ sorted_tok) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= PT) return;
    scatter_pair(p, p < TK ? r.masked_ids[p] : -1, K, TK, E, S, r, r.expert_offsets, tile_base,
                 tile_mask, pair_pos, sorted_tok);
}

hipError_t launch_scatter(const Plan &p, const Routing &r, const Work &w, hipStream_t s) {
    if (p.fuse_scatter) return hipSuccess;
    compact_scatter<<<(p.PT + 255) / 256, 256, 0, s>>>(r, w.tile_base, w.tile_mask, p.PT,
                                                       p.T * p.K, p.K, p.E, p.S, w.pair_pos,
                                                       w.sorted_tok);
    return hipGetLastError();
}

}  // namespace beam
