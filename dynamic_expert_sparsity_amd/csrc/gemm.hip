// The tiled path's expert kernel and its launchers: one launch per
// projection runs the kernel family the compaction picked for the call (the
// streaming bodies of ring_dev.h or the grouped GEMM of gemm_dev.h).
#include <mutex>

#include "gemm_dev.h"
#include "ring_dev.h"

namespace beam {

static int persistent_wgs() {
    static int n = 0;
    static std::once_flag once;
    std::call_once(once, [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            n = cus;
        n = n >= 8 ? n / 8 * 8 : 256;
    });
    return n;
}

static GemmArgs base_args(const Plan &p, const Routing &r, const Work &w) {
    GemmArgs a{};
    a.block_expert = r.block_expert;
    a.num_active = r.num_active;
    a.sorted_tok = w.sorted_tok;
    a.expert_offsets = r.expert_offsets;
    a.expert_counts = r.expert_counts;
    a.mode = w.meta;
    a.pbt = w.pbt;
    a.T = p.T;
    a.d = p.d;
    a.I = p.I;
    a.E = p.E;
    return a;
}

// The tiled path's expert kernel for one projection.  The compaction wrote
// the call's kernel family in the record mode[0] (0: the streaming bodies,
// one or two column groups per unit by mode[3]; 1: 128-row tiles; 2: 256-row
// tiles), so one launch per projection serves every family (the choice is
// made on the device, from the routed counts, with no host round trip).
struct RingArgs {
    const bf16_t *A, *W;
    const int32_t *pbt, *mrec, *sorted_tok;
    bf16_t *out;
    int klen, ncols;
};
using Tile128 = GemmCfg<128, 3, 3, G_DKK128, G_WT128>;
using Tile256 = GemmCfg<GBM, 2, 3, G_DKK, 64>;
static_assert(Tile128::NW == 8 && Tile256::NW == 8, "one workgroup shape for every family");
constexpr int TILED_LDS = RING_LDS > Tile256::LDS_BYTES
                              ? (RING_LDS > Tile128::LDS_BYTES ? RING_LDS : Tile128::LDS_BYTES)
                              : (Tile256::LDS_BYTES > Tile128::LDS_BYTES ? Tile256::LDS_BYTES
                                                                         : Tile128::LDS_BYTES);
static_assert(TILED_LDS <= 160 * 1024, "LDS budget");

template <bool DOWN, bool TAIL>
__global__ __launch_bounds__(512, 1) void expert_tiled(GemmArgs g, RingArgs q) {
    constexpr int MODE = DOWN ? MODE_DOWN : MODE_UP;
    const int family = g.mode[0];
    if (family == 0) {
        if (g.mode[3])
            ring2_body<DOWN, TAIL>(q.A, q.W, q.pbt, q.mrec, q.sorted_tok, q.out, q.klen, q.ncols, 0);
        else
            ring1_body<DOWN, TAIL>(q.A, q.W, q.pbt, q.mrec, q.sorted_tok, q.out, q.klen, q.ncols, 0);
    } else if (family == 1) {
        gemm_body<MODE, 128, 3, 3, G_DKK128, G_WT128>(g);
    } else {
        gemm_body<MODE, GBM, 2, 3, G_DKK, 64>(g);
    }
}

template <bool DOWN, bool TAIL>
static hipError_t launch_tiled_t(const GemmArgs &a, const RingArgs &q, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [] {
        attr_err = hipFuncSetAttribute((const void *)expert_tiled<DOWN, TAIL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, TILED_LDS);
    });
    if (attr_err != hipSuccess) return attr_err;
    expert_tiled<DOWN, TAIL><<<persistent_wgs(), 512, TILED_LDS, s>>>(a, q);
    return hipGetLastError();
}

hipError_t launch_tiled_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                           const Work &w, hipStream_t s) {
    GemmArgs a = base_args(p, r, w);
    a.A = (const bf16_t *)x;
    a.a_bytes = (uint32_t)((size_t)p.T * p.d * 2);
    a.W = (const bf16_t *)W_gu;
    a.out = (bf16_t *)w.h;
    a.n_ntiles = p.I / (GBN / 2);
    const RingArgs q{(const bf16_t *)x, (const bf16_t *)W_gu, w.pbt, w.meta, w.sorted_tok,
                     (bf16_t *)w.h, p.d, p.I};
    // the tiled path needs d % 256 == 0: no short last k-chunk
    return launch_tiled_t<false, false>(a, q, s);
}

hipError_t launch_tiled_down(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                             hipStream_t s) {
    GemmArgs a = base_args(p, r, w);
    a.A = (const bf16_t *)w.h;
    a.a_bytes = (uint32_t)((size_t)p.cap * p.I * 2);
    a.W = (const bf16_t *)W_dt;
    a.out = (bf16_t *)w.o;
    a.n_ntiles = p.d / GBN;
    const RingArgs q{(const bf16_t *)w.h, (const bf16_t *)W_dt, w.pbt, w.meta, w.sorted_tok,
                     (bf16_t *)w.o, p.I, p.d};
    return p.I % 256 == 0 ? launch_tiled_t<true, false>(a, q, s)
                          : launch_tiled_t<true, true>(a, q, s);
}

}  // namespace beam
