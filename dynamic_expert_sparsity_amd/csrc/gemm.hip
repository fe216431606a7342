// a5-a6, prefill: the SwiGLU experts (BEAM paper, section 3.1 Eq. 3) as a
// grouped bf16 GEMM over the block-padded per-expert lists, on the
// v_mfma_f32_32x32x16_bf16 matrix cores.  Only experts with active pairs have
// blocks, so masked pairs cost no FLOPs and their experts no bytes.
//
// Tile: 128 sorted positions (one block of one expert) x 256 output columns,
// k in stages of 64, double-buffered in LDS.  Four waves, each 64 x 128 (2 x 4
// MFMA tiles of 32 x 32).  Up: the 256 columns are 128 gate rows and the 128
// matching up rows of W_gu, so each wave holds gate and up accumulators of the
// same (position, unit) and applies SiLU(a) * u in registers.  Down: A is h
// (contiguous rows), B is W_dt.
//
// LDS layout of a stage: row r of the tile holds its 64 k-values as eight
// 16-byte chunks; chunk c is stored at slot c ^ (r % 8).  Global loads: eight
// threads fetch one row's 128 contiguous bytes.  MFMA reads: lane l reads row
// (l % 32) at chunk 2*kk + l/32; the XOR spreads the 32 rows of a read over
// all banks.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int GBM = 128;  // rows (sorted positions) per tile = block_m
constexpr int GBN = 256;  // output columns per tile
constexpr int GBK = 64;   // k per stage
constexpr int G_A_BYTES = GBM * GBK * 2;
constexpr int G_B_BYTES = GBN * GBK * 2;
constexpr int G_STAGE_BYTES = G_A_BYTES + G_B_BYTES;
constexpr int G_LDS_BYTES = 2 * G_STAGE_BYTES;  // 96 KB

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 &a, const u32x4 &b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int r, int c) { return r * (GBK * 2) + ((c ^ (r & 7)) << 4); }

// UP: A rows = x[token of position], B rows = gate rows j0.. then up rows
// I + j0..; DOWN: A rows = h[position], B rows = W_dt rows c0..
template <bool UP>
__global__ __launch_bounds__(256) void grouped_swiglu_gemm(
    const bf16_t *__restrict__ A_src, const bf16_t *__restrict__ W,
    const int32_t *__restrict__ block_expert, const int32_t *__restrict__ num_active,
    const int32_t *__restrict__ sorted_tok, bf16_t *__restrict__ out, int d, int I,
    int n_ntiles, int n_tiles_total) {
    extern __shared__ __align__(16) unsigned char lds[];
    // XCD-aware order: consecutive workgroup ids go to different XCDs, so XCD
    // x takes the contiguous range of logical tiles [x * per, (x + 1) * per):
    // the column tiles of one block, and the blocks of one expert, share an L2.
    const int per = (int)(gridDim.x / 8);
    const int logical = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (logical >= n_tiles_total) return;
    const int blk = logical / n_ntiles;
    const int nt = logical - blk * n_ntiles;
    if (blk >= num_active[3]) return;
    const int e = block_expert[blk];
    const int pos0 = blk * GBM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int K = UP ? d : I;          // contraction length
    const int ldw = UP ? d : I;        // weight row length
    const int cth = tid & 7;           // chunk this thread loads
    const int rth = tid >> 3;          // first row this thread loads (+32 i)

    // global row pointers of this thread's 4 A rows and 8 B rows
    const bf16_t *ga[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rth + 32 * i;
        if (UP) ga[i] = A_src + (size_t)sorted_tok[pos0 + r] * d + cth * 8;
        else ga[i] = A_src + (size_t)(pos0 + r) * I + cth * 8;
    }
    const bf16_t *gb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = rth + 32 * i;
        size_t wrow;
        if (UP) wrow = (size_t)e * 2 * I + (r < 128 ? nt * 128 + r : I + nt * 128 + (r - 128));
        else wrow = (size_t)e * d + nt * GBN + r;
        gb[i] = W + wrow * ldw + cth * 8;
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.f;

    // B-row base of each of the wave's 4 column fragments
    int brow[4];
    if (UP) {
        brow[0] = wn * 64;
        brow[1] = wn * 64 + 32;
        brow[2] = 128 + wn * 64;
        brow[3] = 128 + wn * 64 + 32;
    } else {
#pragma unroll
        for (int n = 0; n < 4; ++n) brow[n] = wn * 128 + n * 32;
    }

    const int nst = K / GBK;
    u32x4 ra[4], rb[8];
    auto load_stage = [&](int s) {
        const int k0 = s * GBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = ld16(ga[i] + k0);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = ld16(gb[i] + k0);
    };
    auto store_stage = [&](int buf) {
        unsigned char *sa = lds + buf * G_STAGE_BYTES;
        unsigned char *sb = sa + G_A_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4 *>(sa + swz(rth + 32 * i, cth)) = ra[i];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4 *>(sb + swz(rth + 32 * i, cth)) = rb[i];
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    const int lr = lane & 31;
    const int lh = lane >> 5;
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        if (s + 1 < nst) load_stage(s + 1);
        const unsigned char *sa = lds + buf * G_STAGE_BYTES;
        const unsigned char *sb = sa + G_A_BYTES;
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
            const int ch = 2 * kk + lh;
            u32x4 af[2], bfr[4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                af[m] = *reinterpret_cast<const u32x4 *>(sa + swz(wm * 64 + m * 32 + lr, ch));
#pragma unroll
            for (int n = 0; n < 4; ++n)
                bfr[n] = *reinterpret_cast<const u32x4 *>(sb + swz(brow[n] + lr, ch));
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[m][n] = mfma32x32x16(af[m], bfr[n], acc[m][n]);
        }
        if (s + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4) % 2),
    // register 4*(i/8) + i%4.  Pad rows of a block compute values that nothing
    // reads (their A rows are token 0 / unused h rows inside the buffer).
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = wm * 64 + m * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
            const size_t prow = (size_t)(pos0 + row);
            if (UP) {
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int j = nt * 128 + wn * 64 + n * 32 + lr;
                    out[prow * I + j] = f32_to_bf16(silu<false>(acc[m][n][v]) * acc[m][n + 2][v]);
                }
            } else {
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const int c = nt * GBN + wn * 128 + n * 32 + lr;
                    out[prow * d + c] = f32_to_bf16(acc[m][n][v]);
                }
            }
        }
    }
}

template <bool UP>
static hipError_t launch_gemm(const Plan &p, const void *A_src, const void *W, const Routing &r,
                              const Work &w, void *out, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [] {
        attr_err = hipFuncSetAttribute((const void *)grouped_swiglu_gemm<UP>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G_LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int n_ntiles = UP ? p.I / 128 : p.d / GBN;
    const long long tiles = p.n_blocks_cap * n_ntiles;
    const long long grid = (tiles + 7) / 8 * 8;
    grouped_swiglu_gemm<UP><<<(unsigned)grid, 256, G_LDS_BYTES, s>>>(
        (const bf16_t *)A_src, (const bf16_t *)W, r.block_expert, r.num_active, w.sorted_tok,
        (bf16_t *)out, p.d, p.I, n_ntiles, (int)tiles);
    return hipGetLastError();
}

hipError_t launch_gemm_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                          const Work &w, hipStream_t s) {
    return launch_gemm<true>(p, x, W_gu, r, w, w.h, s);
}

hipError_t launch_gemm_down(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                            hipStream_t s) {
    return launch_gemm<false>(p, w.h, W_dt, r, w, w.o, s);
}

}  // namespace beam
