// a5-a6 (and a1 for large batches): the SwiGLU experts (BEAM paper, section
// 3.1 Eq. 3) as a grouped bf16 GEMM over the block-padded per-expert lists,
// on the v_mfma_f32_32x32x16_bf16 matrix cores.  Only experts with active
// pairs have blocks, so masked pairs cost no FLOPs and their experts no bytes.
// The same kernel, in ROUTER mode, computes the two routers' logits (Eq. 4-5)
// of a large batch as one dense GEMM with 2E = 256 columns.
//
// Tile: BM rows (UP/DOWN: one 128-position block of one expert, or 256
// positions = up to two such blocks of one expert; ROUTER: 128 tokens) x 256
// output columns, k in stages of 64.  The call's record says which height
// works: a weight slice is read once per tile, so 256-row tiles halve the
// weight reads of experts with many pairs, 128-row tiles waste fewer rows on
// experts with few.  (BM / WT) (rows) x 2 (columns) waves, each WT x 128
// (WT / 32 x 4 MFMA tiles of 32 x 32; WT = 64 for the 256-row and router
// tiles, 32 for the 128-row expert tiles); a wave whose WT rows are all
// padding of its expert's last block (or past the last token) skips its LDS
// reads and MFMAs, and rows past the expert's segment are never stored.  UP: the 256
// columns are 128 gate rows and the 128 matching up rows of W_gu, so each
// wave holds gate and up accumulators of the same (position, unit) and
// applies SiLU(a) * u in registers.  DOWN: A is h (contiguous rows), B is
// W_dt.  ROUTER: A is x, B is W_gate then W_mask, fp32 out.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4):
// A (32 KB per stage) in a ring of two stages, B (32 KB) in a ring of three,
// so the weights stream two stages ahead (160 KB of LDS; the router tiles use
// three-stage rings of 16 + 32 KB).  Every row segment a load instruction fetches is a whole
// 128-byte line (k = 64 bf16): a wave instruction fills 1 KB = 8 rows, lane l
// fetching chunk (l % 8) ^ f(row) of row l / 8; half-line segments would halve
// the rate at which a CU can pull lines from L2.  LDS layout of a stage: row r
// holds its 64 k-values as eight 16-byte chunks, chunk c at slot c ^ f(r) (see
// swz).  MFMA reads: lane l reads row (l % 32) at chunk 2*kk + l/32,
// conflict-free.
//
// Pipeline: the LDS reads of k-slice kk + 1 are issued before the MFMAs of
// slice kk, across stage boundaries too, so LDS reads overlap MFMAs.  The
// global->LDS loads of a stage are interleaved with the MFMAs of the stage
// before (issued in a burst, they stall every wave on the address unit while
// the matrix cores idle).  A stage boundary waits (explicit vmcnt: the
// compiler does not track LDS written by global_load_lds) for the next stage
// and meets the other waves at a barrier, which frees the buffers just read.
//
// Scheduling: a persistent grid of one workgroup per CU walks the tiles that
// exist on the device (blocks * column tiles); the tiles are split into eight
// contiguous ranges, one per XCD (consecutive workgroup ids go to different
// XCDs), so the column tiles of a block and the blocks of an expert are worked
// on together under one L2.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int GBM = 256;   // rows of the taller expert tile (two 128-row blocks of one expert)
constexpr int GBM_R = 128; // rows per router tile (more tiles for a 2E-column GEMM)
constexpr int GBN = 256;   // output columns per tile
constexpr int GBK = 64;    // k per stage: one 128-byte line per row
constexpr int G_ROWB = GBK * 2;       // bytes per row per stage
constexpr int G_RPI = 1024 / G_ROWB;  // rows per 1 KB wave load (8)
// k-slices (of 4) over which a stage's loads are spread in the expert GEMMs
#ifndef G_DKK
#define G_DKK 4
#endif
#ifndef G_SKIP_A
#define G_SKIP_A 1
#endif
#ifndef G_WN_FAST
#define G_WN_FAST 1
#endif
// the 128-row tiles: rows per wave (32: eight waves, each 32 x 128, half
// the DMA issues per wave of four 64-row waves; 6-7 us faster down
// projections at 70-80 pairs per expert) and the k-slices their loads are
// spread over
#ifndef G_WT128
#define G_WT128 32
#endif
#ifndef G_DKK128
#define G_DKK128 3
#endif

// BM rows per tile, WT rows per wave (BM / WT x 2 waves, each WT x 128);
// A in a ring of NA stages, B in a ring of NB (NA or NA + 1) stages; a
// stage's loads are spread over DKK of its four k-slices
template <int BM, int NA, int NB, int DKK, int WT>
struct GemmCfg {
    static constexpr int WM = BM / WT;                      // waves along the rows
    static constexpr int NW = WM * 2;                       // waves per workgroup
    static constexpr int MF = WT / 32;                      // 32-row MFMA tiles per wave
    static constexpr int MPS = MF * 4;                      // MFMAs per wave per k-slice
    static constexpr int A_BYTES = BM * G_ROWB;             // one stage of A
    static constexpr int B_BYTES = GBN * G_ROWB;            // one stage of B
    static constexpr int B_OFF = NA * A_BYTES;              // B ring after the A ring
    static constexpr int LDS_BYTES = NA * A_BYTES + NB * B_BYTES;
    static constexpr int LA = A_BYTES / 1024 / NW;          // 1 KB wave loads per wave per stage
    static constexpr int LB = B_BYTES / 1024 / NW;
    static constexpr int L = LA + LB;
    static constexpr int PER = L / DKK;                     // loads per k-slice
    static constexpr int KK = GBK / 16;                     // k-slices per stage
    static_assert(LA * NW * 1024 == A_BYTES && LB * NW * 1024 == B_BYTES, "whole wave loads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((NA == 2 && NB == 3) || (NA == 3 && NB == 3), "ring depths");
    static_assert(PER * DKK == L && MPS % PER == 0 && DKK <= KK, "load spread");
    static_assert(WT == 32 || WT == 64 || WT == 128, "wave tile height");
    // Issue slot p (stage p of the loop; p < 0 before it) sends A of stage
    // p + NA - 1, then B of stage p + NB - 1; load u goes out in k-slice
    // u / PER, and slice KK - 1 runs after the boundary p -> p + 1.  Loads
    // that may still be in flight when stage t must have landed (the newer
    // loads only), if stage t + 1 exists (else none):
    //   at the boundary before t > 0: NB = NA + 1: the B loads of slot t - 1
    //     sent before that boundary (A of stage t is the last needed);
    //     NB = NA: every load of slot t - 1 sent before it;
    //   before the loop (t = 0): B of stage 1 (NB = NA + 1), or all of slot -1.
    static constexpr int BEFORE = L < PER * (KK - 1) ? L : PER * (KK - 1);
    static constexpr int S_LOOP = NB == NA + 1 ? (BEFORE > LA ? BEFORE - LA : 0) : BEFORE;
    static constexpr int S_PRO = NB == NA + 1 ? LB : L;
    static_assert(NB == NA || (LA - 1) / PER < KK - 1, "A of a stage is sent before its boundary");
    static_assert(S_LOOP < 64 && S_PRO < 64, "vmcnt range");
};

enum GemmMode { MODE_UP = 0, MODE_DOWN = 1, MODE_ROUTER = 2 };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 &a, const u32x4 &b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// chunk c of a 128-byte row r sits at 16-byte slot c ^ f(r),
// f(r) = (r % 8) ^ ((r / 8) % 2): any 8 consecutive rows, and the even and the
// odd rows of any 16 aligned rows, get distinct slots, so a 32-row fragment
// read is conflict-free whether a read phase serves 8 lanes (32 banks) or 16
// lanes (64 banks).
__device__ __forceinline__ int swz_f(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * G_ROWB + ((c ^ swz_f(r)) << 4); }

// s_waitcnt with only the vector-memory count set (expcnt / lgkmcnt at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 0x3) << 14));
}
// s_waitcnt with only the LDS/scalar count set: at most N of them in flight
template <int N>
__device__ __forceinline__ void wait_lgkm() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (N << 8) | (0x3 << 14));
}

__device__ __forceinline__ void lds_dma16(const void *g, unsigned char *l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

struct GemmArgs {
    const bf16_t *A;        // x (UP, ROUTER) or h (DOWN)
    const bf16_t *W;        // W_gu (UP), W_dt (DOWN), W_gate (ROUTER)
    const bf16_t *W2;       // W_mask (ROUTER)
    const int32_t *block_expert, *num_active, *sorted_tok;
    const int32_t *expert_offsets, *expert_counts;
    bf16_t *out;            // h (UP) or o (DOWN)
    float *gate_logits, *mask_logits;  // ROUTER
    int T, d, I, E;
    int n_ntiles;           // column tiles per block
    int n_rblocks;          // ROUTER: row blocks
    const int32_t *mode;    // UP/DOWN: the call's record {family, max count, records, 0}
    const int32_t *pbt;     // UP/DOWN, 256-row tiles: {expert, first position, segment rows,
                            // valid rows} per tile
};

template <int MODE, int BM, int NA, int NB, int DKK, int WT>
__global__ __launch_bounds__(BM / WT * 128, 1) void grouped_gemm(GemmArgs g) {
    using C = GemmCfg<BM, NA, NB, DKK, WT>;
    constexpr int MF = C::MF;
    constexpr int KK = C::KK;  // 16-wide k-slices per stage
    static_assert(KK % 2 == 0, "fragment sets alternate by slice parity");
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    // column half fastest: consecutive waves sit on different SIMDs (wave w
    // runs on SIMD w % 4), so the live waves of a part-filled tile (the low
    // row groups) spread over the SIMDs instead of sharing one
    const int wn = G_WN_FAST ? wave & 1 : wave / C::WM;
    const int wm = G_WN_FAST ? wave >> 1 : wave % C::WM;
    const int lr = lane & 31;
    const int lh = lane >> 5;

    // the call's kernel family: 1 = 128-row tiles, 2 = 256-row tiles (0 = streaming)
    if (MODE != MODE_ROUTER && g.mode[0] != (BM == 256 ? 2 : 1)) return;
    const int n_blocks = MODE == MODE_ROUTER ? g.n_rblocks : BM == 256 ? g.mode[2] : g.num_active[3];
    const int n_tiles = n_blocks * g.n_ntiles;
    const int xcd = blockIdx.x & 7;
    const int per_xcd_wg = gridDim.x >> 3;
    const int chunk = (n_tiles + 7) >> 3;
    const int t_begin = xcd * chunk;
    const int t_end = min(n_tiles, t_begin + chunk);

    const int K = MODE == MODE_DOWN ? g.I : g.d;
    const int ldw = K;
    const int nst = K / GBK;
    // load i of a stage covers 8-row group q = wave + NW i of its operand;
    // lane l fetches row 8 q + l / 8
    const int lrow = lane >> 3;

    int brow[4];
    if (MODE == MODE_UP) {
        brow[0] = wn * 64;
        brow[1] = wn * 64 + 32;
        brow[2] = 128 + wn * 64;
        brow[3] = 128 + wn * 64 + 32;
    } else {
#pragma unroll
        for (int n = 0; n < 4; ++n) brow[n] = wn * 128 + n * 32;
    }

    for (int tile = t_begin + (int)(blockIdx.x >> 3); tile < t_end; tile += per_xcd_wg) {
        const int blk = tile / g.n_ntiles;
        const int nt = tile - blk * g.n_ntiles;
        // tile: BM rows from pos0 of expert e; seg of them lie in the expert's
        // padded segment (a 256-row tile can end after 128), rows_valid hold
        // real pairs (tokens, for the router)
        int pos0, e, seg, rows_valid;
        if (MODE == MODE_ROUTER) {
            pos0 = blk * BM;
            e = 0;
            seg = BM;
            rows_valid = g.T - pos0;
        } else if (BM == 256) {
            const int4 rec = *reinterpret_cast<const int4 *>(g.pbt + 4 * blk);
            e = rec.x;
            pos0 = rec.y;
            seg = rec.z;
            rows_valid = rec.w;
        } else {
            pos0 = blk * BM;
            e = g.block_expert[blk];
            seg = BM;
            rows_valid = g.expert_offsets[e] + g.expert_counts[e] - pos0;
        }
        const bool live = __builtin_amdgcn_readfirstlane(wm * WT < rows_valid ? 1 : 0) != 0;

        // this lane's 16 bytes land at slot l % 8 of row r: chunk (l % 8) ^ f(r)
        const bf16_t *srcA[C::LA], *srcB[C::LB];
#pragma unroll
        for (int i = 0; i < C::LA; ++i) {
            const int r = G_RPI * (wave + C::NW * i) + lrow;
            // rows past the segment (the next expert's, or past the lists)
            // read the segment's first row; nothing stores them
            const int rs = r < seg ? r : 0;
            if (MODE == MODE_UP) {
                srcA[i] = g.A + (size_t)g.sorted_tok[pos0 + rs] * g.d;
            } else if (MODE == MODE_DOWN) {
                srcA[i] = g.A + (size_t)(pos0 + rs) * g.I;
            } else {
                const int t = min(pos0 + r, g.T - 1);
                srcA[i] = g.A + (size_t)t * g.d;
            }
            srcA[i] += ((lane & 7) ^ swz_f(r)) * 8;
        }
#pragma unroll
        for (int i = 0; i < C::LB; ++i) {
            const int r = G_RPI * (wave + C::NW * i) + lrow;
            if (MODE == MODE_UP) {
                const int wr = r < 128 ? nt * 128 + r : g.I + nt * 128 + (r - 128);
                srcB[i] = g.W + ((size_t)e * 2 * g.I + wr) * ldw;
            } else if (MODE == MODE_DOWN) {
                srcB[i] = g.W + ((size_t)e * g.d + nt * GBN + r) * ldw;
            } else {
                const int n = min(nt * GBN + r, 2 * g.E - 1);
                srcB[i] = n < g.E ? g.W + (size_t)n * ldw : g.W2 + (size_t)(n - g.E) * ldw;
            }
            srcB[i] += ((lane & 7) ^ swz_f(r)) * 8;
        }
        // issue slot p (stage p of the loop; p < 0 before it) loads A of stage
        // p + NA - 1 and then B of stage p + NB - 1, each into the ring buffer
        // the stage before it left free at the last boundary
        // A loads whose 8 rows all lie past the tile's valid rows are not
        // sent (SKIP_A): no MFMA result that is stored for a real pair reads
        // them (a row's products depend on that row only; pad rows of a
        // segment are written but never read), and with NB = NA + 1 every
        // wait allows only B loads to be outstanding, which are always sent
        // (so a missing A load never shortens a wait).  Keeps the weight
        // stream and drops the DMA of a part-filled tile's empty rows.
        constexpr bool SKIP_A = G_SKIP_A && MODE != MODE_ROUTER && NB == NA + 1;
        unsigned a_send = 0;  // bit u: A load u has a valid row (wave-uniform)
#pragma unroll
        for (int i = 0; i < C::LA; ++i)
            if (!SKIP_A || G_RPI * (wave + C::NW * i) < rows_valid) a_send |= 1u << i;
        auto issue = [&](int p, int u) {
            if (u < C::LA) {
                const int j = p + NA - 1;
                if (j >= 0 && j < nst && ((a_send >> u) & 1u))
                    lds_dma16(srcA[u] + j * GBK,
                              lds + (j % NA) * C::A_BYTES + (wave + C::NW * u) * 1024);
            } else {
                const int j = p + NB - 1;
                if (j >= 0 && j < nst)
                    lds_dma16(srcB[u - C::LA] + j * GBK,
                              lds + C::B_OFF + (j % NB) * C::B_BYTES + (wave + C::NW * (u - C::LA)) * 1024);
            }
        };

        f32x16 acc[MF][4];
#pragma unroll
        for (int m = 0; m < MF; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.f;

        // fragments of one 16-wide k-slice, in two alternating sets
        u32x4 af[2][MF], bfr[2][4];
        auto read_frags = [&](int s, int kk, int set) {
            const unsigned char *sa = lds + (s % NA) * C::A_BYTES;
            const unsigned char *sb = lds + C::B_OFF + (s % NB) * C::B_BYTES;
            const int ch = 2 * kk + lh;
#pragma unroll
            for (int m = 0; m < MF; ++m)
                af[set][m] = *reinterpret_cast<const u32x4 *>(sa + swz(wm * WT + m * 32 + lr, ch));
#pragma unroll
            for (int n = 0; n < 4; ++n)
                bfr[set][n] = *reinterpret_cast<const u32x4 *>(sb + swz(brow[n] + lr, ch));
        };
        // one k-slice of stage s: the MF x 4 MFMAs (LIVE waves) with the
        // loads of issue slot s interleaved (spread over the first DKK
        // slices, one after every few MFMAs, so the address unit works while
        // the matrix cores do)
        constexpr int PER = C::PER;
        constexpr int MPS = C::MPS;
        auto slice = [&](auto LIVE, int set, int s, int kk) {
#pragma unroll
            for (int j = 0; j < MPS; ++j) {
                const int m = j >> 2, n = j & 3;
                if constexpr (decltype(LIVE)::value)
                    acc[m][n] = mfma32x32x16(af[set][m], bfr[set][n], acc[m][n]);
                if (kk < DKK && (j % (MPS / PER)) == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    issue(s, kk * PER + j / (MPS / PER));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        // Waves whose rows are all padding run the same loop without reads
        // and MFMAs (a separate copy, so the live copy is straight-line code).
        auto main_loop = [&](auto LIVE) {
            constexpr bool LV = decltype(LIVE)::value;
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's LDS
            asm volatile("" ::: "memory");
            for (int p = -(NB - 1); p < 0; ++p)
#pragma unroll
                for (int u = 0; u < C::L; ++u) issue(p, u);
            if (1 < nst) wait_vmcnt<C::S_PRO>();
            else wait_vmcnt<0>();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if constexpr (LV) read_frags(0, 0, 0);
            for (int s = 0; s < nst; ++s) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (kk + 1 < KK) {
                        if constexpr (LV) read_frags(s, kk + 1, (kk + 1) & 1);
                    } else if (s + 1 < nst) {
                        // stage boundary: stage s + 1 landed for every wave,
                        // stage s read by every wave
                        if (s + 2 < nst) wait_vmcnt<C::S_LOOP>();
                        else wait_vmcnt<0>();
                        if constexpr (LV) wait_lgkm<0>();
                        asm volatile("" ::: "memory");
                        __builtin_amdgcn_s_barrier();
                        asm volatile("" ::: "memory");
                        if constexpr (LV) read_frags(s + 1, 0, 0);
                    }
                    // the slice's own fragments are in (LDS reads complete in
                    // order; only the MF + 4 reads of the next slice may be
                    // pending)
                    if constexpr (LV) wait_lgkm<MF + 4>();
                    __builtin_amdgcn_sched_barrier(0);
                    slice(LIVE, kk & 1, s, kk);
                }
            }
        };
        if (live) main_loop(std::true_type{});
        else main_loop(std::false_type{});

        // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4) % 2),
        // register 4*(i/8) + i%4.  Pad rows of a block compute values nothing
        // reads (their A rows are token 0 / h rows inside the buffer).
#pragma unroll
        for (int m = 0; m < MF; ++m) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * WT + m * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                const size_t prow = (size_t)(pos0 + row);
                if (MODE != MODE_ROUTER && row >= seg) continue;  // the next expert's rows
                if (MODE == MODE_UP) {
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        const int j = nt * 128 + wn * 64 + n * 32 + lr;
                        g.out[prow * g.I + j] =
                            f32_to_bf16(silu<false>(acc[m][n][v]) * acc[m][n + 2][v]);
                    }
                } else if (MODE == MODE_DOWN) {
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        const int c = nt * GBN + wn * 128 + n * 32 + lr;
                        g.out[prow * g.d + c] = f32_to_bf16(acc[m][n][v]);
                    }
                } else {
                    if ((int)prow < g.T) {
#pragma unroll
                        for (int n = 0; n < 4; ++n) {
                            const int c = nt * GBN + wn * 128 + n * 32 + lr;
                            if (c < g.E) g.gate_logits[prow * g.E + c] = acc[m][n][v];
                            else if (c < 2 * g.E) g.mask_logits[prow * g.E + (c - g.E)] = acc[m][n][v];
                        }
                    }
                }
            }
        }
    }
}

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

template <int MODE, int BM, int NA, int NB, int DKK, int WT>
static hipError_t launch_gemm(const GemmArgs &a, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    using C = GemmCfg<BM, NA, NB, DKK, WT>;
    std::call_once(once, [] {
        attr_err = hipFuncSetAttribute((const void *)grouped_gemm<MODE, BM, NA, NB, DKK, WT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    });
    if (attr_err != hipSuccess) return attr_err;
    grouped_gemm<MODE, BM, NA, NB, DKK, WT><<<persistent_wgs(), C::NW * 64, C::LDS_BYTES, s>>>(a);
    return hipGetLastError();
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

hipError_t launch_gemm_up(const Plan &p, const void *x, const void *W_gu, const Routing &r,
                          const Work &w, hipStream_t s) {
    GemmArgs a = base_args(p, r, w);
    a.A = (const bf16_t *)x;
    a.W = (const bf16_t *)W_gu;
    a.out = (bf16_t *)w.h;
    a.n_ntiles = p.I / (GBN / 2);
    // both tile heights; the call's record lets one of them work
    const hipError_t e = launch_gemm<MODE_UP, 128, 3, 3, G_DKK128, G_WT128>(a, s);
    if (e != hipSuccess) return e;
    return launch_gemm<MODE_UP, GBM, 2, 3, G_DKK, 64>(a, s);
}

hipError_t launch_gemm_down(const Plan &p, const void *W_dt, const Routing &r, const Work &w,
                            hipStream_t s) {
    GemmArgs a = base_args(p, r, w);
    a.A = (const bf16_t *)w.h;
    a.W = (const bf16_t *)W_dt;
    a.out = (bf16_t *)w.o;
    a.n_ntiles = p.d / GBN;
    const hipError_t e = launch_gemm<MODE_DOWN, 128, 3, 3, G_DKK128, G_WT128>(a, s);
    if (e != hipSuccess) return e;
    return launch_gemm<MODE_DOWN, GBM, 2, 3, G_DKK, 64>(a, s);
}

hipError_t launch_gemm_router(const Plan &p, const void *x, const void *Wg, const void *Wm,
                              const Routing &r, hipStream_t s) {
    GemmArgs a{};
    a.A = (const bf16_t *)x;
    a.W = (const bf16_t *)Wg;
    a.W2 = (const bf16_t *)Wm;
    a.gate_logits = r.gate_logits;
    a.mask_logits = r.mask_logits;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.n_ntiles = (2 * p.E + GBN - 1) / GBN;
    a.n_rblocks = (p.T + GBM_R - 1) / GBM_R;
    return launch_gemm<MODE_ROUTER, GBM_R, 3, 3, 3, 64>(a, s);
}

}  // namespace beam
