// a5-a6: the SwiGLU experts (BEAM paper, section 3.1 Eq. 3) as a grouped
// bf16 GEMM over the block-padded per-expert lists, on the
// v_mfma_f32_32x32x16_bf16 matrix cores.  Only experts with active pairs
// have blocks, so masked pairs cost no FLOPs and their experts no bytes.
//
// Tile: BM rows (one 128-position block of one expert, or 256 positions =
// up to two such blocks of one expert) x 256 output columns, k in stages of
// 64.  The call's record says which height
// works: a weight slice is read once per tile, so 256-row tiles halve the
// weight reads of experts with many pairs, 128-row tiles waste fewer rows on
// experts with few.  (BM / WT) (rows) x 2 (columns) waves, each WT x 128
// (WT / 32 x 4 MFMA tiles of 32 x 32; WT = 64 for the 256-row tiles, 32 for
// the 128-row tiles); a wave whose WT rows are all
// padding of its expert's last block (or past the last token) skips its LDS
// reads and MFMAs, and rows past the expert's segment are never stored.  UP: the 256
// columns are 128 gate rows and the 128 matching up rows of W_gu, so each
// wave holds gate and up accumulators of the same (position, unit) and
// applies SiLU(a) * u in registers.  DOWN: A is h (contiguous rows), B is
// W_dt.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4):
// A (32 KB per stage) in a ring of two stages, B (32 KB) in a ring of three,
// so the weights stream two stages ahead (160 KB of LDS).  Every row
// segment a load instruction fetches is a whole 128-byte line (k = 64 bf16): a wave instruction fills 1 KB = 8 rows, lane l
// fetching chunk (l % 8) ^ f(row) of row l / 8; half-line segments would halve
// the rate at which a CU can pull lines from L2.  LDS layout of a stage: row r
// holds its 64 k-values as eight 16-byte chunks, chunk c at slot c ^ f(r) (see
// swz).  MFMA reads: lane l reads row (l % 32) at chunk 2*kk + l/32,
// conflict-free.
//
// Pipeline: the LDS reads of k-slice kk + 1 are issued before the MFMAs of
// slice kk, so LDS reads overlap MFMAs.  The global->LDS loads of a stage are
// interleaved with the MFMAs of the stage before (issued in a burst, they
// stall every wave on the address unit while the matrix cores idle).  A
// stage boundary waits (explicit vmcnt: the compiler does not track LDS
// written by global_load_lds) for the next stage and meets the other waves
// at a barrier, which frees the buffers just read.  The boundary sits inside
// the stage's last slice of MFMAs (whose fragments are already in
// registers): halfway through it in the up projection, after it in the down
// projection (main_loop), so the operand loads get 3.5 or 4 slices to land.
//
// Scheduling: a persistent grid of one workgroup per CU walks the tiles that
// exist on the device (blocks * column tiles); the tiles are split into eight
// contiguous ranges, one per XCD (consecutive workgroup ids go to different
// XCDs), so the column tiles of a block and the blocks of an expert are worked
// on together under one L2.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int GBM = 256;   // rows of the taller expert tile (two 128-row blocks of one expert)
constexpr int GBN = 256;   // output columns per tile
constexpr int GBK = 64;    // k per stage: one 128-byte line per row
constexpr int G_ROWB = GBK * 2;       // bytes per row per stage
constexpr int G_RPI = 1024 / G_ROWB;  // rows per 1 KB wave load (8)
// k-slices (of 4) over which a stage's loads are spread in the 256-row
// tiles: the first two, so the A loads of the next stage go out at the start
// of a stage and have all of it to land (against all four: 1-2% faster up
// projections at keep 0.5-1.0, A/B in both orders)
#ifndef G_DKK
#define G_DKK 2
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
    // bf16 stores of one wave's epilogue (UP: SiLU(a) * u of 2 of its 4
    // column blocks; DOWN: all 4), counted for the next tile's first wait
    static constexpr int ST_UP = MF * 16 * 2;
    static constexpr int ST_DOWN = MF * 16 * 4;
};

enum GemmMode { MODE_UP = 0, MODE_DOWN = 1 };

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

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// A raw buffer resource over `bytes` bytes from `base` (word 3: the gfx9
// raw-buffer format); loads at offsets past `bytes` return 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// 16 bytes per lane from buffer offset voff + soff into LDS (the wave's 1 KB
// of destinations starts at l).  The buffer form of the LDS DMA is counted
// in vmcnt only; the flat form is also counted as a possible LDS access,
// which made the compiler drain every LDS read before the next MFMAs.
template <int AUX = 0>
__device__ __forceinline__ void lds_dma16_buf(rsrc_t r, uint32_t voff, uint32_t soff,
                                              unsigned char *l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)l, 16,
                                             voff, soff, 0, AUX);
}

struct GemmArgs {
    const bf16_t *A;        // x (UP) or h (DOWN)
    const bf16_t *W;        // W_gu (UP) or W_dt (DOWN)
    const int32_t *block_expert, *num_active, *sorted_tok;
    const int32_t *expert_offsets, *expert_counts;
    bf16_t *out;            // h (UP) or o (DOWN)
    int T, d, I, E;
    uint32_t a_bytes;       // bytes of A (UP: x, DOWN: h; below 2^31)
    int n_ntiles;           // column tiles per block
    const int32_t *mode;    // UP/DOWN: the call's record {family, max count, records, 0}
    const int32_t *pbt;     // UP/DOWN, 256-row tiles: {expert, first position, segment rows,
                            // valid rows} per tile
};

template <int MODE, int BM, int NA, int NB, int DKK, int WT>
__device__ __forceinline__ void gemm_body(const GemmArgs &g) {
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
    if (g.mode[0] != (BM == 256 ? 2 : 1)) return;
    const int n_blocks = BM == 256 ? g.mode[2] : g.num_active[3];
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

    // One tile's place in the problem and its operand addresses, which go
    // through buffer resources (32-bit byte offsets per lane; the stage's k
    // offset goes in the scalar offset).
    struct Tile {
        int pos0, nt, seg, rows_valid;
        bool live;
        unsigned a_send;   // bit u: A load u has a valid row (wave-uniform)
        rsrc_t rB;         // the expert's weights
        uint32_t offA[C::LA], offB[C::LB];
    };
    const rsrc_t rA = make_rsrc(g.A, g.a_bytes);
    // A loads whose 8 rows all lie past the tile's valid rows are not
    // sent (SKIP_A): no MFMA result that is stored for a real pair reads
    // them (a row's products depend on that row only; pad rows of a
    // segment are written but never read), and with NB = NA + 1 every
    // wait allows only B loads to be outstanding, which are always sent
    // (so a missing A load never shortens a wait).  Keeps the weight
    // stream and drops the DMA of a part-filled tile's empty rows.
    constexpr bool SKIP_A = G_SKIP_A && NB == NA + 1;

    auto setup = [&](int tile, Tile &t) {
        const int blk = tile / g.n_ntiles;
        t.nt = tile - blk * g.n_ntiles;
        // tile: BM rows from pos0 of expert e; seg of them lie in the expert's
        // padded segment (a 256-row tile can end after 128), rows_valid hold
        // real pairs
        int e;
        if (BM == 256) {
            const int4 rec = *reinterpret_cast<const int4 *>(g.pbt + 4 * blk);
            e = rec.x;
            t.pos0 = rec.y;
            t.seg = rec.z;
            t.rows_valid = rec.w;
        } else {
            t.pos0 = blk * BM;
            e = g.block_expert[blk];
            t.seg = BM;
            t.rows_valid = g.expert_offsets[e] + g.expert_counts[e] - t.pos0;
        }
        t.live = __builtin_amdgcn_readfirstlane(wm * WT < t.rows_valid ? 1 : 0) != 0;
        const size_t wrows = MODE == MODE_UP ? (size_t)2 * g.I : (size_t)g.d;
        t.rB = make_rsrc(g.W + (size_t)e * wrows * ldw, (uint32_t)(wrows * ldw * 2));
        // this lane's 16 bytes land at slot l % 8 of row r: chunk (l % 8) ^ f(r)
#pragma unroll
        for (int i = 0; i < C::LA; ++i) {
            const int r = G_RPI * (wave + C::NW * i) + lrow;
            // rows past the segment (the next expert's, or past the lists)
            // read the segment's first row; nothing stores them
            const int rs = r < t.seg ? r : 0;
            const int ch = ((lane & 7) ^ swz_f(r)) * 8;
            if (MODE == MODE_UP)
                t.offA[i] = ((uint32_t)g.sorted_tok[t.pos0 + rs] * (uint32_t)g.d + ch) * 2u;
            else
                t.offA[i] = ((uint32_t)(t.pos0 + rs) * (uint32_t)g.I + ch) * 2u;
        }
#pragma unroll
        for (int i = 0; i < C::LB; ++i) {
            const int r = G_RPI * (wave + C::NW * i) + lrow;
            const int ch = ((lane & 7) ^ swz_f(r)) * 8;
            if (MODE == MODE_UP) {
                const int wr = r < 128 ? t.nt * 128 + r : g.I + t.nt * 128 + (r - 128);
                t.offB[i] = ((uint32_t)wr * (uint32_t)ldw + ch) * 2u;
            } else {
                t.offB[i] = ((uint32_t)(t.nt * GBN + r) * (uint32_t)ldw + ch) * 2u;
            }
        }
        t.a_send = 0;
#pragma unroll
        for (int i = 0; i < C::LA; ++i)
            if (!SKIP_A || G_RPI * (wave + C::NW * i) < t.rows_valid) t.a_send |= 1u << i;
    };

    // issue slot p (stage p of the loop; p < 0 before it) loads A of stage
    // p + NA - 1 and then B of stage p + NB - 1, each into the ring buffer
    // the stage before it left free at the last boundary
    auto issue = [&](const Tile &t, int p, int u) {
        if (u < C::LA) {
            const int j = p + NA - 1;
            if (j >= 0 && j < nst && ((t.a_send >> u) & 1u)) {
                unsigned char *dst = lds + (j % NA) * C::A_BYTES + (wave + C::NW * u) * 1024;
                lds_dma16_buf(rA, t.offA[u], (uint32_t)j * G_ROWB, dst);
            }
        } else {
            const int j = p + NB - 1;
            if (j >= 0 && j < nst) {
                unsigned char *dst =
                    lds + C::B_OFF + (j % NB) * C::B_BYTES + (wave + C::NW * (u - C::LA)) * 1024;
                // 128-row tiles are taken when most experts fill one block:
                // a weight slice is then read by one tile only and streams
                // past the L2 (non-temporal); the 256-row tiles of an expert
                // with several of them share its slices through the L2
                lds_dma16_buf<BM == 128 ? 2 : 0>(t.rB, t.offB[u - C::LA], (uint32_t)j * G_ROWB, dst);
            }
        }
    };
    auto prologue = [&](const Tile &t) {
        for (int p = -(NB - 1); p < 0; ++p)
#pragma unroll
            for (int u = 0; u < C::L; ++u) issue(t, p, u);
    };

    f32x16 acc[MF][4];
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
    auto slice = [&](const Tile &t, auto LIVE, int set, int s, int kk, int at, auto &&mid) {
#pragma unroll
        for (int j = 0; j < MPS; ++j) {
            const int m = j >> 2, n = j & 3;
            if constexpr (decltype(LIVE)::value)
                acc[m][n] = mfma32x32x16(af[set][m], bfr[set][n], acc[m][n]);
            if (kk < DKK && (j % (MPS / PER)) == 0) {
                __builtin_amdgcn_sched_barrier(0);
                issue(t, s, kk * PER + j / (MPS / PER));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j == at) mid();
        }
    };

    // The stages of one tile whose prologue loads were issued.  Waves whose
    // rows are all padding run the same loop without reads and MFMAs (a
    // separate copy, so the live copy is straight-line code).  The waits
    // count this wave's vector-memory operations, which complete in issue
    // order: the epilogue stores of the previous tile, issued after this
    // tile's prologue loads, are the newest (up to ST of them).
    auto main_loop = [&](const Tile &t, auto LIVE, int stores_after_prologue) {
        constexpr bool LV = decltype(LIVE)::value;
        if (stores_after_prologue) {
            // every prologue load is older than the stores: all of them done
            // once at most min(stores, 63) operations are in flight, which
            // also lets the newest stage's B loads finish (a stricter wait)
            wait_vmcnt<(MODE == MODE_UP ? C::ST_UP : C::ST_DOWN) < 63
                           ? (MODE == MODE_UP ? C::ST_UP : C::ST_DOWN) : 63>();
        } else if (1 < nst) {
            wait_vmcnt<C::S_PRO>();
        } else {
            wait_vmcnt<0>();
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (LV) read_frags(0, 0, 0);
        // The stage boundary (the wait for the next stage's operands, the
        // barrier, the first fragment reads of the next stage) sits inside
        // the stage's last k-slice.  Every load of a slot goes out in the
        // slot's first slices, so the waits count the same loads wherever
        // the boundary sits.  Up projection (32 stages per tile at d =
        // 2048): halfway through the last slice's MFMAs, so the loads get
        // 3.5 slices to land and the slice's other half hides the next
        // fragment reads (4% faster at keep 0.5, 1% at keep 1.0 than at the
        // slice's start).  Down projection (12 stages at I = 768): after
        // the slice, 4 slices to land (4-5% faster than at its start; the
        // half-way point measured the same).
        static_assert(DKK < KK, "a slot's loads precede its last slice");
        constexpr int AT = MODE == MODE_UP ? MPS / 2 - 1 : MPS - 1;
        static_assert(AT >= 0 && AT < MPS, "the boundary falls on one of the slice's MFMAs");
        for (int s = 0; s < nst; ++s) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 1 < KK) {
                    if constexpr (LV) read_frags(s, kk + 1, (kk + 1) & 1);
                    // the slice's own fragments are in (LDS reads complete
                    // in order; only the MF + 4 reads of the next slice may
                    // be pending)
                    if constexpr (LV) wait_lgkm<MF + 4>();
                } else {
                    if constexpr (LV) wait_lgkm<0>();
                }
                __builtin_amdgcn_sched_barrier(0);
                const bool bnd = kk + 1 == KK && s + 1 < nst;
                slice(t, LIVE, kk & 1, s, kk, AT, [&] {
                    if (!bnd) return;
                    // stage s + 1 landed for every wave, stage s read by
                    // every wave (this slice's fragments are in registers)
                    __builtin_amdgcn_sched_barrier(0);
                    if (s + 2 < nst) wait_vmcnt<C::S_LOOP>();
                    else wait_vmcnt<0>();
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    if constexpr (LV) read_frags(s + 1, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        }
    };

    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4) % 2),
    // register 4*(i/8) + i%4.  Pad rows of a block compute values nothing
    // reads (their A rows are token 0 / h rows inside the buffer).  A wave
    // whose rows are all pad (or the next expert's) stores nothing: no
    // pair's result lives there, and the down GEMM does not load h rows of
    // an 8-row group that lies wholly past the valid rows.  Every other
    // wave issues all of its C::ST stores.
    auto epilogue = [&](const Tile &t) {
        if (wm * WT >= t.rows_valid) return;  // pad rows only
#pragma unroll
        for (int m = 0; m < MF; ++m) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * WT + m * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                const size_t prow = (size_t)(t.pos0 + row);
                if (MODE == MODE_UP) {
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        const int j = t.nt * 128 + wn * 64 + n * 32 + lr;
                        g.out[prow * g.I + j] =
                            f32_to_bf16(silu_fast(acc[m][n][v]) * acc[m][n + 2][v]);
                    }
                } else {
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        const int c = t.nt * GBN + wn * 128 + n * 32 + lr;
                        g.out[prow * g.d + c] = f32_to_bf16(acc[m][n][v]);
                    }
                }
            }
        }
    };

    int tile = t_begin + (int)(blockIdx.x >> 3);
    if (tile >= t_end) return;
    Tile cur;
    setup(tile, cur);
    prologue(cur);
    int stores = 0;  // epilogue stores issued after the current tile's prologue
    for (;;) {
#pragma unroll
        for (int m = 0; m < MF; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.f;
        if (cur.live) main_loop(cur, std::true_type{}, stores);
        else main_loop(cur, std::false_type{}, stores);
        // the next tile's loads go out before this tile's epilogue, so they
        // overlap its arithmetic and stores; first every wave is done
        // reading this tile's stages
        const int next = tile + per_xcd_wg;
        const bool more = next < t_end;
        Tile nxt;
        if (more) {
            setup(next, nxt);
            wait_lgkm<0>();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            prologue(nxt);
        }
        epilogue(cur);
        if (!more) break;
        stores = wm * WT >= cur.rows_valid ? 0 : 1;
        cur = nxt;
        tile = next;
    }
}

}  // namespace beam
