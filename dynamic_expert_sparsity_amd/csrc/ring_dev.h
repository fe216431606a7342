// The weight-streaming expert kernels' bodies (a5-a6 for few pairs per
// expert): BEAM paper, section 3.1 Eq. 3; only experts with active pairs are
// streamed (section 3.2; the news article's section 5).
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// Up and down projections, ring-streamed (bf16, k length % 64 == 0).  A
// unit is (block of up to 32 positions of one expert, column group): 32 rows
// of the expert's weights (up: 16 gate + 16 up rows; down: 32 output
// channels).  A persistent grid of one 8-wave workgroup per CU walks a
// contiguous range of units, streaming them through RING_NS LDS slots in
// k-chunks of 256 with RING_NS - 1 chunks in flight, so the reduction that
// ends a unit overlaps the loads of the next.  A slot holds the chunk's 32
// weight rows (512 B each, 16-byte piece c of row r at c ^ (r % 16)) and, per
// wave, that wave's 32-wide k-slice of the block's x rows (64 B each, piece
// c of position p at c ^ ((p / 4) % 4)): every operand arrives through
// global_load_lds (weights non-temporal: read once), so the MFMAs read only
// LDS and the compiler tracks no in-flight register loads.  Waits are
// explicit vmcnt counts per wave: a chunk is 2 weight loads and 1 or 2 x
// loads; the h stores that end a unit are not counted, which only makes the
// next waits stricter.  A k length that is not a multiple of 256 ends in a
// short chunk: its loads past the row end are pointed at the chunk's start
// (in bounds, never used) and the waves whose k-slice lies past the end skip
// their MFMAs for it.
// ---------------------------------------------------------------------------
constexpr int RING_NS = 4;                         // LDS slots
constexpr int RING_W = 32 * 512;                   // weight rows of a slot
constexpr int RING_X = 8 * 2 * 1024;               // x: 8 waves x 2 blocks of 16 positions
constexpr int RING_SLOT = RING_W + RING_X;         // 32 KB
constexpr int RING_LDS = RING_NS * RING_SLOT + 8 * 4 * 64 * 16;  // + partial sums (160 KB)

template <int N>
__device__ __forceinline__ void ring_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 0x3) << 14));
}
// at most n vector-memory operations of this wave in flight (n a sum of up to
// two chunks of 3 or 4)
__device__ __forceinline__ void ring_wait_le(int n) {
    if (n >= 8) ring_wait_vm<8>();
    else if (n >= 7) ring_wait_vm<7>();
    else if (n >= 6) ring_wait_vm<6>();
    else if (n >= 4) ring_wait_vm<4>();
    else if (n >= 3) ring_wait_vm<3>();
    else ring_wait_vm<0>();
}
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
template <int AUX>
__device__ __forceinline__ void ring_dma(const void *g, unsigned char *l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 16, 0, AUX);
}

// DOWN = false: up projection (A = x rows of the block's tokens, B = the 16
// gate and 16 up rows of a column group of 16 units; out h = SiLU(a) * u).
// DOWN = true: down projection (A = the block's h rows, B = 32 rows of W_dt,
// one per output channel of a column group of 32; out o).  klen = d (up) or
// I (down), a multiple of 64; ncols = I (up) or d (down).
template <bool DOWN, bool TAIL>
__device__ __forceinline__ void ring1_body(
    const bf16_t *__restrict__ A, const bf16_t *__restrict__ W,
    const int32_t *__restrict__ pbt, const int32_t *__restrict__ mrec,
    const int32_t *__restrict__ sorted_tok, bf16_t *__restrict__ out, int klen, int ncols,
    int check_mode) {
    constexpr int NS = RING_NS;
    extern __shared__ __align__(16) unsigned char lds[];
    f32x4 *red = reinterpret_cast<f32x4 *>(lds + NS * RING_SLOT);  // [wave][2 col blocks x 2 row blocks][lane]
    // mrec = {kernel family, max count, records, layout}; family 1 or 2: the tiled kernels take this call
    if (check_mode && mrec[0] != 0) return;
    const int NCH = (klen + 255) >> 8;             // k-chunks of 256 per row (last may be short)
    // elements of a short last chunk (TAIL instances only; else klen % 256 == 0)
    const int tail = TAIL ? (klen & 255) : 0;
    const int ncg = DOWN ? ncols >> 5 : ncols >> 4;  // column groups per position block
    const int NU = mrec[2] * ncg;
    const int G = gridDim.x, b = blockIdx.x;
    const int u_begin = (int)((long long)NU * b / G);
    const int u_end = (int)((long long)NU * (b + 1) / G);
    if (u_end <= u_begin) return;
    const int nch = (u_end - u_begin) * NCH;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, kg = lane >> 4;

    // request side: the unit whose chunks are being loaded
    int iu = -1, i_rows = 0, i_pos0 = 0, i_cg = 0;
    const bf16_t *wrow0 = W, *wrow1 = W;  // this lane's two weight rows (+ chunk)
    const bf16_t *xa0 = A, *xa1 = A;      // this lane's A source for row blocks 0 / 1 (+ chunk)
    // per slot: this wave's vector-memory ops for the chunk in it, and, when
    // it is the last chunk of its unit, the unit's (first position, rows,
    // column group) for the stores (requests run up to NS - 1 chunks, which
    // can be several units, ahead of the compute)
    int ld[NS], spos[NS], srow[NS], scg[NS];

    // weight loads: instruction i covers rows 4 wave + 2 i + {0, 1}; lane l
    // fetches piece (l % 32) ^ (r % 16) of row r = 4 wave + 2 i + l / 32
    const int wr0 = 4 * wave + (lane >> 5), wr1 = wr0 + 2;
    const int wp0 = (lane & 31) ^ (wr0 & 15), wp1 = (lane & 31) ^ (wr1 & 15);  // weight pieces
    // A loads: lane l -> position 16 blk + l / 4, piece (l % 4) ^ ((l / 16) % 4)
    const int xp = lane >> 2;
    const int xpiece = (lane & 3) ^ ((lane >> 4) & 3);
    // row of the unit's 32 weight rows -> row of W[e] (up: gate rows, then up rows)
    auto wmap = [&](int r, int cg) {
        return DOWN ? cg * 32 + r : (r < 16 ? cg * 16 + r : ncols + cg * 16 + (r - 16));
    };

    auto issue = [&](int jj, int q) {  // chunk jj into slot q (static)
        const int uu = jj / NCH, c = jj - uu * NCH;
        if (uu != iu) {
            iu = uu;
            const int U = u_begin + uu;
            const int pbi = U / ncg, cg = U - pbi * ncg;
            const int4 rec = *reinterpret_cast<const int4 *>(pbt + 4 * pbi);
            const int e = rec.x, pos0 = rec.y, rows = rec.z;
            const size_t wrows = DOWN ? (size_t)ncols : (size_t)2 * ncols;  // rows of W[e]
            const bf16_t *we = W + (size_t)e * wrows * klen;
            wrow0 = we + (size_t)wmap(wr0, cg) * klen + (wp0 << 3);
            wrow1 = we + (size_t)wmap(wr1, cg) * klen + (wp1 << 3);
            int a0, a1;  // A rows of this lane's positions xp and 16 + xp
            if (DOWN) {
                a0 = pos0 + (xp < rows ? xp : 0);
                a1 = pos0 + (16 + xp < rows ? 16 + xp : 0);
            } else {
                // token ids of the block's positions (scalar loads); past rows: token 0
                const int *st = sorted_tok + pos0;
                int t0 = st[0], t1 = st[16];
#pragma unroll
                for (int j = 1; j < 16; ++j) {
                    const int v0 = st[j], v1 = st[16 + j];
                    t0 = xp == j ? v0 : t0;
                    t1 = xp == j ? v1 : t1;
                }
                a0 = xp < rows ? t0 : 0;
                a1 = 16 + xp < rows ? t1 : 0;
            }
            xa0 = A + (size_t)a0 * klen + wave * 32 + xpiece * 8;
            xa1 = A + (size_t)a1 * klen + wave * 32 + xpiece * 8;
            i_rows = rows;
            i_pos0 = pos0;
            i_cg = cg;
        }
        if (c == NCH - 1) {
            spos[q] = i_pos0;
            srow[q] = i_rows;
            scg[q] = i_cg;
        }
        unsigned char *sl = lds + q * RING_SLOT;
        // a short last chunk: pieces past the row end load the chunk's start instead
        const bool shrt = TAIL && tail != 0 && c == NCH - 1;
        const int w0o = shrt && (wp0 << 3) >= tail ? -(wp0 << 3) : 0;
        const int w1o = shrt && (wp1 << 3) >= tail ? -(wp1 << 3) : 0;
        const int xo = shrt && wave * 32 >= tail ? -(wave * 32 + xpiece * 8) : 0;
        ring_dma<2>(wrow0 + c * 256 + w0o, sl + (4 * wave) * 512);
        ring_dma<2>(wrow1 + c * 256 + w1o, sl + (4 * wave + 2) * 512);
        unsigned char *xs = sl + RING_W + wave * 2048;
        ring_dma<0>(xa0 + c * 256 + xo, xs);
        if (i_rows > 16) {
            ring_dma<0>(xa1 + c * 256 + xo, xs + 1024);
            ld[q] = 4;
        } else {
            ld[q] = 3;
        }
    };

    f32x4 c00 = {0.f, 0.f, 0.f, 0.f}, c10 = c00, c01 = c00, c11 = c00;  // [col block][row block]
#pragma unroll
    for (int q = 0; q < NS; ++q) ld[q] = spos[q] = srow[q] = scg[q] = 0;
#pragma unroll
    for (int q = 0; q < NS - 1; ++q)
        if (q < nch) issue(q, q);
    for (int j0 = 0; j0 < nch; j0 += NS) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int j = j0 + q;
            if (j >= nch) break;
            // chunk j landed: only the chunks requested after it may be in flight
            int later = 0;
#pragma unroll
            for (int t = 1; t <= NS - 2; ++t)
                if (j + t < nch) later += ld[(q + t) % NS];
            ring_wait_le(later);
            ring_barrier();  // every wave's part of chunk j is in; slot of chunk j - 1 is free
            const bool rb1 = ld[q] == 4;
            if (j + NS - 1 < nch) issue(j + NS - 1, (q + NS - 1) % NS);
            // this wave's 32-wide k-slice: one k-step of 32
            const unsigned char *sl = lds + q * RING_SLOT;
            const int gc = 4 * wave + kg;  // 16-byte piece of the weight row
            const u32x4 w0 = *reinterpret_cast<const u32x4 *>(sl + li * 512 + ((gc ^ li) << 4));
            const u32x4 w1 = *reinterpret_cast<const u32x4 *>(sl + (16 + li) * 512 + ((gc ^ li) << 4));
            const unsigned char *xs = sl + RING_W + wave * 2048;
            const int xo = li * 64 + ((kg ^ ((li >> 2) & 3)) << 4);
            const int uu = j / NCH;
            // this wave's k-slice lies past the end of a short last chunk
            const bool idle = TAIL && tail != 0 && j - uu * NCH == NCH - 1 && wave * 32 >= tail;
            if (!idle) {
                const u32x4 a0 = *reinterpret_cast<const u32x4 *>(xs + xo);
                c00 = mfma16x16x32(a0, w0, c00);
                c10 = mfma16x16x32(a0, w1, c10);
                if (rb1) {
                    const u32x4 a1 = *reinterpret_cast<const u32x4 *>(xs + 1024 + xo);
                    c01 = mfma16x16x32(a1, w0, c01);
                    c11 = mfma16x16x32(a1, w1, c11);
                }
            }
            if (j - uu * NCH == NCH - 1) {
                // unit done: the eight waves' partial sums meet in LDS
                red[(wave * 4 + 0) * 64 + lane] = c00;
                red[(wave * 4 + 1) * 64 + lane] = c10;
                red[(wave * 4 + 2) * 64 + lane] = c01;
                red[(wave * 4 + 3) * 64 + lane] = c11;
                __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0)
                ring_barrier();
                // all 512 threads reduce: thread t -> row block t / 256, lane
                // (t / 4) % 64 of the partials, component t % 4 (one output
                // row), summing the eight waves in order
                const int rows = srow[q];
                const int tt = threadIdx.x, rb = tt >> 8, L = (tt >> 2) & 63, comp = tt & 3;
                const float *rf = reinterpret_cast<const float *>(red);
                if (rb == 0 || rows > 16) {
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        s0 += rf[((w * 4 + 2 * rb) * 64 + L) * 4 + comp];
                        s1 += rf[((w * 4 + 2 * rb + 1) * 64 + L) * 4 + comp];
                    }
                    // D layout of a 16x16 MFMA: lane L holds column L % 16, rows 4 (L / 16) + comp
                    const int row = 16 * rb + 4 * (L >> 4) + comp;
                    if (row < rows) {
                        bf16_t *o = out + (size_t)(spos[q] + row) * ncols;
                        const int cg = scg[q];
                        if (DOWN) {
                            o[cg * 32 + (L & 15)] = f32_to_bf16(s0);
                            o[cg * 32 + 16 + (L & 15)] = f32_to_bf16(s1);
                        } else {
                            o[cg * 16 + (L & 15)] = f32_to_bf16(silu<false>(s0) * s1);
                        }
                    }
                }
                c00 = f32x4{0.f, 0.f, 0.f, 0.f};
                c10 = c00;
                c01 = c00;
                c11 = c00;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The same projections with two column groups per unit, taken per call when
// the blocks hold more positions (the compaction's layout flag: at least 6
// routed pairs per block of 32 on average), where the x loads of the ring
// above cost about as much as its weight loads: its x rows are then mostly
// distinct tokens, and with more than 16 positions a block needs two x
// loads per chunk.  A unit is (block of up to 32 positions, pair of column
// groups): 64 weight rows, so each k-chunk of the block's x rows serves 64
// weight rows.  The work is still split over the grid in column groups (half
// units), so a workgroup's range may begin or end with half a unit.  A slot
// holds the chunk's 64 weight rows (same swizzle) and the block's x rows as
// eight 32-wide k-slices (same layout as above); wave w loads weight rows
// 8w..8w+7 and k-slice w of x, and computes column group w / 4 of the unit
// over the 64-wide k range w % 4.  A chunk is 4 weight loads per wave (none
// when the wave's column group is outside the range) and 1 or 2 x loads.
// Three slots of 48 KB; the four k-range partial sums of each column group
// meet in the slot of the unit's last chunk once every wave's reads of it
// are complete.  Short last chunks as above (k ranges of 64 lie wholly
// inside or past the end, the k length being a multiple of 64).
// ---------------------------------------------------------------------------
constexpr int RING2_NS = 3;                         // LDS slots
constexpr int RING2_W = 64 * 512;                   // weight rows of a slot
constexpr int RING2_X = 8 * 2 * 1024;               // x: 8 k-slices x 2 blocks of 16 positions
constexpr int RING2_SLOT = RING2_W + RING2_X;         // 48 KB
constexpr int RING2_LDS = RING2_NS * RING2_SLOT;      // 144 KB (partial sums reuse a slot)
static_assert(8 * 4 * 64 * 16 <= RING2_SLOT, "a unit's partial sums fit one slot");

// at most n vector-memory operations of this wave in flight (n: 0 or the
// 1, 2, 5 or 6 operations of one chunk)
__device__ __forceinline__ void ring2_wait_le(int n) {
    if (n >= 6) ring_wait_vm<6>();
    else if (n >= 5) ring_wait_vm<5>();
    else if (n >= 2) ring_wait_vm<2>();
    else if (n >= 1) ring_wait_vm<1>();
    else ring_wait_vm<0>();
}
// DOWN as for ring1_body; ncols = I (up, a multiple of 32) or d (down, a
// multiple of 64).
template <bool DOWN, bool TAIL>
__device__ __forceinline__ void ring2_body(
    const bf16_t *__restrict__ A, const bf16_t *__restrict__ W,
    const int32_t *__restrict__ pbt, const int32_t *__restrict__ mrec,
    const int32_t *__restrict__ sorted_tok, bf16_t *__restrict__ out, int klen, int ncols,
    int check_mode) {
    constexpr int NS = RING2_NS;
    extern __shared__ __align__(16) unsigned char lds[];
    // mrec = {kernel family, max count, records, layout}; family 1 or 2: the tiled kernels take this call
    if (check_mode && mrec[0] != 0) return;
    const int NCH = (klen + 255) >> 8;             // k-chunks of 256 per row (last may be short)
    // elements of a short last chunk (TAIL instances only; else klen % 256 == 0)
    const int tail = TAIL ? (klen & 255) : 0;
    const int ncp = DOWN ? ncols >> 6 : ncols >> 5;  // column-group pairs per position block
    const int NH = 2 * mrec[2] * ncp;                // half units
    const int G = gridDim.x, b = blockIdx.x;
    const int h_begin = (int)((long long)NH * b / G);
    const int h_end = (int)((long long)NH * (b + 1) / G);
    if (h_end <= h_begin) return;
    const int u_first = h_begin >> 1;
    const int nch = (((h_end - 1) >> 1) - u_first + 1) * NCH;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, kg = lane >> 4;
    const int kq = wave & 3, half = wave >> 2;       // compute: k range, half of the rows

    // request side: the unit whose chunks are being loaded
    int iu = -1, i_rows = 0, i_pos0 = 0, i_cp = 0, i_hm = 0;
    const bf16_t *wrow[4] = {W, W, W, W};  // this lane's four weight rows (+ chunk)
    const bf16_t *xa0 = A, *xa1 = A;        // this lane's A source for row blocks 0 / 1 (+ chunk)
    // per slot: this wave's vector-memory ops for the chunk in it, the
    // chunk's halves present (bits 0, 1) and second row block (bit 2), and,
    // when it is the last chunk of its unit, the unit's (first position,
    // rows, column-group pair) for the stores (requests run up to NS - 1
    // chunks, which can be several units, ahead of the compute)
    int ld[NS], fl[NS], spos[NS], srow[NS], scp[NS];

    // weight loads: instruction i covers rows 8 wave + 2 i + {0, 1}; lane l
    // fetches piece (l % 32) ^ (r % 16) of row r = 8 wave + 2 i + l / 32
    int wpc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wpc[i] = (lane & 31) ^ ((8 * wave + 2 * i + (lane >> 5)) & 15);
    // A loads: lane l -> position 16 blk + l / 4, piece (l % 4) ^ ((l / 16) % 4) of k-slice wave
    const int xp = lane >> 2;
    const int xpiece = (lane & 3) ^ ((lane >> 4) & 3);
    // row of the unit's 64 weight rows -> row of W[e] (up: per column group
    // 16 gate rows, then 16 up rows)
    auto wmap = [&](int r, int cp) {
        if (DOWN) return cp * 64 + r;
        const int g = 2 * cp + (r >> 5), rr = r & 31;
        return rr < 16 ? g * 16 + rr : ncols + g * 16 + (rr - 16);
    };

    auto issue = [&](int jj, int q) {  // chunk jj into slot q (static)
        const int uu = jj / NCH, c = jj - uu * NCH;
        if (uu != iu) {
            iu = uu;
            const int U = u_first + uu;
            const int pbi = U / ncp, cp = U - pbi * ncp;
            const int4 rec = *reinterpret_cast<const int4 *>(pbt + 4 * pbi);
            const int e = rec.x, pos0 = rec.y, rows = rec.z;
            const size_t wrows = DOWN ? (size_t)ncols : (size_t)2 * ncols;  // rows of W[e]
            const bf16_t *we = W + (size_t)e * wrows * klen;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wrow[i] = we + (size_t)wmap(8 * wave + 2 * i + (lane >> 5), cp) * klen + (wpc[i] << 3);
            int a0, a1;  // A rows of this lane's positions xp and 16 + xp
            if (DOWN) {
                a0 = pos0 + (xp < rows ? xp : 0);
                a1 = pos0 + (16 + xp < rows ? 16 + xp : 0);
            } else {
                // token ids of the block's positions (scalar loads); past rows: token 0
                const int *st = sorted_tok + pos0;
                int t0 = st[0], t1 = st[16];
#pragma unroll
                for (int j = 1; j < 16; ++j) {
                    const int v0 = st[j], v1 = st[16 + j];
                    t0 = xp == j ? v0 : t0;
                    t1 = xp == j ? v1 : t1;
                }
                a0 = xp < rows ? t0 : 0;
                a1 = 16 + xp < rows ? t1 : 0;
            }
            xa0 = A + (size_t)a0 * klen + wave * 32 + xpiece * 8;
            xa1 = A + (size_t)a1 * klen + wave * 32 + xpiece * 8;
            i_rows = rows;
            i_pos0 = pos0;
            i_cp = cp;
            // halves of this unit inside the range [h_begin, h_end)
            i_hm = (2 * U >= h_begin ? 1 : 0) | (2 * U + 1 < h_end ? 2 : 0);
        }
        if (c == NCH - 1) {
            spos[q] = i_pos0;
            srow[q] = i_rows;
            scp[q] = i_cp;
        }
        unsigned char *sl = lds + q * RING2_SLOT;
        // a short last chunk: pieces past the row end load the chunk's start instead
        const bool shrt = TAIL && tail != 0 && c == NCH - 1;
        int n = 0;
        if ((i_hm >> (wave >> 2)) & 1) {  // this wave's weight rows lie in a present half
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int wo = shrt && (wpc[i] << 3) >= tail ? -(wpc[i] << 3) : 0;
                ring_dma<2>(wrow[i] + c * 256 + wo, sl + (8 * wave + 2 * i) * 512);
            }
            n = 4;
        }
        const int xo = shrt && wave * 32 >= tail ? -(wave * 32 + xpiece * 8) : 0;
        unsigned char *xs = sl + RING2_W + wave * 2048;
        ring_dma<0>(xa0 + c * 256 + xo, xs);
        if (i_rows > 16) {
            ring_dma<0>(xa1 + c * 256 + xo, xs + 1024);
            n += 2;
        } else {
            n += 1;
        }
        ld[q] = n;
        fl[q] = i_hm | (i_rows > 16 ? 4 : 0);
    };

    f32x4 c00 = {0.f, 0.f, 0.f, 0.f}, c10 = c00, c01 = c00, c11 = c00;  // [col block][row block]
#pragma unroll
    for (int q = 0; q < NS; ++q) ld[q] = fl[q] = spos[q] = srow[q] = scp[q] = 0;
#pragma unroll
    for (int q = 0; q < NS - 1; ++q)
        if (q < nch) issue(q, q);
    for (int j0 = 0; j0 < nch; j0 += NS) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int j = j0 + q;
            if (j >= nch) break;
            // chunk j landed: only the chunks requested after it may be in flight
            int later = 0;
#pragma unroll
            for (int t = 1; t <= NS - 2; ++t)
                if (j + t < nch) later += ld[(q + t) % NS];
            ring2_wait_le(later);
            ring_barrier();  // every wave's part of chunk j is in; slot of chunk j - 1 is free
            const int f = fl[q];
            if (j + NS - 1 < nch) issue(j + NS - 1, (q + NS - 1) % NS);
            unsigned char *sl = lds + q * RING2_SLOT;
            const int uu = j / NCH;
            const bool last = j - uu * NCH == NCH - 1;
            // this wave's k range lies past the end of a short last chunk
            const bool idle = TAIL && tail != 0 && last && kq * 64 >= tail;
            if (!idle && ((f >> half) & 1)) {
                const int xo = li * 64 + ((kg ^ ((li >> 2) & 3)) << 4);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int s = 2 * kq + ks;   // k-slice
                    const int gc = 4 * s + kg;   // 16-byte piece of the weight row
                    const u32x4 w0 = *reinterpret_cast<const u32x4 *>(sl + (32 * half + li) * 512 + ((gc ^ li) << 4));
                    const u32x4 w1 =
                        *reinterpret_cast<const u32x4 *>(sl + (32 * half + 16 + li) * 512 + ((gc ^ li) << 4));
                    const unsigned char *xs = sl + RING2_W + s * 2048;
                    const u32x4 a0 = *reinterpret_cast<const u32x4 *>(xs + xo);
                    c00 = mfma16x16x32(a0, w0, c00);
                    c10 = mfma16x16x32(a0, w1, c10);
                    if (f & 4) {
                        const u32x4 a1 = *reinterpret_cast<const u32x4 *>(xs + 1024 + xo);
                        c01 = mfma16x16x32(a1, w0, c01);
                        c11 = mfma16x16x32(a1, w1, c11);
                    }
                }
            }
            if (last) {
                // unit done: the partial sums meet in this slot once every
                // wave's reads of it are complete
                __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0)
                ring_barrier();
                f32x4 *red = reinterpret_cast<f32x4 *>(sl);  // [wave][2 col blocks x 2 row blocks][lane]
                red[(wave * 4 + 0) * 64 + lane] = c00;
                red[(wave * 4 + 1) * 64 + lane] = c10;
                red[(wave * 4 + 2) * 64 + lane] = c01;
                red[(wave * 4 + 3) * 64 + lane] = c11;
                __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0)
                ring_barrier();
                // all 512 threads reduce: thread t -> row block t / 256, lane
                // (t / 4) % 64 of the partials, component t % 4 (one output
                // row), per present half summing its four k ranges in order
                const int rows = srow[q];
                const int tt = threadIdx.x, rb = tt >> 8, L = (tt >> 2) & 63, comp = tt & 3;
                const float *rf = reinterpret_cast<const float *>(red);
                // D layout of a 16x16 MFMA: lane L holds column L % 16, rows 4 (L / 16) + comp
                const int row = 16 * rb + 4 * (L >> 4) + comp;
                if (row < rows) {
                    bf16_t *o = out + (size_t)(spos[q] + row) * ncols;
                    const int cp = scp[q];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if (!((f >> hh) & 1)) continue;
                        float s0 = 0.f, s1 = 0.f;
#pragma unroll
                        for (int k4 = 0; k4 < 4; ++k4) {
                            const int w = 4 * hh + k4;
                            s0 += rf[((w * 4 + 2 * rb) * 64 + L) * 4 + comp];
                            s1 += rf[((w * 4 + 2 * rb + 1) * 64 + L) * 4 + comp];
                        }
                        if (DOWN) {
                            o[cp * 64 + hh * 32 + (L & 15)] = f32_to_bf16(s0);
                            o[cp * 64 + hh * 32 + 16 + (L & 15)] = f32_to_bf16(s1);
                        } else {
                            o[(2 * cp + hh) * 16 + (L & 15)] = f32_to_bf16(silu<false>(s0) * s1);
                        }
                    }
                }
                c00 = f32x4{0.f, 0.f, 0.f, 0.f};
                c10 = c00;
                c01 = c00;
                c11 = c00;
            }
        }
    }
}

}  // namespace beam
