// Measured peaks of the GPU the layer runs on: a streaming copy, a streaming
// read and a loop of bf16 matrix instructions with no memory traffic.  They
// give the attainable HBM bandwidth and MFMA rate that the layer's kernels
// are compared against, next to the vendor figures (8 TB/s, 2.5 PFLOP/s).
//
// Built as its own library (libbeam_peak.so), apart from the layer's
// C-ABI.  Every entry point returns 0 or a HIP error code; they enqueue on
// the given stream and do not synchronise.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BLOCK = 256;      // threads of the copy's and the MFMA loop's workgroups
constexpr int SBLOCK = 512;     // threads of the read's workgroups
constexpr int PER_THREAD = 16;  // 16-byte elements per thread per round
constexpr int ROUND = SBLOCK * PER_THREAD;  // elements of a workgroup round (128 KB)

typedef float f32x16_t __attribute__((ext_vector_type(16)));

int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

// Copy: workgroup b copies the contiguous elements [b*BLOCK*PER_THREAD, ...)
// of n 16-byte elements: every wave instruction moves 1 KB, all PER_THREAD
// loads of a thread are in flight before its stores (one round per
// workgroup measured faster than persistent workgroups for the copy).
__global__ __launch_bounds__(BLOCK) void copy16(const u32x4_t *__restrict__ src,
                                                u32x4_t *__restrict__ dst, size_t n) {
    const size_t base = (size_t)blockIdx.x * BLOCK * PER_THREAD + threadIdx.x;
    u32x4_t v[PER_THREAD];
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
        const size_t i = base + (size_t)u * BLOCK;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
        const size_t i = base + (size_t)u * BLOCK;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

// Read: persistent workgroups (two per CU); workgroup b takes the 128 KB
// rounds b, b + G, ... of the n 16-byte elements, so at any time the grid
// works through one contiguous window; every wave instruction moves 1 KB and
// a thread's PER_THREAD loads of a round are in flight together (7.0-7.1
// TB/s where one round per workgroup gave 6.9).  The xor of everything a
// thread read is stored only if it equals a value that the caller's data does
// not produce in practice, so the loads stay and nothing is written.
__global__ __launch_bounds__(SBLOCK) void read16(const u32x4_t *__restrict__ src, size_t n,
                                                 u32x4_t *__restrict__ sink) {
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (size_t r0 = (size_t)blockIdx.x * ROUND; r0 < n; r0 += (size_t)gridDim.x * ROUND) {
        const size_t base = r0 + threadIdx.x;
        u32x4_t v[PER_THREAD];
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const size_t i = base + (size_t)u * SBLOCK;
            v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) acc ^= v[u];
    }
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0x85ebca6bu &&
        acc[3] == 0xc2b2ae35u)
        sink[0] = acc;
}

constexpr int CHAINS = 4;  // independent accumulators per wave

// iters x CHAINS 32x32x16 bf16 MFMAs per wave, operands held in registers;
// the CHAINS accumulators are independent, so consecutive instructions never
// wait on each other.
__global__ __launch_bounds__(BLOCK) void mfma_loop(int iters, f32x4_t *__restrict__ sink) {
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (float)threadIdx.x + (float)j);
        b[j] = (__bf16)(0.5f * (float)j);
    }
    f32x16_t acc[CHAINS] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    if (s == 12345.f) sink[0] = f32x4_t{s, s, s, s};
}

// two read workgroups per CU, fewer when there are fewer rounds
unsigned stream_grid(size_t n) {
    const size_t rounds = (n + ROUND - 1) / ROUND;
    const size_t g = (size_t)cu_count() * 2;
    return (unsigned)(rounds < g ? rounds : g);
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16, 16-byte aligned pointers) from src to dst.
int beam_peak_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16 != 0) return (int)hipErrorInvalidValue;
    const size_t n = bytes / 16, per = (size_t)BLOCK * PER_THREAD;
    if (n == 0) return 0;
    copy16<<<(unsigned)((n + per - 1) / per), BLOCK, 0, stream>>>((const u32x4_t *)src,
                                                                  (u32x4_t *)dst, n);
    return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from src; sink: 16 bytes of device memory.
int beam_peak_read(const void *src, size_t bytes, void *sink, hipStream_t stream) {
    if (!src || !sink || bytes % 16 != 0) return (int)hipErrorInvalidValue;
    const size_t n = bytes / 16;
    if (n == 0) return 0;
    read16<<<stream_grid(n), SBLOCK, 0, stream>>>((const u32x4_t *)src, n, (u32x4_t *)sink);
    return (int)hipGetLastError();
}

// Runs the MFMA loop; *flops receives the floating-point operations it does.
// sink: 16 bytes of device memory.
int beam_peak_mfma(int iters, void *sink, double *flops, hipStream_t stream) {
    if (iters <= 0 || !sink || !flops) return (int)hipErrorInvalidValue;
    const int blocks = cu_count() * 8;
    mfma_loop<<<blocks, BLOCK, 0, stream>>>(iters, (f32x4_t *)sink);
    *flops = (double)blocks * (BLOCK / 64) * (double)iters * CHAINS * (2.0 * 32 * 32 * 16);
    return (int)hipGetLastError();
}

}  // extern "C"
