// Shared device helpers of libmoe (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest, ties to even
// (gfx950 converts in one instruction, v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<unsigned>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values at once: low half = a, high half = b.
__device__ __forceinline__ unsigned f32x2_to_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ unsigned long long ballot(bool p) { return __ballot(p); }

// Mask of the lanes below the calling lane.
__device__ __forceinline__ unsigned long long lanes_below() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int n = __shfl_up(v, off, kWave);
        if (l >= off) v += n;
    }
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Exclusive scan of s[0..n) in LDS in place, n <= 4096, whole block takes
// part (blockDim.x a multiple of 64, at most 1024). Returns the total.
// `scratch` must hold blockDim.x/64 + 1 ints.
__device__ inline int block_exclusive_scan_lds(int* s, int n, int* scratch) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    const int beg = min(n, tid * per);
    const int end = min(n, beg + per);
    int local = 0;
    for (int i = beg; i < end; ++i) local += s[i];
    const int incl = wave_inclusive_scan(local);
    const int w = tid / kWave;
    if (lane_id() == kWave - 1) scratch[w] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < nt / kWave; ++i) {
            int t = scratch[i];
            scratch[i] = run;
            run += t;
        }
        scratch[nt / kWave] = run;
    }
    __syncthreads();
    int run = scratch[w] + incl - local;
    for (int i = beg; i < end; ++i) {
        int t = s[i];
        s[i] = run;
        run += t;
    }
    const int total = scratch[nt / kWave];
    __syncthreads();
    return total;
}

// Workgroup barrier for pipelined loops that keep global loads in flight
// across it. __syncthreads() carries a workgroup fence, for which the
// compiler waits on every outstanding global load. When the barrier only has
// to order LDS accesses, this is enough: each wave's LDS operations are
// complete (lgkmcnt(0)) when it arrives, register values loaded from global
// memory are waited for exactly where they are used, and the asm memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Buffers streamed once and far larger than the 256 MB Infinity Cache are
// read or written with non-temporal accesses past this size.
constexpr long long kStreamBytes = 1LL << 30;

// ------------------------------------------------------------ debug checks
// Device-side preconditions the release build leaves unchecked (the kernels
// only keep every access inside its buffer when they are broken). A build
// with MOE_DEBUG records each broken one as a bit in a device word of the
// source file that checks it; moe_debug_status() ORs and clears them.
enum DebugFlag : unsigned {
    kDbgIdRange = 1u,      // a router id outside [0, E) reached a packing
    kDbgRecvSum = 2u,      // receive counts negative or not summing to N
    kDbgNonFinite = 4u,    // a router score is not finite
    kDbgOffsets = 8u,      // expert offsets: offsets[0] != 0, decreasing or past N
};
#ifdef MOE_DEBUG
static __device__ unsigned g_debug_flags = 0;   // one word per source file
__device__ __forceinline__ void debug_flag(unsigned bit) { atomicOr(&g_debug_flags, bit); }
#define MOE_DBG_CHECK(cond, bit)            \
    do {                                     \
        if (!(cond)) ::moe::debug_flag(bit); \
    } while (0)
// Host side: the flags of this source file (then cleared when `reset`).
#define MOE_DBG_READER(name)                                                          \
    unsigned debug_read_##name(int reset) {                                           \
        unsigned v = 0;                                                               \
        if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_flags), sizeof v) != hipSuccess) \
            return 0x80000000u;                                                       \
        if (reset) {                                                                  \
            const unsigned z = 0;                                                     \
            (void)hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &z, sizeof z);         \
        }                                                                             \
        return v;                                                                     \
    }
#else
#define MOE_DBG_CHECK(cond, bit) \
    do {                         \
    } while (0)
#define MOE_DBG_READER(name) \
    unsigned debug_read_##name(int) { return 0; }
#endif

// Raw buffer resource (stride 0) that starts at `base` and spans `bytes`:
// the hardware drops a store, and returns zeros for a load without touching
// memory, whose offset (the lane's VGPR offset plus the instruction's
// immediate; the scalar offset is kept at 0) is at or past that size. With
// `bytes` = valid rows x row pitch, the rows of a partial tile past its
// expert's segment are dropped (or read as zeros) without a branch per
// access, and every address is a 32-bit offset from one scalar base instead
// of a 64-bit lane pointer.
// The fourth descriptor word is the gfx9 raw-buffer format (32-bit data,
// no swizzle). `base` and `bytes` must be the same in every lane of the
// wavefront: they pass through readfirstlane, which keeps the descriptor in
// scalar registers (a descriptor the compiler holds in vector registers
// becomes a loop over its distinct values around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
    const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
    void* u = reinterpret_cast<void*>((static_cast<unsigned long long>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

}  // namespace moe
