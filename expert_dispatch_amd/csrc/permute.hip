// Expert-major packing and the receive-side reorder.
//
// "Three axes of Parallelism", Expert Parallel (EP) -> Producing assignments:
// count the assignments routed to each expert, take offsets from the
// cumulative counts, and write every assignment into its expert's region of
// the packed buffer. Same page, Dispatch, expert computation and combine: a
// received buffer is source-major and is permuted expert-major with counts
// recv_matrix.sum(0) and their cumulative sums as offsets. The Modalities EP
// page (Design) builds those indices on the device with no readback.
//
// Token-routed packing, three launches and no host synchronisation:
//  1. perm_hist:  per-chunk expert histogram in LDS (512, 1024 or 4096
//                 assignments per block: small batches get more blocks, large
//                 ones fewer chunk histograms for every ranking block to sum);
//  2. perm_rank:  every block re-derives the global offsets and its own base
//                 per expert from the chunk histograms, then ranks its
//                 assignments stably with wave ballots (a bit-sliced match of
//                 equal expert ids, popcount of the lanes below) -> dest and
//                 perm_src; no atomics decide a position, so the result is the
//                 unique stable order;
//  3. perm_gather: one wavefront per token reads its row once with 16-byte
//                 loads and writes it to its k packed rows.
// The receive-side reorder is one launch: each block rebuilds the (sender,
// expert) block starts from the count matrix in LDS, then each wavefront maps
// its rows and copies them.
#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermMaxE = 1024;
constexpr int kPermSmallTK = 65536;   // up to this many assignments: 1024-chunks
constexpr int kPermTinyTK = 32768;    // up to this many: 512-chunks

// assignments per ranking block
static int perm_chunk(long long TK) {
    return TK <= kPermTinyTK ? 512 : (TK <= kPermSmallTK ? 1024 : 4096);
}

// e_base: the packing covers global expert ids [e_base, e_base + E) (an
// expert-parallel rank's range); any other id is dropped.
// id_hi: router ids are expected in [0, id_hi) (checked in debug builds only)
template <int CHUNK>
__global__ __launch_bounds__(kPermThreads) void perm_hist_kernel(
    const int32_t* __restrict__ idx, int TK, int e_base, int E, int id_hi,
    int32_t* __restrict__ bc)
{
    constexpr int kPermIters = CHUNK / kPermThreads;
    __shared__ int h[kPermMaxE];
    for (int e = threadIdx.x; e < E; e += kPermThreads) h[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * CHUNK;
#pragma unroll 4
    for (int q = 0; q < kPermIters; ++q) {
        const int a = base + threadIdx.x + q * kPermThreads;
        if (a < TK) {
            const int id = idx[a];
            MOE_DBG_CHECK(id >= 0 && id < id_hi, kDbgIdRange);
            (void)id_hi;
            const int e = id - e_base;
            if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kPermThreads) bc[(size_t)blockIdx.x * E + e] = h[e];
}

// cap: assignments an expert keeps (its first cap in ascending a; INT_MAX =
// all); routed (may be null) receives the per-expert counts before the cap.
template <int CHUNK>
__global__ __launch_bounds__(kPermThreads) void perm_rank_kernel(
    const int32_t* __restrict__ idx, int TK, int e_base, int E, int nbits, int cap,
    const int32_t* __restrict__ bc, int nb,
    int32_t* __restrict__ routed, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ dest)
{
    constexpr int kPermIters = CHUNK / kPermThreads;   // per lane
    __shared__ int s_off[kPermMaxE];       // offsets of the kept assignments
    __shared__ int s_base[kPermMaxE];      // assignments of earlier blocks (rank base)
    __shared__ int s_wcnt[4][kPermMaxE];   // per-wave running counts, then wave bases
    __shared__ int s_scan[kPermThreads / kWave + 1];

    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = lane_id();

    for (int e = tid; e < E; e += kPermThreads) {
        // the chunk histograms of expert e, eight loads in flight at a time
        int tot = 0, pre = 0;
        int b = 0;
        for (; b + 8 <= nb; b += 8) {
            int c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = bc[(size_t)(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                tot += c[u];
                if (b + u < (int)blockIdx.x) pre += c[u];
            }
        }
        for (; b < nb; ++b) {
            const int c = bc[(size_t)b * E + e];
            tot += c;
            if (b < (int)blockIdx.x) pre += c;
        }
        const int kept = min(tot, cap);
        s_off[e] = kept;
        s_base[e] = pre;
        if (blockIdx.x == 0) {
            counts[e] = kept;
            if (routed) routed[e] = tot;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) s_wcnt[q][e] = 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan_lds(s_off, E, s_scan);
    if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += kPermThreads) offsets[e] = s_off[e];
        if (tid == 0) offsets[E] = total;
    }
    __syncthreads();

    // stable ranks inside this wave's CHUNK/4 consecutive assignments
    volatile int* wc = s_wcnt[w];
    const int a0 = blockIdx.x * CHUNK + w * (CHUNK / 4);
    int loc[kPermIters];
    int key[kPermIters];
#pragma unroll
    for (int it = 0; it < kPermIters; ++it) {
        const int a = a0 + it * kWave + lane;
        int e = (a < TK) ? idx[a] - e_base : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        if (!valid) e = -1;
        unsigned long long m = ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const unsigned long long bb = ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const unsigned long long below = m & lanes_below();
        int prior = 0;
        if (valid) prior = wc[e];
        __builtin_amdgcn_wave_barrier();
        if (valid && below == 0) wc[e] = prior + __popcll(m);
        __builtin_amdgcn_wave_barrier();
        loc[it] = prior + __popcll(below);
        key[it] = e;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) {
        int run = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = s_wcnt[q][e];
            s_wcnt[q][e] = run;
            run += t;
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kPermIters; ++it) {
        const int a = a0 + it * kWave + lane;
        if (a >= TK) continue;
        const int e = key[it];
        int j = -1;
        if (e >= 0) {
            const int r = s_base[e] + s_wcnt[w][e] + loc[it];   // rank inside expert e
            j = r < cap ? s_off[e] + r : -1;
            if (j >= total) j = -1;
        }
        dest[a] = j;
        if (j >= 0) perm_src[j] = a;
    }
}

// x_perm[dest[t*k+s]] = x[t]: one wavefront per token, V-byte vectors;
// packed rows are out_stride vectors apart. NTS: non-temporal stores.
template <typename V, bool NTS>
__global__ __launch_bounds__(256) void perm_gather_kernel(
    const V* __restrict__ x, int vecs_per_row, int T, int k, const int32_t* __restrict__ dest,
    int rows_out, V* __restrict__ x_perm, int out_stride)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const int my_dest = lane < k ? dest[(size_t)t * k + lane] : -1;
    const V* src = x + (size_t)t * vecs_per_row;
    constexpr int U = 4;
    for (int c0 = 0; c0 < vecs_per_row; c0 += kWave * U) {
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave + lane;
            if (c < vecs_per_row) v[u] = src[c];
        }
        for (int s = 0; s < k; ++s) {
            const int j = __shfl(my_dest, s, kWave);
            if ((unsigned)j >= (unsigned)rows_out) continue;
            V* dst = x_perm + (size_t)j * out_stride;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave + lane;
                if (c < vecs_per_row) {
                    if constexpr (NTS) __builtin_nontemporal_store(v[u], dst + c);
                    else dst[c] = v[u];
                }
            }
        }
    }
}

constexpr int kRecvMaxCells = 4096;
constexpr int kRecvRowsPerBlock = 16;

template <typename V>
__global__ __launch_bounds__(256) void perm_recv_kernel(
    const int32_t* __restrict__ recv, int S, int E, int N,
    const V* __restrict__ x, int vecs_per_row,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ dest, V* __restrict__ x_perm,
    int out_stride)
{
    __shared__ int s_start[kRecvMaxCells];   // first received row of cell (i,j)
    __shared__ int s_dbase[kRecvMaxCells];   // first packed row of cell (i,j)
    __shared__ int s_off[kPermMaxE + 1];
    __shared__ int s_scan[256 / kWave + 1];
    const int tid = threadIdx.x;
    const int C = S * E;
    for (int c = tid; c < C; c += blockDim.x) {
        const int v = max(recv[c], 0);
        s_start[c] = v;
        s_dbase[c] = v;
    }
    __syncthreads();
    // per local expert: rows from earlier senders, and the expert's total
    for (int j = tid; j < E; j += blockDim.x) {
        int run = 0;
        for (int i = 0; i < S; ++i) {
            const int t = s_dbase[i * E + j];
            s_dbase[i * E + j] = run;
            run += t;
        }
        s_off[j] = run;
    }
    __syncthreads();
    const int total_rows = block_exclusive_scan_lds(s_start, C, s_scan);
    const int total_e = block_exclusive_scan_lds(s_off, E, s_scan);
#ifdef MOE_DEBUG
    if (blockIdx.x == 0) {
        for (int c = tid; c < C; c += blockDim.x) MOE_DBG_CHECK(recv[c] >= 0, kDbgRecvSum);
        if (tid == 0) MOE_DBG_CHECK(total_rows == N, kDbgRecvSum);
    }
#endif
    for (int c = tid; c < C; c += blockDim.x) s_dbase[c] += s_off[c % E];
    if (blockIdx.x == 0) {
        for (int j = tid; j < E; j += blockDim.x) {
            const int next = (j + 1 < E) ? s_off[j + 1] : total_e;
            counts[j] = next - s_off[j];
            offsets[j] = s_off[j];
        }
        if (tid == 0) offsets[E] = total_e;
    }
    __syncthreads();

    const int lane = lane_id();
    const int w = tid / kWave;
    for (int q = w; q < kRecvRowsPerBlock; q += blockDim.x / kWave) {
        const int r = blockIdx.x * kRecvRowsPerBlock + q;
        if (r >= N) break;
        int j = -1;
        if (r < total_rows) {
            // last cell whose first row is <= r (a non-empty cell)
            int lo = 0, hi = C - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_start[mid] <= r) lo = mid; else hi = mid - 1;
            }
            j = s_dbase[lo] + (r - s_start[lo]);
            if (j >= N) j = -1;
        }
        if (lane == 0) {
            dest[r] = j;
            if (j >= 0) perm_src[j] = r;
        }
        if (j < 0) continue;
        const V* src = x + (size_t)r * vecs_per_row;
        V* dst = x_perm + (size_t)j * out_stride;
        // four vectors per lane in flight before their stores
        constexpr int U = 4;
        for (int c0 = lane; c0 < vecs_per_row; c0 += kWave * U) {
            V v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u * kWave < vecs_per_row) v[u] = src[c0 + u * kWave];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u * kWave < vecs_per_row) dst[c0 + u * kWave] = v[u];
        }
    }
}

static int ceil_log2(int v) {
    int b = 0;
    while ((1 << b) < v) ++b;
    return b;
}

size_t permute_ws_bytes(int T, int k, int E) {
    const long long TK = (long long)T * k;
    const long long chunk = perm_chunk(TK);
    const long long nb = std::max(1LL, (TK + chunk - 1) / chunk);
    return align_up((size_t)(nb * E) * sizeof(int32_t), 256);
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int e_base, int E, int id_hi, int cap,
                          const void* x, int es, int d, int32_t* routed, int32_t* counts,
                          int32_t* offsets, int32_t* perm_src, int32_t* dest, void* x_perm,
                          int ld, void* ws, hipStream_t st)
{
    const int TK = T * k;
    const int chunk = perm_chunk(TK);
    const int nb = std::max(1, (TK + chunk - 1) / chunk);
    int32_t* bc = static_cast<int32_t*>(ws);
    if (chunk == 512) {
        perm_hist_kernel<512><<<nb, kPermThreads, 0, st>>>(idx, TK, e_base, E, id_hi, bc);
        perm_rank_kernel<512><<<nb, kPermThreads, 0, st>>>(idx, TK, e_base, E, ceil_log2(E), cap, bc,
                                                           nb, routed, counts, offsets,
                                                           perm_src, dest);
    } else if (chunk == 1024) {
        perm_hist_kernel<1024><<<nb, kPermThreads, 0, st>>>(idx, TK, e_base, E, id_hi, bc);
        perm_rank_kernel<1024><<<nb, kPermThreads, 0, st>>>(idx, TK, e_base, E, ceil_log2(E), cap, bc,
                                                            nb, routed, counts, offsets,
                                                            perm_src, dest);
    } else {
        perm_hist_kernel<4096><<<nb, kPermThreads, 0, st>>>(idx, TK, e_base, E, id_hi, bc);
        perm_rank_kernel<4096><<<nb, kPermThreads, 0, st>>>(idx, TK, e_base, E, ceil_log2(E), cap, bc,
                                                            nb, routed, counts, offsets,
                                                            perm_src, dest);
    }
    if (T > 0) {
        const size_t row_bytes = (size_t)d * es;
        const size_t ld_bytes = (size_t)ld * es;
        const dim3 grid((T + 3) / 4);
        // (non-temporal stores of the packed rows measured no faster on the
        // stress layer's routing, whose rows land in ascending order inside
        // each expert's region; plain stores everywhere)
        if (row_bytes % 16 == 0 && ld_bytes % 16 == 0 && (uintptr_t)x % 16 == 0 &&
            (uintptr_t)x_perm % 16 == 0)
            perm_gather_kernel<u32x4, false><<<grid, 256, 0, st>>>(
                (const u32x4*)x, (int)(row_bytes / 16), T, k, dest, TK, (u32x4*)x_perm,
                (int)(ld_bytes / 16));
        else
            perm_gather_kernel<uint16_t, false><<<grid, 256, 0, st>>>(
                (const uint16_t*)x, (int)(row_bytes / 2), T, k, dest, TK, (uint16_t*)x_perm,
                (int)(ld_bytes / 2));
    }
    return hipGetLastError();
}

hipError_t launch_permute_recv(const int32_t* recv, int S, int E, int N, const void* x, int es,
                               int d, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                               int32_t* dest, void* x_perm, int ld, hipStream_t st)
{
    const int nblk = std::max(1, (N + kRecvRowsPerBlock - 1) / kRecvRowsPerBlock);
    const size_t row_bytes = (size_t)d * es;
    const size_t ld_bytes = (size_t)ld * es;
    if (row_bytes % 16 == 0 && ld_bytes % 16 == 0 && (uintptr_t)x % 16 == 0 &&
        (uintptr_t)x_perm % 16 == 0)
        perm_recv_kernel<u32x4><<<nblk, 256, 0, st>>>(recv, S, E, N, (const u32x4*)x,
                                                      (int)(row_bytes / 16), counts, offsets,
                                                      perm_src, dest, (u32x4*)x_perm,
                                                      (int)(ld_bytes / 16));
    else
        perm_recv_kernel<uint16_t><<<nblk, 256, 0, st>>>(recv, S, E, N, (const uint16_t*)x,
                                                         (int)(row_bytes / 2), counts, offsets,
                                                         perm_src, dest, (uint16_t*)x_perm,
                                                         (int)(ld_bytes / 2));
    return hipGetLastError();
}

// ------------------------------------------------ packing without allocation
// Callers that cannot allocate (code under HIP graph capture, tight serving
// loops) take the chunk histograms in this file-scope device array instead
// of a workspace: kStaticPermuteBytes per GPU, held until the process ends.
// In host code the array's name is a stand-in, not a device address: the
// address each device uses comes from hipGetSymbolAddress, once per device,
// with that device current.
constexpr size_t kStaticPermuteBytes = size_t(1) << 20;
static __device__ __align__(256) int32_t scratch[kStaticPermuteBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device, filled on first use
}  // namespace

size_t static_permute_bytes() { return kStaticPermuteBytes; }

// The current device's address of `scratch`, or nullptr (with the HIP error
// in *err) if it cannot be had.
void* static_permute_scratch(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    *err = hipSuccess;
    return g_scratch_ptr[dev];
}

MOE_DBG_READER(permute)

}  // namespace moe
