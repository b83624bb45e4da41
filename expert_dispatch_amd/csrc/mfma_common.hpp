// Pieces shared by the grouped matrix-core kernels (forward expert MLPs and
// their backward): the device-side tile scheduler over expert-contiguous
// rows, the LDS swizzles and fragment conventions of
// v_mfma_f32_32x32x16_bf16, and the persistent grid size.
#pragma once

#include <algorithm>

#include "common.hpp"

namespace moe {

constexpr int kMaxE = 4096;
constexpr int kGroupM = 4;   // row tiles per scheduling group inside an expert

// ----------------------------------------------------------- tile scheduler

struct Tile {
    int e, m0, seg_end, n_tile, bm;
    int stream;   // matrix-core kernel: the tile's weight panel is read by no other tile
};

// All threads of the block must call it. s_off needs E+1 ints, s_pre E ints.
__device__ bool schedule_tile(const int32_t* __restrict__ offsets, int N, int E, int bm,
                              int n_tiles, int* s_off, int* s_pre, int* scratch, Tile& tile)
{
    const int tid = threadIdx.x;
    // offsets NULL: one group of all N rows
    for (int e = tid; e <= E; e += blockDim.x)
        s_off[e] = offsets ? min(max(offsets[e], 0), N) : (e == 0 ? 0 : N);
#ifdef MOE_DEBUG
    if (offsets && blockIdx.x == 0)
        for (int e = tid; e <= E; e += blockDim.x)
            MOE_DBG_CHECK(offsets[e] >= 0 && offsets[e] <= N && (e > 0 || offsets[0] == 0) &&
                              (e == 0 || offsets[e] >= offsets[e - 1]),
                          kDbgOffsets);
#endif
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        const int lo = s_off[e];
        const int hi = max(lo, s_off[e + 1]);
        s_pre[e] = (hi - lo + bm - 1) / bm * n_tiles;
    }
    __syncthreads();
    const int total = block_exclusive_scan_lds(s_pre, E, scratch);
    const int per_xcd = (total + 7) / 8;
    const int b = blockIdx.x;
    const int slot = b / 8;
    if (slot >= per_xcd) return false;
    const int t = (b % 8) * per_xcd + slot;
    if (t >= total) return false;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int rows_lo = s_off[e];
    const int rows_hi = max(rows_lo, s_off[e + 1]);
    const int mt = (rows_hi - rows_lo + bm - 1) / bm;
    const int local = t - s_pre[e];
    // inside an expert, groups of kGroupM row tiles sweep all column tiles
    // (row tile fastest): the tiles resident on an XCD at one time share a
    // few A row panels and a few weight panels through its L2
    const int grp = local / (kGroupM * n_tiles);
    const int within = local - grp * (kGroupM * n_tiles);
    const int gsz = min(kGroupM, mt - grp * kGroupM);
    tile.e = e;
    tile.n_tile = within / gsz;
    tile.m0 = rows_lo + (grp * kGroupM + within % gsz) * bm;
    tile.seg_end = rows_hi;
    tile.bm = bm;
    return true;
}

// Tile list of the matrix-core kernel, two tile heights in one launch. An
// expert with n rows gets n / 256 tiles of 256 rows; a remainder above 128
// rows one more 256-row tile, a remainder of at most 128 rows one 128-row tile
// (a 256-row tile would be more than half padding there). Every row tile
// spans all n_tiles column tiles. Tile indices [0, big - split) are 256-row
// tiles (expert by expert; inside an expert groups of kGroupM row tiles sweep
// all column tiles, row tile fastest); [big - split, big + split) the last
// `split` 256-row tiles of that order, each as two 128-row halves (upper half
// first); then the small 128-row tiles.
struct TileList {
    const int* off;     // [E+1] clamped offsets
    const int* big;     // [E] exclusive prefix of 256-row tiles x n_tiles
    const int* small;   // [E] exclusive prefix of 128-row tiles x n_tiles
    int E, n_tiles, total_big, total_small;
    int split;          // 256-row tiles run as two 128-row halves
};

// Cost, in eighths of a 256-row tile, of the busiest block of a persistent
// grid of G blocks when the list holds nb 256-row tiles followed by ns
// 128-row tiles of cost c8 each, dealt cyclically (block position r takes
// tiles r, r + G, ...): every position gets nb / G and ns / G of them; the
// first nb % G positions one more 256-row tile, and the ns % G positions
// from nb % G on (wrapping past G onto the first ones) one more 128-row tile.
__device__ __forceinline__ int tail_cost(int nb, int ns, int G, int c8) {
    const int qb = nb / G, rb = nb % G, qs = ns / G, ms = ns % G;
    int extra = 0;
    if (rb > 0) extra = 8 + (rb + ms > G ? c8 : 0);
    if (ms > 0) extra = max(extra, c8);
    return 8 * qb + c8 * qs + extra;
}

// All threads of the block must call it. s_off needs E+1 ints, s_big and
// s_small E ints each. half_c8 > 0: the cost of a 128-row tile in eighths of a
// 256-row one; when the last, partial round of 256-row tiles over the grid
// (gridDim.x blocks) would end the launch later than running those tiles as
// 128-row halves, by tail_cost, they are split. 0 keeps every tile whole.
__device__ TileList build_tile_list(const int32_t* __restrict__ offsets, int N, int E,
                                    int n_tiles, int* s_off, int* s_big, int* s_small,
                                    int* scratch, int half_c8 = 0)
{
    const int tid = threadIdx.x;
    // offsets NULL: one group of all N rows
    for (int e = tid; e <= E; e += blockDim.x)
        s_off[e] = offsets ? min(max(offsets[e], 0), N) : (e == 0 ? 0 : N);
#ifdef MOE_DEBUG
    if (offsets && blockIdx.x == 0)
        for (int e = tid; e <= E; e += blockDim.x)
            MOE_DBG_CHECK(offsets[e] >= 0 && offsets[e] <= N && (e > 0 || offsets[0] == 0) &&
                              (e == 0 || offsets[e] >= offsets[e - 1]),
                          kDbgOffsets);
#endif
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        const int n = max(0, s_off[e + 1] - s_off[e]);
        const int rem = n & 255;
        s_big[e] = ((n >> 8) + (rem > 128 ? 1 : 0)) * n_tiles;
        s_small[e] = (rem > 0 && rem <= 128) ? n_tiles : 0;
    }
    __syncthreads();
    TileList L;
    L.off = s_off;
    L.big = s_big;
    L.small = s_small;
    L.E = E;
    L.n_tiles = n_tiles;
    L.total_big = __builtin_amdgcn_readfirstlane(block_exclusive_scan_lds(s_big, E, scratch));
    L.total_small = __builtin_amdgcn_readfirstlane(block_exclusive_scan_lds(s_small, E, scratch));
    L.split = 0;
    const int G = gridDim.x;
    const int rem = L.total_big % G;
    if (half_c8 > 0 && rem > 0 &&
        tail_cost(L.total_big - rem, L.total_small + 2 * rem, G, half_c8) <
            tail_cost(L.total_big, L.total_small, G, half_c8))
        L.split = rem;
    return L;
}

// Largest e with pre[e] <= t (pre is an exclusive prefix over E entries, so
// experts owning no tile are skipped).
__device__ __forceinline__ int find_owner(const int* pre, int E, int t) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Tile t of the list, 0 <= t < total_big + split + total_small.
__device__ Tile decode_tile(const TileList& L, int t) {
    Tile tile;
    int half = -1;   // 0, 1: upper or lower half of a split 256-row tile
    if (t >= L.total_big - L.split && t < L.total_big + L.split) {
        const int u = t - (L.total_big - L.split);
        half = u & 1;
        t = L.total_big - L.split + (u >> 1);
    } else if (t >= L.total_big + L.split) {
        t -= L.split;   // the small tiles, shifted by the split's extra entries
    }
    if (t < L.total_big) {
        const int e = find_owner(L.big, L.E, t);
        const int rows_lo = L.off[e];
        const int rows_hi = max(rows_lo, L.off[e + 1]);
        const int n = rows_hi - rows_lo;
        const int mt = (n >> 8) + ((n & 255) > 128 ? 1 : 0);
        const int local = t - L.big[e];
        const int grp = local / (kGroupM * L.n_tiles);
        const int within = local - grp * (kGroupM * L.n_tiles);
        const int gsz = min(kGroupM, mt - grp * kGroupM);
        tile.e = e;
        tile.n_tile = within / gsz;
        tile.m0 = rows_lo + (grp * kGroupM + within % gsz) * 256;
        tile.seg_end = rows_hi;
        tile.bm = 256;
        tile.stream = mt < 2;
        if (half >= 0) {
            // both halves read the same weight panel at about the same time
            // on one XCD (consecutive list entries): keep it cacheable
            tile.m0 += 128 * half;
            tile.bm = 128;
            tile.stream = 0;
        }
    } else {
        t -= L.total_big;
        const int e = find_owner(L.small, L.E, t);
        const int rows_lo = L.off[e];
        const int rows_hi = max(rows_lo, L.off[e + 1]);
        tile.e = e;
        tile.n_tile = t - L.small[e];
        tile.m0 = rows_lo + ((rows_hi - rows_lo) >> 8) * 256;
        tile.seg_end = rows_hi;
        tile.bm = 128;
        // remainder tiles run after all 256-row tiles: whatever the expert's
        // other tiles read is long gone from L2
        tile.stream = 1;
    }
    // uniform over the block: keep the fields in scalar registers
    tile.e = __builtin_amdgcn_readfirstlane(tile.e);
    tile.m0 = __builtin_amdgcn_readfirstlane(tile.m0);
    tile.seg_end = __builtin_amdgcn_readfirstlane(tile.seg_end);
    tile.n_tile = __builtin_amdgcn_readfirstlane(tile.n_tile);
    tile.bm = __builtin_amdgcn_readfirstlane(tile.bm);
    tile.stream = __builtin_amdgcn_readfirstlane(tile.stream);
    return tile;
}

inline long long max_row_tiles(int N, int E, int bm) {
    // sum_e ceil(n_e / bm) <= (N + E * (bm - 1)) / bm
    return ((long long)N + (long long)E * (bm - 1)) / bm;
}

#define LDS_AS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// silu(z) = z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp
// each; h is rounded to bf16 right after, up to 2^-8 relative). For z -> -inf,
// 1 + exp(-z) overflows to +inf and the reciprocal gives 0, so silu -> -0.
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Stage layouts in LDS (no padding; XOR swizzles of 16-byte chunks inside a
// row keep the fragment reads and the staging writes free of bank conflicts,
// both for LDS phases of 8 lanes x 16 bytes over 32 banks and of 16 lanes x
// 16 bytes (32 lanes x 8 bytes) over 64 banks):
//  A: [rows][BK], chunk c of row r stored at a_swz(c, r);
//  B: [BK k-rows][BNB columns], N-contiguous as in memory, chunk c of k-row r
//     stored at b_swz(c, r). B fragments are read with the gfx950 LDS
//     transpose read (ds_read_b64_tr_b16): in each 16-lane group, lane j
//     points at k-row j/4, columns 4*(j%4)..+3 of a 4 x 16 block and receives
//     the 4 k-values of column j.
__device__ __forceinline__ int a_swz(int c, int r) {
    return c ^ (((r >> 1) ^ (r >> 3)) & 3);
}
__device__ __forceinline__ int b_swz(int c, int r) {
    return c ^ (2 * (r & 3)) ^ (8 * ((c >> 1) & 1));
}

// Persistent grid: one block per compute unit (the kernel's LDS and registers
// allow no second one), rounded down to a multiple of 8, and no more blocks
// than there can be tiles (sum_e ceil(n_e / 128) row tiles at most).
inline unsigned mfma_grid(int N, int E, int n_tiles) {
    static int cus[64] = {0};
    int dev = 0;
    (void)hipGetDevice(&dev);
    int& c = cus[dev & 63];
    if (c == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        c = v;
    }
    const long long cap = std::max(8, c / 8 * 8);
    const long long tiles = max_row_tiles(N, E, 128) * n_tiles;
    return (unsigned)std::max(8LL, std::min(cap, (tiles + 7) / 8 * 8));
}

}  // namespace moe
