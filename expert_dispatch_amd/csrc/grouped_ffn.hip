// Grouped SwiGLU expert MLPs over expert-contiguous rows.
//
// "Three axes of Parallelism", Mapping experts to EP ranks: each rank holds
// W_gate, W_val [E_local,d,f] and W_out [E_local,f,d], experts contiguous;
// Dispatch, expert computation and combine: once the rows of every local
// expert are contiguous the work is E_local independent MLPs.
//
// Two launches: gate_up (h = silu(x.W_gate) * (x.W_val), stored bf16) and
// down (y = h.W_out, stored fp32). Both use one kernel shape:
//  * a device-side tile scheduler: every block reads offsets[0..E], turns the
//    per-expert row counts into a prefix of tiles and finds its own
//    (expert, column tile, row tile) by binary search. Nothing is read back
//    to the host, empty experts own no tile, the grid is an upper bound and
//    surplus blocks leave at once;
//  * XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs,
//    so block b works on tile (b % 8) * ceil(tiles / 8) + b / 8. Each XCD
//    then walks a contiguous run of the tile list, ordered expert by expert
//    and, inside an expert, by groups of 4 row tiles that sweep all column
//    tiles, so the tiles resident on an XCD share row and weight panels
//    through its L2;
//  * block tile 256 rows x 256 B-columns (gate_up: 128 gate + 128 val columns
//    of the same hidden units), BK = 64, 4 wavefronts of 128 x 128, each a
//    4 x 4 grid of v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 / lane,
//    held in AGPRs), so every fragment read from LDS feeds four MFMAs;
//  * a register-staged pipeline: two stages of global loads in flight in
//    registers while one LDS buffer (of two, 128 KB) is consumed. A is
//    K-contiguous in LDS; the weight panel stays N-contiguous as in memory and
//    the MFMA B fragments come from the gfx950 LDS transpose read. XOR
//    swizzles keep both fragment reads and the staging writes conflict-free;
//  * the fused epilogue applies SwiGLU on the two accumulator sets of a lane
//    (gate and val of the same element sit in the same lane and register).
// A plain fp32-FMA kernel covers fp32 data and shapes the matrix-core path
// does not tile.
#include <algorithm>

#include "common.hpp"

namespace moe {

constexpr int kMaxE = 4096;
constexpr int kGroupM = 4;   // row tiles per scheduling group inside an expert

// ----------------------------------------------------------- tile scheduler

struct Tile {
    int e, m0, seg_end, n_tile;
};

// All threads of the block must call it. s_off needs E+1 ints, s_pre E ints.
__device__ bool schedule_tile(const int32_t* __restrict__ offsets, int N, int E, int bm,
                              int n_tiles, int* s_off, int* s_pre, int* scratch, Tile& tile)
{
    const int tid = threadIdx.x;
    for (int e = tid; e <= E; e += blockDim.x) s_off[e] = min(max(offsets[e], 0), N);
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
    return true;
}

static long long max_row_tiles(int N, int E, int bm) {
    // sum_e ceil(n_e / bm) <= (N + E * (bm - 1)) / bm
    return ((long long)N + (long long)E * (bm - 1)) / bm;
}

// ------------------------------------------------------ matrix-core kernel

constexpr int BM = 256;       // rows per tile
constexpr int BK = 64;        // k per pipeline stage
constexpr int BNB = 256;      // B-panel columns per tile
constexpr int kMfmaThreads = 256;
constexpr int kMI = BM / 64;   // 32-row accumulator blocks per wavefront (2 x 2 wavefronts)
constexpr int kAChunks = BM * BK / 8 / kMfmaThreads;   // 16-byte A chunks per thread per stage

#define LDS_AS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Workgroup barrier of the pipelined main loop. __syncthreads() carries a
// workgroup fence, for which the compiler waits on every outstanding global
// load, draining the prefetched stages held in registers. The loop needs no
// fence: the LDS writes before the barrier and the LDS reads after it are
// ordered by the barrier itself, the compiler waits on each register load
// exactly where its value is written to LDS, and the asm memory clobber keeps
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Stage layouts in LDS (no padding; XOR swizzles keep the fragment reads
// conflict-free):
//  A: [BM rows][BK], 16-byte chunk c of row r stored at chunk c ^ (r & 7);
//  B: [BK k-rows][BNB columns], N-contiguous as in memory, 16-byte chunk c of
//     k-row r stored at chunk c ^ 2*(r & 3). B fragments are read with the
//     gfx950 LDS transpose read (ds_read_b64_tr_b16): in each 16-lane group,
//     lane j points at k-row j/4, columns 4*(j%4)..+3 of a 4 x 16 block and
//     receives the 4 k-values of column j.

template <bool GATE_UP, bool Y_BF16>
__global__ __launch_bounds__(kMfmaThreads, 1) void ffn_mfma_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int N, int K, int NC,
    int E, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    void* __restrict__ C)
{
    constexpr int BNT = GATE_UP ? 128 : 256;   // output columns per tile
    __shared__ __attribute__((aligned(1024))) uint16_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(1024))) uint16_t sB[2][BK * BNB];
    __shared__ int scratch[kMfmaThreads / kWave + 1];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    Tile tile;
    {
        int* s_pre = reinterpret_cast<int*>(&sB[0][0]);   // 4096 ints fit in 32 KB
        int* s_off = reinterpret_cast<int*>(&sB[1][0]);   // 4097 ints fit in 32 KB
        const bool ok = schedule_tile(offsets, N, E, BM, NC / BNT, s_off, s_pre, scratch, tile);
        if (!ok) return;  // uniform over the block
        __syncthreads();  // the scheduler's LDS is reused below
    }
    const int m0 = tile.m0;
    const int seg_last = tile.seg_end - 1;
    const size_t wbase = (size_t)tile.e * (size_t)K * (size_t)NC;
    const int n0 = tile.n_tile * BNT;

    // ---- global sources and LDS destinations of this thread's 16-byte chunks
    // A: chunk id q = tid + 256 i -> row tid/8 + 32 i, chunk tid%8 (8 lanes per
    // 128-byte row); the swizzle term (row & 7) does not depend on i.
    const uint16_t* a_src[kAChunks];
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        const int r = (tid >> 3) + 32 * i;
        a_src[i] = A + (size_t)min(m0 + r, seg_last) * K + (tid & 7) * 8;
    }
    const int a_dst = (tid >> 3) * BK + (((tid & 7) ^ ((tid >> 3) & 7)) * 8);   // + 32 i rows
    // B: chunk id q = tid + 256 i -> k-row tid/32 + 8 i, chunk tid%32 (32 lanes
    // per 512-byte row); again the swizzle term (k-row & 3) does not depend on i.
    const uint16_t* b_src;
    {
        const int c = tid & 31;
        const uint16_t* base;
        int col;
        if (GATE_UP) {
            base = (c < 16) ? B0 : B1;
            col = n0 + (c & 15) * 8;
        } else {
            base = B0;
            col = n0 + c * 8;
        }
        b_src = base + wbase + (size_t)(tid >> 5) * NC + col;                      // + 8 i k-rows
    }
    const int b_dst = (tid >> 5) * BNB + (((tid & 31) ^ (2 * ((tid >> 5) & 3))) * 8);  // + 8 i k-rows

    // ---- fragment addressing (element offsets inside a stage buffer)
    // A (row (BM/2)wm + 32mi + lane%32, logical chunk 2ks + lane/32): the mi term
    // is a constant 32 rows; the ks term goes through the XOR, one base per ks.
    int a_lane[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int r = (BM / 2) * wm + (lane & 31);
        a_lane[ks] = r * BK + ((((2 * ks + (lane >> 5)) ^ (r & 7))) * 8);
    }
    // B: 16-lane group g = lane/16, j = lane%16 points at k-row
    // 16ks + 8(g/2) + 4h + j/4 and column nbase[q] + 16(g%2) + 4(j%4); the
    // swizzle term (k-row & 3) = j/4 is lane-constant, so ks and h are
    // constant offsets and only q needs a per-lane base.
    const int g = lane >> 4, j = lane & 15;
    int b_lane[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int nb;
        if (GATE_UP) nb = (q < 2) ? (64 * wn + 32 * q) : (128 + 64 * wn + 32 * (q - 2));
        else nb = 128 * wn + 32 * q;
        const int n = nb + 16 * (g & 1) + 4 * (j & 3);
        b_lane[q] = (8 * (g >> 1) + (j >> 2)) * BNB + (((n >> 3) ^ (2 * (j >> 2))) * 8) + (n & 7);
    }

    f32x16 acc[kMI][4];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][q][r] = 0.0f;

    // two register stages in flight; LDS double buffer
    u32x4 ra0[kAChunks], rb0[8], ra1[kAChunks], rb1[8];
    auto load_regs = [&](int kt, u32x4 (&ra)[kAChunks], u32x4 (&rb)[8]) {
        const size_t ka = (size_t)kt * BK;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + ka);
        const uint16_t* bs = b_src + ka * NC;
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bs + (size_t)(8 * i) * NC);
    };
    auto store_lds = [&](int buf, const u32x4 (&ra)[kAChunks], const u32x4 (&rb)[8]) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) *reinterpret_cast<u32x4*>(&sA[buf][a_dst + 32 * i * BK]) = ra[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&sB[buf][b_dst + 8 * i * BNB]) = rb[i];
    };
    auto compute = [&](int buf) {
        const uint16_t* sa = sA[buf];
        const uint16_t* sb = sB[buf];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[kMI], bfr[4];
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8*>(sa + a_lane[ks] + 32 * mi * BK);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint16_t* p = sb + b_lane[q] + 16 * ks * BNB;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * BNB));
                const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                bfr[q] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[mi][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[q], acc[mi][q], 0, 0, 0);
            // keep each substep's fragment reads next to its MFMAs (bounds live registers)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int KT = K / BK;
    // Loads and LDS writes past the last stage are issued anyway with the
    // stage index clamped (a valid address, written into a buffer that is
    // free and never read again): branch-free, so the compiler's wait
    // analysis sees one straight path and waits only for the stage it stores.
    auto clampk = [&](int k) { return min(k, KT - 1); };
    load_regs(0, ra0, rb0);
    load_regs(clampk(1), ra1, rb1);
    store_lds(0, ra0, rb0);
    load_regs(clampk(2), ra0, rb0);
    // iteration kt: barrier (stage kt is in LDS buffer kt&1 and buffer
    // (kt+1)&1 is free); write stage kt+1 from its registers; reload those
    // registers with stage kt+3; compute stage kt. Loads get two iterations.
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        lds_barrier();
        store_lds(1, ra1, rb1);
        load_regs(clampk(kt + 3), ra1, rb1);
        compute(0);
        lds_barrier();
        store_lds(0, ra0, rb0);
        load_regs(clampk(kt + 4), ra0, rb0);
        compute(1);
    }
    if (kt < KT) {  // odd number of stages: the last one sits in buffer 0
        lds_barrier();
        compute(0);
    }

    // epilogue: lane holds column (lane % 32) of each 32x32 accumulator and
    // rows 8*(r/4) + 4*(lane/32) + r%4 for register r
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
    if (GATE_UP) {
        uint16_t* H = static_cast<uint16_t*>(C);
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int col = n0 + 64 * wn + 32 * q + col_l;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + (BM / 2) * wm + 32 * mi + 8 * (r >> 2) + row_l + (r & 3);
                    if (row <= seg_last) {
                        const float gv = acc[mi][q][r];
                        const float v = acc[mi][q + 2][r];
                        const float h = __fdividef(gv, 1.0f + __expf(-gv)) * v;
                        H[(size_t)row * NC + col] = f32_to_bf16(h);
                    }
                }
            }
    } else {
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + 128 * wn + 32 * q + col_l;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + (BM / 2) * wm + 32 * mi + 8 * (r >> 2) + row_l + (r & 3);
                    if (row <= seg_last) {
                        if (Y_BF16)
                            static_cast<uint16_t*>(C)[(size_t)row * NC + col] = f32_to_bf16(acc[mi][q][r]);
                        else
                            static_cast<float*>(C)[(size_t)row * NC + col] = acc[mi][q][r];
                    }
                }
            }
    }
}

// ------------------------------------------------------------ generic kernel

constexpr int GBM = 64, GBN = 64, GBK = 16;

template <typename XT, typename OT, bool GATE_UP>
__global__ __launch_bounds__(256) void ffn_generic_kernel(
    const XT* __restrict__ A, const int32_t* __restrict__ offsets, int N, int K, int NC, int E,
    const XT* __restrict__ B0, const XT* __restrict__ B1, OT* __restrict__ C)
{
    __shared__ float sAg[GBM][GBK + 1];
    __shared__ float sB0[GBK][GBN];
    __shared__ float sB1[GBK][GBN];
    __shared__ int s_sched[2 * kMaxE + 1];
    __shared__ int scratch[256 / kWave + 1];

    Tile tile;
    if (!schedule_tile(offsets, N, E, GBM, (NC + GBN - 1) / GBN, s_sched, s_sched + kMaxE + 1,
                       scratch, tile))
        return;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int m0 = tile.m0, seg_last = tile.seg_end - 1;
    const int n0 = tile.n_tile * GBN;
    const size_t wbase = (size_t)tile.e * (size_t)K * (size_t)NC;

    float acc0[4][4], acc1[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) { acc0[i][j] = 0.f; acc1[i][j] = 0.f; }

    for (int k0 = 0; k0 < K; k0 += GBK) {
        for (int q = tid; q < GBM * GBK; q += 256) {
            const int r = q / GBK, kk = q % GBK;
            const int row = min(m0 + r, seg_last);
            const int kx = k0 + kk;
            sAg[r][kk] = kx < K ? Elem<XT>::load(A, (size_t)row * K + kx) : 0.f;
        }
        for (int q = tid; q < GBK * GBN; q += 256) {
            const int kk = q / GBN, c = q % GBN;
            const int kx = k0 + kk, col = n0 + c;
            const bool in = kx < K && col < NC;
            const size_t o = wbase + (size_t)kx * NC + col;
            sB0[kk][c] = in ? Elem<XT>::load(B0, o) : 0.f;
            if (GATE_UP) sB1[kk][c] = in ? Elem<XT>::load(B1, o) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GBK; ++kk) {
            float a[4], b0[4], b1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sAg[ty * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b0[j] = sB0[kk][tx * 4 + j];
                if (GATE_UP) b1[j] = sB1[kk][tx * 4 + j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0[i][j] = __builtin_fmaf(a[i], b0[j], acc0[i][j]);
                    if (GATE_UP) acc1[i][j] = __builtin_fmaf(a[i], b1[j], acc1[i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + ty * 4 + i;
        if (row > seg_last) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + tx * 4 + j;
            if (col >= NC) continue;
            float v = acc0[i][j];
            if (GATE_UP) v = v / (1.0f + __expf(-v)) * acc1[i][j];
            Elem<OT>::store(C, (size_t)row * NC + col, v);
        }
    }
}

// ----------------------------------------------------------------- launches

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool ffn_gate_up_uses_mfma(moe_dtype dt, int d, int f, const void* x, const void* wg,
                           const void* wv, const void* h) {
    return dt == MOE_BF16 && d % BK == 0 && f % 128 == 0 && aligned16(x) && aligned16(wg) &&
           aligned16(wv) && aligned16(h);
}
bool ffn_down_uses_mfma(moe_dtype dt, int f, int d, const void* h, const void* wo) {
    return dt == MOE_BF16 && f % BK == 0 && d % 256 == 0 && aligned16(h) && aligned16(wo);
}

static unsigned grid_for(long long tiles) {
    long long g = (tiles + 7) / 8 * 8;
    return (unsigned)std::max(8LL, g);
}

hipError_t launch_gate_up(const void* x, moe_dtype dt, int N, int d, int f, int E,
                          const int32_t* offsets, const void* wg, const void* wv, void* h,
                          hipStream_t st)
{
    if (ffn_gate_up_uses_mfma(dt, d, f, x, wg, wv, h)) {
        const long long tiles = max_row_tiles(N, E, BM) * (f / 128);
        ffn_mfma_kernel<true, false><<<grid_for(tiles), kMfmaThreads, 0, st>>>(
            (const uint16_t*)x, offsets, N, d, f, E, (const uint16_t*)wg, (const uint16_t*)wv, h);
    } else {
        const long long tiles = max_row_tiles(N, E, GBM) * ((f + GBN - 1) / GBN);
        if (dt == MOE_BF16)
            ffn_generic_kernel<uint16_t, uint16_t, true><<<grid_for(tiles), 256, 0, st>>>(
                (const uint16_t*)x, offsets, N, d, f, E, (const uint16_t*)wg,
                (const uint16_t*)wv, (uint16_t*)h);
        else
            ffn_generic_kernel<float, float, true><<<grid_for(tiles), 256, 0, st>>>(
                (const float*)x, offsets, N, d, f, E, (const float*)wg, (const float*)wv,
                (float*)h);
    }
    return hipGetLastError();
}

hipError_t launch_down(const void* h, moe_dtype dt, int N, int f, int d, int E,
                       const int32_t* offsets, const void* wo, void* y, moe_dtype y_dt,
                       hipStream_t st)
{
    if (ffn_down_uses_mfma(dt, f, d, h, wo) && aligned16(y)) {
        const long long tiles = max_row_tiles(N, E, BM) * (d / 256);
        if (y_dt == MOE_BF16)
            ffn_mfma_kernel<false, true><<<grid_for(tiles), kMfmaThreads, 0, st>>>(
                (const uint16_t*)h, offsets, N, f, d, E, (const uint16_t*)wo, nullptr, y);
        else
            ffn_mfma_kernel<false, false><<<grid_for(tiles), kMfmaThreads, 0, st>>>(
                (const uint16_t*)h, offsets, N, f, d, E, (const uint16_t*)wo, nullptr, y);
    } else {
        const long long tiles = max_row_tiles(N, E, GBM) * ((d + GBN - 1) / GBN);
        const unsigned g = grid_for(tiles);
        if (dt == MOE_BF16) {
            if (y_dt == MOE_BF16)
                ffn_generic_kernel<uint16_t, uint16_t, false><<<g, 256, 0, st>>>(
                    (const uint16_t*)h, offsets, N, f, d, E, (const uint16_t*)wo, nullptr,
                    (uint16_t*)y);
            else
                ffn_generic_kernel<uint16_t, float, false><<<g, 256, 0, st>>>(
                    (const uint16_t*)h, offsets, N, f, d, E, (const uint16_t*)wo, nullptr,
                    (float*)y);
        } else {
            if (y_dt == MOE_BF16)
                ffn_generic_kernel<float, uint16_t, false><<<g, 256, 0, st>>>(
                    (const float*)h, offsets, N, f, d, E, (const float*)wo, nullptr, (uint16_t*)y);
            else
                ffn_generic_kernel<float, float, false><<<g, 256, 0, st>>>(
                    (const float*)h, offsets, N, f, d, E, (const float*)wo, nullptr, (float*)y);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
