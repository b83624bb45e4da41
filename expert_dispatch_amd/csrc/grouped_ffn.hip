// Grouped SwiGLU expert MLPs over expert-contiguous rows.
//
// "Three axes of Parallelism", Mapping experts to EP ranks: each rank holds
// W_gate, W_val [E_local,d,f] and W_out [E_local,f,d], experts contiguous;
// Dispatch, expert computation and combine: once the rows of every local
// expert are contiguous the work is E_local independent MLPs.
//
// Two launches: gate_up (h = silu(x.W_gate) * (x.W_val), stored bf16) and
// down (y = h.W_out, stored fp32 or bf16). Both use one kernel shape:
//  * a device-side tile list: every block reads offsets[0..E] and turns the
//    per-expert row counts into a prefix of tiles in LDS (256-row tiles, and
//    one 128-row tile for a remainder of at most 128 rows). Nothing is read
//    back to the host and empty experts own no tile;
//  * a persistent grid (one block per CU, a multiple of 8) in XCD-aware
//    order: block b works through tiles i*G + (b % 8) * (G / 8) + b / 8, so in
//    every pass each XCD takes a contiguous run of the list, which is ordered
//    expert by expert and, inside an expert, by groups of 4 row tiles that
//    sweep all column tiles: the tiles resident on an XCD share row and
//    weight panels through its L2;
//  * block tile TM rows x 256 B-columns (gate_up: 128 gate + 128 val columns
//    of the same hidden units), BK = 32, 4 wavefronts of TM/2 x 128, each a
//    (TM/64) x 4 grid of v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per
//    lane at TM = 256, held in AGPRs), so every fragment read from LDS feeds
//    several MFMAs;
//  * a register-staged pipeline: three stages of global loads in flight in
//    registers and a three-buffer LDS ring (96 KB). A is K-contiguous in LDS;
//    the weight panel stays N-contiguous as in memory and the MFMA B
//    fragments come from the gfx950 LDS transpose read. XOR swizzles keep
//    both fragment reads and the staging writes conflict-free;
//  * fused epilogues: SwiGLU on the two accumulator sets of a lane (gate and
//    val of the same element sit in the same lane and register); outputs
//    leave through buffer stores bounded by the expert's segment.
// A plain fp32-FMA kernel covers fp32 data and shapes the matrix-core path
// does not tile.
#include <algorithm>
#include <type_traits>

#include "mfma_common.hpp"

namespace moe {

// ------------------------------------------------------ matrix-core kernel

constexpr int BM = 256;       // rows of a full tile (a remainder tile has 128)
constexpr int BK = 32;        // k per pipeline stage
constexpr int BNB = 256;      // B-panel columns per tile
constexpr int kMfmaThreads = 256;
constexpr int kBChunks = BK * BNB / 8 / kMfmaThreads;   // 16-byte B chunks per thread per stage
constexpr int kRing = 3;      // LDS stage buffers
constexpr int kSets = 3;      // register stages in flight (global-load prefetch distance)

// Barrier that lets up to P of this wave's most recent LDS operations still be
// in flight (LDS operations of a wave complete in order). The main loop issues
// the fragment reads of the next stage last; they read a buffer no wave
// writes before the following barrier, so only what precedes them (this
// step's LDS writes and the reads of the buffer about to be refilled) must
// be complete here.
template <int P>
__device__ __forceinline__ void lds_barrier_pending() {
    static_assert(P == 10 || P == 12, "pending count");
    if constexpr (P == 12)
        asm volatile("s_waitcnt lgkmcnt(12)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(10)\n\ts_barrier" ::: "memory");
}

// LDS of the kernel: the stage ring (96 KB, sized for 256-row tiles; the
// epilogue reuses it) and the tile list (built once per block, kept).
constexpr int kSmemElems = kRing * (BM * BK + BK * BNB);

// Global-load stage in registers: 16-byte A and B chunks of one thread (a
// 128-row tile uses the first half of a[]).
struct Stage {
    u32x4 a[BM * BK / 8 / kMfmaThreads];
    u32x4 b[kBChunks];
};

// Per-thread global sources of one tile (A rows lda elements apart). A: chunk q = tid + 256 i -> row
// tid/4 + 64 i, chunk tid%4 (4 lanes per 64-byte row); rows past the expert's
// segment re-read its last row (never stored). B: chunk q = tid + 256 i ->
// k-row tid/32 + 8 i, chunk tid%32 (32 lanes per 512-byte row; gate_up: 16
// chunks of W_gate, then 16 of W_val).
template <bool GATE_UP, int TM, bool STREAM>
struct TileSrc {
    static constexpr int kAChunks = TM * BK / 8 / kMfmaThreads;
    const uint16_t* a[kAChunks];
    const uint16_t* b;

    __device__ __forceinline__ TileSrc(const uint16_t* A, int lda, int K, int NC,
                                       const uint16_t* B0, const uint16_t* B1, const Tile& tile) {
        const int tid = threadIdx.x;
        const int seg_last = tile.seg_end - 1;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int r = (tid >> 2) + 64 * i;
            a[i] = A + (size_t)min(tile.m0 + r, seg_last) * lda + (tid & 3) * 8;
        }
        const size_t wbase = (size_t)tile.e * (size_t)K * (size_t)NC;
        const int c = tid & 31;
        if (GATE_UP) {
            b = ((c < 16) ? B0 : B1) + wbase + (size_t)(tid >> 5) * NC + tile.n_tile * 128 + (c & 15) * 8;
        } else {
            b = B0 + wbase + (size_t)(tid >> 5) * NC + tile.n_tile * 256 + c * 8;
        }
    }
    __device__ __forceinline__ void load(int kt, int NC, Stage& r) const {
        const size_t ka = (size_t)kt * BK;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) r.a[i] = *reinterpret_cast<const u32x4*>(a[i] + ka);
        // STREAM: no other tile reads this weight panel; a non-temporal load
        // keeps it from pushing the A rows (read again by the next stage) out
        // of the caches. Otherwise the panel is left in L2 for the expert's
        // other row tiles.
        const uint16_t* bs = b + ka * NC;
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const u32x4* p = reinterpret_cast<const u32x4*>(bs + (size_t)(8 * i) * NC);
            r.b[i] = STREAM ? __builtin_nontemporal_load(p) : *p;
        }
    }
};

// One output tile of TM rows (256 or 128) x 256 B-columns. The 4 wavefronts
// form a 2 x 2 grid, each computing TM/2 x 128 as a (TM/64) x 4 grid of
// v_mfma_f32_32x32x16_bf16 accumulators held in AGPRs.
template <bool GATE_UP, bool Y_BF16, int TM, bool STREAM, bool SAVE>
__device__ __forceinline__ void ffn_mfma_tile(
    const uint16_t* __restrict__ A, int lda, int K, int NC, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ C, uint16_t* __restrict__ act,
    const Tile& tile, uint16_t* smem)
{
    constexpr int kMI = TM / 64;                               // 32-row blocks per wavefront
    constexpr int kAChunks = TM * BK / 8 / kMfmaThreads;       // 16-byte A chunks per thread per stage
    constexpr int kReads = kMI + 8;                            // LDS reads per fragment set
    constexpr int BNT = GATE_UP ? 128 : 256;                   // output columns per tile
    auto sA = [&](int buf) { return smem + buf * (TM * BK); };
    auto sB = [&](int buf) { return smem + kRing * (TM * BK) + buf * (BK * BNB); };

    // The thread index passes through an empty asm statement, so the compiler
    // recomputes the addresses derived from it for every tile instead of
    // hoisting them out of the block's tile loop (where they would stay live
    // next to the full register budget of the main loop).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const int m0 = tile.m0;
    const int seg_last = tile.seg_end - 1;
    const int n0 = tile.n_tile * BNT;
    const TileSrc<GATE_UP, TM, STREAM> src(A, lda, K, NC, B0, B1, tile);

    // LDS destinations of this thread's chunks: A + 64 i rows, B + 8 i k-rows
    // (the swizzle terms do not depend on i)
    const int a_dst = (tid >> 2) * BK + (a_swz(tid & 3, tid >> 2) * 8);
    const int b_dst = (tid >> 5) * BNB + (b_swz(tid & 31, tid >> 5) * 8);

    // ---- fragment addressing (element offsets inside a stage buffer)
    // A (row (TM/2)wm + 32mi + lane%32, logical chunk 2ks + lane/32): the mi
    // term is a constant 32 rows (the swizzle term does not change with it).
    int a_lane[BK / 16];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int r = (TM / 2) * wm + (lane & 31);
        a_lane[ks] = r * BK + (a_swz(2 * ks + (lane >> 5), r) * 8);
    }
    // B: 16-lane group g = lane/16, j = lane%16 points at k-row
    // 16ks + 8(g/2) + 4h + j/4 and column nb[q] + 16(g%2) + 4(j%4); the swizzle
    // term (k-row & 3) = j/4 is lane-constant, so ks and h are constant
    // offsets and only q needs a per-lane base.
    const int g = lane >> 4, j = lane & 15;
    int b_lane[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int nb;
        if (GATE_UP) nb = (q < 2) ? (64 * wn + 32 * q) : (128 + 64 * wn + 32 * (q - 2));
        else nb = 128 * wn + 32 * q;
        const int n = nb + 16 * (g & 1) + 4 * (j & 3);
        const int kr = 8 * (g >> 1) + (j >> 2);
        b_lane[q] = kr * BNB + (b_swz(n >> 3, kr) * 8) + (n & 7);
    }

    f32x16 acc[kMI][4];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][q][r] = 0.0f;

    struct Frags {
        bf16x8 a[kMI];
        bf16x8 b[4];
    };
    auto store_lds = [&](int buf, const Stage& r) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) *reinterpret_cast<u32x4*>(sA(buf) + a_dst + 64 * i * BK) = r.a[i];
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) *reinterpret_cast<u32x4*>(sB(buf) + b_dst + 8 * i * BNB) = r.b[i];
    };
    auto read_frags = [&](int buf, int ks, Frags& f) {
        const uint16_t* sa = sA(buf);
        const uint16_t* sb = sB(buf);
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
            f.a[mi] = *reinterpret_cast<const bf16x8*>(sa + a_lane[ks] + 32 * mi * BK);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint16_t* p = sb + b_lane[q] + 16 * ks * BNB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * BNB));
            const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            f.b[q] = __builtin_bit_cast(bf16x8, v);
        }
    };
    auto mfmas = [&](const Frags& f) {
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[mi][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[q], acc[mi][q], 0, 0, 0);
    };

    const int KT = K / BK;
    // Loads and LDS writes past the last stage are issued anyway with the
    // stage index clamped (a valid address, written into a buffer no later
    // step reads): the loop body stays branch-free, so the compiler's wait
    // analysis waits only for the stage it stores.
    auto clampk = [&](int k) { return min(k, KT - 1); };

    // Pipeline: stage s lives in LDS buffer s % 3 and, before that, in
    // register set s % 3 (the loop body is three steps, so the set is static
    // and the buffer index is carried along). Step kt (after a barrier that
    // publishes stage kt+1 and retires every read of buffer (kt-1) % 3):
    //   read the second k-substep fragments of stage kt,
    //   MFMAs of stage kt, first k-substep (fragments read in step kt-1),
    //   write stage kt+2 from its registers into buffer (kt+2) % 3 and
    //   reload those registers with stage kt+5,
    //   read the first k-substep fragments of stage kt+1,
    //   MFMAs of stage kt, second k-substep.
    // Global loads get three steps to land; LDS reads of a stage start one
    // step before its MFMAs.
    Stage rs[kSets];
#pragma unroll
    for (int i = 0; i < kSets; ++i) src.load(clampk(i), NC, rs[i]);
    Frags f0, f1;
    lds_barrier();   // the block's previous tile is done with the ring
    store_lds(0, rs[0]);
    src.load(clampk(kSets), NC, rs[0]);
    store_lds(1, rs[1]);
    src.load(clampk(kSets + 1), NC, rs[1]);
    lds_barrier();
    read_frags(0, 0, f0);

    auto step = [&](int kt, int buf, Stage& r) {
        const int nxt = (buf == kRing - 1) ? 0 : buf + 1;
        const int wr = (nxt == kRing - 1) ? 0 : nxt + 1;
        lds_barrier_pending<kReads>();
        read_frags(buf, 1, f1);
        mfmas(f0);
        store_lds(wr, r);
        src.load(clampk(kt + 2 + kSets), NC, r);
        read_frags(nxt, 0, f0);
        mfmas(f1);
        // issue order, so that every MFMA has LDS or global-memory work beside it
        if constexpr (TM == 256) {
            // the 12 fragment reads of the second k-substep between the first
            // 12 MFMAs, the stage's 8 LDS writes and 8 global loads over the
            // next 8, the 12 fragment reads of the next stage over the last 12
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        } else {
            // 16 MFMAs: 10 reads over the first 5, 6 LDS writes and 6 global
            // loads over the next 3, the 10 reads of the next stage over the
            // last 8
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        return nxt;
    };
    int kt = 0, buf = 0;
    for (; kt + kSets <= KT; kt += kSets) {
#pragma unroll
        for (int u = 0; u < kSets; ++u) buf = step(kt + u, buf, rs[(u + 2) % kSets]);
    }
#pragma unroll
    for (int u = 0; u < kSets - 1; ++u)
        if (kt + u < KT) buf = step(kt + u, buf, rs[(u + 2) % kSets]);

    // Epilogue. A lane holds column lane%32 of each 32x32 accumulator block and
    // rows 8*(r/4) + 4*(lane/32) + r%4 for register r.
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
    const int nrows = min(TM, seg_last + 1 - m0);   // rows of the tile inside the segment
    if (GATE_UP) {
        // The bf16 h tile is staged row-major through the (now idle) LDS ring
        // and leaves with 16-byte row-contiguous stores instead of one 2-byte
        // store per element. With `act` (training) the pre-activations a and v
        // of the tile follow the same way, into act[:, 0:f] and act[:, f:2f].
        // h tile: TM rows x 128 hidden columns, bf16, row stride 136 elements
        // (256 rows: 69632 bytes of the 96 KB ring)
        constexpr int HS = 136;
        uint16_t* sh = smem;
        // which = 0: h, 1: a, 2: v
        auto stage_out = [&](int which, uint16_t* dst, int ld, int col0) {
            lds_barrier();   // every wave is done with the ring (stages or the last tile)
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        // rows r and r+1 of a lane are adjacent: one packed conversion
                        const int row = (TM / 2) * wm + 32 * mi + 8 * (r >> 2) + row_l + (r & 3);
                        const int col = 64 * wn + 32 * q + col_l;
                        const float g0 = acc[mi][q][r], g1 = acc[mi][q][r + 1];
                        const float v0 = acc[mi][q + 2][r], v1 = acc[mi][q + 2][r + 1];
                        float o0, o1;
                        if (which == 0) { o0 = silu_fast(g0) * v0; o1 = silu_fast(g1) * v1; }
                        else if (which == 1) { o0 = g0; o1 = g1; }
                        else { o0 = v0; o1 = v1; }
                        const unsigned pk = f32x2_to_bf16x2(o0, o1);
                        sh[row * HS + col] = (uint16_t)pk;
                        sh[(row + 1) * HS + col] = (uint16_t)(pk >> 16);
                    }
            lds_barrier();
            // TM rows x 16 chunks of 8 columns; thread -> chunk tid%16, rows
            // tid/16 + 16 i; rows past the segment fall outside the resource
            const __amdgpu_buffer_rsrc_t out =
                tile_rsrc(dst + (size_t)m0 * ld + col0, nrows * ld * 2);
            const int c8 = (tid & 15) * 8;
            const int voff = ((tid >> 4) * ld + c8) * 2;
#pragma unroll
            for (int i = 0; i < TM / 16; ++i) {
                const int row = (tid >> 4) + 16 * i;
                const u32x4 v = *reinterpret_cast<const u32x4*>(&sh[row * HS + c8]);
                __builtin_amdgcn_raw_buffer_store_b128(v, out, voff + 16 * i * ld * 2, 0, 0);
            }
        };
        stage_out(0, static_cast<uint16_t*>(C), NC, n0);
        if constexpr (SAVE) {
            stage_out(1, act, 2 * NC, n0);
            stage_out(2, act, 2 * NC, NC + n0);
        }
    } else if (Y_BF16) {
        // y in bf16: registers r, r+1 of a lane are rows i, i+1 of one column and
        // neighbouring lanes hold neighbouring columns, so a swap between lane
        // pairs (DPP quad_perm [1,0,3,2]) gives every even lane columns c, c+1 of
        // row i and every odd lane columns c-1, c of row i+1: one 4-byte store
        // per two values
        const int odd = lane & 1;
        const __amdgpu_buffer_rsrc_t out =
            tile_rsrc(static_cast<uint16_t*>(C) + (size_t)m0 * NC + n0, nrows * NC * 2);
        const int voff = (((TM / 2) * wm + row_l + odd) * NC + 128 * wn + col_l - odd) * 2;
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int roff = voff + (32 * mi + 8 * (r >> 2) + (r & 3)) * NC * 2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x = acc[mi][q][r], y = acc[mi][q][r + 1];
                    const float xs = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
                    const float ys = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0xB1, 0xF, 0xF, false));
                    const unsigned pk = f32x2_to_bf16x2(odd ? ys : x, odd ? y : xs);
                    __builtin_amdgcn_raw_buffer_store_b32(pk, out, roff + 64 * q, 0, 0);
                }
            }
    } else {
        // y in fp32: 32 lanes cover 32 consecutive columns of a row per
        // register, so direct stores already write whole 128-byte row segments
        const __amdgpu_buffer_rsrc_t out =
            tile_rsrc(static_cast<float*>(C) + (size_t)m0 * NC + n0, nrows * NC * 4);
        const int voff = (((TM / 2) * wm + row_l) * NC + 128 * wn + col_l) * 4;
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int roff = voff + (32 * mi + 8 * (r >> 2) + (r & 3)) * NC * 4;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[mi][q][r]), out,
                                                          roff + 128 * q, 0, 0);
            }
    }
}

// Persistent: the grid is a multiple of 8 no larger than the number of
// compute units; block b works through tiles t_i = i*G + (b%8)*(G/8) + b/8
// (G = grid size), so in every pass i each XCD (block b runs on XCD b % 8)
// takes a contiguous run of the tile list and the tiles of one expert meet
// on one XCD and share its L2.
template <bool GATE_UP, bool Y_BF16, bool SAVE>
__global__ __launch_bounds__(kMfmaThreads, 1) void ffn_mfma_kernel(
    const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ offsets, int N, int K,
    int NC, int E, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    void* __restrict__ C, uint16_t* __restrict__ act)
{
    constexpr int BNT = GATE_UP ? 128 : 256;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmemElems];
    __shared__ int s_sched[3 * kMaxE + 1];
    __shared__ int scratch[kMfmaThreads / kWave + 1];
    // a 128-row tile costs about 7/8 (gate_up) and 3/4 (down) of a 256-row one
    // (the weight panel it streams is the same): the cost ratio for splitting
    // the last partial round of 256-row tiles
    const TileList L = build_tile_list(offsets, N, E, NC / BNT, s_sched, s_sched + kMaxE + 1,
                                       s_sched + 2 * kMaxE + 1, scratch, GATE_UP ? 7 : 6);
    const int total = L.total_big + L.split + L.total_small;
    const int G = gridDim.x;
    const int base = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    for (int t = base; t < total; t += G) {
        const Tile tile = decode_tile(L, t);
        if (tile.bm == 128 && tile.stream)
            ffn_mfma_tile<GATE_UP, Y_BF16, 128, true, SAVE>(A, lda, K, NC, B0, B1, C, act, tile, smem);
        else if (tile.bm == 128)
            ffn_mfma_tile<GATE_UP, Y_BF16, 128, false, SAVE>(A, lda, K, NC, B0, B1, C, act, tile, smem);
        else if (tile.stream)
            ffn_mfma_tile<GATE_UP, Y_BF16, 256, true, SAVE>(A, lda, K, NC, B0, B1, C, act, tile, smem);
        else
            ffn_mfma_tile<GATE_UP, Y_BF16, 256, false, SAVE>(A, lda, K, NC, B0, B1, C, act, tile, smem);
    }
}

// ------------------------------------------------------------ generic kernel

constexpr int GBM = 64, GBN = 64, GBK = 16;

template <typename XT, typename OT, bool GATE_UP>
__global__ __launch_bounds__(256) void ffn_generic_kernel(
    const XT* __restrict__ A, int lda, const int32_t* __restrict__ offsets, int N, int K, int NC,
    int E, const XT* __restrict__ B0, const XT* __restrict__ B1, OT* __restrict__ C,
    OT* __restrict__ act)
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
            sAg[r][kk] = kx < K ? Elem<XT>::load(A, (size_t)row * lda + kx) : 0.f;
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
            if (GATE_UP) {
                if (act) {
                    Elem<OT>::store(act, (size_t)row * 2 * NC + col, v);
                    Elem<OT>::store(act, (size_t)row * 2 * NC + NC + col, acc1[i][j]);
                }
                v = v / (1.0f + __expf(-v)) * acc1[i][j];
            }
            Elem<OT>::store(C, (size_t)row * NC + col, v);
        }
    }
}

// ----------------------------------------------------------------- launches

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// (f, d < 2^20 keep a tile's byte offsets in the epilogue's buffer stores in
// 31 bits)
bool ffn_gate_up_uses_mfma(moe_dtype dt, int d, int ldx, int f, const void* x, const void* wg,
                           const void* wv, const void* h) {
    return dt == MOE_BF16 && d % BK == 0 && ldx % 8 == 0 && f % 128 == 0 && f < (1 << 20) &&
           aligned16(x) &&
           aligned16(wg) && aligned16(wv) && aligned16(h);
}
bool ffn_down_uses_mfma(moe_dtype dt, int f, int d, const void* h, const void* wo) {
    return dt == MOE_BF16 && f % BK == 0 && d % 256 == 0 && d < (1 << 20) && aligned16(h) &&
           aligned16(wo);
}

static unsigned grid_for(long long tiles) {
    long long g = (tiles + 7) / 8 * 8;
    return (unsigned)std::max(8LL, g);
}

hipError_t launch_gate_up(const void* x, int ldx, moe_dtype dt, int N, int d, int f, int E,
                          const int32_t* offsets, const void* wg, const void* wv, void* h,
                          void* act, hipStream_t st)
{
    if (ffn_gate_up_uses_mfma(dt, d, ldx, f, x, wg, wv, h) && aligned16(act)) {
        const unsigned g = mfma_grid(N, E, f / 128);
        if (act)
            ffn_mfma_kernel<true, false, true><<<g, kMfmaThreads, 0, st>>>(
                (const uint16_t*)x, ldx, offsets, N, d, f, E, (const uint16_t*)wg,
                (const uint16_t*)wv, h, (uint16_t*)act);
        else
            ffn_mfma_kernel<true, false, false><<<g, kMfmaThreads, 0, st>>>(
                (const uint16_t*)x, ldx, offsets, N, d, f, E, (const uint16_t*)wg,
                (const uint16_t*)wv, h, nullptr);
    } else {
        const long long tiles = max_row_tiles(N, E, GBM) * ((f + GBN - 1) / GBN);
        if (dt == MOE_BF16)
            ffn_generic_kernel<uint16_t, uint16_t, true><<<grid_for(tiles), 256, 0, st>>>(
                (const uint16_t*)x, ldx, offsets, N, d, f, E, (const uint16_t*)wg,
                (const uint16_t*)wv, (uint16_t*)h, (uint16_t*)act);
        else
            ffn_generic_kernel<float, float, true><<<grid_for(tiles), 256, 0, st>>>(
                (const float*)x, ldx, offsets, N, d, f, E, (const float*)wg, (const float*)wv,
                (float*)h, (float*)act);
    }
    return hipGetLastError();
}

hipError_t launch_down(const void* h, moe_dtype dt, int N, int f, int d, int E,
                       const int32_t* offsets, const void* wo, void* y, moe_dtype y_dt,
                       hipStream_t st)
{
    if (ffn_down_uses_mfma(dt, f, d, h, wo) && aligned16(y)) {
        const unsigned grid = mfma_grid(N, E, d / 256);
        if (y_dt == MOE_BF16)
            ffn_mfma_kernel<false, true, false><<<grid, kMfmaThreads, 0, st>>>(
                (const uint16_t*)h, f, offsets, N, f, d, E, (const uint16_t*)wo, nullptr, y,
                nullptr);
        else
            ffn_mfma_kernel<false, false, false><<<grid, kMfmaThreads, 0, st>>>(
                (const uint16_t*)h, f, offsets, N, f, d, E, (const uint16_t*)wo, nullptr, y,
                nullptr);
    } else {
        const long long tiles = max_row_tiles(N, E, GBM) * ((d + GBN - 1) / GBN);
        const unsigned g = grid_for(tiles);
        if (dt == MOE_BF16) {
            if (y_dt == MOE_BF16)
                ffn_generic_kernel<uint16_t, uint16_t, false><<<g, 256, 0, st>>>(
                    (const uint16_t*)h, f, offsets, N, f, d, E, (const uint16_t*)wo, nullptr,
                    (uint16_t*)y, nullptr);
            else
                ffn_generic_kernel<uint16_t, float, false><<<g, 256, 0, st>>>(
                    (const uint16_t*)h, f, offsets, N, f, d, E, (const uint16_t*)wo, nullptr,
                    (float*)y, nullptr);
        } else {
            if (y_dt == MOE_BF16)
                ffn_generic_kernel<float, uint16_t, false><<<g, 256, 0, st>>>(
                    (const float*)h, f, offsets, N, f, d, E, (const float*)wo, nullptr, (uint16_t*)y,
                    nullptr);
            else
                ffn_generic_kernel<float, float, false><<<g, 256, 0, st>>>(
                    (const float*)h, f, offsets, N, f, d, E, (const float*)wo, nullptr, (float*)y,
                    nullptr);
        }
    }
    return hipGetLastError();
}

MOE_DBG_READER(ffn)

}  // namespace moe
