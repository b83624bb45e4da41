// Backward of the grouped SwiGLU expert MLPs (and of the router's score
// product), as grouped matrix-core GEMMs.
//
// The pages' systems train the layer: gradients flow back through the expert
// MLPs and the permutation pair, and an expert's weight gradient is divided
// by the EP group size ("Three axes of Parallelism", EP backward pass). With
// a = x.W_gate[e], v = x.W_val[e], h = silu(a) * v, y = h.W_out[e] on the rows
// of expert e, the chain rule gives two product shapes:
//
//  * data gradients, rows grouped by expert, C = A . B_e^T (both operands
//    K-contiguous in memory):
//      dh   = dy . W_out[e]^T            (K = d),  fused SwiGLU backward:
//             da = dh * v * silu'(a), dv = dh * silu(a)  -> d_act = [da | dv]
//      dx   = [da | dv] . [W_gate[e] ; W_val[e]]^T   (K = 2f, two sources)
//      router: dx += dl . W_r^T          (one group, K = E)
//  * weight gradients, one output tile per (expert, m, n) with the expert's
//    rows as the reduction, C_e = scale * A_e^T . B_e (both operands row-major
//    with the rows as K):
//      dW_out[e]            = h^T . dy
//      [dW_gate | dW_val][e] = x^T . [da | dv]   (paired column tiles)
//      router: dW_r          = x^T . dl         (one group of all T rows)
//
// Both shapes reuse the forward's machinery: 256 threads as a 2 x 2 grid of
// wavefronts, v_mfma_f32_32x32x16_bf16 with fp32 accumulators, BK = 32 stages
// through a three-buffer LDS ring fed by three register stages of 16-byte
// global loads. A K-contiguous operand is staged [rows][32] with the a_swz
// swizzle and read as plain 16-byte fragments; a row-major operand whose rows
// are the reduction is staged [32][256] with b_swz and read with the gfx950
// LDS transpose read. Rows of the data-gradient kernel are scheduled by the
// forward's device-side tile list (256-row tiles, 128-row remainder tiles);
// the weight-gradient kernel walks the E x M/256 x N/256 tile list
// persistently, every pass giving each XCD a contiguous run, with a
// reduction of ceil(n_e/32) stages (rows past the expert's end load as
// zeros; an expert with no rows writes zeros). A plain fp32-FMA kernel covers fp32 data and shapes the
// matrix-core path does not tile.
#include "mfma_common.hpp"

namespace moe {

namespace {

constexpr int kT = 256;     // threads
constexpr int kK = 32;      // k per stage
constexpr int kN = 256;     // columns per tile
constexpr int kRingB = 3;   // LDS stage buffers
constexpr int kSetsB = 3;   // register stages in flight

// sigmoid with the hardware exp2 and reciprocal
__device__ __forceinline__ float sigmoid_fast(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Barrier that leaves this wavefront's P most recent LDS operations in flight
// (LDS operations of a wavefront complete in order; lgkmcnt counts to 15).
// The main loops issue the next stage's first fragment reads last in a step;
// they read a buffer no wavefront writes before the following barrier.
template <int P>
__device__ __forceinline__ void lds_barrier_keep() {
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" :: "n"(P < 15 ? P : 15) : "memory");
}

// SwiGLU backward of one element: h = silu(a) * v, silu(a) = a s, s = sigmoid(a),
// silu'(a) = s (1 + a (1 - s)).
__device__ __forceinline__ void swiglu_bwd(float dh, float a, float v, float& da, float& dv) {
    const float s = sigmoid_fast(a);
    da = dh * v * (s * (1.0f + a * (1.0f - s)));
    dv = dh * (a * s);
}

}  // namespace

enum NtEpi { kNtSwigluBwd = 0, kNtStoreF32 = 1, kNtAccumF32 = 2, kNtStoreBf16 = 3 };

// ----------------------------------------------- data gradients: C = A . B^T

struct NtArgs {
    const uint16_t* A;    // [rows, K], row stride K
    int K;                // reduction length (multiple of 32)
    const uint16_t* B0;   // per expert [N, K0]: B(k, n) = B0[e][n][k] for k < K0
    const uint16_t* B1;   // per expert [N, K - K0]: B(k, n) = B1[e][n][k - K0]
    int K0;               // multiple of 32
    int N;                // output columns
    void* C;              // swiglu-bwd: d_act [rows, 2N] bf16; else [rows, N]
    const uint16_t* act;  // swiglu-bwd: [rows, 2N] bf16, (a | v)
};

struct NtStage {
    u32x4 a[4];
    u32x4 b[4];
};

template <int EPI, int TM>
__device__ __forceinline__ void nt_tile(const NtArgs& p, const Tile& tile, uint16_t* smem)
{
    constexpr int kMI = TM / 64;                 // 32-row blocks per wavefront
    constexpr int kAC = TM * kK / 8 / kT;        // 16-byte A chunks per thread per stage
    constexpr int kBC = kN * kK / 8 / kT;        // 16-byte B chunks per thread per stage
    auto sA = [&](int b) { return smem + b * (TM * kK); };
    auto sB = [&](int b) { return smem + kRingB * (TM * kK) + b * (kN * kK); };

    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = tile.m0, seg_last = tile.seg_end - 1;
    const int n0 = tile.n_tile * kN;
    const int K = p.K, KT = K / kK, KT0 = p.K0 / kK, K1 = K - p.K0;

    // sources: A chunk i -> row tid/4 + 64 i (rows past the segment re-read
    // its last row, never stored), 16-byte chunk tid%4 of the stage's 64
    // bytes; B chunk i -> output column n0 + tid/4 + 64 i (clamped to N-1)
    const uint16_t* ap[kAC];
#pragma unroll
    for (int i = 0; i < kAC; ++i)
        ap[i] = p.A + (size_t)min(m0 + (tid >> 2) + 64 * i, seg_last) * K + (tid & 3) * 8;
    const uint16_t* bp0[kBC];
    const uint16_t* bp1[kBC];
#pragma unroll
    for (int i = 0; i < kBC; ++i) {
        const size_t n = (size_t)tile.e * p.N + min(n0 + (tid >> 2) + 64 * i, p.N - 1);
        bp0[i] = p.B0 + n * p.K0 + (tid & 3) * 8;
        bp1[i] = (K1 > 0 ? p.B1 + n * K1 : p.B0) + (tid & 3) * 8;
    }
    auto load = [&](int kt, NtStage& r) {
#pragma unroll
        for (int i = 0; i < kAC; ++i) r.a[i] = *reinterpret_cast<const u32x4*>(ap[i] + (size_t)kt * kK);
        const bool first = kt < KT0;
#pragma unroll
        for (int i = 0; i < kBC; ++i) {
            const uint16_t* q = first ? bp0[i] + (size_t)kt * kK : bp1[i] + (size_t)(kt - KT0) * kK;
            r.b[i] = *reinterpret_cast<const u32x4*>(q);
        }
    };
    // LDS destinations (the swizzle term does not change with + 64 rows)
    const int dst = (tid >> 2) * kK + a_swz(tid & 3, tid >> 2) * 8;
    auto store = [&](int buf, const NtStage& r) {
#pragma unroll
        for (int i = 0; i < kAC; ++i) *reinterpret_cast<u32x4*>(sA(buf) + dst + 64 * i * kK) = r.a[i];
#pragma unroll
        for (int i = 0; i < kBC; ++i) *reinterpret_cast<u32x4*>(sB(buf) + dst + 64 * i * kK) = r.b[i];
    };
    // fragments: row (or column) base + lane%32, 16-byte chunk 2 ks + lane/32;
    // + 32 rows per block (the swizzle term does not change with it)
    int a_lane[2], b_lane[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int ra = (TM / 2) * wm + (lane & 31);
        const int rb = 128 * wn + (lane & 31);
        a_lane[ks] = ra * kK + a_swz(2 * ks + (lane >> 5), ra) * 8;
        b_lane[ks] = rb * kK + a_swz(2 * ks + (lane >> 5), rb) * 8;
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
    auto read_frags = [&](int buf, int ks, Frags& fr) {
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
            fr.a[mi] = *reinterpret_cast<const bf16x8*>(sA(buf) + a_lane[ks] + 32 * mi * kK);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            fr.b[q] = *reinterpret_cast<const bf16x8*>(sB(buf) + b_lane[ks] + 32 * q * kK);
    };
    auto mfmas = [&](const Frags& fr) {
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[mi][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[mi], fr.b[q], acc[mi][q], 0, 0, 0);
    };

    // Stage s lives in register set s % 3, then LDS buffer s % 3. Step kt,
    // after a barrier that publishes stage kt+1 and retires every read of
    // buffer (kt-1) % 3: read the second k-substep of stage kt, MFMAs of the
    // first (read in the step before), store stage kt+2 into buffer
    // (kt-1) % 3 and reload its register set with stage kt+5, read the first
    // k-substep of stage kt+1, MFMAs of the second. Loads past the last stage
    // re-read it.
    auto clampk = [&](int k) { return min(k, KT - 1); };
    NtStage rs[kSetsB];
#pragma unroll
    for (int i = 0; i < kSetsB; ++i) load(clampk(i), rs[i]);
    lds_barrier();   // the block's previous tile is done with the ring
    store(0, rs[0]);
    load(clampk(3), rs[0]);
    store(1, rs[1]);
    load(clampk(4), rs[1]);
    lds_barrier();
    Frags f0, f1;
    read_frags(0, 0, f0);
    auto step = [&](int kt, int buf, NtStage& r) {
        const int nxt = buf == kRingB - 1 ? 0 : buf + 1;
        const int wr = nxt == kRingB - 1 ? 0 : nxt + 1;
        lds_barrier_keep<kMI + 4>();
        read_frags(buf, 1, f1);
        mfmas(f0);
        store(wr, r);
        load(clampk(kt + 5), r);
        read_frags(nxt, 0, f0);
        mfmas(f1);
        // issue order, so that every MFMA has LDS or global-memory work beside it:
        // the second k-substep's fragment reads over the first MFMAs, the
        // stage's LDS writes and global loads over the next, the next stage's
        // first fragment reads over the ones after
        if constexpr (TM == 256) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
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
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
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
    for (; kt + kSetsB <= KT; kt += kSetsB) {
#pragma unroll
        for (int u = 0; u < kSetsB; ++u) buf = step(kt + u, buf, rs[(u + 2) % kSetsB]);
    }
#pragma unroll
    for (int u = 0; u < kSetsB - 1; ++u)
        if (kt + u < KT) buf = step(kt + u, buf, rs[(u + 2) % kSetsB]);

    // Epilogue. A lane holds column lane%32 of each 32 x 32 block and rows
    // 8 (r/4) + 4 (lane/32) + r%4 for register r.
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
    if constexpr (EPI == kNtSwigluBwd) {
        // The SwiGLU backward reads a and v and writes da and dv, two bf16
        // tensors each: done element by element from the accumulator layout
        // that is four 2-byte accesses per element. Instead every wavefront
        // stages its dh rows, 32 at a time, row-major in its own slice of the
        // idle ring (fp32, row stride 136: the two rows a register spans fall
        // in different banks), and reads them back as 8 consecutive columns
        // per lane, so that a, v, da and dv move in 16-byte chunks.
        constexpr int SS = 136;
        lds_barrier();   // every wavefront is done with the stage buffers
        float* sw = reinterpret_cast<float*>(smem) + wave * (32 * SS);
        const int rr0 = lane >> 4;           // row within a group of 4
        const int c8 = (lane & 15) * 8;      // 8 columns of the wavefront's 128
        const int col = n0 + 128 * wn + c8;
        // act and d_act [rows, 2N] through buffer resources over the tile's
        // rows inside the segment; a lane whose columns lie past N gets an
        // offset outside them (its loads read zeros, its stores are dropped)
        const int nrows = min(TM, seg_last + 1 - m0);
        const int lim = nrows * 2 * p.N * 2;
        const __amdgpu_buffer_rsrc_t act_r = tile_rsrc(p.act + (size_t)m0 * 2 * p.N, lim);
        const __amdgpu_buffer_rsrc_t dact_r =
            tile_rsrc(static_cast<uint16_t*>(p.C) + (size_t)m0 * 2 * p.N, lim);
        const int vcol = col < p.N ? (((TM / 2) * wm + rr0) * 2 * p.N + col) * 2 : lim;
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sw[(8 * (r >> 2) + row_l + (r & 3)) * SS + 32 * q + col_l] = acc[mi][q][r];
            // LDS operations of a wavefront complete in order: the reads below
            // see these writes, and the next block's writes follow the reads
#pragma unroll 2
            for (int it = 0; it < 8; ++it) {
                const int rr = rr0 + 4 * it;
                const f32x4 h0 = *reinterpret_cast<const f32x4*>(&sw[rr * SS + c8]);
                const f32x4 h1 = *reinterpret_cast<const f32x4*>(&sw[rr * SS + c8 + 4]);
                const int o = vcol + (32 * mi + 4 * it) * 2 * p.N * 2;
                const u32x4 av = __builtin_amdgcn_raw_buffer_load_b128(act_r, o, 0, 0);
                const u32x4 vv = __builtin_amdgcn_raw_buffer_load_b128(act_r, o + p.N * 2, 0, 0);
                const float dh[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                u32x4 da_out, dv_out;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float da0, dv0, da1, dv1;
                    swiglu_bwd(dh[2 * w], __uint_as_float(av[w] << 16), __uint_as_float(vv[w] << 16), da0, dv0);
                    swiglu_bwd(dh[2 * w + 1], __uint_as_float(av[w] & 0xffff0000u),
                               __uint_as_float(vv[w] & 0xffff0000u), da1, dv1);
                    da_out[w] = f32x2_to_bf16x2(da0, da1);
                    dv_out[w] = f32x2_to_bf16x2(dv0, dv1);
                }
                __builtin_amdgcn_raw_buffer_store_b128(da_out, dact_r, o, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(dv_out, dact_r, o + p.N * 2, 0, 0);
            }
        }
        return;
    }
    // C [rows, N] through a buffer resource over the tile's rows inside the
    // segment; columns past N get an offset outside it (dropped, and read as
    // zero by the accumulating form)
    constexpr int ES = EPI == kNtStoreBf16 ? 2 : 4;
    const int nrows = min(TM, seg_last + 1 - m0);
    const int lim = nrows * p.N * ES;
    const __amdgpu_buffer_rsrc_t out =
        tile_rsrc(static_cast<char*>(p.C) + (size_t)m0 * p.N * ES, lim);
    int vq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int col = n0 + 128 * wn + 32 * q + col_l;
        vq[q] = col < p.N ? (((TM / 2) * wm + row_l) * p.N + col) * ES : lim;
    }
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ro = (32 * mi + 8 * (r >> 2) + (r & 3)) * p.N * ES;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v = acc[mi][q][r];
                if constexpr (EPI == kNtStoreF32) {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out, vq[q] + ro, 0, 0);
                } else if constexpr (EPI == kNtAccumF32) {
                    const float c = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(out, vq[q] + ro, 0, 0));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c + v), out, vq[q] + ro, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), out, vq[q] + ro, 0, 0);
                }
            }
        }
}

// LDS: ring of three stages sized for 256-row tiles (96 KB) + the tile list.
constexpr int kNtSmem = kRingB * (256 * kK + kN * kK);

template <int EPI>
__global__ __launch_bounds__(kT, 1) void nt_mfma_kernel(NtArgs p, const int32_t* __restrict__ offsets,
                                                       int rows, int E)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kNtSmem];
    __shared__ int s_sched[3 * kMaxE + 1];
    __shared__ int scratch[kT / kWave + 1];
    const TileList L = build_tile_list(offsets, rows, E, (p.N + kN - 1) / kN, s_sched,
                                       s_sched + kMaxE + 1, s_sched + 2 * kMaxE + 1, scratch);
    const int total = L.total_big + L.split + L.total_small;
    const int G = gridDim.x;
    const int base = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    for (int t = base; t < total; t += G) {
        const Tile tile = decode_tile(L, t);
        if (tile.bm == 128) nt_tile<EPI, 128>(p, tile, smem);
        else nt_tile<EPI, 256>(p, tile, smem);
    }
}

// ---------------------------------------- weight gradients: C_e = s A_e^T B_e

struct TnArgs {
    const uint16_t* A;  // [rows, lda]: A(k = row j, m) = A[j][m], m < M
    int lda, M;
    const uint16_t* B;  // [rows, ldb]: B(k = row j, n) = B[j][n]
    int ldb, Nc;        // Nc: output columns (per half when paired)
    int pair;           // > 0: paired tiles; tile column c < 128 is B column n0 + c
                        // (-> C0), c >= 128 is B column pair + n0 + c - 128 (-> C1)
    float* C0;          // [E, M, Nc] fp32
    float* C1;          // paired: second output [E, M, Nc]
    float scale;
    int split;          // offsets NULL and split > 0: group e is rows [e*split, (e+1)*split)
};

// Rows [j0, j1) of group e: the expert's segment, all rows, or one split.
__device__ __forceinline__ void group_rows(const int32_t* offsets, int split, int rows, int e,
                                           int& j0, int& j1) {
    if (offsets) {
        j0 = min(max(offsets[e], 0), rows);
        j1 = max(j0, min(offsets[e + 1], rows));
    } else if (split > 0) {
        j0 = min(e * split, rows);
        j1 = min(j0 + split, rows);
    } else {
        j0 = 0;
        j1 = rows;
    }
}

// One output tile of 256 x 256 per block iteration, 256 fp32 accumulators per
// lane (one block per CU). Measured against a 128-row tile with two blocks
// per CU: 12.6 against 14.8 ms on the stress-shaped backward, and no slower
// on the Qwen3 shape.
struct TnStage {
    u32x4 a[4];
    u32x4 b[4];
};

__global__ __launch_bounds__(kT, 1) void tn_mfma_kernel(
    TnArgs p, const int32_t* __restrict__ offsets, int rows, int E)
{
    constexpr int TM = 256;               // output rows (of M) per tile
    constexpr int kMI = TM / 64;          // 32-row blocks per wavefront (= A chunks per thread)
    constexpr int kAT = TM / 8;           // threads per A k-row (16-byte chunks)
    constexpr int kAR = kT / kAT;         // A k-rows per pass
    constexpr int kS = 3;                 // register stages in flight
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kRingB * kK * (TM + kN)];
    auto sA = [&](int b) { return smem + b * (kK * TM); };
    auto sB = [&](int b) { return smem + kRingB * (kK * TM) + b * (kK * kN); };

    const int mt_n = (p.M + TM - 1) / TM;
    const int ncols = p.pair > 0 ? 128 : kN;
    const int nt_n = (p.Nc + ncols - 1) / ncols;
    const int per_e = mt_n * nt_n;
    const int tiles = E * per_e;
    // Persistent: block b takes tiles t_i = i G + (b % 8) (G / 8) + b / 8, so in
    // every pass i each XCD (block b runs on XCD b % 8) works through a
    // contiguous run of the expert-major tile list at the same time, and the
    // tiles of one expert meet on one XCD at the same reduction position and
    // share their rows through its L2.
    const int G = gridDim.x;
    const int base = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    for (int t = base; t < tiles; t += G) {
    if (t != base) lds_barrier();   // the previous tile is done with the ring
    const int e = t / per_e;
    const int mt = (t % per_e) / nt_n;
    const int nt = t % nt_n;
    const int m0 = mt * TM, n0 = nt * ncols;
    int j0, j1;
    group_rows(offsets, p.split, rows, e, j0, j1);
    // uniform over the block: keep them (and what derives from them) scalar
    j0 = __builtin_amdgcn_readfirstlane(j0);
    j1 = __builtin_amdgcn_readfirstlane(j1);
    // stages of 32 rows, rounded up to a whole number of kS-step loop bodies
    // (the rows past the expert's end load as zeros and add nothing)
    const int KT = (j1 - j0 + kS * kK - 1) / (kS * kK) * kS;

    int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    f32x16 acc[kMI][4];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][q][r] = 0.0f;

    if (KT > 0) {
        // A chunk i: k-row tid/kAT + kAR i, 16-byte chunk tid%kAT of the TM
        // columns; B chunk i: k-row tid/32 + 8 i, chunk tid%32 of the 256
        // columns (columns clamped inside the operand; rows past the expert's
        // end load as zeros)
        const int ca = tid % kAT, cb = tid & 31;
        const int acol = min(m0 + 8 * ca, p.M - 8);
        int bcol;
        if (p.pair > 0) bcol = (cb < 16) ? min(n0 + 8 * cb, p.Nc - 8) : p.pair + min(n0 + 8 * (cb - 16), p.Nc - 8);
        else bcol = min(n0 + 8 * cb, p.Nc - 8);
        // A stage is read through buffer resources over its own 32 rows,
        // clipped at the group's end: rows past j1 (the padding of the last
        // loop body, and every stage past it) load as zeros without a memory
        // access, and the lane offsets stay small whatever the operand size.
        const int a_off = ((tid / kAT) * p.lda + acol) * 2;
        const int b_off = ((tid >> 5) * p.ldb + bcol) * 2;
        auto load = [&](int kt, TnStage& r) {
            const int j = j0 + kt * kK;
            const int live = min(max(j1 - j, 0), kK);   // rows of the stage inside the group
            const __amdgpu_buffer_rsrc_t ar = tile_rsrc(p.A + (size_t)j * p.lda, live * p.lda * 2);
            const __amdgpu_buffer_rsrc_t br = tile_rsrc(p.B + (size_t)j * p.ldb, live * p.ldb * 2);
#pragma unroll
            for (int i = 0; i < kMI; ++i)
                r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, a_off + kAR * i * p.lda * 2, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(br, b_off + 8 * i * p.ldb * 2, 0, 0);
        };
        const int adst = (tid / kAT) * TM + b_swz(ca, tid / kAT) * 8;
        const int bdst = (tid >> 5) * kN + b_swz(cb, tid >> 5) * 8;
        auto store = [&](int buf, const TnStage& r) {
#pragma unroll
            for (int i = 0; i < kMI; ++i)
                *reinterpret_cast<u32x4*>(sA(buf) + adst + kAR * i * TM) = r.a[i];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(sB(buf) + bdst + 8 * i * kN) = r.b[i];
        };
        // transpose-read fragments: in each 16-lane group g, lane j points at
        // k-row 8 (g/2) + j/4 and columns base + 16 (g%2) + 4 (j%4)..+3
        const int g = lane >> 4, jl = lane & 15;
        const int kr = 8 * (g >> 1) + (jl >> 2);
        int a_lane[kMI], b_lane[4];
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi) {
            const int m = (TM / 2) * wm + 32 * mi + 16 * (g & 1) + 4 * (jl & 3);
            a_lane[mi] = kr * TM + b_swz(m >> 3, kr) * 8 + (m & 7);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = 128 * wn + 32 * q + 16 * (g & 1) + 4 * (jl & 3);
            b_lane[q] = kr * kN + b_swz(n >> 3, kr) * 8 + (n & 7);
        }
        auto tr8 = [&](const uint16_t* s, int row_elems) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(s));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(s + 4 * row_elems));
            const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, v);
        };
        struct Frags {
            bf16x8 a[kMI];
            bf16x8 b[4];
        };
        auto read_frags = [&](int buf, int ks, Frags& fr) {
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi) fr.a[mi] = tr8(sA(buf) + a_lane[mi] + 16 * ks * TM, TM);
#pragma unroll
            for (int q = 0; q < 4; ++q) fr.b[q] = tr8(sB(buf) + b_lane[q] + 16 * ks * kN, kN);
        };
        auto mfmas = [&](const Frags& fr) {
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[mi][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[mi], fr.b[q], acc[mi][q], 0, 0, 0);
        };
        // The data-gradient kernel's pipeline: stage s lives in register set
        // s % 3, then LDS buffer s % 3; step kt reads the second k-substep of
        // stage kt, runs the MFMAs of the first (read in the step before),
        // stores stage kt+2 into the buffer stage kt-1 used (every wavefront
        // passed the barrier after its last read of it) and reloads its set
        // with stage kt+5, reads the first k-substep of stage kt+1, and runs
        // the MFMAs of the second. Stages past the last one load as zeros.
        TnStage rs[kS];
#pragma unroll
        for (int i = 0; i < kS; ++i) load(i, rs[i]);
        store(0, rs[0]);
        load(kS, rs[0]);
        store(1, rs[1]);
        load(kS + 1, rs[1]);
        lds_barrier();
        Frags f0, f1;
        read_frags(0, 0, f0);
        auto step = [&](int kt, int buf, TnStage& r) {
            const int nxt = buf == kRingB - 1 ? 0 : buf + 1;
            const int wr = nxt == kRingB - 1 ? 0 : nxt + 1;
            lds_barrier_keep<2 * (kMI + 4)>();
            read_frags(buf, 1, f1);
            mfmas(f0);
            store(wr, r);
            load(kt + 2 + kS, r);
            read_frags(nxt, 0, f0);
            mfmas(f1);
            // issue order: the 16 transpose reads of the second k-substep over
            // the first 16 MFMAs, the stage's LDS writes and global loads over
            // the next 8, the next stage's first 16 reads over the last 8
#pragma unroll
            for (int i = 0; i < 16; ++i) {
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
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            return nxt;
        };
        int buf = 0;
        for (int kt = 0; kt < KT; kt += kS) {
#pragma unroll
            for (int u = 0; u < kS; ++u) buf = step(kt + u, buf, rs[(u + 2) % kS]);
        }
    }

    // Epilogue: 32 lanes write 32 consecutive fp32 of one row per register.
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
    // Stores go through a buffer resource over the tile's rows below M;
    // columns past Nc get an offset outside it and are dropped.
    float* C = p.C0;
    int cbase = n0 + 128 * wn;
    if (p.pair > 0) {
        // wavefront column half wn: 0 -> first output, 1 -> second
        C = __builtin_amdgcn_readfirstlane(wn) ? p.C1 : p.C0;
        cbase = n0;
    }
    const int nrows = min(TM, p.M - m0);
    const int lim = nrows * p.Nc * 4;
    const __amdgpu_buffer_rsrc_t out = tile_rsrc(C + ((size_t)e * p.M + m0) * p.Nc, lim);
    int vq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int col = cbase + 32 * q + col_l;
        vq[q] = col < p.Nc ? (((TM / 2) * wm + row_l) * p.Nc + col) * 4 : lim;
    }
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ro = (32 * mi + 8 * (r >> 2) + (r & 3)) * p.Nc * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p.scale * acc[mi][q][r]), out,
                                                      vq[q] + ro, 0, 0);
        }
    }
}

// ------------------------------------------------------------ generic kernels

constexpr int kGM = 64, kGN = 64, kGK = 16;

// Data gradients, any shape and element type: 64 x 64 output tiles of the
// row-grouped product, one thread 4 x 4 outputs.
template <typename XT, int EPI>
__global__ __launch_bounds__(256) void nt_generic_kernel(
    const XT* __restrict__ A, int K, const XT* __restrict__ B0, const XT* __restrict__ B1, int K0,
    int N, void* __restrict__ C, const XT* __restrict__ act, const int32_t* __restrict__ offsets,
    int rows, int E)
{
    __shared__ float sA[kGM][kGK + 1];
    __shared__ float sB[kGK][kGN + 1];
    __shared__ int s_sched[2 * kMaxE + 1];
    __shared__ int scratch[256 / kWave + 1];
    Tile tile;
    if (!schedule_tile(offsets, rows, E, kGM, (N + kGN - 1) / kGN, s_sched, s_sched + kMaxE + 1,
                       scratch, tile))
        return;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int m0 = tile.m0, seg_last = tile.seg_end - 1;
    const int n0 = tile.n_tile * kGN;
    const int K1 = K - K0;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int k0 = 0; k0 < K; k0 += kGK) {
        for (int q = tid; q < kGM * kGK; q += 256) {
            const int r = q / kGK, kk = q % kGK;
            const int kx = k0 + kk;
            sA[r][kk] = kx < K ? Elem<XT>::load(A, (size_t)min(m0 + r, seg_last) * K + kx) : 0.f;
        }
        for (int q = tid; q < kGK * kGN; q += 256) {
            const int kk = q / kGN, c = q % kGN;
            const int kx = k0 + kk, n = n0 + c;
            float v = 0.f;
            if (kx < K && n < N) {
                const size_t nr = (size_t)tile.e * N + n;
                v = kx < K0 ? Elem<XT>::load(B0, nr * K0 + kx) : Elem<XT>::load(B1, nr * K1 + (kx - K0));
            }
            sB[kk][c] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[ty * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
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
            if (col >= N) continue;
            const float v = acc[i][j];
            if constexpr (EPI == kNtSwigluBwd) {
                const size_t o = (size_t)row * 2 * N + col;
                float da, dv;
                swiglu_bwd(v, Elem<XT>::load(act, o), Elem<XT>::load(act, o + N), da, dv);
                Elem<XT>::store(static_cast<XT*>(C), o, da);
                Elem<XT>::store(static_cast<XT*>(C), o + N, dv);
            } else if constexpr (EPI == kNtStoreF32) {
                static_cast<float*>(C)[(size_t)row * N + col] = v;
            } else if constexpr (EPI == kNtAccumF32) {
                static_cast<float*>(C)[(size_t)row * N + col] += v;
            } else {
                Elem<uint16_t>::store(static_cast<uint16_t*>(C), (size_t)row * N + col, v);
            }
        }
    }
}

// Weight gradients, any shape and element type: one 64 x 64 tile of
// C_e = scale * A_e^T B_e per block.
template <typename XT>
__global__ __launch_bounds__(256) void tn_generic_kernel(
    const XT* __restrict__ A, int lda, int M, const XT* __restrict__ B, int ldb, int Nc, int pair,
    float* __restrict__ C0, float* __restrict__ C1, float scale,
    const int32_t* __restrict__ offsets, int split, int rows, int E)
{
    __shared__ float sA[kGK][kGM + 1];
    __shared__ float sB[kGK][kGN + 1];
    const int mt_n = (M + kGM - 1) / kGM;
    const int halves = pair > 0 ? 2 : 1;
    const int nt_n = (Nc + kGN - 1) / kGN;
    const int per_e = mt_n * nt_n * halves;
    const int t = blockIdx.x;
    if (t >= E * per_e) return;
    const int e = t / per_e;
    const int rest = t % per_e;
    const int half = rest / (mt_n * nt_n);
    const int mt = (rest % (mt_n * nt_n)) / nt_n;
    const int nt = rest % nt_n;
    const int m0 = mt * kGM, n0 = nt * kGN;
    const int bcol0 = half ? pair : 0;
    int j0, j1;
    group_rows(offsets, split, rows, e, j0, j1);
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int k0 = j0; k0 < j1; k0 += kGK) {
        for (int q = tid; q < kGK * kGM; q += 256) {
            const int kk = q / kGM, c = q % kGM;
            const int j = k0 + kk, m = m0 + c;
            sA[kk][c] = (j < j1 && m < M) ? Elem<XT>::load(A, (size_t)j * lda + m) : 0.f;
        }
        for (int q = tid; q < kGK * kGN; q += 256) {
            const int kk = q / kGN, c = q % kGN;
            const int j = k0 + kk, n = n0 + c;
            sB[kk][c] = (j < j1 && n < Nc) ? Elem<XT>::load(B, (size_t)j * ldb + bcol0 + n) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* C = (half ? C1 : C0) + (size_t)e * M * Nc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < Nc) C[(size_t)m * Nc + n] = scale * acc[i][j];
        }
    }
}

// ----------------------------------------------------------------- launches

static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// C[rows, N] = A[rows, K] . B_e^T on the rows of each group (offsets NULL:
// one group of all rows), with epilogue `epi`.
hipError_t launch_nt(int epi, const void* A, moe_dtype dt, int rows, int K, int K0, int N, int E,
                     const int32_t* offsets, const void* B0, const void* B1, void* C,
                     const void* act, hipStream_t st)
{
    // (N < 2^20 keeps a tile's byte offsets in 31 bits)
    const bool mfma = dt == MOE_BF16 && K % kK == 0 && K0 % kK == 0 && K0 > 0 && N % 8 == 0 &&
                      N < (1 << 20) && al16(A) && al16(B0) && al16(B1) && al16(C) &&
                      (epi != kNtSwigluBwd || al16(act));
    if (mfma) {
        NtArgs p{(const uint16_t*)A, K, (const uint16_t*)B0, (const uint16_t*)B1, K0, N, C,
                 (const uint16_t*)act};
        const unsigned g = mfma_grid(rows, E, (N + kN - 1) / kN);
        switch (epi) {
        case kNtSwigluBwd: nt_mfma_kernel<kNtSwigluBwd><<<g, kT, 0, st>>>(p, offsets, rows, E); break;
        case kNtStoreF32: nt_mfma_kernel<kNtStoreF32><<<g, kT, 0, st>>>(p, offsets, rows, E); break;
        case kNtAccumF32: nt_mfma_kernel<kNtAccumF32><<<g, kT, 0, st>>>(p, offsets, rows, E); break;
        default: nt_mfma_kernel<kNtStoreBf16><<<g, kT, 0, st>>>(p, offsets, rows, E); break;
        }
        return hipGetLastError();
    }
    const long long tiles = max_row_tiles(rows, E, kGM) * ((N + kGN - 1) / kGN);
    const unsigned g = (unsigned)std::max(8LL, (tiles + 7) / 8 * 8);
#define NT_GEN(XT)                                                                                  \
    switch (epi) {                                                                                  \
    case kNtSwigluBwd: nt_generic_kernel<XT, kNtSwigluBwd><<<g, 256, 0, st>>>(                     \
        (const XT*)A, K, (const XT*)B0, (const XT*)B1, K0, N, C, (const XT*)act, offsets, rows, E); \
        break;                                                                                      \
    case kNtStoreF32: nt_generic_kernel<XT, kNtStoreF32><<<g, 256, 0, st>>>(                       \
        (const XT*)A, K, (const XT*)B0, (const XT*)B1, K0, N, C, (const XT*)act, offsets, rows, E); \
        break;                                                                                      \
    case kNtAccumF32: nt_generic_kernel<XT, kNtAccumF32><<<g, 256, 0, st>>>(                       \
        (const XT*)A, K, (const XT*)B0, (const XT*)B1, K0, N, C, (const XT*)act, offsets, rows, E); \
        break;                                                                                      \
    default: nt_generic_kernel<XT, kNtStoreBf16><<<g, 256, 0, st>>>(                               \
        (const XT*)A, K, (const XT*)B0, (const XT*)B1, K0, N, C, (const XT*)act, offsets, rows, E); \
        break;                                                                                      \
    }
    if (dt == MOE_BF16) { NT_GEN(uint16_t) } else { NT_GEN(float) }
#undef NT_GEN
    return hipGetLastError();
}

// C_e[M, Nc] = scale * A_e^T B_e over the rows of each group (offsets NULL:
// one group of all rows, or with split > 0 groups of `split` consecutive
// rows); pair > 0: B columns [0, Nc) -> C0 and [pair, pair + Nc) -> C1.
hipError_t launch_tn(const void* A, int lda, int M, const void* B, int ldb, int Nc, int pair,
                     moe_dtype dt, int rows, int E, const int32_t* offsets, float scale,
                     float* C0, float* C1, hipStream_t st, int split)
{
    // (Nc, lda, ldb < 2^20 keep a tile's byte offsets in 31 bits)
    const bool mfma = dt == MOE_BF16 && lda % 8 == 0 && ldb % 8 == 0 && M % 8 == 0 &&
                      Nc % 8 == 0 && Nc < (1 << 20) && lda < (1 << 20) && ldb < (1 << 20) &&
                      pair % 8 == 0 && M >= 8 && Nc >= 8 && al16(A) && al16(B);
    if (mfma) {
        TnArgs p{(const uint16_t*)A, lda, M, (const uint16_t*)B, ldb, Nc, pair, C0, C1, scale,
                 split};
        const long long tiles = (long long)E * ((M + kN - 1) / kN) *
                                ((Nc + (pair > 0 ? 128 : kN) - 1) / (pair > 0 ? 128 : kN));
        // resident blocks: one per CU, a multiple of 8
        const long long cap = (long long)mfma_grid(1 << 30, 1, 1);
        const unsigned g = (unsigned)std::max(8LL, std::min(cap, (tiles + 7) / 8 * 8));
        tn_mfma_kernel<<<g, kT, 0, st>>>(p, offsets, rows, E);
        return hipGetLastError();
    }
    const long long tiles = (long long)E * ((M + kGM - 1) / kGM) * ((Nc + kGN - 1) / kGN) *
                            (pair > 0 ? 2 : 1);
    if (dt == MOE_BF16)
        tn_generic_kernel<uint16_t><<<(unsigned)tiles, 256, 0, st>>>(
            (const uint16_t*)A, lda, M, (const uint16_t*)B, ldb, Nc, pair, C0, C1, scale, offsets,
            split, rows, E);
    else
        tn_generic_kernel<float><<<(unsigned)tiles, 256, 0, st>>>(
            (const float*)A, lda, M, (const float*)B, ldb, Nc, pair, C0, C1, scale, offsets, split,
            rows, E);
    return hipGetLastError();
}

// out[i] = sum over g ascending of part[g * n + i] (a fixed order: the result
// does not depend on the launch)
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int S,
                                                        long long n, float* __restrict__ out)
{
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    if (i + 4 <= n) {
        // eight partials in flight at a time, added in ascending g
        f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
        int g = 1;
        for (; g + 8 <= S; g += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *reinterpret_cast<const f32x4*>(part + (size_t)(g + u) * n + i);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc[0] += v[u][0]; acc[1] += v[u][1]; acc[2] += v[u][2]; acc[3] += v[u][3];
            }
        }
        for (; g < S; ++g) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)g * n + i);
            acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
        }
        *reinterpret_cast<f32x4*>(out + i) = acc;
    } else {
        for (long long q = i; q < n; ++q) {
            float acc = part[q];
            for (int g = 1; g < S; ++g) acc += part[(size_t)g * n + q];
            out[q] = acc;
        }
    }
}

// Row splits of the router's weight gradient (one output reduced over all T
// tokens): at most 16 groups, each a whole number of the kernel's 96-row loop
// bodies. More groups put more tiles in flight but write (and sum back) one
// fp32 [d, E] partial each: 16 took the step from 34.7 to 23.7 us at the
// Qwen3 shape against 43 (one group per 96 rows), and from 108 to 72 us on
// the stress shape against 64.
int router_splits(int T, int& split) {
    if (T <= 96) { split = 0; return 1; }
    const int S0 = std::min(16, (T + 95) / 96);
    split = ((T + S0 - 1) / S0 + 95) / 96 * 96;
    return (T + split - 1) / split;
}

hipError_t launch_sum_splits(const float* part, int S, long long n, float* out, hipStream_t st)
{
    const long long blocks = (n + 1023) / 1024;
    sum_splits_kernel<<<(unsigned)blocks, 256, 0, st>>>(part, S, n, out);
    return hipGetLastError();
}

MOE_DBG_READER(bwd)

}  // namespace moe
