// Router: scores, then top-k selection and router weights.
//
// "Three axes of Parallelism", Expert Parallel (EP) -> Producing assignments:
// the router scores every token against all E experts ([T,E]); top-K
// selection gives the expert ids and the weight with which each was chosen
// ([T,K] each).
//
// Scores are fixed bit for bit: an fp32 sum in index order, one fused
// multiply-add per term from +0, then one fp32 bias add. That makes the work
// T*E independent chains of d dependent FMAs on the vector ALUs (a matrix
// core would sum in its own order). route_scores_pc_kernel tiles the [T,E]
// score matrix 64 tokens x 32 experts per block; each of four wavefronts'
// threads runs the chains of 2 tokens x 4 experts side by side, reading x and
// W_r from LDS (d-chunks double-buffered in LDS), while four more wavefronts
// stage the chunks. route_scores_kernel_any does the same without the
// staging wavefronts for shapes and pointers vector loads do not fit. Zero
// padding of a chunk past d adds +-0 to a sum that is never -0, so no bit
// changes. route_topk_kernel then gives each
// token one wavefront: its E <= 1024 scores spread over the 64 lanes, k
// rounds of a wave-wide arg-max under (score descending, index ascending)
// with DPP and ballots, then the softmax weights.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace moe {

constexpr int kRT = 64;       // tokens per block
constexpr int kRE = 32;       // experts per block
constexpr int kRG = 8;        // steps per register group

// Score tile of this block in a 1-D grid of score_blocks(T, E) blocks: the
// expert tiles of one token tile go to blocks b, b + 8, b + 16, ..., which
// the hardware places on one XCD (blocks are dealt to the 8 XCDs round
// robin), so the token rows are read from HBM once and from that XCD's L2
// by the other expert tiles. Returns false for a block past the last token
// tile.
__device__ __forceinline__ bool score_tile(int T, int E, int& t0, int& e0) {
    const int et = (E + kRE - 1) / kRE;
    const int slot = blockIdx.x / 8;
    const int tt = (slot / et) * 8 + blockIdx.x % 8;
    t0 = tt * kRT;
    e0 = (slot % et) * kRE;
    return t0 < T;
}
inline unsigned score_blocks(int T, int E) {
    const long long tt = (T + kRT - 1) / kRT, et = (E + kRE - 1) / kRE;
    return (unsigned)((tt + 7) / 8 * 8 * et);
}

// Any d, E and alignment (element loads). Block: 64 tokens x 32 experts;
// thread (eg, tg) = (tid % 8, tid / 8) owns experts 4eg..4eg+3 and tokens tg,
// tg+32: eight FMA chains. x is staged [token][i] (rows padded to 132 floats:
// the 8 token rows a wavefront reads at once fall in distinct banks) and W_r
// as it is laid out, [i][expert], so one 16-byte LDS read gives four steps of
// a token or one step of four experts. d is walked in chunks of 128, double-
// buffered in LDS with one barrier per chunk; inside a chunk the LDS reads of
// the next 8 steps are issued before the 64 FMAs of the current 8.
__global__ __launch_bounds__(256) void route_scores_kernel_any(
    const void* __restrict__ xv, const void* __restrict__ wv, bool bf16,
    const float* __restrict__ bias, int T, int d, int E, float* __restrict__ logits)
{
    constexpr int kRD = 128;                        // d-chunk
    constexpr int kRS = kRD + 4;                    // x tile row stride (floats)
    constexpr int kXU = kRT * kRD / 1024;           // x groups of 4 per thread per chunk
    constexpr int kWU = kRD * kRE / 1024;           // W_r groups of 4 per thread per chunk
    constexpr int kRBuf = kRT * kRS + kRD * kRE;    // floats per LDS buffer
    __shared__ __attribute__((aligned(16))) float smem[2 * kRBuf];

    const int tid = threadIdx.x;
    const int eg = tid & 7;
    const int tg = tid >> 3;
    int t0, e0;
    if (!score_tile(T, E, t0, e0)) return;
    const int nchunks = (d + kRD - 1) / kRD;
    auto ld = [&](const void* p, size_t i) {
        return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
    };

    // staging of chunk c into LDS buffer c % 2 (zeros past T, d and E)
    auto stage = [&](int c) {
        const int i0 = c * kRD;
        float* xs = smem + (c & 1) * kRBuf;
        float* ws = xs + kRT * kRS;
#pragma unroll
        for (int u = 0; u < kXU; ++u) {
            const int gq = tid + 256 * u;
            const int tl = gq / (kRD / 4), i4 = (gq % (kRD / 4)) * 4;
            const int t = t0 + tl, i = i0 + i4;
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = (t < T && i + q < d) ? ld(xv, (size_t)t * d + i + q) : 0.0f;
            *reinterpret_cast<f32x4*>(&xs[tl * kRS + i4]) = v;
        }
#pragma unroll
        for (int u = 0; u < kWU; ++u) {
            const int gq = tid + 256 * u;
            const int il = gq >> 3, e4 = (gq & 7) * 4;
            const int i = i0 + il, e = e0 + e4;
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = (i < d && e + q < E) ? ld(wv, (size_t)i * E + e + q) : 0.0f;
            *reinterpret_cast<f32x4*>(&ws[il * kRE + e4]) = v;
        }
    };

    float acc[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[b][a] = 0.0f;

    // one group: x of 2 tokens x 8 steps, W_r of 8 steps x 4 experts
    struct Group {
        f32x4 x[2][2];
        f32x4 w[kRG];
    };
    auto read_group = [&](const float* xs, const float* ws, int i, Group& g) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                g.x[b][h] = *reinterpret_cast<const f32x4*>(&xs[(tg + 32 * b) * kRS + i + 4 * h]);
#pragma unroll
        for (int q = 0; q < kRG; ++q)
            g.w[q] = *reinterpret_cast<const f32x4*>(&ws[(i + q) * kRE + 4 * eg]);
    };
    auto fma_group = [&](const Group& g) {
#pragma unroll
        for (int q = 0; q < kRG; ++q)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    acc[b][a] = __builtin_fmaf(g.x[b][q >> 2][q & 3], g.w[q][a], acc[b][a]);
    };

    stage(0);
    lds_barrier();
    for (int c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) stage(c + 1);
        const float* xs = smem + (c & 1) * kRBuf;
        const float* ws = xs + kRT * kRS;
        // groups up to d rounded up to 8 (the tile holds zeros past d)
        const int n = min(kRD, d - c * kRD + kRG - 1) / kRG;
        Group g;
        for (int j = 0; j < n; ++j) {
            read_group(xs, ws, j * kRG, g);
            fma_group(g);
        }
        lds_barrier();
    }

#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int e = e0 + 4 * eg + a;
        if (e >= E) continue;
        const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int t = t0 + tg + 32 * b;
            if (t >= T) continue;
            float l = acc[b][a];
            if (bias) l = l + bv;
            logits[(size_t)t * E + e] = l;
        }
    }
}

// 4-element vector loads (d % 4 == 0, E % 4 == 0, aligned pointers): eight
// wavefronts, the first four run the FMA chains with the same thread mapping
// and order as route_scores_kernel_any, the last four only stage: global
// loads of chunk c + 2, conversion to fp32, the LDS writes of chunk c + 1
// while chunk c is consumed. One barrier per chunk. KRD is the d-chunk: 128
// (100 KB of LDS, one block per CU) when the grid has about one block per CU;
// 64 (50 KB, more blocks per CU) when there are many more blocks than CUs.
template <typename XT, int KRD>
__global__ __launch_bounds__(512) void route_scores_pc_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias,
    int T, int d, int E, float* __restrict__ logits)
{
    constexpr int kRD = KRD;                        // d-chunk
    constexpr int kRS = kRD + 4;                    // x tile row stride (floats)
    constexpr int kXU = kRT * kRD / 1024;           // x groups of 4 per staging thread per chunk
    constexpr int kWU = kRD * kRE / 1024;           // W_r groups of 4 per staging thread per chunk
    constexpr int kRBuf = kRT * kRS + kRD * kRE;    // floats per LDS buffer
    __shared__ __attribute__((aligned(16))) float smem[2 * kRBuf];

    int t0, e0;
    if (!score_tile(T, E, t0, e0)) return;
    const int nchunks = (d + kRD - 1) / kRD;
    const bool stager = threadIdx.x >= 256;          // wavefronts 4..7

    using Raw = typename std::conditional<sizeof(XT) == 2, u32x2, f32x4>::type;
    auto unpack = [&](const Raw& r, bool in, float (&v)[4]) {
        if constexpr (sizeof(XT) == 2) {
            v[0] = __uint_as_float(r[0] << 16);
            v[1] = __uint_as_float(r[0] & 0xffff0000u);
            v[2] = __uint_as_float(r[1] << 16);
            v[3] = __uint_as_float(r[1] & 0xffff0000u);
        } else {
            v[0] = r[0]; v[1] = r[1]; v[2] = r[2]; v[3] = r[3];
        }
        if (!in) v[0] = v[1] = v[2] = v[3] = 0.0f;
    };

    if (stager) {
        // x: 64 tokens x 128 values (8 groups of 4 per thread), W_r: 128 rows x
        // 32 experts (4 groups of 4), raw bits from clamped (always valid)
        // addresses, out-of-range groups zeroed when written to LDS
        const int tid = threadIdx.x - 256;
        Raw rx[kXU], rw[kWU];
        bool xin[kXU], win[kWU];
        auto load = [&](int c) {
            const int i0 = c * kRD;
#pragma unroll
            for (int u = 0; u < kXU; ++u) {
                const int gq = tid + 256 * u;
                const int tl = gq / (kRD / 4), i4 = (gq % (kRD / 4)) * 4;
                const int t = t0 + tl, i = i0 + i4;
                xin[u] = t < T && i < d;
                rx[u] = *reinterpret_cast<const Raw*>(x + (size_t)min(t, T - 1) * d + min(i, d - 4));
            }
#pragma unroll
            for (int u = 0; u < kWU; ++u) {
                const int gq = tid + 256 * u;
                const int il = gq >> 3, e4 = (gq & 7) * 4;
                const int i = i0 + il, e = e0 + e4;
                win[u] = i < d && e < E;
                rw[u] = *reinterpret_cast<const Raw*>(w + (size_t)min(i, d - 1) * E + min(e, E - 4));
            }
        };
        auto store = [&](int c) {
            float* xs = smem + (c & 1) * kRBuf;
            float* ws = xs + kRT * kRS;
#pragma unroll
            for (int u = 0; u < kXU; ++u) {
                const int gq = tid + 256 * u;
                const int tl = gq / (kRD / 4), i4 = (gq % (kRD / 4)) * 4;
                float v[4];
                unpack(rx[u], xin[u], v);
                const f32x4 q = {v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4*>(&xs[tl * kRS + i4]) = q;
            }
#pragma unroll
            for (int u = 0; u < kWU; ++u) {
                const int gq = tid + 256 * u;
                const int il = gq >> 3, e4 = (gq & 7) * 4;
                float v[4];
                unpack(rw[u], win[u], v);
                const f32x4 q = {v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4*>(&ws[il * kRE + e4]) = q;
            }
        };
        load(0);
        store(0);
        load(1);   // past the last chunk: clamped addresses, never stored
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) store(c + 1);
            if (c + 2 < nchunks) load(c + 2);
            lds_barrier();
        }
        return;
    }

    const int tid = threadIdx.x;
    const int eg = tid & 7;
    const int tg = tid >> 3;
    float acc[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[b][a] = 0.0f;
    struct Group {
        f32x4 x[2][2];
        f32x4 w[kRG];
    };
    auto read_group = [&](const float* xs, const float* ws, int i, Group& g) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                g.x[b][h] = *reinterpret_cast<const f32x4*>(&xs[(tg + 32 * b) * kRS + i + 4 * h]);
#pragma unroll
        for (int q = 0; q < kRG; ++q)
            g.w[q] = *reinterpret_cast<const f32x4*>(&ws[(i + q) * kRE + 4 * eg]);
    };
    auto fma_group = [&](const Group& g) {
#pragma unroll
        for (int q = 0; q < kRG; ++q)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    acc[b][a] = __builtin_fmaf(g.x[b][q >> 2][q & 3], g.w[q][a], acc[b][a]);
    };
    lds_barrier();   // chunk 0 is in LDS
    for (int c = 0; c < nchunks; ++c) {
        const float* xs = smem + (c & 1) * kRBuf;
        const float* ws = xs + kRT * kRS;
        Group g[2];
        if ((c + 1) * kRD <= d) {
            read_group(xs, ws, 0, g[0]);
#pragma unroll
            for (int j = 0; j < kRD / kRG; ++j) {
                if (j + 1 < kRD / kRG) read_group(xs, ws, (j + 1) * kRG, g[(j + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                fma_group(g[j & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // last, partial chunk: groups up to d rounded up to 8 (zeros past d)
            const int n = (d - c * kRD + kRG - 1) / kRG;
            for (int j = 0; j < n; ++j) {
                read_group(xs, ws, j * kRG, g[0]);
                fma_group(g[0]);
            }
        }
        lds_barrier();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int e = e0 + 4 * eg + a;
        if (e >= E) continue;
        const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int t = t0 + tg + 32 * b;
            if (t >= T) continue;
            float l = acc[b][a];
            if (bias) l = l + bv;
            logits[(size_t)t * E + e] = l;
        }
    }
}

// Maximum over the wavefront, in every lane: an inclusive max-scan with DPP
// row shifts (1, 2, 4, 8 lanes inside each row of 16) and row broadcasts
// (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3) leaves the maximum in
// lane 63, which is read out. Lanes without a source keep -inf, the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float v) {
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(-__builtin_inff()), __float_as_int(v),
                                              CTRL, ROW_MASK, 0xf, false);
    return fmaxf(v, __int_as_float(o));
}
__device__ __forceinline__ float wave_max_f32_dpp(float x) {
    x = dpp_max_step<0x111, 0xf>(x);   // row_shr:1
    x = dpp_max_step<0x112, 0xf>(x);   // row_shr:2
    x = dpp_max_step<0x114, 0xf>(x);   // row_shr:4
    x = dpp_max_step<0x118, 0xf>(x);   // row_shr:8
    x = dpp_max_step<0x142, 0xa>(x);   // row_bcast:15
    x = dpp_max_step<0x143, 0xc>(x);   // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}

// One wavefront per token; lane l holds scores l, l + 64, ... (EJ of them,
// E <= 64 EJ). Each of the k rounds takes the wavefront's maximum m of the
// scores not taken yet (DPP max-scan, no LDS round trips), then the lowest
// index holding m (a ballot per register; the indices of register j all lie
// below those of register j + 1), which is the order (score descending, index
// ascending). Then the softmax weights.
template <int EJ>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ gates)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const float* l = logits + (size_t)t * E;
    float v[EJ];
    unsigned avail = 0;   // bit j: score lane + 64 j exists and is not taken yet
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? l[e] : -__builtin_inff();
        if (e < E) avail |= 1u << j;
        MOE_DBG_CHECK(e >= E || __builtin_isfinite(v[j]), kDbgNonFinite);
    }
    float myv = 0.0f;
    int mye = 0;
    for (int s = 0; s < k; ++s) {
        float lv = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < EJ; ++j)
            if ((avail >> j) & 1u) lv = fmaxf(lv, v[j]);
        const float m = wave_max_f32_dpp(lv);
        // registers from the last to the first: the lowest one with a hit wins
        int be = 0x7fffffff;
#pragma unroll
        for (int j = EJ - 1; j >= 0; --j) {
            const unsigned long long hit = __ballot(((avail >> j) & 1u) && v[j] == m);
            if (hit) be = kWave * j + (__ffsll((long long)hit) - 1);
        }
        if (be != 0x7fffffff && (be & (kWave - 1)) == lane) avail &= ~(1u << (be / kWave));
        if (lane == s) { myv = m; mye = be; }
    }
    const float m = __shfl(myv, 0, kWave);
    const float u = lane < k ? expf(myv - m) : 0.0f;
    float denom;
    if (renorm) {
        denom = wave_sum_f32(u);
    } else {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            const int e = lane + kWave * j;
            if (e < E) part += expf(v[j] - m);
        }
        denom = wave_sum_f32(part);
    }
    if (lane < k) {
        const size_t o = (size_t)t * k + lane;
        topk_idx[o] = mye;
        gates[o] = u / denom;
    }
}

// Top-k with 16 lanes (one DPP row) per token, four tokens per wavefront, for
// k <= 16 and E <= 16 EJ: lane r of a row holds scores r, r + 16, ...; each
// round takes the row's maximum m of the scores not taken yet (DPP max-scan
// inside the row, lane 15 read back), then the lowest index holding m (a
// DPP min-scan of each lane's lowest candidate index), which is the order
// (score descending, index ascending). A quarter of the wavefronts of the
// one-token-per-wavefront kernel, for the same result.
template <int CTRL>
__device__ __forceinline__ float row_max_step(float v) {
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(-__builtin_inff()), __float_as_int(v),
                                              CTRL, 0xf, 0xf, false);
    return fmaxf(v, __int_as_float(o));
}
template <int CTRL>
__device__ __forceinline__ int row_min_step(int v) {
    const int o = __builtin_amdgcn_update_dpp(0x7fffffff, v, CTRL, 0xf, 0xf, false);
    return min(v, o);
}
// value of lane 15 of the calling lane's row, in every lane of the row
__device__ __forceinline__ float row_last_f32(float v) {
    return __int_as_float(__shfl(__float_as_int(v), lane_id() | 15, kWave));
}
__device__ __forceinline__ float row_max_f32(float v) {
    v = row_max_step<0x111>(v);   // row_shr:1
    v = row_max_step<0x112>(v);   // row_shr:2
    v = row_max_step<0x114>(v);   // row_shr:4
    v = row_max_step<0x118>(v);   // row_shr:8
    return row_last_f32(v);
}
__device__ __forceinline__ int row_min_i32(int v) {
    v = row_min_step<0x111>(v);
    v = row_min_step<0x112>(v);
    v = row_min_step<0x114>(v);
    v = row_min_step<0x118>(v);
    return __shfl(v, lane_id() | 15, kWave);
}
__device__ __forceinline__ float row_sum_f32(float v) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

template <int EJ>
__global__ __launch_bounds__(256) void route_topk_row_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ gates)
{
    // every lane runs every round (rows past T hold -inf and write nothing),
    // so the DPP row operations always read active lanes
    const int t = blockIdx.x * 16 + threadIdx.x / 16;
    const int r = threadIdx.x & 15;
    const bool live = t < T;
    const float* l = logits + (size_t)(live ? t : 0) * E;
    float v[EJ];
    unsigned avail = 0;   // bit j: score r + 16 j exists and is not taken yet
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = r + 16 * j;
        const bool in = live && e < E;
        v[j] = in ? l[e] : -__builtin_inff();
        if (in) avail |= 1u << j;
        MOE_DBG_CHECK(!in || __builtin_isfinite(v[j]), kDbgNonFinite);
    }
    float myv = 0.0f;
    int mye = 0;
    for (int s = 0; s < k; ++s) {
        float lv = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < EJ; ++j)
            if ((avail >> j) & 1u) lv = fmaxf(lv, v[j]);
        const float m = row_max_f32(lv);
        int cand = 0x7fffffff;
#pragma unroll
        for (int j = EJ - 1; j >= 0; --j)
            if (((avail >> j) & 1u) && v[j] == m) cand = r + 16 * j;
        const int be = row_min_i32(cand);
        if (be != 0x7fffffff && (be & 15) == r) avail &= ~(1u << (be >> 4));
        if (r == s) { myv = m; mye = be; }
    }
    const float m0 = __shfl(myv, threadIdx.x & ~15 & (kWave - 1), kWave);
    const float u = r < k ? expf(myv - m0) : 0.0f;
    float denom;
    if (renorm) {
        denom = row_sum_f32(u);
    } else {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < EJ; ++j)
            if (live && r + 16 * j < E) part += expf(v[j] - m0);
        denom = row_sum_f32(part);
    }
    if (live && r < k) {
        const size_t o = (size_t)t * k + r;
        topk_idx[o] = mye;
        gates[o] = u / denom;
    }
}

// Backward of the router weights, one wavefront per token. With g the
// weights of the k selected experts and dg their gradients, gdg = sum_s g_s dg_s:
//  renorm:    g = softmax over the selected logits, so
//             d_l[e_s] = g_s (dg_s - gdg) and 0 for every other expert;
//  otherwise: g_s = p_{e_s} with p the softmax over all E, so
//             d_l[e] = p_e ([e = e_s] dg_s - gdg).
// The selection itself is piecewise constant and passes no gradient. d_l is
// written in fp32 and, if asked, as a bf16 copy for the matrix-core products
// with x and W_r.
__global__ __launch_bounds__(256) void route_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ gates, const float* __restrict__ d_gates, int T, int E, int k,
    int renorm, float* __restrict__ d_logits, uint16_t* __restrict__ d_logits_bf16)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    int my_e = -1;
    float my_g = 0.0f, my_dg = 0.0f;
    if (lane < k) {
        my_e = topk_idx[(size_t)t * k + lane];
        my_g = gates[(size_t)t * k + lane];
        my_dg = d_gates[(size_t)t * k + lane];
    }
    const float gdg = wave_sum_f32(my_g * my_dg);
    const float* l = logits + (size_t)t * E;
    float m = 0.0f, denom = 1.0f;
    if (!renorm) {
        // the softmax over all E from the top logit (slot 0 holds it)
        m = l[min(max(__shfl(my_e, 0, kWave), 0), E - 1)];
        float part = 0.0f;
        for (int e = lane; e < E; e += kWave) part += expf(l[e] - m);
        denom = wave_sum_f32(part);
    }
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        // the slot that selected e, if any
        float sel_g = 0.0f, sel_dg = 0.0f;
        bool sel = false;
        for (int s = 0; s < k; ++s) {
            const int es = __shfl(my_e, s, kWave);
            const float gs = __shfl(my_g, s, kWave);
            const float dgs = __shfl(my_dg, s, kWave);
            if (es == e) { sel = true; sel_g = gs; sel_dg = dgs; }
        }
        if (e >= E) continue;
        float v;
        if (renorm) v = sel ? sel_g * (sel_dg - gdg) : 0.0f;
        else v = (expf(l[e] - m) / denom) * ((sel ? sel_dg : 0.0f) - gdg);
        if (d_logits) d_logits[(size_t)t * E + e] = v;
        if (d_logits_bf16) d_logits_bf16[(size_t)t * E + e] = f32_to_bf16(v);
    }
}

hipError_t launch_route_bwd(const float* logits, const int32_t* idx, const float* gates,
                            const float* d_gates, int T, int E, int k, int renorm,
                            float* d_logits, uint16_t* d_logits_bf16, hipStream_t st)
{
    route_bwd_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, idx, gates, d_gates, T, E, k, renorm,
                                                  d_logits, d_logits_bf16);
    return hipGetLastError();
}

// ------------------------------------------------------- load statistics
//
// p_mean[e] = (1/T) sum_t softmax(l[t,:])[e] and aux = E sum_e (counts[e] /
// (T k)) p_mean[e]. Two launches, no atomics (the same result on every run).
// Pass 1: block c takes the c-th of C equal token ranges in sub-chunks of 16
// tokens: sixteen threads per token find the maximum and the sum of exp of
// its logits (into LDS), then every thread adds the softmax probabilities of
// its experts (e = tid, tid + 256, ...) over the sub-chunk's tokens in
// ascending order, in fp64, into part[c][e].
constexpr int kStatSub = 16;
__global__ __launch_bounds__(256) void route_stats_partial_kernel(
    const float* __restrict__ logits, int T, int E, int C, double* __restrict__ part)
{
    __shared__ float s_m[kStatSub], s_z[kStatSub];
    const int tid = threadIdx.x;
    const int tc = (T + C - 1) / C;
    const int t0 = blockIdx.x * tc, t1 = min(T, t0 + tc);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};   // experts tid + 256 j (E <= 1024)
    for (int s0 = t0; s0 < t1; s0 += kStatSub) {
        const int n = min(kStatSub, t1 - s0);
        {
            // thread (i, p) = (tid / 16, tid % 16) takes logits p, p + 16, ... of
            // token i; the sixteen combine through lane shuffles
            const int i = tid >> 4, p = tid & 15;
            const float* l = logits + (size_t)(s0 + min(i, n - 1)) * E;
            float m = -__builtin_inff(), z = 0.0f;
            for (int e = p; e < E; e += 16) m = fmaxf(m, l[e]);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
            for (int e = p; e < E; e += 16) z += expf(l[e] - m);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, kWave);
            if (i < n && p == 0) { s_m[i] = m; s_z[i] = z; }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + 256 * j;
            if (e >= E) continue;
            const float* l = logits + (size_t)s0 * E + e;
            double a = acc[j];
            if (n == kStatSub) {
                // all sixteen tokens' logits in flight, added in ascending order
                float v[kStatSub];
#pragma unroll
                for (int u = 0; u < kStatSub; ++u) v[u] = l[(size_t)u * E];
#pragma unroll
                for (int u = 0; u < kStatSub; ++u) a += (double)(expf(v[u] - s_m[u]) / s_z[u]);
            } else {
                for (int i = 0; i < n; ++i) a += (double)(expf(l[(size_t)i * E] - s_m[i]) / s_z[i]);
            }
            acc[j] = a;
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + 256 * j;
        if (e < E) part[(size_t)blockIdx.x * E + e] = acc[j];
    }
}

// Pass 2, one block of 256 threads, experts in passes of 256 / G: G = 256 / E
// (a power of two, at least 1) threads per expert, thread (e, g) sums
// part[c][e] over c = g, g + G, ... ascending; the G sums are added pairwise
// in a fixed tree. p_mean[e] = sum / T; then, if asked, the load-balance
// statistic E * sum_e (counts_e / (T k)) p_mean_e (per-thread sums over the
// passes, then a fixed tree).
__global__ __launch_bounds__(256) void route_aux_kernel(const double* __restrict__ part, int C,
                                                       const int32_t* __restrict__ counts, int T,
                                                       int E, int G, int k,
                                                       float* __restrict__ p_mean,
                                                       float* __restrict__ aux)
{
    __shared__ double s[256];
    const int tid = threadIdx.x;
    const int g = tid % G;
    double acc = 0.0;
    for (int e0 = 0; e0 < E; e0 += 256 / G) {
        const int e = e0 + tid / G;
        double sum = 0.0;
        if (e < E) {
            int c = g;
            for (; c + 7 * G < C; c += 8 * G) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(c + u * G) * E + e];
#pragma unroll
                for (int u = 0; u < 8; ++u) sum += v[u];
            }
            for (; c < C; c += G) sum += part[(size_t)c * E + e];
        }
        s[tid] = sum;
        __syncthreads();
        for (int w = G >> 1; w > 0; w >>= 1) {
            if (g < w) s[tid] += s[tid + w];
            __syncthreads();
        }
        if (g == 0 && e < E) {
            const float pm = (float)(s[tid] / (double)T);
            p_mean[e] = pm;
            if (aux) acc += ((double)counts[e] / ((double)T * k)) * (double)pm;
        }
        __syncthreads();
    }
    if (!aux) return;
    s[tid] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) s[tid] += s[tid + w];
        __syncthreads();
    }
    if (tid == 0) *aux = (float)((double)E * s[0]);
}

int route_stat_chunks(int T) { return std::max(1, std::min(256, (T + 15) / 16)); }

hipError_t launch_route_stats(const float* logits, const int32_t* counts, int T, int E, int k,
                              float* p_mean, float* aux, double* part, hipStream_t st)
{
    const int C = route_stat_chunks(T);
    int G = 1;
    while (G * 2 * E <= 256) G *= 2;
    route_stats_partial_kernel<<<C, 256, 0, st>>>(logits, T, E, C, part);
    route_aux_kernel<<<1, 256, 0, st>>>(part, C, counts, T, E, G, k, p_mean, aux);
    return hipGetLastError();
}

template <typename XT>
static hipError_t launch_scores_t(const void* x, const void* w, const float* bias, int T, int d,
                                  int E, float* logits, hipStream_t st)
{
    const unsigned grid = score_blocks(T, E);
    const bool vec = d % 4 == 0 && E % 4 == 0 && (uintptr_t)x % (4 * sizeof(XT)) == 0 &&
                     (uintptr_t)w % (4 * sizeof(XT)) == 0;
    // many more blocks than compute units: the narrower chunk (more blocks per CU)
    const bool many = (long long)((T + kRT - 1) / kRT) * ((E + kRE - 1) / kRE) >= 2LL * 256;
    if (vec && many)
        route_scores_pc_kernel<XT, 64><<<grid, 512, 0, st>>>((const XT*)x, (const XT*)w, bias, T, d,
                                                             E, logits);
    else if (vec)
        route_scores_pc_kernel<XT, 128><<<grid, 512, 0, st>>>((const XT*)x, (const XT*)w, bias, T,
                                                              d, E, logits);
    else
        route_scores_kernel_any<<<grid, 256, 0, st>>>(x, w, sizeof(XT) == 2, bias, T, d, E, logits);
    return hipGetLastError();
}

hipError_t launch_route(const void* x, moe_dtype dt, const void* w, const float* bias, int T,
                        int d, int E, int k, int renorm, float* logits, int32_t* idx,
                        float* gates, hipStream_t st)
{
    hipError_t e = (dt == MOE_BF16) ? launch_scores_t<uint16_t>(x, w, bias, T, d, E, logits, st)
                                    : launch_scores_t<float>(x, w, bias, T, d, E, logits, st);
    if (e != hipSuccess) return e;
    if (k <= 16 && E <= 256) {
        const unsigned g16 = (T + 15) / 16;
        if (E <= 64)
            route_topk_row_kernel<4><<<g16, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
        else if (E <= 128)
            route_topk_row_kernel<8><<<g16, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
        else
            route_topk_row_kernel<16><<<g16, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
        return hipGetLastError();
    }
    const unsigned g = (T + 3) / 4;
    if (E <= 64) route_topk_kernel<1><<<g, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
    else if (E <= 128) route_topk_kernel<2><<<g, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
    else if (E <= 256) route_topk_kernel<4><<<g, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
    else if (E <= 512) route_topk_kernel<8><<<g, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
    else route_topk_kernel<16><<<g, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
    return hipGetLastError();
}

MOE_DBG_READER(route)

}  // namespace moe
