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
// core would sum in its own order). route_scores_kernel tiles the [T,E]
// score matrix 32 tokens x 32 experts per block; each thread runs the chains
// of 2 tokens x 2 experts side by side, reading x and W_r from LDS (staged
// in 64-wide d-chunks, the next chunk prefetched into registers while the
// current one is consumed). Zero padding of a chunk past d adds +-0 to a sum
// that is never -0, so no bit changes. route_topk_kernel then gives each
// token one wavefront: its E <= 1024 scores spread over the 64 lanes, k
// rounds of a wave-wide arg-max under (score descending, index ascending),
// then the softmax weights.
#include <algorithm>

#include "common.hpp"

namespace moe {

constexpr int kRT = 32;       // tokens per block
constexpr int kRE = 32;       // experts per block
constexpr int kRD = 64;       // d-chunk
constexpr int kRS = kRD + 4;  // LDS row stride (floats) of both staged tiles

template <typename XT, bool VEC>
__device__ __forceinline__ void load4(const XT* p, size_t i, bool in, float (&v)[4]) {
    if (!in) { v[0] = v[1] = v[2] = v[3] = 0.0f; return; }
    if constexpr (VEC) {
        if constexpr (sizeof(XT) == 2) {
            const u32x2 u = *reinterpret_cast<const u32x2*>(p + i);
            v[0] = __uint_as_float(u[0] << 16);
            v[1] = __uint_as_float(u[0] & 0xffff0000u);
            v[2] = __uint_as_float(u[1] << 16);
            v[3] = __uint_as_float(u[1] & 0xffff0000u);
        } else {
            const f32x4 u = *reinterpret_cast<const f32x4*>(p + i);
            v[0] = u[0]; v[1] = u[1]; v[2] = u[2]; v[3] = u[3];
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = Elem<XT>::load(p, i + q);
    }
}

// VEC: d % 4 == 0, E % 4 == 0 and aligned pointers (4-element vector loads).
// Block: 32 tokens x 32 experts; thread (tx, ty) owns tokens ty, ty+16 and
// experts tx, tx+16. x is staged [token][i] and W_r transposed to
// [expert][i], so both operands of four consecutive FMA steps are one
// 16-byte LDS read; rows are padded to 68 floats, which puts the eight
// lanes of each 16-byte read phase in distinct banks.
template <typename XT, bool VEC>
__global__ __launch_bounds__(256) void route_scores_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias,
    int T, int d, int E, float* __restrict__ logits)
{
    __shared__ __attribute__((aligned(16))) float xs[kRT * kRS];
    __shared__ __attribute__((aligned(16))) float wt[kRE * kRS];

    const int tid = threadIdx.x;
    const int tx = tid & 15;
    const int ty = tid >> 4;
    const int t0 = blockIdx.x * kRT;
    const int e0 = blockIdx.y * kRE;

    // staging: x 32 tokens x 64 values and W_r 64 rows x 32 experts, each as
    // 512 groups of 4 consecutive values, two groups of each per thread
    float xr[2][4], wr[2][4];
    auto load_chunk = [&](int i0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int gq = tid + 256 * u;
            const int tl = gq >> 4, i4 = (gq & 15) * 4;
            const int t = t0 + tl, i = i0 + i4;
            if (VEC) {
                load4<XT, true>(x, (size_t)t * d + i, t < T && i < d, xr[u]);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    xr[u][c] = (t < T && i + c < d) ? Elem<XT>::load(x, (size_t)t * d + i + c) : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int gq = tid + 256 * u;
            const int il = gq >> 3, e4 = (gq & 7) * 4;
            const int i = i0 + il, e = e0 + e4;
            if (VEC) {
                load4<XT, true>(w, (size_t)i * E + e, i < d && e < E, wr[u]);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    wr[u][c] = (i < d && e + c < E) ? Elem<XT>::load(w, (size_t)i * E + e + c) : 0.0f;
            }
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int gq = tid + 256 * u;
            const int tl = gq >> 4, i4 = (gq & 15) * 4;
            f32x4 v = {xr[u][0], xr[u][1], xr[u][2], xr[u][3]};
            *reinterpret_cast<f32x4*>(&xs[tl * kRS + i4]) = v;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int gq = tid + 256 * u;
            const int il = gq >> 3, e4 = (gq & 7) * 4;
#pragma unroll
            for (int c = 0; c < 4; ++c) wt[(e4 + c) * kRS + il] = wr[u][c];
        }
    };

    float acc[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) { acc[b][0] = 0.0f; acc[b][1] = 0.0f; }

    load_chunk(0);
    for (int i0 = 0; i0 < d; i0 += kRD) {
        __syncthreads();          // previous chunk fully consumed
        store_chunk();
        __syncthreads();
        if (i0 + kRD < d) load_chunk(i0 + kRD);
        const int dc = min(kRD, ((d - i0) + 3) & ~3);
#pragma unroll 4
        for (int i = 0; i < dc; i += 4) {
            f32x4 xv[2], wv[2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
                xv[b] = *reinterpret_cast<const f32x4*>(&xs[(ty + 16 * b) * kRS + i]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
                wv[a] = *reinterpret_cast<const f32x4*>(&wt[(tx + 16 * a) * kRS + i]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int a = 0; a < 2; ++a)
                        acc[b][a] = __builtin_fmaf(xv[b][c], wv[a][c], acc[b][a]);
        }
    }

#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int e = e0 + tx + 16 * a;
        if (e >= E) continue;
        const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int t = t0 + ty + 16 * b;
            if (t >= T) continue;
            float l = acc[b][a];
            if (bias) l = l + bv;
            logits[(size_t)t * E + e] = l;
        }
    }
}

__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ gates)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const int EJ = (E + kWave - 1) / kWave;
    const float* l = logits + (size_t)t * E;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = lane + kWave * j;
        v[j] = (j < EJ && e < E) ? l[e] : 0.0f;
    }
    unsigned used = 0;
    float myv = 0.0f;
    int mye = 0;
    for (int s = 0; s < k; ++s) {
        float bv = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + kWave * j;
            if (j < EJ && e < E && !((used >> j) & 1u)) {
                if (v[j] > bv || (v[j] == bv && e < be)) { bv = v[j]; be = e; }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oe = __shfl_xor(be, off, kWave);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if ((be % kWave) == lane) used |= 1u << (be / kWave);
        if (lane == s) { myv = bv; mye = be; }
    }
    const float m = __shfl(myv, 0, kWave);
    const float u = lane < k ? expf(myv - m) : 0.0f;
    float denom;
    if (renorm) {
        denom = wave_sum_f32(u);
    } else {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + kWave * j;
            if (j < EJ && e < E) part += expf(v[j] - m);
        }
        denom = wave_sum_f32(part);
    }
    if (lane < k) {
        const size_t o = (size_t)t * k + lane;
        topk_idx[o] = mye;
        gates[o] = u / denom;
    }
}

template <typename XT>
static hipError_t launch_scores_t(const void* x, const void* w, const float* bias, int T, int d,
                                  int E, float* logits, hipStream_t st)
{
    const dim3 grid((T + kRT - 1) / kRT, (E + kRE - 1) / kRE);
    const bool vec = d % 4 == 0 && E % 4 == 0 && (uintptr_t)x % (4 * sizeof(XT)) == 0 &&
                     (uintptr_t)w % (4 * sizeof(XT)) == 0;
    if (vec)
        route_scores_kernel<XT, true><<<grid, 256, 0, st>>>((const XT*)x, (const XT*)w, bias, T,
                                                            d, E, logits);
    else
        route_scores_kernel<XT, false><<<grid, 256, 0, st>>>((const XT*)x, (const XT*)w, bias, T,
                                                             d, E, logits);
    return hipGetLastError();
}

hipError_t launch_route(const void* x, moe_dtype dt, const void* w, const float* bias, int T,
                        int d, int E, int k, int renorm, float* logits, int32_t* idx,
                        float* gates, hipStream_t st)
{
    hipError_t e = (dt == MOE_BF16) ? launch_scores_t<uint16_t>(x, w, bias, T, d, E, logits, st)
                                    : launch_scores_t<float>(x, w, bias, T, d, E, logits, st);
    if (e != hipSuccess) return e;
    route_topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, renorm, idx, gates);
    return hipGetLastError();
}

}  // namespace moe
