// Router: scores, top-k selection and router weights in one kernel.
//
// "Three axes of Parallelism", Expert Parallel (EP) -> Producing assignments:
// the router scores every token against all E experts ([T,E]); top-K
// selection gives the expert ids and the weight with which each was chosen
// ([T,K] each).
//
// Scores are fixed bit for bit: an fp32 sum in index order, one fused
// multiply-add per term from +0, then one fp32 bias add. Each thread owns a
// few (token, expert) scores and runs their chains side by side; x and W_r
// are staged through LDS in d-chunks (zero padding of a chunk adds +-0 to a
// nonzero-or-+0 sum and so changes no bit). The scores of a block's tokens
// then sit in LDS and one wavefront per token picks the top k: E <= 1024
// scores spread over the 64 lanes, k rounds of a wave-wide arg-max under
// (score descending, index ascending).
#include "common.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouteTB = 4;          // tokens per thread
constexpr int kRouteXs = 4096;       // floats of the x tile
constexpr int kRouteWs = 8192;       // floats of the W_r chunk (reused for scores)

struct RouteGeom {
    int EC;   // expert lanes (power of two, <= 256)
    int EA;   // experts per thread
    int TG;   // token lanes = 256 / EC
    int TT;   // tokens per block
    int DC;   // d-chunk (multiple of 4)
};

static RouteGeom route_geom(int E) {
    RouteGeom g;
    g.EC = 1;
    while (g.EC * 2 <= E && g.EC * 2 <= 256) g.EC *= 2;
    g.EA = (E + g.EC - 1) / g.EC;
    g.TG = kRouteThreads / g.EC;
    g.TT = g.TG * kRouteTB;
    int dc = 64;
    dc = std::min(dc, kRouteWs / E);
    dc = std::min(dc, kRouteXs / g.TT);
    dc = (dc / 4) * 4;
    g.DC = std::max(dc, 4);
    return g;
}

template <typename XT, bool VEC>
__device__ __forceinline__ void load4(const XT* p, size_t i, float (&v)[4]) {
    if constexpr (VEC) {
        if constexpr (sizeof(XT) == 2) {
            u32x2 u = *reinterpret_cast<const u32x2*>(p + i);
            v[0] = __uint_as_float(u[0] << 16);
            v[1] = __uint_as_float(u[0] & 0xffff0000u);
            v[2] = __uint_as_float(u[1] << 16);
            v[3] = __uint_as_float(u[1] & 0xffff0000u);
        } else {
            f32x4 u = *reinterpret_cast<const f32x4*>(p + i);
            v[0] = u[0]; v[1] = u[1]; v[2] = u[2]; v[3] = u[3];
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = Elem<XT>::load(p, i + q);
    }
}

template <typename XT, int EA, bool VEC>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias,
    int T, int d, int E, int k, int renorm, int EC, int TG, int TT, int DC,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ gates)
{
    __shared__ __attribute__((aligned(16))) float xs[kRouteXs];
    __shared__ __attribute__((aligned(16))) float ws[kRouteWs];

    const int tid = threadIdx.x;
    const int te = tid % EC;
    const int tg = tid / EC;
    const int t0 = blockIdx.x * TT;
    const int DCP = DC;  // x tile row stride

    float acc[EA][kRouteTB];
#pragma unroll
    for (int a = 0; a < EA; ++a)
#pragma unroll
        for (int b = 0; b < kRouteTB; ++b) acc[a][b] = 0.0f;

    for (int i0 = 0; i0 < d; i0 += DC) {
        const int dc = min(DC, d - i0);
        const int dc4 = (dc + 3) & ~3;
        // x tile: TT tokens x dc4 values (zero beyond d or T)
        for (int q = tid; q < TT * (dc4 / 4); q += kRouteThreads) {
            const int tl = q / (dc4 / 4);
            const int i4 = (q % (dc4 / 4)) * 4;
            const int t = t0 + tl;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (t < T) {
                if (VEC) {
                    load4<XT, true>(x, (size_t)t * d + i0 + i4, v);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (i4 + c < dc) v[c] = Elem<XT>::load(x, (size_t)t * d + i0 + i4 + c);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) xs[tl * DCP + i4 + c] = v[c];
        }
        // W_r chunk: rows i0 .. i0+dc of [d,E], contiguous; zero rows to dc4
        {
            const size_t base = (size_t)i0 * E;
            const int n = dc * E;
            if (VEC) {
                for (int q = tid * 4; q < n; q += kRouteThreads * 4) {
                    float v[4];
                    load4<XT, true>(w, base + q, v);
#pragma unroll
                    for (int c = 0; c < 4; ++c) ws[q + c] = v[c];
                }
            } else {
                for (int q = tid; q < n; q += kRouteThreads) ws[q] = Elem<XT>::load(w, base + q);
            }
            for (int q = n + tid; q < dc4 * E; q += kRouteThreads) ws[q] = 0.0f;
        }
        __syncthreads();
        for (int i = 0; i < dc4; i += 4) {
            float wv[EA][4];
#pragma unroll
            for (int a = 0; a < EA; ++a) {
                const int e = min(te + EC * a, E - 1);
#pragma unroll
                for (int c = 0; c < 4; ++c) wv[a][c] = ws[(i + c) * E + e];
            }
#pragma unroll
            for (int b = 0; b < kRouteTB; ++b) {
                const f32x4 xv = *reinterpret_cast<const f32x4*>(&xs[(tg + TG * b) * DCP + i]);
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int a = 0; a < EA; ++a) acc[a][b] = __builtin_fmaf(xv[c], wv[a][c], acc[a][b]);
            }
        }
        __syncthreads();
    }

    // scores of this block's tokens -> LDS (reusing the W_r chunk)
    float* sl = ws;
#pragma unroll
    for (int a = 0; a < EA; ++a) {
        const int e = te + EC * a;
        if (e < E) {
            const float b = bias ? bias[e] : 0.0f;
#pragma unroll
            for (int bb = 0; bb < kRouteTB; ++bb) {
                float l = acc[a][bb];
                if (bias) l = l + b;
                sl[(tg + TG * bb) * E + e] = l;
            }
        }
    }
    __syncthreads();

    const int ntok = min(TT, T - t0);
    if (logits) {
        for (int q = tid; q < ntok * E; q += kRouteThreads)
            logits[(size_t)t0 * E + q] = sl[q];
    }

    // top-k: one wavefront per token
    const int wv_id = tid / kWave;
    const int lane = lane_id();
    const int EJ = (E + kWave - 1) / kWave;
    for (int tl = wv_id; tl < ntok; tl += kRouteThreads / kWave) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + kWave * j;
            v[j] = (j < EJ && e < E) ? sl[tl * E + e] : 0.0f;
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
            const size_t o = (size_t)(t0 + tl) * k + lane;
            topk_idx[o] = mye;
            gates[o] = u / denom;
        }
    }
}

template <typename XT, int EA>
static hipError_t launch_route_ea(const RouteGeom& g, bool vec, const void* x, const void* w,
                                  const float* bias, int T, int d, int E, int k, int renorm,
                                  float* logits, int32_t* idx, float* gates, hipStream_t st)
{
    const dim3 grid((T + g.TT - 1) / g.TT);
    if (vec)
        route_kernel<XT, EA, true><<<grid, kRouteThreads, 0, st>>>(
            (const XT*)x, (const XT*)w, bias, T, d, E, k, renorm, g.EC, g.TG, g.TT, g.DC,
            logits, idx, gates);
    else
        route_kernel<XT, EA, false><<<grid, kRouteThreads, 0, st>>>(
            (const XT*)x, (const XT*)w, bias, T, d, E, k, renorm, g.EC, g.TG, g.TT, g.DC,
            logits, idx, gates);
    return hipGetLastError();
}

template <typename XT>
static hipError_t launch_route_t(const void* x, const void* w, const float* bias, int T, int d,
                                 int E, int k, int renorm, float* logits, int32_t* idx,
                                 float* gates, hipStream_t st)
{
    const RouteGeom g = route_geom(E);
    const bool vec = (d % 4 == 0) && ((uintptr_t)x % (4 * sizeof(XT)) == 0) &&
                     ((uintptr_t)w % (4 * sizeof(XT)) == 0);
    switch (g.EA) {
        case 1: return launch_route_ea<XT, 1>(g, vec, x, w, bias, T, d, E, k, renorm, logits, idx, gates, st);
        case 2: return launch_route_ea<XT, 2>(g, vec, x, w, bias, T, d, E, k, renorm, logits, idx, gates, st);
        default: return launch_route_ea<XT, 4>(g, vec, x, w, bias, T, d, E, k, renorm, logits, idx, gates, st);
    }
}

hipError_t launch_route(const void* x, moe_dtype dt, const void* w, const float* bias, int T,
                        int d, int E, int k, int renorm, float* logits, int32_t* idx,
                        float* gates, hipStream_t st)
{
    if (dt == MOE_BF16)
        return launch_route_t<uint16_t>(x, w, bias, T, d, E, k, renorm, logits, idx, gates, st);
    return launch_route_t<float>(x, w, bias, T, d, E, k, renorm, logits, idx, gates, st);
}

}  // namespace moe
