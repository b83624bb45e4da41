// Weighted combine / un-permute.
//
// "Three axes of Parallelism", Dispatch, expert computation and combine: each
// packed expert output goes back to its token, scaled by that slot's router
// weight, and a token's k contributions are added, giving the [T,D] layout
// again. Written as a gather per
// token (the deterministic form of the scatter-add, no atomics): one
// wavefront per token reads its k packed rows (indices and weights held in
// lanes 0..k-1 and broadcast by shuffles), sums them in fp32 in slot order,
// adds the always-on shared-expert row if given, and writes the token once.
#include "common.hpp"

namespace moe {

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(p);
        v[0] = u[0]; v[1] = u[1]; v[2] = u[2]; v[3] = u[3];
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
        f32x4 u = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(p) = u;
    }
    // non-temporal: the row is written once and read by a later kernel only
    static __device__ __forceinline__ void store_nt(float* p, const float (&v)[4]) {
        f32x4 u = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(u, reinterpret_cast<f32x4*>(p));
    }
};
template <> struct Vec4<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[4]) {
        const u32x2 u = *reinterpret_cast<const u32x2*>(p);
        v[0] = __uint_as_float(u[0] << 16);
        v[1] = __uint_as_float(u[0] & 0xffff0000u);
        v[2] = __uint_as_float(u[1] << 16);
        v[3] = __uint_as_float(u[1] & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[4]) {
        u32x2 u;
        u[0] = (unsigned)f32_to_bf16(v[0]) | ((unsigned)f32_to_bf16(v[1]) << 16);
        u[1] = (unsigned)f32_to_bf16(v[2]) | ((unsigned)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<u32x2*>(p) = u;
    }
    static __device__ __forceinline__ void store_nt(uint16_t* p, const float (&v)[4]) {
        u32x2 u;
        u[0] = (unsigned)f32_to_bf16(v[0]) | ((unsigned)f32_to_bf16(v[1]) << 16);
        u[1] = (unsigned)f32_to_bf16(v[2]) | ((unsigned)f32_to_bf16(v[3]) << 16);
        __builtin_nontemporal_store(u, reinterpret_cast<u32x2*>(p));
    }
};

template <typename YT, typename ST, typename OT, bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(
    const YT* __restrict__ y, const int32_t* __restrict__ dest, const float* __restrict__ gates,
    int T, int k, int d, const ST* __restrict__ shared, OT* __restrict__ out)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const long long rows = (long long)T * k;
    int my_j = -1;
    float my_g = 0.0f;
    if (lane < k) {
        my_j = dest[(size_t)t * k + lane];
        if (my_j < 0 || my_j >= rows) my_j = -1;
        my_g = gates ? gates[(size_t)t * k + lane] : 1.0f;
    }
    OT* o = out + (size_t)t * d;
    if constexpr (VEC) {
        constexpr int U = 2;
        for (int c0 = lane * 4; c0 < d; c0 += kWave * 4 * U) {
            float acc[U][4];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u][q] = 0.0f;
            for (int s = 0; s < k; ++s) {
                const int j = __shfl(my_j, s, kWave);
                const float g = __shfl(my_g, s, kWave);
                if (j < 0) continue;
                const YT* yr = y + (size_t)j * d;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * kWave * 4;
                    if (c < d) {
                        float v[4];
                        Vec4<YT>::load(yr + c, v);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[u][q] = __builtin_fmaf(g, v[q], acc[u][q]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave * 4;
                if (c < d) {
                    if (shared) {
                        float v[4];
                        Vec4<ST>::load(shared + (size_t)t * d + c, v);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[u][q] += v[q];
                    }
                    Vec4<OT>::store(o + c, acc[u]);
                }
            }
        }
    } else {
        for (int c = lane; c < d; c += kWave) {
            float acc = 0.0f;
            for (int s = 0; s < k; ++s) {
                const int j = __shfl(my_j, s, kWave);
                const float g = __shfl(my_g, s, kWave);
                if (j < 0) continue;
                acc = __builtin_fmaf(g, Elem<YT>::load(y, (size_t)j * d + c), acc);
            }
            if (shared) acc += Elem<ST>::load(shared, (size_t)t * d + c);
            Elem<OT>::store(out, (size_t)t * d + c, acc);
        }
    }
}

// k <= 8 with 4-element vectors: the k slots' row indices and weights are read
// out of lanes 0..k-1 once per token into scalar registers and each slot's
// row gets a buffer descriptor. A token with every slot kept has the loads
// of all its rows of a column window in flight before the first FMA (slots
// past k have empty descriptors: zeros without a memory access, weight 0); a
// token with dropped slots loads its kept rows one slot after the other. The
// sum runs in slot order as in the general kernel.
// AUX: the loads' cache policy; 2 = non-temporal (nt), for expert outputs
// far larger than the 256 MB Infinity Cache, which are read once: with nt
// loads and stores the combine's 8:1 read:write stream ran 5-7 % faster at
// T = 32768, d = 4096 (4.3 GB of fp32 rows).
template <typename YT, int AUX = 0> struct RowLoad;
template <int AUX> struct RowLoad<float, AUX> {
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off, float (&v)[4]) {
        const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
        v[0] = __uint_as_float(u[0]); v[1] = __uint_as_float(u[1]);
        v[2] = __uint_as_float(u[2]); v[3] = __uint_as_float(u[3]);
    }
};
template <int AUX> struct RowLoad<uint16_t, AUX> {
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off, float (&v)[4]) {
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
        v[0] = __uint_as_float(u[0] << 16);
        v[1] = __uint_as_float(u[0] & 0xffff0000u);
        v[2] = __uint_as_float(u[1] << 16);
        v[3] = __uint_as_float(u[1] & 0xffff0000u);
    }
};

// KM: slots held (k <= KM); U: 4-column groups per lane per window (k <= 2
// takes eight, so that a row's loads are in flight together).
template <typename YT, typename ST, typename OT, int KM, int U, bool NT>
__global__ __launch_bounds__(256) void combine_k8_kernel(
    const YT* __restrict__ y, const int32_t* __restrict__ dest, const float* __restrict__ gates,
    int T, int k, int d, const ST* __restrict__ shared, OT* __restrict__ out)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const long long rows = (long long)T * k;
    int my_j = -1;
    float my_g = 0.0f;
    if (lane < k) {
        my_j = dest[(size_t)t * k + lane];
        if (my_j < 0 || my_j >= rows) my_j = -1;
        my_g = gates ? gates[(size_t)t * k + lane] : 1.0f;
    }
    __amdgpu_buffer_rsrc_t row[KM];
    float g[KM];
    unsigned live = 0;   // slots with a kept row (the same in every lane)
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        const int j = __builtin_amdgcn_readlane(my_j, s);
        g[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), s));
        const bool on = s < k && j >= 0;
        if (on) live |= 1u << s;
        row[s] = tile_rsrc(y + (size_t)(on ? j : 0) * d, on ? d * (int)sizeof(YT) : 0);
    }
    OT* o = out + (size_t)t * d;
    if (live != (1u << k) - 1) {
        // some slot dropped (fixed capacity, or experts of other ranks): load
        // only the kept rows, one slot after the other, in slot order
        for (int c0 = lane * 4; c0 < d; c0 += kWave * 4 * U) {
            float acc[U][4];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u][q] = 0.0f;
            for (int s = 0; s < k; ++s) {
                if (!((live >> s) & 1u)) continue;
                __amdgpu_buffer_rsrc_t r = row[0];
                float gs = g[0];
#pragma unroll
                for (int q = 1; q < KM; ++q)
                    if (q == s) { r = row[q]; gs = g[q]; }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float v[4];
                    RowLoad<YT, NT ? 2 : 0>::load(r, (c0 + u * kWave * 4) * (int)sizeof(YT), v);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[u][q] = __builtin_fmaf(gs, v[q], acc[u][q]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave * 4;
                if (c < d) {
                    if (shared) {
                        float w[4];
                        Vec4<ST>::load(shared + (size_t)t * d + c, w);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[u][q] += w[q];
                    }
                    if constexpr (NT) Vec4<OT>::store_nt(o + c, acc[u]);
                    else Vec4<OT>::store(o + c, acc[u]);
                }
            }
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t srow =
        tile_rsrc(shared ? shared + (size_t)t * d : nullptr, shared ? d * (int)sizeof(ST) : 0);
    for (int c0 = lane * 4; c0 < d; c0 += kWave * 4 * U) {
        float v[KM][U][4], sv[U][4];
#pragma unroll
        for (int s = 0; s < KM; ++s)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // columns past d fall outside the row's descriptor: zeros
                const int c = c0 + u * kWave * 4;
                RowLoad<YT, NT ? 2 : 0>::load(row[s], c * (int)sizeof(YT), v[s][u]);
            }
        if (shared) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                RowLoad<ST, NT ? 2 : 0>::load(srow, (c0 + u * kWave * 4) * (int)sizeof(ST), sv[u]);
        }
        float acc[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[u][q] = 0.0f;
        // slots past k (and dropped ones) have weight 0 or zero rows: they
        // add +0, so every slot runs and the loads stay ahead of the FMAs
#pragma unroll
        for (int s = 0; s < KM; ++s) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u][q] = __builtin_fmaf(g[s], v[s][u][q], acc[u][q]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave * 4;
            if (c < d) {
                if (shared) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[u][q] += sv[u][q];
                }
                if constexpr (NT) Vec4<OT>::store_nt(o + c, acc[u]);
                else Vec4<OT>::store(o + c, acc[u]);
            }
        }
    }
}

template <typename YT, typename ST, typename OT>
static hipError_t launch_combine_t(const void* y, const int32_t* dest, const float* gates, int T,
                                   int k, int d, const void* sh, void* out, hipStream_t st)
{
    const dim3 grid((T + 3) / 4);
    auto al = [](const void* p, size_t a) { return p == nullptr || (uintptr_t)p % a == 0; };
    const bool vec = d % 4 == 0 && al(y, 4 * sizeof(YT)) && al(sh, 4 * sizeof(ST)) &&
                     al(out, 4 * sizeof(OT));
    const bool rows_ok = (long long)d * sizeof(YT) < (1LL << 31) && (long long)d * sizeof(ST) < (1LL << 31);
    // rows far past the Infinity Cache are streamed with non-temporal accesses
    const bool nt = (long long)T * k * d * (long long)sizeof(YT) > kStreamBytes;
    if (vec && k <= 2 && rows_ok && !nt)
        combine_k8_kernel<YT, ST, OT, 2, 8, false><<<grid, 256, 0, st>>>(
            (const YT*)y, dest, gates, T, k, d, (const ST*)sh, (OT*)out);
    else if (vec && k <= 2 && rows_ok)
        combine_k8_kernel<YT, ST, OT, 2, 8, true><<<grid, 256, 0, st>>>(
            (const YT*)y, dest, gates, T, k, d, (const ST*)sh, (OT*)out);
    else if (vec && k <= 8 && rows_ok && !nt)
        combine_k8_kernel<YT, ST, OT, 8, 2, false><<<grid, 256, 0, st>>>(
            (const YT*)y, dest, gates, T, k, d, (const ST*)sh, (OT*)out);
    else if (vec && k <= 8 && rows_ok)
        combine_k8_kernel<YT, ST, OT, 8, 2, true><<<grid, 256, 0, st>>>(
            (const YT*)y, dest, gates, T, k, d, (const ST*)sh, (OT*)out);
    else if (vec)
        combine_kernel<YT, ST, OT, true><<<grid, 256, 0, st>>>(
            (const YT*)y, dest, gates, T, k, d, (const ST*)sh, (OT*)out);
    else
        combine_kernel<YT, ST, OT, false><<<grid, 256, 0, st>>>(
            (const YT*)y, dest, gates, T, k, d, (const ST*)sh, (OT*)out);
    return hipGetLastError();
}

template <typename YT, typename ST>
static hipError_t launch_combine_o(moe_dtype out_dt, const void* y, const int32_t* dest,
                                   const float* gates, int T, int k, int d, const void* sh,
                                   void* out, hipStream_t st)
{
    if (out_dt == MOE_BF16) return launch_combine_t<YT, ST, uint16_t>(y, dest, gates, T, k, d, sh, out, st);
    return launch_combine_t<YT, ST, float>(y, dest, gates, T, k, d, sh, out, st);
}

template <typename YT>
static hipError_t launch_combine_s(moe_dtype sh_dt, moe_dtype out_dt, const void* y,
                                   const int32_t* dest, const float* gates, int T, int k, int d,
                                   const void* sh, void* out, hipStream_t st)
{
    if (sh_dt == MOE_BF16) return launch_combine_o<YT, uint16_t>(out_dt, y, dest, gates, T, k, d, sh, out, st);
    return launch_combine_o<YT, float>(out_dt, y, dest, gates, T, k, d, sh, out, st);
}

hipError_t launch_combine(const void* y, moe_dtype y_dt, const int32_t* dest, const float* gates,
                          int T, int k, int d, const void* sh, moe_dtype sh_dt, void* out,
                          moe_dtype out_dt, hipStream_t st)
{
    if (y_dt == MOE_BF16)
        return launch_combine_s<uint16_t>(sh_dt, out_dt, y, dest, gates, T, k, d, sh, out, st);
    return launch_combine_s<float>(sh_dt, out_dt, y, dest, gates, T, k, d, sh, out, st);
}

// ------------------------------------------------------------------ backward
//
// Gradient of the combine: with out[t] = sum_s g[t,s] y[dest[t*k+s]],
//   d_y[dest[t*k+s]] = g[t,s] d_out[t]    (written in the activation type: the
//                                          input of the expert backward GEMMs)
//   d_g[t,s]        = <d_out[t], y[dest[t*k+s]]>
// One wavefront per token: for each slot it streams d_out[t] (cached after
// the first slot) and the slot's y row, writes the scaled row and reduces the
// dot product over the wave. A dropped assignment (dest < 0) gets d_g = 0 and
// no row.
template <typename GT, typename YT, typename DT, bool VEC>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const GT* __restrict__ d_out, const YT* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ gates, int T, int k, int d, DT* __restrict__ d_y,
    float* __restrict__ d_gates)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const long long rows = (long long)T * k;
    int my_j = -1;
    float my_g = 0.0f;
    if (lane < k) {
        my_j = dest[(size_t)t * k + lane];
        if (my_j < 0 || my_j >= rows) my_j = -1;
        my_g = gates[(size_t)t * k + lane];
    }
    const GT* go = d_out + (size_t)t * d;
    for (int s = 0; s < k; ++s) {
        const int j = __shfl(my_j, s, kWave);
        const float g = __shfl(my_g, s, kWave);
        float dot = 0.0f;
        if (j >= 0) {
            const YT* yr = y + (size_t)j * d;
            DT* dyr = d_y + (size_t)j * d;
            if constexpr (VEC) {
                for (int c = lane * 4; c < d; c += kWave * 4) {
                    float o[4], v[4], w[4];
                    Vec4<GT>::load(go + c, o);
                    Vec4<YT>::load(yr + c, v);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        dot = __builtin_fmaf(o[q], v[q], dot);
                        w[q] = g * o[q];
                    }
                    Vec4<DT>::store(dyr + c, w);
                }
            } else {
                for (int c = lane; c < d; c += kWave) {
                    const float o = Elem<GT>::load(go, c);
                    dot = __builtin_fmaf(o, Elem<YT>::load(yr, c), dot);
                    Elem<DT>::store(dyr, c, g * o);
                }
            }
        }
        dot = wave_sum_f32(dot);
        if (lane == 0) d_gates[(size_t)t * k + s] = dot;
    }
}

// 4-element vectors and d <= 4096: the token's d_out row stays in registers
// (one 4-element vector per lane per 256 columns) and is read once; each
// kept slot's y row is read through a scalar buffer descriptor with all of
// the row's loads in flight at once, d_y written through another. The dot
// product keeps the general kernel's order (per lane ascending columns, then
// the wavefront sum).
template <typename T> struct Raw4;
template <> struct Raw4<float> {
    typedef u32x4 type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
    static __device__ __forceinline__ void unpack(const type& u, float (&v)[4]) {
        v[0] = __uint_as_float(u[0]); v[1] = __uint_as_float(u[1]);
        v[2] = __uint_as_float(u[2]); v[3] = __uint_as_float(u[3]);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int off, const float (&v)[4]) {
        const u32x4 u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                         __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, 0);
    }
};
template <> struct Raw4<uint16_t> {
    typedef u32x2 type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
    static __device__ __forceinline__ void unpack(const type& u, float (&v)[4]) {
        v[0] = __uint_as_float(u[0] << 16);
        v[1] = __uint_as_float(u[0] & 0xffff0000u);
        v[2] = __uint_as_float(u[1] << 16);
        v[3] = __uint_as_float(u[1] & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int off, const float (&v)[4]) {
        const u32x2 u = {f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
    }
};

// NCH 256-column chunks per row (d <= 256 NCH): every chunk is loaded and
// stored unconditionally, the ones past d fall outside the row's descriptor.
template <typename GT, typename YT, typename DT, int NCH>
__global__ __launch_bounds__(256) void combine_bwd_reg_kernel(
    const GT* __restrict__ d_out, const YT* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ gates, int T, int k, int d, DT* __restrict__ d_y,
    float* __restrict__ d_gates)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const long long rows = (long long)T * k;
    int my_j = -1;
    float my_g = 0.0f;
    if (lane < k) {
        my_j = dest[(size_t)t * k + lane];
        if (my_j < 0 || my_j >= rows) my_j = -1;
        my_g = gates[(size_t)t * k + lane];
    }
    const __amdgpu_buffer_rsrc_t gr = tile_rsrc(d_out + (size_t)t * d, d * (int)sizeof(GT));
    typename Raw4<GT>::type o[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) o[i] = Raw4<GT>::load(gr, (lane * 4 + 256 * i) * (int)sizeof(GT));
    for (int s = 0; s < k; ++s) {
        const int j = __builtin_amdgcn_readlane(my_j, s);
        const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), s));
        float dot = 0.0f;
        if (j >= 0) {
            const __amdgpu_buffer_rsrc_t yr = tile_rsrc(y + (size_t)j * d, d * (int)sizeof(YT));
            const __amdgpu_buffer_rsrc_t dr = tile_rsrc(d_y + (size_t)j * d, d * (int)sizeof(DT));
            typename Raw4<YT>::type v[NCH];
#pragma unroll
            for (int i = 0; i < NCH; ++i) v[i] = Raw4<YT>::load(yr, (lane * 4 + 256 * i) * (int)sizeof(YT));
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                float of[4], vf[4], w[4];
                Raw4<GT>::unpack(o[i], of);
                Raw4<YT>::unpack(v[i], vf);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    dot = __builtin_fmaf(of[q], vf[q], dot);
                    w[q] = g * of[q];
                }
                Raw4<DT>::store(dr, (lane * 4 + 256 * i) * (int)sizeof(DT), w);
            }
        }
        dot = wave_sum_f32(dot);
        if (lane == 0) d_gates[(size_t)t * k + s] = dot;
    }
}

template <typename GT, typename YT, typename DT>
static hipError_t launch_combine_bwd_t(const void* d_out, const void* y, const int32_t* dest,
                                       const float* gates, int T, int k, int d, void* d_y,
                                       float* d_gates, hipStream_t st)
{
    const dim3 grid((T + 3) / 4);
    auto al = [](const void* p, size_t a) { return (uintptr_t)p % a == 0; };
    const bool vec = d % 4 == 0 && al(d_out, 4 * sizeof(GT)) && al(y, 4 * sizeof(YT)) &&
                     al(d_y, 4 * sizeof(DT));
    if (vec && d <= 2048)
        combine_bwd_reg_kernel<GT, YT, DT, 8><<<grid, 256, 0, st>>>(
            (const GT*)d_out, (const YT*)y, dest, gates, T, k, d, (DT*)d_y, d_gates);
    else if (vec && d <= 4096)
        combine_bwd_reg_kernel<GT, YT, DT, 16><<<grid, 256, 0, st>>>(
            (const GT*)d_out, (const YT*)y, dest, gates, T, k, d, (DT*)d_y, d_gates);
    else if (vec)
        combine_bwd_kernel<GT, YT, DT, true><<<grid, 256, 0, st>>>(
            (const GT*)d_out, (const YT*)y, dest, gates, T, k, d, (DT*)d_y, d_gates);
    else
        combine_bwd_kernel<GT, YT, DT, false><<<grid, 256, 0, st>>>(
            (const GT*)d_out, (const YT*)y, dest, gates, T, k, d, (DT*)d_y, d_gates);
    return hipGetLastError();
}

template <typename GT, typename YT>
static hipError_t launch_combine_bwd_d(moe_dtype dy_dt, const void* d_out, const void* y,
                                       const int32_t* dest, const float* gates, int T, int k,
                                       int d, void* d_y, float* d_gates, hipStream_t st)
{
    if (dy_dt == MOE_BF16)
        return launch_combine_bwd_t<GT, YT, uint16_t>(d_out, y, dest, gates, T, k, d, d_y, d_gates, st);
    return launch_combine_bwd_t<GT, YT, float>(d_out, y, dest, gates, T, k, d, d_y, d_gates, st);
}

template <typename GT>
static hipError_t launch_combine_bwd_y(moe_dtype y_dt, moe_dtype dy_dt, const void* d_out,
                                       const void* y, const int32_t* dest, const float* gates,
                                       int T, int k, int d, void* d_y, float* d_gates,
                                       hipStream_t st)
{
    if (y_dt == MOE_BF16)
        return launch_combine_bwd_d<GT, uint16_t>(dy_dt, d_out, y, dest, gates, T, k, d, d_y, d_gates, st);
    return launch_combine_bwd_d<GT, float>(dy_dt, d_out, y, dest, gates, T, k, d, d_y, d_gates, st);
}

// ------------------------------------------------- token input gradient
//
// d_x[t] = sum_s d_x_perm[dest[t*k+s]] + sum_s d_l[t,e_s] W_r[:,e_s], the
// packing's backward (every token sums its rows' input gradients) and the
// router scores' backward in one pass, for renormalised router weights:
// there d_l is nonzero only at the k selected experts, d_l[t,e_s] =
// g_s (dg_s - sum_r g_r dg_r), so the product with W_r^T is a gather of k
// rows of W_r^T (staged once per call, [E,d], L2-resident). One wavefront
// per token; lanes 0..k-1 hold the slot's row, expert and d_l, broadcast by
// shuffles; sums in fp32 in slot order; no atomics.
template <typename PT, typename WT, bool VEC>
__global__ __launch_bounds__(256) void token_grad_kernel(
    const PT* __restrict__ d_xp, const int32_t* __restrict__ dest, const int32_t* __restrict__ idx,
    const float* __restrict__ gates, const float* __restrict__ d_gates,
    const WT* __restrict__ w_t, int T, int k, int d, int E, float* __restrict__ d_x)
{
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const long long rows = (long long)T * k;
    int my_j = -1, my_e = 0;
    float my_g = 0.0f, my_dg = 0.0f;
    if (lane < k) {
        const size_t a = (size_t)t * k + lane;
        my_j = dest[a];
        if (my_j < 0 || my_j >= rows) my_j = -1;
        my_e = min(max(idx[a], 0), E - 1);
        my_g = gates[a];
        my_dg = d_gates[a];
    }
    const float gdg = wave_sum_f32(my_g * my_dg);
    const float my_dl = my_g * (my_dg - gdg);
    float* o = d_x + (size_t)t * d;
    if constexpr (VEC) {
        // two 4-column groups per lane per pass (more loads in flight)
        constexpr int U = 2;
        for (int c0 = lane * 4; c0 < d; c0 += kWave * 4 * U) {
            float acc[U][4];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u][q] = 0.0f;
            for (int s = 0; s < k; ++s) {
                const int j = __shfl(my_j, s, kWave);
                if (j < 0) continue;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * kWave * 4;
                    if (c < d) {
                        float v[4];
                        Vec4<PT>::load(d_xp + (size_t)j * d + c, v);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[u][q] += v[q];
                    }
                }
            }
            for (int s = 0; s < k; ++s) {
                const int e = __shfl(my_e, s, kWave);
                const float dl = __shfl(my_dl, s, kWave);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * kWave * 4;
                    if (c < d) {
                        float v[4];
                        Vec4<WT>::load(w_t + (size_t)e * d + c, v);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[u][q] = __builtin_fmaf(dl, v[q], acc[u][q]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave * 4;
                if (c < d) Vec4<float>::store(o + c, acc[u]);
            }
        }
    } else {
        for (int c = lane; c < d; c += kWave) {
            float acc = 0.0f;
            for (int s = 0; s < k; ++s) {
                const int j = __shfl(my_j, s, kWave);
                if (j >= 0) acc += Elem<PT>::load(d_xp, (size_t)j * d + c);
            }
            for (int s = 0; s < k; ++s) {
                const int e = __shfl(my_e, s, kWave);
                const float dl = __shfl(my_dl, s, kWave);
                acc = __builtin_fmaf(dl, Elem<WT>::load(w_t, (size_t)e * d + c), acc);
            }
            d_x[(size_t)t * d + c] = acc;
        }
    }
}

// w_t[e][i] = w[i][e] through 64 x 64 LDS tiles (w: [d, E])
template <typename WT>
__global__ __launch_bounds__(256) void transpose_kernel(const WT* __restrict__ w, int d, int E,
                                                       WT* __restrict__ w_t)
{
    __shared__ WT tile[64][65];
    const int i0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    for (int q = threadIdx.x; q < 64 * 64; q += 256) {
        const int r = q / 64, c = q % 64;
        if (i0 + r < d && e0 + c < E) tile[r][c] = w[(size_t)(i0 + r) * E + e0 + c];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * 64; q += 256) {
        const int r = q / 64, c = q % 64;
        if (e0 + r < E && i0 + c < d) w_t[(size_t)(e0 + r) * d + i0 + c] = tile[c][r];
    }
}

// k <= 8 with 4-element vectors: the slots' rows, experts and logit
// gradients read out of lanes 0..k-1 once per token into scalar registers,
// every row through a buffer descriptor (empty for a dropped slot or a slot
// past k: zeros without a memory access), and the k rows of d_x_perm and of
// W_r^T of a column window all in flight before the sums, which keep the
// general kernel's order (the d_x_perm rows in slot order, then the W_r^T
// terms in slot order).
template <typename PT, typename WT>
__global__ __launch_bounds__(256) void token_grad_k8_kernel(
    const PT* __restrict__ d_xp, const int32_t* __restrict__ dest, const int32_t* __restrict__ idx,
    const float* __restrict__ gates, const float* __restrict__ d_gates,
    const WT* __restrict__ w_t, int T, int k, int d, int E, float* __restrict__ d_x)
{
    constexpr int KM = 8, U = 2;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const long long rows = (long long)T * k;
    int my_j = -1, my_e = 0;
    float my_g = 0.0f, my_dg = 0.0f;
    if (lane < k) {
        const size_t a = (size_t)t * k + lane;
        my_j = dest[a];
        if (my_j < 0 || my_j >= rows) my_j = -1;
        my_e = min(max(idx[a], 0), E - 1);
        my_g = gates[a];
        my_dg = d_gates[a];
    }
    const float gdg = wave_sum_f32(my_g * my_dg);
    const float my_dl = my_g * (my_dg - gdg);
    __amdgpu_buffer_rsrc_t prow[KM], wrow[KM];
    float dl[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        const int j = __builtin_amdgcn_readlane(my_j, s);
        const int e = __builtin_amdgcn_readlane(my_e, s);
        dl[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_dl), s));
        const bool pon = s < k && j >= 0, won = s < k;
        prow[s] = tile_rsrc(d_xp + (size_t)(pon ? j : 0) * d, pon ? d * (int)sizeof(PT) : 0);
        wrow[s] = tile_rsrc(w_t + (size_t)e * d, won ? d * (int)sizeof(WT) : 0);
    }
    float* o = d_x + (size_t)t * d;
    for (int c0 = lane * 4; c0 < d; c0 += kWave * 4 * U) {
        float pv[KM][U][4], wv[KM][U][4];
#pragma unroll
        for (int s = 0; s < KM; ++s)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave * 4;
                RowLoad<PT>::load(prow[s], c * (int)sizeof(PT), pv[s][u]);
                RowLoad<WT>::load(wrow[s], c * (int)sizeof(WT), wv[s][u]);
            }
        float acc[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[u][q] = 0.0f;
#pragma unroll
        for (int s = 0; s < KM; ++s)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u][q] += pv[s][u][q];
#pragma unroll
        for (int s = 0; s < KM; ++s)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[u][q] = __builtin_fmaf(dl[s], wv[s][u][q], acc[u][q]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave * 4;
            if (c < d) Vec4<float>::store(o + c, acc[u]);
        }
    }
}

template <typename PT, typename WT>
static hipError_t launch_token_grad_t(const void* d_xp, const int32_t* dest, const int32_t* idx,
                                      const float* gates, const float* d_gates, const void* w,
                                      int T, int k, int d, int E, float* d_x, void* w_t,
                                      hipStream_t st)
{
    const dim3 tg((d + 63) / 64, (E + 63) / 64);
    transpose_kernel<WT><<<tg, 256, 0, st>>>((const WT*)w, d, E, (WT*)w_t);
    auto al = [](const void* p, size_t a) { return (uintptr_t)p % a == 0; };
    const bool vec = d % 4 == 0 && al(d_xp, 4 * sizeof(PT)) && al(w_t, 4 * sizeof(WT)) &&
                     al(d_x, 16);
    const dim3 grid((T + 3) / 4);
    if (vec && k <= 8 && d < (1 << 28))
        token_grad_k8_kernel<PT, WT><<<grid, 256, 0, st>>>(
            (const PT*)d_xp, dest, idx, gates, d_gates, (const WT*)w_t, T, k, d, E, d_x);
    else if (vec)
        token_grad_kernel<PT, WT, true><<<grid, 256, 0, st>>>(
            (const PT*)d_xp, dest, idx, gates, d_gates, (const WT*)w_t, T, k, d, E, d_x);
    else
        token_grad_kernel<PT, WT, false><<<grid, 256, 0, st>>>(
            (const PT*)d_xp, dest, idx, gates, d_gates, (const WT*)w_t, T, k, d, E, d_x);
    return hipGetLastError();
}

hipError_t launch_token_grad(const void* d_xp, moe_dtype p_dt, const int32_t* dest,
                             const int32_t* idx, const float* gates, const float* d_gates,
                             const void* w, moe_dtype w_dt, int T, int k, int d, int E,
                             float* d_x, void* w_t, hipStream_t st)
{
    if (p_dt == MOE_BF16) {
        if (w_dt == MOE_BF16)
            return launch_token_grad_t<uint16_t, uint16_t>(d_xp, dest, idx, gates, d_gates, w, T, k, d, E, d_x, w_t, st);
        return launch_token_grad_t<uint16_t, float>(d_xp, dest, idx, gates, d_gates, w, T, k, d, E, d_x, w_t, st);
    }
    if (w_dt == MOE_BF16)
        return launch_token_grad_t<float, uint16_t>(d_xp, dest, idx, gates, d_gates, w, T, k, d, E, d_x, w_t, st);
    return launch_token_grad_t<float, float>(d_xp, dest, idx, gates, d_gates, w, T, k, d, E, d_x, w_t, st);
}

hipError_t launch_combine_bwd(const void* d_out, moe_dtype g_dt, const void* y, moe_dtype y_dt,
                              const int32_t* dest, const float* gates, int T, int k, int d,
                              void* d_y, moe_dtype dy_dt, float* d_gates, hipStream_t st)
{
    if (g_dt == MOE_BF16)
        return launch_combine_bwd_y<uint16_t>(y_dt, dy_dt, d_out, y, dest, gates, T, k, d, d_y, d_gates, st);
    return launch_combine_bwd_y<float>(y_dt, dy_dt, d_out, y, dest, gates, T, k, d, d_y, d_gates, st);
}

}  // namespace moe
