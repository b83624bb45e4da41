// C ABI of libmoe: host-side argument checks, workspace sizes and launches.
// Every check happens before anything is enqueued; nothing here waits on the
// device or copies device -> host.
#include <algorithm>

#include "common.hpp"

namespace moe {
hipError_t launch_route(const void* x, moe_dtype dt, const void* w, const float* bias, int T,
                        int d, int E, int k, int renorm, float* logits, int32_t* idx,
                        float* gates, hipStream_t st);
size_t permute_ws_bytes(int T, int k, int E);
hipError_t launch_permute(const int32_t* idx, int T, int k, int e_base, int E, int cap,
                          const void* x, int es, int d, int32_t* routed,
                          int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* dest,
                          void* x_perm, void* ws, hipStream_t st);
hipError_t launch_permute_recv(const int32_t* recv, int S, int E, int N, const void* x, int es,
                               int d, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                               int32_t* dest, void* x_perm, hipStream_t st);
hipError_t launch_gate_up(const void* x, moe_dtype dt, int N, int d, int f, int E,
                          const int32_t* offsets, const void* wg, const void* wv, void* h,
                          hipStream_t st);
hipError_t launch_down(const void* h, moe_dtype dt, int N, int f, int d, int E,
                       const int32_t* offsets, const void* wo, void* y, moe_dtype y_dt,
                       hipStream_t st);
hipError_t launch_combine(const void* y, moe_dtype y_dt, const int32_t* dest, const float* gates,
                          int T, int k, int d, const void* sh, moe_dtype sh_dt, void* out,
                          moe_dtype out_dt, hipStream_t st);
}  // namespace moe

namespace {

constexpr int kMaxRouteE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxFfnE = 4096;
constexpr int kMaxRecvCells = 4096;

bool valid_dtype(moe_dtype t) { return t == MOE_F32 || t == MOE_BF16; }
int elem_size(moe_dtype t) { return t == MOE_BF16 ? 2 : 4; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

size_t h_bytes(int N, int f, moe_dtype dt) {
    return moe::align_up((size_t)N * (size_t)f * (size_t)elem_size(dt), 256);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported size or type";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

int moe_version(void) { return 100; }

moe_status moe_route(const void* x, moe_dtype dt, const void* w_router, const float* bias,
                     int T, int d, int E, int k, int renorm, float* logits, int32_t* topk_idx,
                     float* gates, void* stream)
{
    if (!valid_dtype(dt) || T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E)
        return MOE_ERR_INVALID_ARG;
    if (E > kMaxRouteE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * E > INT32_MAX || (long long)T * d > (1LL << 40))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !logits || !topk_idx || !gates) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_route(x, dt, w_router, bias, T, d, E, k, renorm, logits,
                                        topk_idx, gates, as_stream(stream)));
}

size_t moe_permute_workspace(int T, int k, int E) {
    if (T < 0 || k <= 0 || E <= 0) return 0;
    return moe::permute_ws_bytes(T, k, E);
}

moe_status moe_permute(const int32_t* topk_idx, int T, int k, int E, const void* x,
                       moe_dtype dt, int d, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                       int32_t* dest, void* x_perm, void* ws, size_t ws_bytes, void* stream)
{
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E <= 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe::permute_ws_bytes(T, k, E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_idx, T, k, 0, E, INT32_MAX, x, elem_size(dt), d,
                                          nullptr, counts, offsets, perm_src, dest, x_perm, ws,
                                          as_stream(stream)));
}

moe_status moe_permute_capacity(const int32_t* topk_idx, int T, int k, int E, int capacity,
                                const void* x, moe_dtype dt, int d, int32_t* routed,
                                int32_t* counts, int32_t* offsets, int32_t* perm_src,
                                int32_t* dest, void* x_perm, void* ws, size_t ws_bytes,
                                void* stream)
{
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E <= 0 || d <= 0 || capacity < 0)
        return MOE_ERR_INVALID_ARG;
    if (E > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe::permute_ws_bytes(T, k, E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_idx, T, k, 0, E, capacity, x, elem_size(dt), d,
                                          routed, counts, offsets, perm_src, dest, x_perm, ws,
                                          as_stream(stream)));
}

moe_status moe_permute_range(const int32_t* topk_idx, int T, int k, int e_first, int E_loc,
                             const void* x, moe_dtype dt, int d, int32_t* counts,
                             int32_t* offsets, int32_t* perm_src, int32_t* dest, void* x_perm,
                             void* ws, size_t ws_bytes, void* stream)
{
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E_loc <= 0 || e_first < 0 || d <= 0)
        return MOE_ERR_INVALID_ARG;
    if (E_loc > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe::permute_ws_bytes(T, k, E_loc)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_idx, T, k, e_first, E_loc, INT32_MAX, x,
                                          elem_size(dt), d, nullptr, counts, offsets, perm_src,
                                          dest, x_perm, ws, as_stream(stream)));
}

size_t moe_permute_recv_workspace(int S, int E_loc, int N) {
    (void)S; (void)E_loc; (void)N;
    return 0;
}

moe_status moe_permute_recv(const int32_t* recv_counts, int S, int E_loc, int N,
                            const void* x_recv, moe_dtype dt, int d, int32_t* counts,
                            int32_t* offsets, int32_t* perm_src, int32_t* dest, void* x_perm,
                            void* ws, size_t ws_bytes, void* stream)
{
    (void)ws; (void)ws_bytes;
    if (!valid_dtype(dt) || S <= 0 || E_loc <= 0 || N < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    if ((long long)S * E_loc > kMaxRecvCells || E_loc > kMaxRouteE) return MOE_ERR_UNSUPPORTED;
    if (!recv_counts || !counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (N > 0 && (!x_recv || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_permute_recv(recv_counts, S, E_loc, N, x_recv, elem_size(dt), d,
                                               counts, offsets, perm_src, dest, x_perm,
                                               as_stream(stream)));
}

size_t moe_grouped_ffn_workspace(int N, int d, int f, int E, moe_dtype dt) {
    (void)d; (void)E;
    if (N < 0 || f <= 0 || !valid_dtype(dt)) return 0;
    return h_bytes(N, f, dt);
}

static moe_status check_ffn(moe_dtype dt, int N, int d, int f, int E, const int32_t* offsets) {
    if (!valid_dtype(dt) || N < 0 || d <= 0 || f <= 0 || E <= 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxFfnE) return MOE_ERR_UNSUPPORTED;
    if ((long long)N * std::max(d, f) > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
    if (!offsets) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status moe_ffn_gate_up(const void* x_perm, moe_dtype dt, int N, int d, int f, int E,
                           const int32_t* offsets, const void* w_gate, const void* w_val,
                           void* h, void* stream)
{
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    if (N == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_val || !h) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_gate_up(x_perm, dt, N, d, f, E, offsets, w_gate, w_val, h,
                                          as_stream(stream)));
}

moe_status moe_ffn_down(const void* h, moe_dtype dt, int N, int f, int d, int E,
                        const int32_t* offsets, const void* w_out, void* y, moe_dtype y_dt,
                        void* stream)
{
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    if (!valid_dtype(y_dt)) return MOE_ERR_INVALID_ARG;
    if (N == 0) return MOE_OK;
    if (!h || !w_out || !y) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_down(h, dt, N, f, d, E, offsets, w_out, y, y_dt,
                                       as_stream(stream)));
}

moe_status moe_grouped_ffn(const void* x_perm, moe_dtype dt, int N, int d, int f, int E,
                           const int32_t* offsets, const void* w_gate, const void* w_val,
                           const void* w_out, void* y, moe_dtype y_dt, void* ws, size_t ws_bytes,
                           void* stream)
{
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    if (!valid_dtype(y_dt)) return MOE_ERR_INVALID_ARG;
    if (N == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_val || !w_out || !y) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < h_bytes(N, f, dt)) return MOE_ERR_WORKSPACE;
    hipStream_t st = as_stream(stream);
    hipError_t e = moe::launch_gate_up(x_perm, dt, N, d, f, E, offsets, w_gate, w_val, ws, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(moe::launch_down(ws, dt, N, f, d, E, offsets, w_out, y, y_dt, st));
}

moe_status moe_combine(const void* y_perm, moe_dtype y_dt, const int32_t* dest,
                       const float* gates, int T, int k, int d, const void* y_shared,
                       moe_dtype sh_dt, void* out, moe_dtype out_dt, void* stream)
{
    if (!valid_dtype(y_dt) || !valid_dtype(out_dt) || T < 0 || k <= 0 || d <= 0)
        return MOE_ERR_INVALID_ARG;
    if (y_shared && !valid_dtype(sh_dt)) return MOE_ERR_INVALID_ARG;
    if (k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_perm || !dest || !out) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_combine(y_perm, y_dt, dest, gates, T, k, d, y_shared,
                                          y_shared ? sh_dt : MOE_F32, out, out_dt,
                                          as_stream(stream)));
}

}  // extern "C"
