// C ABI of libmoe: host-side argument checks, workspace sizes and launches.
// Every check happens before anything is enqueued; nothing here waits on the
// device or copies device -> host.
#include <algorithm>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "common.hpp"

namespace moe {
hipError_t launch_route(const void* x, moe_dtype dt, const void* w, const float* bias, int T,
                        int d, int E, int k, int renorm, float* logits, int32_t* idx,
                        float* gates, hipStream_t st);
size_t permute_ws_bytes(int T, int k, int E);
size_t static_permute_bytes();
void* static_permute_scratch(hipError_t* err);
hipError_t launch_permute(const int32_t* idx, int T, int k, int e_base, int E, int id_hi, int cap,
                          const void* x, int es, int d, int32_t* routed,
                          int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* dest,
                          void* x_perm, int ld, void* ws, hipStream_t st);
hipError_t launch_permute_recv(const int32_t* recv, int S, int E, int N, const void* x, int es,
                               int d, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                               int32_t* dest, void* x_perm, int ld, hipStream_t st);
hipError_t launch_gate_up(const void* x, int ldx, moe_dtype dt, int N, int d, int f, int E,
                          const int32_t* offsets, const void* wg, const void* wv, void* h,
                          void* act, hipStream_t st);
hipError_t launch_down(const void* h, moe_dtype dt, int N, int f, int d, int E,
                       const int32_t* offsets, const void* wo, void* y, moe_dtype y_dt,
                       hipStream_t st);
hipError_t launch_combine(const void* y, moe_dtype y_dt, const int32_t* dest, const float* gates,
                          int T, int k, int d, const void* sh, moe_dtype sh_dt, void* out,
                          moe_dtype out_dt, hipStream_t st);
hipError_t launch_combine_bwd(const void* d_out, moe_dtype g_dt, const void* y, moe_dtype y_dt,
                              const int32_t* dest, const float* gates, int T, int k, int d,
                              void* d_y, moe_dtype dy_dt, float* d_gates, hipStream_t st);
hipError_t launch_route_bwd(const float* logits, const int32_t* idx, const float* gates,
                            const float* d_gates, int T, int E, int k, int renorm,
                            float* d_logits, uint16_t* d_logits_bf16, hipStream_t st);
hipError_t launch_nt(int epi, const void* A, moe_dtype dt, int rows, int K, int K0, int N, int E,
                     const int32_t* offsets, const void* B0, const void* B1, void* C,
                     const void* act, hipStream_t st);
hipError_t launch_tn(const void* A, int lda, int M, const void* B, int ldb, int Nc, int pair,
                     moe_dtype dt, int rows, int E, const int32_t* offsets, float scale,
                     float* C0, float* C1, hipStream_t st, int split);
int router_splits(int T, int& split);
hipError_t launch_sum_splits(const float* part, int S, long long n, float* out, hipStream_t st);
enum NtEpi { kNtSwigluBwd = 0, kNtStoreF32 = 1, kNtAccumF32 = 2, kNtStoreBf16 = 3 };
unsigned debug_read_route(int reset);
unsigned debug_read_permute(int reset);
unsigned debug_read_ffn(int reset);
unsigned debug_read_bwd(int reset);
hipError_t launch_route_stats(const float* logits, const int32_t* counts, int T, int E, int k,
                              float* p_mean, float* aux, double* part, hipStream_t st);
int route_stat_chunks(int T);
hipError_t launch_token_grad(const void* d_xp, moe_dtype p_dt, const int32_t* dest,
                             const int32_t* idx, const float* gates, const float* d_gates,
                             const void* w, moe_dtype w_dt, int T, int k, int d, int E,
                             float* d_x, void* w_t, hipStream_t st);
}  // namespace moe

namespace {

constexpr int kMaxRouteE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxFfnE = 4096;
constexpr int kMaxRecvCells = 4096;

bool valid_dtype(moe_dtype t) { return t == MOE_F32 || t == MOE_BF16; }

// Row stride of a packed-row buffer: 0 selects dense rows (d); anything
// below d is rejected (returns -1).
int resolve_ld(int ld, int d) {
    if (ld == 0) return d;
    return ld >= d ? ld : -1;
}
int elem_size(moe_dtype t) { return t == MOE_BF16 ? 2 : 4; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// A roctx range named after the entry point, open while the call checks its
// arguments and enqueues its kernels: a marker trace (rocprofv3
// --marker-trace) shows each call on the host timeline beside the kernels it
// launched. Without a profiler attached a push/pop is a cheap no-op.
struct Range {
    explicit Range(const char* name) { roctxRangePushA(name); }
    ~Range() { roctxRangePop(); }
    Range(const Range&) = delete;
    Range& operator=(const Range&) = delete;
};
#define MOE_RANGE() Range moe_range_(__func__)

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

int moe_version(void) { return 102; }

moe_status moe_debug_status(unsigned* flags, int reset)
{
    if (!flags) return MOE_ERR_INVALID_ARG;
    *flags = 0;
#ifdef MOE_DEBUG
    // test-only: waits for the device so that every enqueued kernel has run
    if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
    const unsigned v = moe::debug_read_route(reset) | moe::debug_read_permute(reset) |
                       moe::debug_read_ffn(reset) | moe::debug_read_bwd(reset);
    if (v & 0x80000000u) return MOE_ERR_HIP;
    *flags = v;
    return MOE_OK;
#else
    (void)reset;
    return MOE_ERR_UNSUPPORTED;
#endif
}

int moe_x_perm_ld(int d, moe_dtype dt) {
    if (d <= 0 || !valid_dtype(dt)) return 0;
    // one 128-byte line past the row: rows of a power-of-two byte length
    // would otherwise start on the same memory channel
    return d + 128 / (int)elem_size(dt);
}

moe_status moe_route(const void* x, moe_dtype dt, const void* w_router, const float* bias,
                     int T, int d, int E, int k, int renorm, float* logits, int32_t* topk_idx,
                     float* gates, void* stream)
{
    MOE_RANGE();
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
                       int32_t* dest, void* x_perm, int ld_x_perm, void* ws, size_t ws_bytes,
                       void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E <= 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    const int ld = resolve_ld(ld_x_perm, d);
    if (ld < 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe::permute_ws_bytes(T, k, E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_idx, T, k, 0, E, E, INT32_MAX, x, elem_size(dt), d,
                                          nullptr, counts, offsets, perm_src, dest, x_perm, ld,
                                          ws, as_stream(stream)));
}

moe_status moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, const void* x,
                               moe_dtype dt, int d, int32_t* counts, int32_t* offsets,
                               int32_t* perm_src, int32_t* dest, void* x_perm, int ld_x_perm,
                               void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E <= 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    const int ld = resolve_ld(ld_x_perm, d);
    if (ld < 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    // the chunk histograms must fit the library's static per-GPU array
    if (moe::permute_ws_bytes(T, k, E) > moe::static_permute_bytes()) return MOE_ERR_WORKSPACE;
    hipError_t err = hipSuccess;
    void* ws = moe::static_permute_scratch(&err);
    if (!ws) return MOE_ERR_HIP;
    return hip_status(moe::launch_permute(topk_idx, T, k, 0, E, E, INT32_MAX, x, elem_size(dt), d,
                                          nullptr, counts, offsets, perm_src, dest, x_perm, ld,
                                          ws, as_stream(stream)));
}

moe_status moe_permute_capacity(const int32_t* topk_idx, int T, int k, int E, int capacity,
                                const void* x, moe_dtype dt, int d, int32_t* routed,
                                int32_t* counts, int32_t* offsets, int32_t* perm_src,
                                int32_t* dest, void* x_perm, int ld_x_perm, void* ws,
                                size_t ws_bytes, void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E <= 0 || d <= 0 || capacity < 0)
        return MOE_ERR_INVALID_ARG;
    const int ld = resolve_ld(ld_x_perm, d);
    if (ld < 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe::permute_ws_bytes(T, k, E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_idx, T, k, 0, E, E, capacity, x, elem_size(dt), d,
                                          routed, counts, offsets, perm_src, dest, x_perm, ld,
                                          ws, as_stream(stream)));
}

moe_status moe_permute_range(const int32_t* topk_idx, int T, int k, int e_first, int E_loc,
                             const void* x, moe_dtype dt, int d, int32_t* counts,
                             int32_t* offsets, int32_t* perm_src, int32_t* dest, void* x_perm,
                             int ld_x_perm, void* ws, size_t ws_bytes, void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(dt) || T < 0 || k <= 0 || E_loc <= 0 || e_first < 0 || d <= 0)
        return MOE_ERR_INVALID_ARG;
    const int ld = resolve_ld(ld_x_perm, d);
    if (ld < 0) return MOE_ERR_INVALID_ARG;
    if (E_loc > kMaxRouteE || k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !x || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe::permute_ws_bytes(T, k, E_loc)) return MOE_ERR_WORKSPACE;
    // (global ids: only their sign is known to be wrong here)
    return hip_status(moe::launch_permute(topk_idx, T, k, e_first, E_loc, INT32_MAX, INT32_MAX, x,
                                          elem_size(dt), d, nullptr, counts, offsets, perm_src,
                                          dest, x_perm, ld, ws, as_stream(stream)));
}

size_t moe_permute_recv_workspace(int S, int E_loc, int N) {
    (void)S; (void)E_loc; (void)N;
    return 0;
}

moe_status moe_permute_recv(const int32_t* recv_counts, int S, int E_loc, int N,
                            const void* x_recv, moe_dtype dt, int d, int32_t* counts,
                            int32_t* offsets, int32_t* perm_src, int32_t* dest, void* x_perm,
                            int ld_x_perm, void* ws, size_t ws_bytes, void* stream)
{
    MOE_RANGE();
    (void)ws; (void)ws_bytes;
    if (!valid_dtype(dt) || S <= 0 || E_loc <= 0 || N < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    const int ld = resolve_ld(ld_x_perm, d);
    if (ld < 0) return MOE_ERR_INVALID_ARG;
    if ((long long)S * E_loc > kMaxRecvCells || E_loc > kMaxRouteE) return MOE_ERR_UNSUPPORTED;
    if (!recv_counts || !counts || !offsets) return MOE_ERR_INVALID_ARG;
    if (N > 0 && (!x_recv || !perm_src || !dest || !x_perm)) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_permute_recv(recv_counts, S, E_loc, N, x_recv, elem_size(dt), d,
                                               counts, offsets, perm_src, dest, x_perm, ld,
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
    // offsets NULL: one group of all N rows (E must be 1), e.g. shared experts
    if (!offsets && E != 1) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status moe_ffn_gate_up(const void* x_perm, int ld_x_perm, moe_dtype dt, int N, int d, int f,
                           int E, const int32_t* offsets, const void* w_gate, const void* w_val,
                           void* h, void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    const int ldx = resolve_ld(ld_x_perm, d);
    if (ldx < 0) return MOE_ERR_INVALID_ARG;
    if (N == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_val || !h) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_gate_up(x_perm, ldx, dt, N, d, f, E, offsets, w_gate, w_val, h,
                                          nullptr, as_stream(stream)));
}

moe_status moe_ffn_down(const void* h, moe_dtype dt, int N, int f, int d, int E,
                        const int32_t* offsets, const void* w_out, void* y, moe_dtype y_dt,
                        void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    if (!valid_dtype(y_dt)) return MOE_ERR_INVALID_ARG;
    if (N == 0) return MOE_OK;
    if (!h || !w_out || !y) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_down(h, dt, N, f, d, E, offsets, w_out, y, y_dt,
                                       as_stream(stream)));
}

moe_status moe_grouped_ffn(const void* x_perm, int ld_x_perm, moe_dtype dt, int N, int d, int f,
                           int E, const int32_t* offsets, const void* w_gate, const void* w_val,
                           const void* w_out, void* y, moe_dtype y_dt, void* ws, size_t ws_bytes,
                           void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    const int ldx = resolve_ld(ld_x_perm, d);
    if (ldx < 0) return MOE_ERR_INVALID_ARG;
    if (!valid_dtype(y_dt)) return MOE_ERR_INVALID_ARG;
    if (N == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_val || !w_out || !y) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < h_bytes(N, f, dt)) return MOE_ERR_WORKSPACE;
    hipStream_t st = as_stream(stream);
    hipError_t e = moe::launch_gate_up(x_perm, ldx, dt, N, d, f, E, offsets, w_gate, w_val, ws,
                                       nullptr, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(moe::launch_down(ws, dt, N, f, d, E, offsets, w_out, y, y_dt, st));
}

moe_status moe_combine(const void* y_perm, moe_dtype y_dt, const int32_t* dest,
                       const float* gates, int T, int k, int d, const void* y_shared,
                       moe_dtype sh_dt, void* out, moe_dtype out_dt, void* stream)
{
    MOE_RANGE();
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

size_t moe_route_stats_workspace(int T, int E)
{
    if (T <= 0 || E <= 0) return 0;
    // per token-range fp64 partial sums per expert
    return moe::align_up((size_t)moe::route_stat_chunks(T) * E * sizeof(double), 256);
}

moe_status moe_route_stats(const float* logits, const int32_t* counts, int T, int E, int k,
                           float* p_mean, float* aux, void* ws, size_t ws_bytes, void* stream)
{
    MOE_RANGE();
    if (T <= 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID_ARG;
    if ((long long)T * E > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!logits || !p_mean || (aux && !counts)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe_route_stats_workspace(T, E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_route_stats(logits, counts, T, E, k, p_mean, aux,
                                              static_cast<double*>(ws), as_stream(stream)));
}

// ------------------------------------------------------------------ backward

moe_status moe_ffn_gate_up_train(const void* x_perm, int ld_x_perm, moe_dtype dt, int N, int d,
                                 int f, int E, const int32_t* offsets, const void* w_gate,
                                 const void* w_val, void* h, void* act, void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    const int ldx = resolve_ld(ld_x_perm, d);
    if (ldx < 0) return MOE_ERR_INVALID_ARG;
    if (N == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_val || !h || !act) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_gate_up(x_perm, ldx, dt, N, d, f, E, offsets, w_gate, w_val, h,
                                          act, as_stream(stream)));
}

moe_status moe_combine_backward(const void* d_out, moe_dtype d_out_dt, const void* y_perm,
                                moe_dtype y_dt, const int32_t* dest, const float* gates,
                                int T, int k, int d, void* d_y, moe_dtype d_y_dt,
                                float* d_gates, void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(d_out_dt) || !valid_dtype(y_dt) || !valid_dtype(d_y_dt) || T < 0 ||
        k <= 0 || d <= 0)
        return MOE_ERR_INVALID_ARG;
    if (k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!d_out || !y_perm || !dest || !gates || !d_y || !d_gates) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_combine_bwd(d_out, d_out_dt, y_perm, y_dt, dest, gates, T, k, d,
                                              d_y, d_y_dt, d_gates, as_stream(stream)));
}

moe_status moe_ffn_down_backward(const void* d_y, moe_dtype dt, int N, int d, int f, int E,
                                 const int32_t* offsets, const void* w_out, const void* act,
                                 void* d_act, void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    if (N == 0) return MOE_OK;
    if (!d_y || !w_out || !act || !d_act) return MOE_ERR_INVALID_ARG;
    // dh [N,f] = d_y [N,d] . W_out[e]^T, W_out[e] [f,d] read as [N = f][K = d]
    return hip_status(moe::launch_nt(moe::kNtSwigluBwd, d_y, dt, N, d, d, f, E, offsets, w_out,
                                     nullptr, d_act, act, as_stream(stream)));
}

moe_status moe_ffn_gate_up_backward(const void* d_act, moe_dtype dt, int N, int d, int f, int E,
                                    const int32_t* offsets, const void* w_gate,
                                    const void* w_val, void* d_x_perm, moe_dtype dx_dt,
                                    int accumulate, void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    if (!valid_dtype(dx_dt)) return MOE_ERR_INVALID_ARG;
    if (accumulate && dx_dt != MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (dt == MOE_F32 && dx_dt != MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (N == 0) return MOE_OK;
    if (!d_act || !w_gate || !w_val || !d_x_perm) return MOE_ERR_INVALID_ARG;
    // d_x [N,d] = d_act [N,2f] . [W_gate[e] ; W_val[e]]^T: K = 2f, the first f
    // from W_gate[e] [d,f] read as [N = d][K = f], the rest from W_val[e]
    const int epi = accumulate ? moe::kNtAccumF32 : (dx_dt == MOE_BF16 ? moe::kNtStoreBf16
                                                                       : moe::kNtStoreF32);
    return hip_status(moe::launch_nt(epi, d_act, dt, N, 2 * f, f, d, E, offsets, w_gate, w_val,
                                     d_x_perm, nullptr, as_stream(stream)));
}

moe_status moe_ffn_weight_grads(const void* x_perm, int ld_x_perm, const void* h, const void* d_y,
                                const void* d_act, moe_dtype dt, int N, int d, int f, int E,
                                const int32_t* offsets, float scale, float* d_w_gate,
                                float* d_w_val, float* d_w_out, void* stream)
{
    MOE_RANGE();
    moe_status s = check_ffn(dt, N, d, f, E, offsets);
    if (s != MOE_OK) return s;
    const int ldx = resolve_ld(ld_x_perm, d);
    if (ldx < 0) return MOE_ERR_INVALID_ARG;
    if (!d_w_gate || !d_w_val || !d_w_out) return MOE_ERR_INVALID_ARG;
    if (N > 0 && (!x_perm || !h || !d_y || !d_act)) return MOE_ERR_INVALID_ARG;
    hipStream_t st = as_stream(stream);
    // dW_out[e] [f,d] = h_e^T . d_y_e
    hipError_t e = moe::launch_tn(h, f, f, d_y, d, d, 0, dt, N, E, offsets, scale, d_w_out,
                                  nullptr, st, 0);
    if (e != hipSuccess) return MOE_ERR_HIP;
    // [dW_gate | dW_val][e] [d,f] = x_e^T . d_act_e[:, 0:f | f:2f]
    return hip_status(moe::launch_tn(x_perm, ldx, d, d_act, 2 * f, f, f, dt, N, E, offsets, scale,
                                     d_w_gate, d_w_val, st, 0));
}

size_t moe_token_backward_workspace(int d, int E, moe_dtype dt)
{
    if (d <= 0 || E <= 0 || !valid_dtype(dt)) return 0;
    return moe::align_up((size_t)d * E * elem_size(dt), 256);
}

moe_status moe_token_backward(const void* d_x_perm, moe_dtype dxp_dt, const int32_t* dest,
                              const int32_t* topk_idx, const float* gates, const float* d_gates,
                              const void* w_router, moe_dtype dt, int T, int k, int d, int E,
                              float* d_x, void* ws, size_t ws_bytes, void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(dxp_dt) || !valid_dtype(dt) || T < 0 || k <= 0 || k > E || d <= 0)
        return MOE_ERR_INVALID_ARG;
    if (k > kMaxK || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!d_x_perm || !dest || !topk_idx || !gates || !d_gates || !w_router || !d_x)
        return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe_token_backward_workspace(d, E, dt)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_token_grad(d_x_perm, dxp_dt, dest, topk_idx, gates, d_gates,
                                             w_router, dt, T, k, d, E, d_x, ws,
                                             as_stream(stream)));
}

moe_status moe_route_backward(const float* logits, const int32_t* topk_idx, const float* gates,
                              const float* d_gates, int T, int E, int k, int renorm,
                              float* d_logits, void* d_logits_bf16, void* stream)
{
    MOE_RANGE();
    if (T < 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID_ARG;
    if (k > kMaxK || (long long)T * E > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_idx || !gates || !d_gates) return MOE_ERR_INVALID_ARG;
    if (!d_logits && !d_logits_bf16) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_route_bwd(logits, topk_idx, gates, d_gates, T, E, k, renorm,
                                            d_logits, static_cast<uint16_t*>(d_logits_bf16),
                                            as_stream(stream)));
}

size_t moe_router_backward_workspace(int T, int d, int E)
{
    if (T <= 0 || d <= 0 || E <= 0) return 0;
    int split = 0;
    const int S = moe::router_splits(T, split);
    return S > 1 ? (size_t)S * d * E * sizeof(float) : 0;
}

moe_status moe_router_backward(const void* x, const void* w_router, moe_dtype dt,
                               const void* d_logits, int T, int d, int E, float* d_x,
                               int accumulate, float* d_w_router, void* ws, size_t ws_bytes,
                               void* stream)
{
    MOE_RANGE();
    if (!valid_dtype(dt) || T < 0 || d <= 0 || E <= 0) return MOE_ERR_INVALID_ARG;
    if ((long long)T * std::max(d, E) > (1LL << 40) || (long long)T * E > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if (!d_x && !d_w_router) return MOE_OK;
    if (T > 0 && (!x || !w_router || !d_logits)) return MOE_ERR_INVALID_ARG;
    hipStream_t st = as_stream(stream);
    if (d_x && T > 0) {
        // d_x [T,d] (+)= d_logits [T,E] . W_r^T, W_r [d,E] read as [N = d][K = E]
        hipError_t e = moe::launch_nt(accumulate ? moe::kNtAccumF32 : moe::kNtStoreF32, d_logits,
                                      dt, T, E, E, d, 1, nullptr, w_router, nullptr, d_x, nullptr,
                                      st);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (d_w_router) {
        // d_w_router [d,E] = x^T . d_logits over all T rows (T = 0: zeros). A
        // large T is split into row groups whose partial products land in the
        // workspace and are then summed in group order.
        int split = 0;
        const int S = T > 0 ? moe::router_splits(T, split) : 1;
        if (S > 1) {
            if (!ws || ws_bytes < moe_router_backward_workspace(T, d, E)) return MOE_ERR_WORKSPACE;
            float* part = static_cast<float*>(ws);
            hipError_t e = moe::launch_tn(x, d, d, d_logits, E, E, 0, dt, T, S, nullptr, 1.0f,
                                          part, nullptr, st, split);
            if (e != hipSuccess) return MOE_ERR_HIP;
            e = moe::launch_sum_splits(part, S, (long long)d * E, d_w_router, st);
            if (e != hipSuccess) return MOE_ERR_HIP;
        } else {
            hipError_t e = moe::launch_tn(x, d, d, d_logits, E, E, 0, dt, T, 1, nullptr, 1.0f,
                                          d_w_router, nullptr, st, 0);
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
    }
    return MOE_OK;
}

}  // extern "C"
