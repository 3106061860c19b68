// api.hip -- the C ABI of libmoe.so (declared in include/moe.h): argument validation,
// workspace carving and the stage chain.  No device memory is allocated here and nothing
// synchronises; every launch goes to the caller's stream.
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "../../include/moe.h"
#include "launch.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dt(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

moe_status_t check_route(int T, int E, int k) {
    if (T < 0 || E < 1 || k < 1) return MOE_ERR_INVALID_VALUE;
    if (E > MOE_E_MAX || k > MOE_K_MAX || k > E) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_dim(int d) {
    if (d <= 0) return MOE_ERR_INVALID_VALUE;
    if (d % 64 != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps) {
        if (!p) return MOE_ERR_INVALID_VALUE;
        if (!aligned16(p)) return MOE_ERR_MISALIGNED;
    }
    return MOE_OK;
}

bool valid_routing(moe_routing_t r) { return r == MOE_ROUTE_SOFTMAX || r == MOE_ROUTE_SIGMOID; }

moe_status_t launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

#define MOE_TRY(expr)                        \
    do {                                     \
        const moe_status_t st_ = (expr);     \
        if (st_ != MOE_OK) return st_;       \
    } while (0)

// Gate workspace: a 256-byte header (int32 1: tokens decided from exact logits), then the
// fp32 partial logits [split][T][E].
constexpr size_t kGateHeader = 256;
size_t gate_ws(int dt, int T, int H, int E) {
    return kGateHeader + round_up((size_t)moe::gate_splits(dt, T, H, E) * T * E * sizeof(float));
}
size_t pft_ws(int T, int k, int E) { return round_up(moe::pft_ws_bytes((long long)T * k, E)); }
size_t gemm_ws(long long N, int E) { return round_up(moe::gemm_ws_bytes(N, E)); }
size_t pft_layer_ws(int T, int k, int E) { return round_up(moe::pft_layer_ws_bytes(T, k, E)); }
size_t layer_ws(int dt, int T, int H, int E, int k) {
    return pft_layer_ws(T, k, E) + gate_ws(dt, T, H, E) + gemm_ws((long long)T * k, E);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

MOE_API size_t moe_workspace_bytes(int kind, int T, int H, int E, int F, int k, moe_dtype_t dt) {
    (void)F;
    if (!valid_dt(dt) || check_route(T, E, k) != MOE_OK || check_dim(H) != MOE_OK) return 0;
    switch (kind) {
        case MOE_WS_GATE: return gate_ws(dt, T, H, E);
        case MOE_WS_PFT: return pft_ws(T, k, E);
        case MOE_WS_GEMM: return gemm_ws((long long)T * k, E);
        case MOE_WS_LAYER: return layer_ws(dt, T, H, E, k);
        case MOE_WS_BACKWARD:
            if (check_dim(F) != MOE_OK) return 0;
            return round_up(moe::backward_ws_bytes(dt, T, H, E, F, k));
        default: return 0;
    }
}

MOE_API const char* moe_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_VALUE: return "MOE_ERR_INVALID_VALUE: argument out of range or NULL";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the supported limits";
        case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: device pointer not 16-byte aligned";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: the HIP runtime refused a kernel launch";
        case MOE_ERR_SCRATCH_TOO_SMALL:
            return "MOE_ERR_SCRATCH_TOO_SMALL: the call needs more scratch than the library's "
                   "static buffer holds (MOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown moe_status_t";
    }
}

MOE_API moe_status_t moe_gate_topk(moe_dtype_t dt, int T, int H, int E, int k,
                                   moe_routing_t routing, const void* x,
                                   const void* wg, const float* bias, int32_t* top_experts,
                                   float* top_weights, void* ws, size_t ws_bytes, void* stream) {
    if (!valid_dt(dt) || !valid_routing(routing)) return MOE_ERR_INVALID_VALUE;
    MOE_TRY(check_route(T, E, k));
    MOE_TRY(check_dim(H));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, wg, top_experts, top_weights, ws}));
    if (bias && !aligned16(bias)) return MOE_ERR_MISALIGNED;
    if (ws_bytes < gate_ws(dt, T, H, E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    int* refined = static_cast<int*>(ws) + 1;
    float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kGateHeader);
    MOE_TRY(launched(moe::launch_gate_logits(dt, T, H, E, x, wg, partials, refined, nullptr, 0,
                                             as_stream(stream))));
    return launched(moe::launch_topk(dt, T, E, k, routing, moe::gate_splits(dt, T, H, E),
                                     partials, bias, x, wg, H, top_experts, top_weights, refined,
                                     nullptr, as_stream(stream)));
}

MOE_API moe_status_t moe_pft_build(int T, int k, int E, const int32_t* top_experts,
                                   int32_t* counts, int32_t* offsets, int32_t* token_ids,
                                   int32_t* expert_ids, int32_t* dest_pos, void* ws,
                                   size_t ws_bytes, void* stream) {
    MOE_TRY(check_route(T, E, k));
    MOE_TRY(check_ptrs({counts, offsets, ws}));
    if (T > 0) MOE_TRY(check_ptrs({top_experts, token_ids, expert_ids, dest_pos}));
    if (ws_bytes < pft_ws(T, k, E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return launched(moe::launch_pft(T, k, E, top_experts, counts, offsets, token_ids, expert_ids,
                                    dest_pos, ws, as_stream(stream)));
}

MOE_API moe_status_t moe_dispatch(moe_dtype_t dt, int T, int k, int H, const void* x,
                                  const int32_t* dest_pos, void* xd, void* stream) {
    if (!valid_dt(dt)) return MOE_ERR_INVALID_VALUE;
    if (T < 0 || k < 1) return MOE_ERR_INVALID_VALUE;
    if (k > MOE_K_MAX || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_dim(H));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, dest_pos, xd}));
    return launched(moe::launch_dispatch(dt, T, k, H, x, dest_pos, xd, as_stream(stream)));
}

MOE_API moe_status_t moe_grouped_gemm_swiglu(moe_dtype_t dt, int N, int E, int H, int F,
                                             const void* xd, const int32_t* token_ids,
                                             int src_rows, const int32_t* offsets,
                                             const void* w1, const void* w3, const void* w2,
                                             void* h, void* y, void* ws, size_t ws_bytes,
                                             void* stream) {
    if (!valid_dt(dt)) return MOE_ERR_INVALID_VALUE;
    if (N < 0 || E < 1) return MOE_ERR_INVALID_VALUE;
    if (E > MOE_E_MAX) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_dim(H));
    MOE_TRY(check_dim(F));
    if ((w2 == nullptr) != (y == nullptr)) return MOE_ERR_INVALID_VALUE;
    if (token_ids && src_rows < 1) return MOE_ERR_INVALID_VALUE;
    if (N == 0) return MOE_OK;
    MOE_TRY(check_ptrs({xd, offsets, w1, w3, h, ws}));
    if (w2) MOE_TRY(check_ptrs({w2, y}));
    if (token_ids) MOE_TRY(check_ptrs({token_ids}));
    if (ws_bytes < gemm_ws(N, E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (token_ids)
        return launched(moe::launch_grouped_gemm_gather(dt, N, E, H, F, xd, src_rows, token_ids,
                                                        offsets, w1, w3, w2, h, y, ws,
                                                        as_stream(stream)));
    return launched(moe::launch_grouped_gemm(dt, N, E, H, F, xd, offsets, w1, w3, w2, h, y, ws,
                                             as_stream(stream)));
}

MOE_API moe_status_t moe_combine(moe_dtype_t dt, int T, int k, int H, const void* y,
                                 const int32_t* dest_pos, const float* top_weights, void* out,
                                 void* stream) {
    if (!valid_dt(dt)) return MOE_ERR_INVALID_VALUE;
    if (T < 0 || k < 1) return MOE_ERR_INVALID_VALUE;
    if (k > MOE_K_MAX || (long long)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_dim(H));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({y, dest_pos, top_weights, out}));
    return launched(moe::launch_combine(dt, T, k, H, y, dest_pos, top_weights, out,
                                        as_stream(stream)));
}

namespace {

// Validation shared by the two layer-forward entry points (everything but the workspace).
moe_status_t check_layer_forward(moe_dtype_t dt, int T, int H, int E, int F, int k,
                                 moe_routing_t routing, const void* x, const void* wg,
                                 const float* bias, const void* w1, const void* w3,
                                 const void* w2, void* out, const moe_layer_bufs* b) {
    if (!valid_dt(dt) || !valid_routing(routing) || !b) return MOE_ERR_INVALID_VALUE;
    MOE_TRY(check_route(T, E, k));
    MOE_TRY(check_dim(H));
    MOE_TRY(check_dim(F));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, wg, w1, w3, w2, out, b->top_experts, b->top_weights, b->counts,
                        b->offsets, b->token_ids, b->expert_ids, b->dest_pos, b->h, b->y}));
    if (b->xd && !aligned16(b->xd)) return MOE_ERR_MISALIGNED;
    if ((b->a == nullptr) != (b->g == nullptr)) return MOE_ERR_INVALID_VALUE;
    if (b->a && (!aligned16(b->a) || !aligned16(b->g))) return MOE_ERR_MISALIGNED;
    if (bias && !aligned16(bias)) return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

// The stage chain on a validated call with T > 0 and a workspace of layer_ws() bytes.
moe_status_t run_layer_forward(moe_dtype_t dt, int T, int H, int E, int F, int k,
                               moe_routing_t routing, const void* x, const void* wg,
                               const float* bias, const void* w1, const void* w3,
                               const void* w2, void* out, const moe_layer_bufs* b, void* ws,
                               hipStream_t s) {
    const size_t need_pft = pft_layer_ws(T, k, E), need_gate = gate_ws(dt, T, H, E);
    const long long N = (long long)T * k;
    char* w = static_cast<char*>(ws);
    void* ws_pft = w;                       // error word stays at byte 0
    int* refined = reinterpret_cast<int*>(w) + 1;   // beside the error word
    float* partials = reinterpret_cast<float*>(w + need_pft + kGateHeader);
    void* ws_gemm = w + need_pft + need_gate;
    // Buffer build in one launch when the segment counts are small: the gate kernel clears
    // them, the top-k step adds its picks to them, and the place kernel derives counts,
    // offsets, the buffer arrays and the GEMM's tile tables from them.
    const bool fast = moe::pft_layer_fast(T, E);
    int* hist = fast ? moe::pft_layer_hist(ws_pft, T, k) : nullptr;
    const int hist_n = fast ? ((T + moe::kPftSegTokens - 1) / moe::kPftSegTokens) * E : 0;
    const moe::TileTables tables = moe::gemm_tables(ws_gemm, N, E, F);
    MOE_TRY(launched(moe::launch_gate_logits(dt, T, H, E, x, wg, partials, refined, hist, hist_n,
                                             s)));
    MOE_TRY(launched(moe::launch_topk(dt, T, E, k, routing, moe::gate_splits(dt, T, H, E),
                                      partials, bias, x, wg, H, b->top_experts, b->top_weights,
                                      refined, hist, s)));
    if (fast)
        MOE_TRY(launched(moe::launch_pft_layer(T, k, E, b->top_experts, b->counts, b->offsets,
                                               b->token_ids, b->expert_ids, b->dest_pos, ws_pft,
                                               tables, s)));
    else
        MOE_TRY(launched(moe::launch_pft(T, k, E, b->top_experts, b->counts, b->offsets,
                                         b->token_ids, b->expert_ids, b->dest_pos, ws_pft, s)));
    if (b->xd) {
        MOE_TRY(launched(moe::launch_dispatch(dt, T, k, H, x, b->dest_pos, b->xd, s)));
        MOE_TRY(launched(moe::launch_grouped_gemm(dt, (int)N, E, H, F, b->xd, b->offsets, w1, w3,
                                                  w2, b->h, b->y, ws_gemm, s, b->a, b->g, fast)));
    } else {  // dispatch fused into the expert product: rows gathered from x on load
        MOE_TRY(launched(moe::launch_grouped_gemm_gather(dt, (int)N, E, H, F, x, T, b->token_ids,
                                                         b->offsets, w1, w3, w2, b->h, b->y,
                                                         ws_gemm, s, b->a, b->g, fast)));
    }
    return launched(moe::launch_combine(dt, T, k, H, b->y, b->dest_pos, b->top_weights, out, s));
}

}  // namespace

MOE_API moe_status_t moe_layer_forward(moe_dtype_t dt, int T, int H, int E, int F, int k,
                                       moe_routing_t routing, const void* x, const void* wg,
                                       const float* bias, const void* w1, const void* w3,
                                       const void* w2,
                                       void* out, const moe_layer_bufs* b, void* ws,
                                       size_t ws_bytes, void* stream) {
    MOE_TRY(check_layer_forward(dt, T, H, E, F, k, routing, x, wg, bias, w1, w3, w2, out, b));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({ws}));
    if (ws_bytes < layer_ws(dt, T, H, E, k)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return run_layer_forward(dt, T, H, E, F, k, routing, x, wg, bias, w1, w3, w2, out, b, ws,
                             as_stream(stream));
}

// ---- the layer forward without a caller workspace ----
// Its scratch is one file-scope device array per GPU.  In host code `scratch` names a
// host-side stand-in, not device memory: the array's device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is ever handed to kernels.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array (looked up on the first call made
// on that device, then cached).
moe_status_t current_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return MOE_ERR_LAUNCH;
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

MOE_API moe_status_t moe_layer_forward_noalloc(moe_dtype_t dt, int T, int H, int E, int F,
                                               int k, moe_routing_t routing, const void* x,
                                               const void* wg, const float* bias,
                                               const void* w1, const void* w3, const void* w2,
                                               void* out, const moe_layer_bufs* b,
                                               void* stream) {
    MOE_TRY(check_layer_forward(dt, T, H, E, F, k, routing, x, wg, bias, w1, w3, w2, out, b));
    if (T == 0) return MOE_OK;
    if (layer_ws(dt, T, H, E, k) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_TOO_SMALL;
    void* ws = nullptr;
    MOE_TRY(current_scratch(&ws));
    return run_layer_forward(dt, T, H, E, F, k, routing, x, wg, bias, w1, w3, w2, out, b, ws,
                             as_stream(stream));
}

MOE_API moe_status_t moe_layer_backward(moe_dtype_t dt, int T, int H, int E, int F, int k,
                                        moe_routing_t routing, const void* x, const void* wg,
                                        const float* bias, const void* w1, const void* w3,
                                        const void* w2, const moe_layer_bufs* fwd,
                                        const void* dout, void* dx, void* dwg, float* dbias,
                                        void* dw1, void* dw3, void* dw2, float* dtop_weights,
                                        void* ws, size_t ws_bytes, void* stream) {
    if (!valid_dt(dt) || !valid_routing(routing) || !fwd) return MOE_ERR_INVALID_VALUE;
    MOE_TRY(check_route(T, E, k));
    MOE_TRY(check_dim(H));
    MOE_TRY(check_dim(F));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, wg, w1, w3, w2, dout, dx, dwg, dbias, dw1, dw3, dw2, ws,
                        fwd->top_experts, fwd->top_weights, fwd->counts, fwd->offsets,
                        fwd->token_ids, fwd->dest_pos, fwd->h, fwd->y}));
    if (fwd->xd && !aligned16(fwd->xd)) return MOE_ERR_MISALIGNED;
    if ((fwd->a == nullptr) != (fwd->g == nullptr)) return MOE_ERR_INVALID_VALUE;
    if (fwd->a && (!aligned16(fwd->a) || !aligned16(fwd->g))) return MOE_ERR_MISALIGNED;
    if (bias && !aligned16(bias)) return MOE_ERR_MISALIGNED;
    if (dtop_weights && !aligned16(dtop_weights)) return MOE_ERR_MISALIGNED;
    if (ws_bytes < round_up(moe::backward_ws_bytes(dt, T, H, E, F, k)))
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    moe::BwdParams b{};
    b.dt = dt; b.T = T; b.H = H; b.E = E; b.F = F; b.k = k; b.routing = routing;
    b.x = x; b.wg = wg; b.bias = bias; b.w1 = w1; b.w3 = w3; b.w2 = w2;
    b.top_experts = fwd->top_experts; b.top_weights = fwd->top_weights;
    b.counts = fwd->counts; b.offsets = fwd->offsets; b.token_ids = fwd->token_ids;
    b.dest_pos = fwd->dest_pos; b.xd = fwd->xd; b.h = fwd->h; b.y = fwd->y; b.dout = dout;
    b.a = fwd->a; b.g = fwd->g;
    b.dx = dx; b.dwg = dwg; b.dbias = dbias; b.dw1 = dw1; b.dw3 = dw3; b.dw2 = dw2;
    b.dtw = dtop_weights; b.ws = ws;
    return launched(moe::launch_layer_backward(b, as_stream(stream)));
}
