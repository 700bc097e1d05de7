// C-ABI layer of libfsa: argument validation, error reporting, and the
// per-shape plan cache behind fsa_attention. Kernels live in bounds.hip and
// forward.hip; the plan builder in plan.cpp.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <tuple>

#include "fsa_internal.h"

namespace fsa {

namespace {
thread_local char g_last_error[512] = "";
}

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
}

}  // namespace fsa

using fsa::set_error;

namespace {

bool good_scale(float scale) { return std::isfinite(scale) && scale > 0.0f; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(const fsa_plan& p) { return p.shape.dtype == FSA_BF16 ? 2 : 4; }

// Bytes of Q or O: [B][H][F*T][d].
size_t tensor_bytes(const fsa_plan& p) {
    const fsa_shape& s = p.shape;
    return size_t(s.B) * s.H * s.F * s.T * s.d * elem_bytes(p);
}

// Bytes of K or V: [B][H][key tokens][d] (F*T, or M for a cross plan).
size_t kv_bytes(const fsa_plan& p) {
    const fsa_shape& s = p.shape;
    return size_t(s.B) * s.H * size_t(p.key_tokens()) * s.d * elem_bytes(p);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" const char* fsa_status_string(fsa_status st) {
    switch (st) {
        case FSA_OK: return "FSA_OK";
        case FSA_ERR_INVALID_ARG: return "FSA_ERR_INVALID_ARG";
        case FSA_ERR_UNSUPPORTED: return "FSA_ERR_UNSUPPORTED";
        case FSA_ERR_WORKSPACE: return "FSA_ERR_WORKSPACE";
        case FSA_ERR_HIP: return "FSA_ERR_HIP";
        case FSA_ERR_NOMEM: return "FSA_ERR_NOMEM";
    }
    return "FSA_ERR_UNKNOWN";
}

extern "C" const char* fsa_last_error(void) { return fsa::g_last_error; }

extern "C" fsa_status fsa_bounds(const fsa_plan* plan, const void* Q, const void* K, void* ws,
                                 float scale, hipStream_t stream) {
    if (!plan || !Q || !K) {
        set_error("fsa_bounds: NULL plan, Q or K");
        return FSA_ERR_INVALID_ARG;
    }
    if (!good_scale(scale)) {
        set_error("fsa_bounds: scale must be finite and > 0 (got %g)", double(scale));
        return FSA_ERR_INVALID_ARG;
    }
    if (!aligned(Q, 16) || !aligned(K, 16)) {
        set_error("fsa_bounds: Q and K must be 16-byte aligned");
        return FSA_ERR_INVALID_ARG;
    }
    if (!ws || !aligned(ws, 256)) {
        set_error("fsa_bounds: workspace missing or not 256-byte aligned");
        return FSA_ERR_WORKSPACE;
    }
    return fsa::launch_bounds(*plan, Q, K, ws, scale, stream);
}

extern "C" fsa_status fsa_forward(const fsa_plan* plan, const void* Q, const void* K,
                                  const void* V, void* O, const void* ws, float scale,
                                  int32_t mode, hipStream_t stream) {
    if (!plan || !Q || !K || !V || !O) {
        set_error("fsa_forward: NULL plan, Q, K, V or O");
        return FSA_ERR_INVALID_ARG;
    }
    if (!good_scale(scale)) {
        set_error("fsa_forward: scale must be finite and > 0 (got %g)", double(scale));
        return FSA_ERR_INVALID_ARG;
    }
    const int32_t route = mode & ~FSA_MODE_RECORD_PMAX;
    if (route != FSA_MODE_AUTO && route != FSA_MODE_ONLINE_ONLY && route != FSA_MODE_FIXED_ONLY &&
        route != FSA_MODE_AUTO_FRAME && route != FSA_MODE_AUTO_ROWS) {
        set_error("fsa_forward: unknown mode %d", mode);
        return FSA_ERR_INVALID_ARG;
    }
    if ((mode & FSA_MODE_RECORD_PMAX) && plan->shape.dtype != FSA_BF16) {
        set_error("fsa_forward: FSA_MODE_RECORD_PMAX needs a bf16 plan");
        return FSA_ERR_UNSUPPORTED;
    }
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16)) {
        set_error("fsa_forward: Q, K, V and O must be 16-byte aligned");
        return FSA_ERR_INVALID_ARG;
    }
    if (!ws || !aligned(ws, 256)) {
        set_error("fsa_forward: workspace missing or not 256-byte aligned");
        return FSA_ERR_WORKSPACE;
    }
    const size_t nb = tensor_bytes(*plan), kb = kv_bytes(*plan);
    if (overlaps(O, nb, Q, nb) || overlaps(O, nb, K, kb) || overlaps(O, nb, V, kb) ||
        overlaps(O, nb, ws, plan->ws.total)) {
        set_error("fsa_forward: O overlaps Q, K, V or the workspace");
        return FSA_ERR_INVALID_ARG;
    }
    return fsa::launch_forward(*plan, Q, K, V, O, ws, scale, mode, stream);
}

extern "C" fsa_status fsa_copy_eligibility(const fsa_plan* plan, const void* ws,
                                           uint8_t* host_out, hipStream_t stream) {
    if (!plan || !host_out) {
        set_error("fsa_copy_eligibility: NULL plan or host_out");
        return FSA_ERR_INVALID_ARG;
    }
    if (!ws || !aligned(ws, 256)) {
        set_error("fsa_copy_eligibility: workspace missing or not 256-byte aligned");
        return FSA_ERR_WORKSPACE;
    }
    const size_t n = size_t(plan->shape.B) * plan->shape.H;
    hipError_t err = hipMemcpyAsync(host_out, static_cast<const char*>(ws) + plan->ws.elig, n,
                                    hipMemcpyDeviceToHost, stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    if (err != hipSuccess) {
        set_error("fsa_copy_eligibility: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return FSA_OK;
}

namespace {

// (B, H, F, T, d, window, ref_frame, dtype, M); M = 0 for self-attention.
using Key = std::tuple<int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                       int32_t>;

// Cached plans are shared: a call holds its own reference while it uses the
// plan, so fsa_cache_clear on another thread only drops the cache's.
using PlanRef = std::shared_ptr<const fsa_plan>;
std::mutex g_cache_mu;
std::map<Key, PlanRef> g_cache;

// Looks up or builds the plan of a shape (bq = bk = 0; M > 0: a cross plan).
// Caller holds no lock.
fsa_status cached_plan(const fsa_shape& s, int32_t M, PlanRef* out) {
    const Key key{s.B, s.H, s.F, s.T, s.d, s.window, s.ref_frame, s.dtype, M};
    std::lock_guard<std::mutex> lock(g_cache_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) {
        *out = it->second;
        return FSA_OK;
    }
    fsa_plan* p = nullptr;
    fsa_status st = M > 0 ? fsa_plan_create_cross(&s, M, &p) : fsa_plan_create(&s, &p);
    if (st != FSA_OK) return st;
    try {
        PlanRef ref(p, [](const fsa_plan* q) { fsa_plan_destroy(const_cast<fsa_plan*>(q)); });
        g_cache.emplace(key, ref);
        *out = std::move(ref);
    } catch (...) {
        set_error("fsa_attention: out of host memory");
        return FSA_ERR_NOMEM;
    }
    return FSA_OK;
}

fsa_shape make_shape(int32_t F, int32_t T, int32_t window, int32_t ref_frame, int32_t B,
                     int32_t H, int32_t d, int32_t dtype) {
    fsa_shape s;
    s.B = B; s.H = H; s.F = F; s.T = T; s.d = d;
    s.window = window; s.ref_frame = ref_frame; s.bq = 0; s.bk = 0; s.dtype = dtype;
    return s;
}

}  // namespace

extern "C" void fsa_cache_clear(void) {
    std::lock_guard<std::mutex> lock(g_cache_mu);
    g_cache.clear();     // plans still in use by a call are freed when it ends
}

extern "C" size_t fsa_attention_workspace_bytes(int32_t F, int32_t T, int32_t window,
                                                int32_t ref_frame, int32_t B, int32_t H,
                                                int32_t d, int32_t dtype) {
    PlanRef p;
    if (cached_plan(make_shape(F, T, window, ref_frame, B, H, d, dtype), 0, &p) != FSA_OK)
        return 0;
    return p->ws.total;
}

namespace {

// Checks of Q, K, V, O, scale and mode shared by the calls that run bounds
// then forward (before a plan is at hand).
fsa_status check_call(const char* who, const void* Q, const void* K, const void* V,
                      const void* O, float scale, int32_t mode) {
    if (!Q || !K || !V || !O) {
        set_error("%s: NULL Q, K, V or O", who);
        return FSA_ERR_INVALID_ARG;
    }
    if (!good_scale(scale)) {
        set_error("%s: scale must be finite and > 0 (got %g)", who, double(scale));
        return FSA_ERR_INVALID_ARG;
    }
    if (mode != FSA_MODE_AUTO && mode != FSA_MODE_ONLINE_ONLY && mode != FSA_MODE_FIXED_ONLY &&
        mode != FSA_MODE_AUTO_FRAME && mode != FSA_MODE_AUTO_ROWS) {
        set_error("%s: unknown mode %d", who, mode);
        return FSA_ERR_INVALID_ARG;
    }
    return FSA_OK;
}

// bounds then forward on a plan, every argument validated before either
// launch.
fsa_status attend_plan(const char* who, const fsa_plan* p, const void* Q, const void* K,
                       const void* V, void* O, float scale, int32_t mode, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    fsa_status st;
    if (!ws || ws_bytes < p->ws.total) {
        set_error("%s: workspace of %zu bytes, %zu needed", who, ws ? ws_bytes : size_t(0),
                  p->ws.total);
        return FSA_ERR_WORKSPACE;
    }
    const size_t nb = tensor_bytes(*p), kb = kv_bytes(*p);
    if (overlaps(O, nb, K, kb)) {
        set_error("%s: O overlaps K", who);
        return FSA_ERR_INVALID_ARG;
    }
    // Validate both calls before launching either.
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16)) {
        set_error("%s: Q, K, V and O must be 16-byte aligned", who);
        return FSA_ERR_INVALID_ARG;
    }
    if (!aligned(ws, 256)) {
        set_error("%s: workspace not 256-byte aligned", who);
        return FSA_ERR_WORKSPACE;
    }
    if (overlaps(O, nb, Q, nb) || overlaps(O, nb, V, kb) || overlaps(O, nb, ws, p->ws.total)) {
        set_error("%s: O overlaps Q, V or the workspace", who);
        return FSA_ERR_INVALID_ARG;
    }
    st = fsa_bounds(p, Q, K, ws, scale, stream);
    if (st != FSA_OK) return st;
    return fsa_forward(p, Q, K, V, O, ws, scale, mode, stream);
}

// bounds then forward with a cached plan; M > 0: cross-attention.
fsa_status attend(const char* who, const void* Q, const void* K, const void* V, void* O,
                  const fsa_shape& shape, int32_t M, float scale, int32_t mode, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
    fsa_status st = check_call(who, Q, K, V, O, scale, mode);
    if (st != FSA_OK) return st;
    PlanRef ref;
    st = cached_plan(shape, M, &ref);
    if (st != FSA_OK) return st;
    return attend_plan(who, ref.get(), Q, K, V, O, scale, mode, ws, ws_bytes, stream);
}

}  // namespace

extern "C" fsa_status fsa_attention(const void* Q, const void* K, const void* V, void* O,
                                    int32_t F, int32_t T, int32_t window, int32_t ref_frame,
                                    float scale, int32_t B, int32_t H, int32_t d, int32_t dtype,
                                    int32_t mode, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    return attend("fsa_attention", Q, K, V, O, make_shape(F, T, window, ref_frame, B, H, d, dtype),
                  0, scale, mode, ws, ws_bytes, stream);
}

extern "C" size_t fsa_cross_attention_workspace_bytes(int32_t F, int32_t T, int32_t M, int32_t B,
                                                      int32_t H, int32_t d, int32_t dtype) {
    PlanRef p;
    if (M <= 0) {
        set_error("fsa_cross_attention_workspace_bytes: M=%d must be positive", M);
        return 0;
    }
    if (cached_plan(make_shape(F, T, 0, 0, B, H, d, dtype), M, &p) != FSA_OK) return 0;
    return p->ws.total;
}

extern "C" fsa_status fsa_cross_attention(const void* Q, const void* Kr, const void* Vr, void* O,
                                          int32_t F, int32_t T, int32_t M, float scale, int32_t B,
                                          int32_t H, int32_t d, int32_t dtype, int32_t mode,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
    if (M <= 0) {
        set_error("fsa_cross_attention: M=%d must be positive", M);
        return FSA_ERR_INVALID_ARG;
    }
    return attend("fsa_cross_attention", Q, Kr, Vr, O, make_shape(F, T, 0, 0, B, H, d, dtype), M,
                  scale, mode, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ static workspace

// The workspace of fsa_attention_static: one file-scope device array, of
// which every GPU the library runs on holds its own copy until the process
// ends. Host code never uses the array's name as an address (on the host it
// is a stand-in, not device memory): the address comes from
// hipGetSymbolAddress, taken once per device with that device current, on
// the device's first call.
static __device__ __align__(256) unsigned char scratch[FSA_STATIC_WS_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of scratch, or an error status.
fsa_status static_workspace(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error("fsa_attention_static: no usable current device (%s, device %d)",
                  hipGetErrorString(err), dev);
        return FSA_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr) {
            set_error("fsa_attention_static: address of the static workspace on device %d: %s",
                      dev, hipGetErrorString(err));
            return FSA_ERR_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return FSA_OK;
}

}  // namespace

extern "C" fsa_status fsa_attention_static(const fsa_plan* plan, const void* Q, const void* K,
                                           const void* V, void* O, float scale, int32_t mode,
                                           hipStream_t stream) {
    const char* who = "fsa_attention_static";
    if (!plan) {
        set_error("%s: NULL plan", who);
        return FSA_ERR_INVALID_ARG;
    }
    if (plan->ws.total > FSA_STATIC_WS_BYTES) {
        set_error("%s: the plan needs a workspace of %zu bytes, above the static workspace's "
                  "%zu (use fsa_attention with a workspace of its own)", who, plan->ws.total,
                  size_t(FSA_STATIC_WS_BYTES));
        return FSA_ERR_WORKSPACE;
    }
    fsa_status st = check_call(who, Q, K, V, O, scale, mode);
    if (st != FSA_OK) return st;
    void* ws = nullptr;
    st = static_workspace(&ws);
    if (st != FSA_OK) return st;
    return attend_plan(who, plan, Q, K, V, O, scale, mode, ws, FSA_STATIC_WS_BYTES, stream);
}

// ------------------------------------------------------------------ producer

namespace {

bool prep_shape_ok(const fsa_plan& p, const char* who) {
    const fsa_shape& s = p.shape;
    if (p.cross) {
        set_error("%s: the producer makes self-attention inputs; the plan is a cross plan", who);
        return false;
    }
    if (s.d != 128 || s.dtype != FSA_BF16) {
        set_error("%s: the producer supports d = 128, bf16 (got d=%d dtype=%d)", who, s.d,
                  s.dtype);
        return false;
    }
    return true;
}

}  // namespace

extern "C" size_t fsa_prep_weight_bytes(int32_t H, int32_t d) {
    if (H < 1 || d < 1) return 0;
    const size_t C = size_t(H) * d;
    return 3 * C * C * 2;
}

extern "C" fsa_status fsa_prep_pack_weights(const void* W, const float* gamma, void* Wp, int32_t H,
                                            int32_t d, hipStream_t stream) {
    if (!W || !gamma || !Wp) {
        set_error("fsa_prep_pack_weights: NULL W, gamma or Wp");
        return FSA_ERR_INVALID_ARG;
    }
    if (H < 1 || d != 128) {
        set_error("fsa_prep_pack_weights: H=%d must be >= 1 and d=%d must be 128", H, d);
        return d != 128 && H >= 1 ? FSA_ERR_UNSUPPORTED : FSA_ERR_INVALID_ARG;
    }
    if (!aligned(W, 16) || !aligned(Wp, 16) || !aligned(gamma, 4)) {
        set_error("fsa_prep_pack_weights: W and Wp must be 16-byte aligned");
        return FSA_ERR_INVALID_ARG;
    }
    const size_t nb = fsa_prep_weight_bytes(H, d);
    if (overlaps(W, nb, Wp, nb)) {
        set_error("fsa_prep_pack_weights: Wp overlaps W");
        return FSA_ERR_INVALID_ARG;
    }
    return fsa::launch_prep_fold(W, gamma, Wp, H * d, stream);
}

extern "C" fsa_status fsa_prep(const fsa_plan* plan, int32_t grid_h, int32_t grid_w,
                               const void* X, const void* Wp, void* Q, void* K, void* V,
                               void* ws, hipStream_t stream) {
    if (!plan || !X || !Wp || !Q || !K || !V) {
        set_error("fsa_prep: NULL plan, X, Wp, Q, K or V");
        return FSA_ERR_INVALID_ARG;
    }
    if (!prep_shape_ok(*plan, "fsa_prep")) return FSA_ERR_UNSUPPORTED;
    const fsa_shape& s = plan->shape;
    if (grid_h < 1 || grid_w < 1 || int64_t(grid_h) * grid_w != s.T) {
        set_error("fsa_prep: grid %d x %d does not hold T=%d tokens", grid_h, grid_w, s.T);
        return FSA_ERR_INVALID_ARG;
    }
    if (!aligned(X, 16) || !aligned(Wp, 16) || !aligned(Q, 16) || !aligned(K, 16) ||
        !aligned(V, 16)) {
        set_error("fsa_prep: X, Wp, Q, K and V must be 16-byte aligned");
        return FSA_ERR_INVALID_ARG;
    }
    if (!ws || !aligned(ws, 256)) {
        set_error("fsa_prep: workspace missing or not 256-byte aligned");
        return FSA_ERR_WORKSPACE;
    }
    const size_t nb = tensor_bytes(*plan), wb = fsa_prep_weight_bytes(s.H, s.d);
    const void* outs[3] = {Q, K, V};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], nb, X, nb) || overlaps(outs[i], nb, Wp, wb) ||
            overlaps(outs[i], nb, ws, plan->ws.total)) {
            set_error("fsa_prep: an output overlaps X, Wp or the workspace");
            return FSA_ERR_INVALID_ARG;
        }
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], nb, outs[j], nb)) {
                set_error("fsa_prep: Q, K and V overlap");
                return FSA_ERR_INVALID_ARG;
            }
    }
    return fsa::launch_prep(*plan, grid_w, X, Wp, Q, K, V, ws, stream);
}

extern "C" fsa_status fsa_bounds_after_prep(const fsa_plan* plan, const void* K, void* ws,
                                            float scale, hipStream_t stream) {
    if (!plan || !K) {
        set_error("fsa_bounds_after_prep: NULL plan or K");
        return FSA_ERR_INVALID_ARG;
    }
    if (!prep_shape_ok(*plan, "fsa_bounds_after_prep")) return FSA_ERR_UNSUPPORTED;
    if (!good_scale(scale)) {
        set_error("fsa_bounds_after_prep: scale must be finite and > 0 (got %g)", double(scale));
        return FSA_ERR_INVALID_ARG;
    }
    if (!aligned(K, 16)) {
        set_error("fsa_bounds_after_prep: K must be 16-byte aligned");
        return FSA_ERR_INVALID_ARG;
    }
    if (!ws || !aligned(ws, 256)) {
        set_error("fsa_bounds_after_prep: workspace missing or not 256-byte aligned");
        return FSA_ERR_WORKSPACE;
    }
    return fsa::launch_bounds_after_prep(*plan, K, ws, scale, stream);
}
