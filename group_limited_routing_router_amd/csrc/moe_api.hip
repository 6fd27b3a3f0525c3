// moe_api.hip -- the C ABI of libmoe.so (declared in include/moe.h).
//
// Host side only: argument checks, workspace layout and kernel launches.  All
// checks run before the first HIP call, so a rejected call enqueues nothing
// and touches no output.  No allocation, no synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "moe.h"
#include "kernels.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

moe_status ok() {
    g_last_error.clear();
    return MOE_OK;
}

constexpr size_t kAlign = 256;
constexpr int kMaxDim = 65536;  // largest H and I the kernels take
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t ids, weights, offsets, sorted, rows, counts, h, total;
};

Layout layout_of(const moe_problem& p) {
    const size_t P = static_cast<size_t>(p.T) * static_cast<size_t>(p.k);
    const size_t nb = static_cast<size_t>(moe::permute_blocks(static_cast<int64_t>(P)));
    Layout L{};
    size_t o = 0;
    L.ids = o;     o += align_up(P * 4);
    L.weights = o; o += align_up(P * 4);
    L.offsets = o; o += align_up((static_cast<size_t>(p.E) + 1) * 4);
    L.sorted = o;  o += align_up(P * 4);
    L.rows = o;    o += align_up(P * 4);
    L.counts = o;  o += align_up(nb * static_cast<size_t>(p.E) * 4);
    L.h = o;       o += align_up(P * static_cast<size_t>(p.I) * 2);
    L.total = o;
    return L;
}

// Shape checks shared by every entry point.
moe_status check_problem(const moe_problem* p) {
    if (!p) return fail(MOE_ERR_INVALID_ARG, "problem is NULL");
    if (p->T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%lld < 0", (long long)p->T);
    if (p->H <= 0 || p->H % 64 != 0)
        return fail(MOE_ERR_INVALID_ARG, "H=%d must be a positive multiple of 64", p->H);
    if (p->I <= 0 || p->I % 64 != 0)
        return fail(MOE_ERR_INVALID_ARG, "I=%d must be a positive multiple of 64", p->I);
    if (p->E <= 0) return fail(MOE_ERR_INVALID_ARG, "E=%d must be positive", p->E);
    if (p->G <= 0 || p->E % p->G != 0)
        return fail(MOE_ERR_INVALID_ARG, "G=%d must divide E=%d", p->G, p->E);
    if (p->TG < 1 || p->TG > p->G)
        return fail(MOE_ERR_INVALID_ARG, "TG=%d must be in [1, G=%d]", p->TG, p->G);
    const int64_t cand = static_cast<int64_t>(p->TG) * (p->E / p->G);
    if (p->k < 1 || p->k > cand)
        return fail(MOE_ERR_INVALID_ARG, "k=%d must be in [1, TG*E/G=%lld]", p->k, (long long)cand);
    if (!isfinite(p->scale)) return fail(MOE_ERR_INVALID_ARG, "scale is not finite");
    if (p->T * static_cast<int64_t>(p->k) > 0x7fffffffLL)
        return fail(MOE_ERR_INVALID_ARG, "T*k=%lld exceeds int32", (long long)(p->T * p->k));
    if (p->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E=%d > 256", p->E);
    if (p->k > 16) return fail(MOE_ERR_UNSUPPORTED, "k=%d > 16", p->k);
    if (p->H % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "H=%d is not a multiple of 128", p->H);
    // the expert GEMMs form 32-bit byte offsets within one tile's rows of a
    // weight matrix, h or y (at most 256 rows x 65536 x 4 bytes)
    if (p->H > kMaxDim) return fail(MOE_ERR_UNSUPPORTED, "H=%d > %d", p->H, kMaxDim);
    if (p->I > kMaxDim) return fail(MOE_ERR_UNSUPPORTED, "I=%d > %d", p->I, kMaxDim);
    return MOE_OK;
}

moe_status check_ptr(const void* ptr, const char* name, bool nullable = false) {
    if (!ptr) {
        if (nullable) return MOE_OK;
        return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    }
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
        return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return MOE_OK;
}

moe_status check_ws(const moe_problem& p, const void* ws, size_t ws_bytes) {
    const size_t need = layout_of(p).total;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        return fail(MOE_ERR_WORKSPACE, "workspace is not 16-byte aligned");
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
    return MOE_OK;
}

moe::Problem to_internal(const moe_problem& p) {
    return moe::Problem{p.T, p.H, p.I, p.E, p.G, p.TG, p.k, p.scale};
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY(expr)                      \
    do {                                   \
        const moe_status _s = (expr);      \
        if (_s != MOE_OK) return _s;       \
    } while (0)

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// The workspace of moe_forward_noalloc: a fixed array in device memory, one
// copy per GPU that holds it until the process ends.  Host code never uses
// its name as an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress (looked up on the first call on that GPU).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array (looked up once per GPU).
moe_status device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

MOE_EXPORT size_t moe_workspace_bytes(const moe_problem* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return layout_of(*p).total;
}

MOE_EXPORT moe_status moe_route(const moe_problem* p, const moe_bf16* x, const moe_bf16* w_router,
                                const float* bias, int32_t* topk_ids, float* topk_weights,
                                hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(w_router, "w_router"));
    MOE_TRY(check_ptr(bias, "bias", true));
    MOE_TRY(check_ptr(topk_ids, "topk_ids"));
    MOE_TRY(check_ptr(topk_weights, "topk_weights"));
    return hip_status(moe::launch_route(to_internal(*p), x, w_router, bias, topk_ids, topk_weights,
                                        stream),
                      "route launch");
}

MOE_EXPORT moe_status moe_permute(const moe_problem* p, const int32_t* topk_ids,
                                  int32_t* expert_offsets, int32_t* sorted_pairs,
                                  int32_t* pair_rows, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(topk_ids, "topk_ids"));
    MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
    MOE_TRY(check_ptr(sorted_pairs, "sorted_pairs"));
    MOE_TRY(check_ptr(pair_rows, "pair_rows"));
    MOE_TRY(check_ws(*p, ws, ws_bytes));
    const Layout L = layout_of(*p);
    return hip_status(moe::launch_permute(to_internal(*p), topk_ids, expert_offsets, sorted_pairs,
                                          pair_rows, at<int32_t>(ws, L.counts), stream),
                      "permute launch");
}

MOE_EXPORT moe_status moe_expert_ffn(const moe_problem* p, const moe_bf16* x,
                                     const int32_t* sorted_pairs, const int32_t* expert_offsets,
                                     const moe_bf16* w_gate, const moe_bf16* w_up,
                                     const moe_bf16* w_down, float* y, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(sorted_pairs, "sorted_pairs"));
    MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ws(*p, ws, ws_bytes));
    const Layout L = layout_of(*p);
    return hip_status(moe::launch_expert_ffn(to_internal(*p), x, sorted_pairs, expert_offsets,
                                             w_gate, w_up, w_down, at<uint16_t>(ws, L.h), y,
                                             stream),
                      "expert ffn launch");
}

MOE_EXPORT moe_status moe_expert_gate_up(const moe_problem* p, const moe_bf16* x,
                                         const int32_t* sorted_pairs,
                                         const int32_t* expert_offsets, const moe_bf16* w_gate,
                                         const moe_bf16* w_up, moe_bf16* h, hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(sorted_pairs, "sorted_pairs"));
    MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(h, "h"));
    return hip_status(moe::launch_gate_up(to_internal(*p), x, sorted_pairs, expert_offsets, w_gate,
                                          w_up, h, stream),
                      "gate/up launch");
}

MOE_EXPORT moe_status moe_expert_down(const moe_problem* p, const moe_bf16* h,
                                      const int32_t* expert_offsets, const moe_bf16* w_down,
                                      float* y, hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(h, "h"));
    MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(y, "y"));
    return hip_status(moe::launch_down(to_internal(*p), h, expert_offsets, w_down, y, stream),
                      "down launch");
}

MOE_EXPORT moe_status moe_combine(const moe_problem* p, const float* y, const int32_t* pair_rows,
                                  const float* topk_weights, void* out, moe_dtype out_dtype,
                                  hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d is not MOE_DTYPE_F32/BF16", (int)out_dtype);
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ptr(pair_rows, "pair_rows"));
    MOE_TRY(check_ptr(topk_weights, "topk_weights"));
    MOE_TRY(check_ptr(out, "out"));
    return hip_status(moe::launch_combine(to_internal(*p), y, pair_rows, topk_weights, out,
                                          out_dtype == MOE_DTYPE_BF16, stream),
                      "combine launch");
}

MOE_EXPORT moe_status moe_combine_residual(const moe_problem* p, const float* y,
                                           const int32_t* pair_rows, const float* topk_weights,
                                           const float* norm_weight, float eps, int32_t step,
                                           float* residual, hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (!(eps > 0.0f) || !isfinite(eps))
        return fail(MOE_ERR_INVALID_ARG, "eps=%g must be finite and > 0", (double)eps);
    if (step < 1) return fail(MOE_ERR_INVALID_ARG, "step=%d must be >= 1", step);
    if (p->H > moe::kResidualMaxH)
        return fail(MOE_ERR_UNSUPPORTED, "H=%d > %d for the fused epilogue", p->H, moe::kResidualMaxH);
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ptr(pair_rows, "pair_rows"));
    MOE_TRY(check_ptr(topk_weights, "topk_weights"));
    MOE_TRY(check_ptr(norm_weight, "norm_weight"));
    MOE_TRY(check_ptr(residual, "residual"));
    // the stream weights in fp32, as the oracle takes them
    const float wa = sqrtf(static_cast<float>(step - 1) / static_cast<float>(step));
    const float wb = 1.0f / sqrtf(static_cast<float>(step));
    return hip_status(moe::launch_combine_residual(to_internal(*p), y, pair_rows, topk_weights,
                                                   norm_weight, eps, wa, wb, residual, stream),
                      "combine/residual launch");
}

MOE_EXPORT moe_status moe_dense_mlp(const moe_problem* p, const moe_bf16* x,
                                    const moe_bf16* w_gate, const moe_bf16* w_up,
                                    const moe_bf16* w_down, float* out, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->E != 1 || p->G != 1 || p->TG != 1 || p->k != 1)
        return fail(MOE_ERR_INVALID_ARG, "a dense MLP needs E=G=TG=k=1 (got E=%d G=%d TG=%d k=%d)",
                    p->E, p->G, p->TG, p->k);
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(out, "out"));
    MOE_TRY(check_ws(*p, ws, ws_bytes));
    const Layout L = layout_of(*p);
    const moe::Problem q = to_internal(*p);
    int32_t* off = at<int32_t>(ws, L.offsets);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    hipError_t e = moe::launch_identity_dispatch(p->T, off, sorted, stream);
    if (e != hipSuccess) return hip_status(e, "dispatch launch");
    e = moe::launch_expert_ffn(q, x, sorted, off, w_gate, w_up, w_down, at<uint16_t>(ws, L.h), out,
                               stream);
    return hip_status(e, "dense mlp launch");
}

MOE_EXPORT moe_status moe_expert_ffn_fp8(const moe_problem* p, const moe_bf16* x,
                                         const int32_t* sorted_pairs,
                                         const int32_t* expert_offsets, const uint8_t* w_gate,
                                         const float* s_gate, const uint8_t* w_up,
                                         const float* s_up, const uint8_t* w_down,
                                         const float* s_down, float* y, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(sorted_pairs, "sorted_pairs"));
    MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(s_gate, "s_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(s_up, "s_up"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(s_down, "s_down"));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ws(*p, ws, ws_bytes));
    const Layout L = layout_of(*p);
    return hip_status(moe::launch_expert_ffn_fp8(to_internal(*p), x, sorted_pairs, expert_offsets,
                                                 w_gate, s_gate, w_up, s_up, w_down, s_down,
                                                 at<uint16_t>(ws, L.h), y, stream),
                      "fp8 expert ffn launch");
}

MOE_EXPORT moe_status moe_forward_fp8(const moe_problem* p, const moe_bf16* x,
                                      const moe_bf16* w_router, const float* bias,
                                      const uint8_t* w_gate, const float* s_gate,
                                      const uint8_t* w_up, const float* s_up,
                                      const uint8_t* w_down, const float* s_down, void* out,
                                      moe_dtype out_dtype, int32_t* topk_ids,
                                      float* topk_weights, float* y, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d is not MOE_DTYPE_F32/BF16", (int)out_dtype);
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(w_router, "w_router"));
    MOE_TRY(check_ptr(bias, "bias", true));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(s_gate, "s_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(s_up, "s_up"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(s_down, "s_down"));
    MOE_TRY(check_ptr(out, "out"));
    MOE_TRY(check_ptr(topk_ids, "topk_ids", true));
    MOE_TRY(check_ptr(topk_weights, "topk_weights", true));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ws(*p, ws, ws_bytes));
    const Layout L = layout_of(*p);
    const moe::Problem q = to_internal(*p);
    int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
    float* wts = topk_weights ? topk_weights : at<float>(ws, L.weights);
    int32_t* off = at<int32_t>(ws, L.offsets);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    int32_t* rows = at<int32_t>(ws, L.rows);
    // the h region is written only by the expert step, after routing: it
    // doubles as the router's score scratch
    const size_t h_bytes = static_cast<size_t>(p->T) * static_cast<size_t>(p->k) *
                           static_cast<size_t>(p->I) * 2;
    hipError_t e = moe::launch_route_scratch(q, x, w_router, bias, ids, wts, at<uint16_t>(ws, L.h),
                                             h_bytes, stream);
    if (e != hipSuccess) return hip_status(e, "route launch");
    e = moe::launch_permute(q, ids, off, sorted, rows, at<int32_t>(ws, L.counts), stream);
    if (e != hipSuccess) return hip_status(e, "permute launch");
    e = moe::launch_expert_ffn_fp8(q, x, sorted, off, w_gate, s_gate, w_up, s_up, w_down, s_down,
                                   at<uint16_t>(ws, L.h), y, stream);
    if (e != hipSuccess) return hip_status(e, "fp8 expert ffn launch");
    e = moe::launch_combine(q, y, rows, wts, out, out_dtype == MOE_DTYPE_BF16, stream);
    return hip_status(e, "combine launch");
}

MOE_EXPORT moe_status moe_forward(const moe_problem* p, const moe_bf16* x,
                                  const moe_bf16* w_router, const float* bias,
                                  const moe_bf16* w_gate, const moe_bf16* w_up,
                                  const moe_bf16* w_down, void* out, moe_dtype out_dtype,
                                  int32_t* topk_ids, float* topk_weights, float* y, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d is not MOE_DTYPE_F32/BF16", (int)out_dtype);
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(w_router, "w_router"));
    MOE_TRY(check_ptr(bias, "bias", true));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(out, "out"));
    MOE_TRY(check_ptr(topk_ids, "topk_ids", true));
    MOE_TRY(check_ptr(topk_weights, "topk_weights", true));
    MOE_TRY(check_ptr(y, "y"));
    MOE_TRY(check_ws(*p, ws, ws_bytes));
    const Layout L = layout_of(*p);
    const moe::Problem q = to_internal(*p);
    int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
    float* wts = topk_weights ? topk_weights : at<float>(ws, L.weights);
    int32_t* off = at<int32_t>(ws, L.offsets);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    int32_t* rows = at<int32_t>(ws, L.rows);
    // the h region is written only by the expert step, after routing: it
    // doubles as the router's score scratch
    const size_t h_bytes = static_cast<size_t>(p->T) * static_cast<size_t>(p->k) *
                           static_cast<size_t>(p->I) * 2;
    hipError_t e = moe::launch_route_scratch(q, x, w_router, bias, ids, wts, at<uint16_t>(ws, L.h),
                                             h_bytes, stream);
    if (e != hipSuccess) return hip_status(e, "route launch");
    e = moe::launch_permute(q, ids, off, sorted, rows, at<int32_t>(ws, L.counts), stream);
    if (e != hipSuccess) return hip_status(e, "permute launch");
    e = moe::launch_expert_ffn(q, x, sorted, off, w_gate, w_up, w_down, at<uint16_t>(ws, L.h), y,
                               stream);
    if (e != hipSuccess) return hip_status(e, "expert ffn launch");
    e = moe::launch_combine(q, y, rows, wts, out, out_dtype == MOE_DTYPE_BF16, stream);
    return hip_status(e, "combine launch");
}

MOE_EXPORT moe_status moe_forward_noalloc(const moe_problem* p, const moe_bf16* x,
                                          const moe_bf16* w_router, const float* bias,
                                          const moe_bf16* w_gate, const moe_bf16* w_up,
                                          const moe_bf16* w_down, void* out, moe_dtype out_dtype,
                                          int32_t* topk_ids, float* topk_weights, float* y,
                                          hipStream_t stream) {
    MOE_TRY(check_problem(p));
    if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d is not MOE_DTYPE_F32/BF16", (int)out_dtype);
    if (p->T == 0) return ok();
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(w_router, "w_router"));
    MOE_TRY(check_ptr(bias, "bias", true));
    MOE_TRY(check_ptr(w_gate, "w_gate"));
    MOE_TRY(check_ptr(w_up, "w_up"));
    MOE_TRY(check_ptr(w_down, "w_down"));
    MOE_TRY(check_ptr(out, "out"));
    MOE_TRY(check_ptr(topk_ids, "topk_ids", true));
    MOE_TRY(check_ptr(topk_weights, "topk_weights", true));
    MOE_TRY(check_ptr(y, "y"));
    const size_t need = layout_of(*p).total;
    if (need > static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES))
        return fail(MOE_ERR_UNSUPPORTED,
                    "the problem needs %zu bytes of scratch; the static scratch holds %zu "
                    "(call moe_forward with a workspace)",
                    need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    MOE_TRY(device_scratch(&ws));
    // the same kernels and workspace layout as moe_forward; nothing in the
    // workspace has to start at zero (every scratch value is written before
    // it is read), so the previous call's contents need no clearing
    return moe_forward(p, x, w_router, bias, w_gate, w_up, w_down, out, out_dtype, topk_ids,
                       topk_weights, y, ws, need, stream);
}

MOE_EXPORT const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

MOE_EXPORT const char* moe_last_error(void) { return g_last_error.c_str(); }
