// vq_api.hip -- the C ABI of include/vq.h: host-side validation, error state,
// dispatch witness counters and the launches.
//
// Validation follows vllm.cpp PR #2890, commit "kROCM keep-quant provider"
// (an unsupported dtype is an error that names the dtype, never a silent
// fallback) and commit "grouped Q8_0 delegation" (the capability query and
// the activation type each weight type pairs with).  Nothing here computes:
// the only compute path is the gfx950 kernels.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/vq.h"
#include "vq_device.h"
#include "vq_internal.h"

namespace vqk {
thread_local DebugCtx g_dbg;
}  // namespace vqk

namespace {

thread_local std::string g_last_error;

struct Counters {
    std::atomic<uint64_t> quantize_q8k{0}, quantize_q8_1{0}, quantize_weights{0};
    std::atomic<uint64_t> gemv_q4k{0}, gemv_q6k{0}, gemv_q8_0{0};
    std::atomic<uint64_t> gemm_q4k{0}, gemm_q6k{0}, gemm_q8_0{0};
    std::atomic<uint64_t> route{0}, gemm_grouped_q4k{0}, weighted_sum{0};
    std::atomic<uint64_t> gemm_grouped_q6k{0}, gemm_grouped_q8_0{0}, gemm_grouped_rows{0};
    std::atomic<uint64_t> gemm_skinny{0}, rmsnorm_quant{0}, silu_mul_quant{0};
    std::atomic<uint64_t> gemv_q5k{0}, gemm_q5k{0}, gemm_grouped_q5k{0};
};
Counters g_stats;

// Largest M that vq_gemm runs on the GEMV kernel, per weight type (Q4_K,
// Q6_K, Q8_0, Q5_K): the GEMV <-> GEMM crossover, measured on the decode
// shapes against the MFMA GEMM with its split K (GEMV / GEMM at M = 8 and
// 12: Q4_K 10.7 / 14.1 and 16.4 / 14.0 us, Q6_K 17.3 / 22.9 and 23.2 /
// 23.1, Q5_K 10.7 / 16.7 and 17.5 / 16.8; Q8_0 at 32 and 48: 25.0 / 34.6
// and 35.1 / 35.1).
constexpr int64_t kSmallMaxDefault[4] = {8, 8, 32, 8};
// Per calling thread, so a test's override never reaches another thread's calls.
thread_local int64_t g_small_max[4] = {kSmallMaxDefault[0], kSmallMaxDefault[1], kSmallMaxDefault[2],
                                       kSmallMaxDefault[3]};

vq_status fail(vq_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

vq_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return VQ_OK;
    return fail(VQ_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool is_weight(int t) { return t == VQ_Q4_K || t == VQ_Q6_K || t == VQ_Q8_0 || t == VQ_Q5_K; }
// index of a weight type in the per-type tables (Q4_K, Q6_K, Q8_0, Q5_K)
int widx(int w) { return w == VQ_Q4_K ? 0 : (w == VQ_Q6_K ? 1 : (w == VQ_Q8_0 ? 2 : 3)); }
bool is_act(int t) { return t == VQ_Q8_K || t == VQ_Q8_1; }

int64_t qk_of(int t) { return (t == VQ_Q8_0 || t == VQ_Q8_1) ? 32 : 256; }

bool aligned(const void* p, uintptr_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

constexpr int64_t kMaxDim = (int64_t)1 << 24;
constexpr int64_t kMaxK = (int64_t)1 << 20;

vq_status check_weight(int w, const char* fn) {
    if (!is_weight(w))
        return fail(VQ_ERR_UNSUPPORTED_TYPE, "%s: weight type %s (%d) is not a weight type (Q4_K, Q5_K, Q6_K, Q8_0)",
                    fn, vq_type_name(w), w);
    return VQ_OK;
}

vq_status check_pair(int w, int act, const char* fn) {
    if (!is_act(act))
        return fail(VQ_ERR_UNSUPPORTED_TYPE, "%s: activation type %s (%d) is not an activation type (Q8_K, Q8_1)",
                    fn, vq_type_name(act), act);
    const int want = (w == VQ_Q8_0) ? VQ_Q8_1 : VQ_Q8_K;
    if (act != want)
        return fail(VQ_ERR_TYPE_PAIR, "%s: weight type %s pairs with %s activations, not %s", fn, vq_type_name(w),
                    vq_type_name(want), vq_type_name(act));
    return VQ_OK;
}

vq_status check_k(int t, int64_t K, const char* fn) {
    if (K <= 0 || K % qk_of(t) != 0)
        return fail(VQ_ERR_SHAPE, "%s: K = %lld is not a positive multiple of %lld (block length of %s)", fn,
                    (long long)K, (long long)qk_of(t), vq_type_name(t));
    if (K > kMaxK) return fail(VQ_ERR_SHAPE, "%s: K = %lld exceeds %lld", fn, (long long)K, (long long)kMaxK);
    return VQ_OK;
}

vq_status check_dim(int64_t v, const char* name, const char* fn) {
    if (v < 0) return fail(VQ_ERR_SHAPE, "%s: %s = %lld is negative", fn, name, (long long)v);
    if (v > kMaxDim) return fail(VQ_ERR_SHAPE, "%s: %s = %lld exceeds %lld", fn, name, (long long)v,
                                 (long long)kMaxDim);
    return VQ_OK;
}

vqk::ActQ8K act_q8k(void* base, int64_t M, int64_t K) {
    uint8_t* b = (uint8_t*)base;
    vqk::ActQ8K a;
    a.qs = (int8_t*)b;
    a.d = (float*)(b + vq_act_d_offset(VQ_Q8_K, M, K));
    a.bsums = (int16_t*)(b + vq_act_aux_offset(VQ_Q8_K, M, K));
    return a;
}

vqk::ActQ81 act_q81(void* base, int64_t M, int64_t K) {
    uint8_t* b = (uint8_t*)base;
    vqk::ActQ81 a;
    a.qs = (int8_t*)b;
    a.d = (uint16_t*)(b + vq_act_d_offset(VQ_Q8_1, M, K));
    a.s = (uint16_t*)(b + vq_act_aux_offset(VQ_Q8_1, M, K));
    return a;
}

#define VQ_TRY(expr)                    \
    do {                                \
        vq_status _s = (expr);          \
        if (_s != VQ_OK) return _s;     \
    } while (0)

}  // namespace

// Routing workspace of vq_gemm_grouped_noalloc, for callers that cannot
// allocate: a static device array, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = VQ_GROUPED_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
// The device error word: bits that kernels set when a bounded wait gives up
// (1) or, in debug mode, for invalid expert ids (2: outside [0, E), 4:
// repeated within a token).  One per GPU; read and cleared by
// vq_device_status.
static __device__ __align__(64) unsigned int err_word[1];
static std::mutex g_sym_mu;
static std::atomic<void*> g_scratch_ptr[vqk::kMaxDevices] = {};
static std::atomic<void*> g_err_ptr[vqk::kMaxDevices] = {};

// A device symbol's address on the current device, looked up once per device
// with that device current (the host-side name is only a stand-in).
static vq_status symbol_ptr(const char* fn, std::atomic<void*>* cache, const void* symbol, const char* what,
                            void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= vqk::kMaxDevices)
        return fail(VQ_ERR_INVALID_ARG, "%s: device %d outside [0, %d)", fn, dev, vqk::kMaxDevices);
    void* p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_sym_mu);
        p = cache[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, symbol);
            if (e != hipSuccess) return fail(VQ_ERR_HIP, "%s: hipGetSymbolAddress(%s): HIP error %d (%s)", fn, what,
                                             (int)e, hipGetErrorString(e));
            if (!p) return fail(VQ_ERR_HIP, "%s: hipGetSymbolAddress(%s) returned NULL", fn, what);
            cache[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return VQ_OK;
}

// The current device's scratch address.
static vq_status scratch_ptr(const char* fn, void** out) {
    return symbol_ptr(fn, g_scratch_ptr, HIP_SYMBOL(scratch), "scratch", out);
}

// Before a call's launches: the kernels' error word for the current device.
static vq_status prepare_launch(const char* fn) {
    void* p = nullptr;
    VQ_TRY(symbol_ptr(fn, g_err_ptr, HIP_SYMBOL(err_word), "err_word", &p));
    vqk::g_dbg.err_word = (unsigned int*)p;
    return VQ_OK;
}

// Per calling thread: debug flags (VQ_DEBUG_*).
static thread_local int g_debug_flags = 0;

// Reads and clears the current device's error word after `stream` drains.
static vq_status read_device_status(const char* fn, hipStream_t stream) {
    void* p = nullptr;
    VQ_TRY(symbol_ptr(fn, g_err_ptr, HIP_SYMBOL(err_word), "err_word", &p));
    VQ_TRY(hip_status(hipStreamSynchronize(stream), fn));
    unsigned int v = 0;
    VQ_TRY(hip_status(hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost), fn));
    if (v == 0) return VQ_OK;
    const unsigned int zero = 0;
    VQ_TRY(hip_status(hipMemcpy(p, &zero, sizeof(zero), hipMemcpyHostToDevice), fn));
    return fail(VQ_ERR_DEVICE, "%s: device error word 0x%x:%s%s%s", fn, v,
                (v & 1u) ? " a decode GEMV workgroup's loader wait gave up (its rows were written as NaN);" : "",
                (v & 2u) ? " an expert id outside [0, E);" : "", (v & 4u) ? " an expert id repeated within a token;" : "");
}

// After a call's launches: in debug mode, wait for them and report the error word.
static vq_status finish_launch(const char* fn, vq_status s, hipStream_t stream) {
    if (s != VQ_OK || !(g_debug_flags & VQ_DEBUG_SYNC)) return s;
    return read_device_status(fn, stream);
}

extern "C" {

const char* vq_status_string(vq_status s) {
    switch (s) {
        case VQ_OK: return "VQ_OK";
        case VQ_ERR_INVALID_ARG: return "VQ_ERR_INVALID_ARG";
        case VQ_ERR_UNSUPPORTED_TYPE: return "VQ_ERR_UNSUPPORTED_TYPE";
        case VQ_ERR_TYPE_PAIR: return "VQ_ERR_TYPE_PAIR";
        case VQ_ERR_SHAPE: return "VQ_ERR_SHAPE";
        case VQ_ERR_ALIAS: return "VQ_ERR_ALIAS";
        case VQ_ERR_WORKSPACE: return "VQ_ERR_WORKSPACE";
        case VQ_ERR_HIP: return "VQ_ERR_HIP";
        case VQ_ERR_DEVICE: return "VQ_ERR_DEVICE";
    }
    return "VQ_ERR_UNKNOWN";
}

const char* vq_last_error(void) { return g_last_error.c_str(); }

const char* vq_type_name(int t) {
    switch (t) {
        case VQ_Q4_K: return "Q4_K";
        case VQ_Q6_K: return "Q6_K";
        case VQ_Q8_0: return "Q8_0";
        case VQ_Q8_K: return "Q8_K";
        case VQ_Q8_1: return "Q8_1";
        case VQ_Q5_K: return "Q5_K";
    }
    return "unknown";
}

int vq_is_supported(int w, int act, int op) {
    if (!is_weight(w) || !is_act(act)) return 0;
    const int want = (w == VQ_Q8_0) ? VQ_Q8_1 : VQ_Q8_K;
    if (act != want) return 0;
    if (op == VQ_OP_GEMV || op == VQ_OP_GEMM) return 1;
    if (op == VQ_OP_GEMM_GROUPED) return 1;
    return 0;
}

int vq_block_values(int t) {
    if (t == VQ_Q4_K || t == VQ_Q5_K || t == VQ_Q6_K || t == VQ_Q8_K) return 256;
    if (t == VQ_Q8_0 || t == VQ_Q8_1) return 32;
    return 0;
}

size_t vq_block_bytes(int t) {
    switch (t) {
        case VQ_Q4_K: return 144;
        case VQ_Q5_K: return 176;
        case VQ_Q6_K: return 210;
        case VQ_Q8_0: return 34;
        case VQ_Q8_K: return 256 + 4 + 32;
        case VQ_Q8_1: return 32 + 2 + 2;
    }
    return 0;
}

size_t vq_weight_bytes(int w, int64_t N, int64_t K) {
    if (!is_weight(w) || N < 0 || K <= 0 || K % qk_of(w) != 0) return 0;
    return (size_t)N * (size_t)(K / qk_of(w)) * vq_block_bytes(w);
}

size_t vq_act_d_offset(int act, int64_t M, int64_t K) {
    if (!is_act(act) || M < 0 || K <= 0 || K % qk_of(act) != 0) return 0;
    return vqk::align256((size_t)M * (size_t)K);
}

size_t vq_act_aux_offset(int act, int64_t M, int64_t K) {
    if (!is_act(act) || M < 0 || K <= 0 || K % qk_of(act) != 0) return 0;
    const size_t dbytes = (act == VQ_Q8_K) ? (size_t)M * (size_t)(K / 256) * 4 : (size_t)M * (size_t)(K / 32) * 2;
    return vq_act_d_offset(act, M, K) + vqk::align256(dbytes);
}

size_t vq_act_bytes(int act, int64_t M, int64_t K) {
    if (!is_act(act) || M < 0 || K <= 0 || K % qk_of(act) != 0) return 0;
    const size_t abytes = (act == VQ_Q8_K) ? (size_t)M * (size_t)(K / 16) * 2 : (size_t)M * (size_t)(K / 32) * 2;
    return vq_act_aux_offset(act, M, K) + vqk::align256(abytes);
}

vq_status vq_quantize_act(int act, const float* X, int64_t M, int64_t K, int64_t ldx, void* Xq,
                          hipStream_t stream) {
    const char* fn = "vq_quantize_act";
    if (!is_act(act))
        return fail(VQ_ERR_UNSUPPORTED_TYPE, "%s: type %s (%d) is not an activation type (Q8_K, Q8_1)", fn,
                    vq_type_name(act), act);
    VQ_TRY(check_k(act, K, fn));
    VQ_TRY(check_dim(M, "M", fn));
    if (ldx < K) return fail(VQ_ERR_SHAPE, "%s: ldx = %lld < K = %lld", fn, (long long)ldx, (long long)K);
    if (M == 0) return VQ_OK;
    if (!X || !Xq) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer (X=%p, Xq=%p)", fn, (const void*)X, Xq);
    if (!aligned(X, 4) || !aligned(Xq, 16))
        return fail(VQ_ERR_INVALID_ARG, "%s: X must be 4-byte and Xq 16-byte aligned", fn);
    const size_t xb = ((size_t)(M - 1) * (size_t)ldx + (size_t)K) * 4;
    if (overlap(X, xb, Xq, vq_act_bytes(act, M, K)))
        return fail(VQ_ERR_ALIAS, "%s: Xq overlaps X", fn);
    hipError_t e;
    if (act == VQ_Q8_K) {
        g_stats.quantize_q8k++;
        e = vqk::launch_quantize_q8k(X, M, K, ldx, act_q8k(Xq, M, K), stream);
    } else {
        g_stats.quantize_q8_1++;
        e = vqk::launch_quantize_q8_1(X, M, K, ldx, act_q81(Xq, M, K), stream);
    }
    return hip_status(e, fn);
}

// Shared checks and launch of the two producers (kind 0: RMSNorm, 1: SiLU-mul).
static vq_status produce_impl(const char* fn, int kind, int act, const float* A, const float* B, int64_t M,
                              int64_t K, int64_t ldx, float eps, float* Y, int64_t ldy, void* Xq,
                              hipStream_t stream) {
    if (!is_act(act))
        return fail(VQ_ERR_UNSUPPORTED_TYPE, "%s: type %s (%d) is not an activation type (Q8_K, Q8_1)", fn,
                    vq_type_name(act), act);
    VQ_TRY(check_k(act, K, fn));
    VQ_TRY(check_dim(M, "M", fn));
    if (ldx < K) return fail(VQ_ERR_SHAPE, "%s: ldx = %lld < K = %lld", fn, (long long)ldx, (long long)K);
    if (Y && ldy < K) return fail(VQ_ERR_SHAPE, "%s: ldy = %lld < K = %lld", fn, (long long)ldy, (long long)K);
    if (kind == 0 && !(eps >= 0.0f && eps < INFINITY))
        return fail(VQ_ERR_INVALID_ARG, "%s: eps = %g must be finite and >= 0", fn, (double)eps);
    if (M == 0) return VQ_OK;
    if (!A || !B || !Xq) return fail(VQ_ERR_INVALID_ARG, "%s: null input or Xq pointer", fn);
    if (!aligned(A, 4) || !aligned(B, 4) || (Y && !aligned(Y, 4)) || !aligned(Xq, 16))
        return fail(VQ_ERR_INVALID_ARG, "%s: inputs and Y must be 4-byte, Xq 16-byte aligned", fn);
    const size_t ab = ((size_t)(M - 1) * (size_t)ldx + (size_t)K) * 4;
    const size_t bb = (kind == 0) ? (size_t)K * 4 : ab;
    const size_t qb = vq_act_bytes(act, M, K);
    if (overlap(Xq, qb, A, ab) || overlap(Xq, qb, B, bb)) return fail(VQ_ERR_ALIAS, "%s: Xq overlaps an input", fn);
    if (Y) {
        const size_t yb = ((size_t)(M - 1) * (size_t)ldy + (size_t)K) * 4;
        if (overlap(Y, yb, A, ab) || overlap(Y, yb, B, bb) || overlap(Y, yb, Xq, qb))
            return fail(VQ_ERR_ALIAS, "%s: Y overlaps an input or Xq", fn);
    }
    if (kind == 1 && M * ((K + 1023) / 1024) > INT32_MAX)
        return fail(VQ_ERR_SHAPE, "%s: M * ceil(K / 1024) exceeds the grid limit", fn);
    if (kind == 0) g_stats.rmsnorm_quant++;
    else g_stats.silu_mul_quant++;
    return hip_status(vqk::launch_produce_quant(kind, act == VQ_Q8_K ? 0 : 1, A, B, ldx, M, K, eps, Y, ldy,
                                                act == VQ_Q8_K ? act_q8k(Xq, M, K) : vqk::ActQ8K{},
                                                act == VQ_Q8_1 ? act_q81(Xq, M, K) : vqk::ActQ81{}, stream),
                      fn);
}

vq_status vq_rmsnorm_quant(int act, const float* X, const float* gamma, int64_t M, int64_t K, int64_t ldx,
                           float eps, float* Y, int64_t ldy, void* Xq, hipStream_t stream) {
    return produce_impl("vq_rmsnorm_quant", 0, act, X, gamma, M, K, ldx, eps, Y, ldy, Xq, stream);
}

vq_status vq_silu_mul_quant(int act, const float* G, const float* U, int64_t M, int64_t K, int64_t ldx, float* Y,
                            int64_t ldy, void* Xq, hipStream_t stream) {
    return produce_impl("vq_silu_mul_quant", 1, act, G, U, M, K, ldx, 0.0f, Y, ldy, Xq, stream);
}

vq_status vq_quantize_weights(int w, const float* W, int64_t N, int64_t K, void* Wq, hipStream_t stream) {
    const char* fn = "vq_quantize_weights";
    VQ_TRY(check_weight(w, fn));
    VQ_TRY(check_k(w, K, fn));
    VQ_TRY(check_dim(N, "N", fn));
    if (N == 0) return VQ_OK;
    if (!W || !Wq) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(W, 16) || !aligned(Wq, 16))
        return fail(VQ_ERR_INVALID_ARG, "%s: W and Wq must be 16-byte aligned", fn);
    if (overlap(W, (size_t)N * (size_t)K * 4, Wq, vq_weight_bytes(w, N, K)))
        return fail(VQ_ERR_ALIAS, "%s: Wq overlaps W", fn);
    g_stats.quantize_weights++;
    return hip_status(vqk::launch_quantize_weights(w, W, N, K, (uint8_t*)Wq, stream), fn);
}

vq_status vq_gemv(int w, const void* W, int64_t N, int64_t K, const float* x, float* y, void* xq_out,
                  hipStream_t stream) {
    const char* fn = "vq_gemv";
    VQ_TRY(check_weight(w, fn));
    VQ_TRY(check_k(w, K, fn));
    VQ_TRY(check_dim(N, "N", fn));
    const int act = (w == VQ_Q8_0) ? VQ_Q8_1 : VQ_Q8_K;
    if (vqk::gemv_lds_bytes(w, N > 0 ? N : 1, K, 1) > 160 * 1024)
        return fail(VQ_ERR_SHAPE, "%s: K = %lld is too long for the fused %s GEMV (one row and the quantized "
                    "activation must fit the 160 KiB LDS)", fn, (long long)K, vq_type_name(w));
    if (N == 0) return VQ_OK;
    if (!W || !x || !y) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer (W=%p, x=%p, y=%p)", fn, W,
                                    (const void*)x, (void*)y);
    if (!aligned(W, 16) || !aligned(x, 4) || !aligned(y, 4) || (xq_out && !aligned(xq_out, 16)))
        return fail(VQ_ERR_INVALID_ARG, "%s: W and xq_out must be 16-byte, x and y 4-byte aligned", fn);
    const size_t wb = vq_weight_bytes(w, N, K), xb = (size_t)K * 4, yb = (size_t)N * 4;
    const size_t qb = vq_act_bytes(act, 1, K);
    if (overlap(y, yb, W, wb) || overlap(y, yb, x, xb))
        return fail(VQ_ERR_ALIAS, "%s: y overlaps an input", fn);
    if (xq_out && (overlap(xq_out, qb, W, wb) || overlap(xq_out, qb, x, xb) || overlap(xq_out, qb, y, yb)))
        return fail(VQ_ERR_ALIAS, "%s: xq_out overlaps another buffer", fn);
    if (w == VQ_Q4_K) g_stats.gemv_q4k++;
    else if (w == VQ_Q6_K) g_stats.gemv_q6k++;
    else if (w == VQ_Q5_K) g_stats.gemv_q5k++;
    else g_stats.gemv_q8_0++;
    VQ_TRY(prepare_launch(fn));
    return finish_launch(fn, hip_status(vqk::launch_gemv(w, (const uint8_t*)W, N, K, x, y, (uint8_t*)xq_out, stream), fn),
                         stream);
}

vq_status vq_stream_probe(int w, const void* W, int64_t N, int64_t K, void* sink, size_t sink_bytes,
                          hipStream_t stream) {
    const char* fn = "vq_stream_probe";
    VQ_TRY(check_weight(w, fn));
    VQ_TRY(check_k(w, K, fn));
    VQ_TRY(check_dim(N, "N", fn));
    if (N == 0) return VQ_OK;
    if (!W || !sink) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(W, 16) || !aligned(sink, 4))
        return fail(VQ_ERR_INVALID_ARG, "%s: W must be 16-byte, sink 4-byte aligned", fn);
    if (sink_bytes < (size_t)N * 4)
        return fail(VQ_ERR_WORKSPACE, "%s: sink of %zu bytes, %lld needed", fn, sink_bytes, (long long)(4 * N));
    if (overlap(sink, sink_bytes, W, vq_weight_bytes(w, N, K)))
        return fail(VQ_ERR_ALIAS, "%s: sink overlaps W", fn);
    const hipError_t e = vqk::launch_stream_probe(w, (const uint8_t*)W, N, K, (uint32_t*)sink, nullptr, stream);
    if (e == hipErrorInvalidValue)
        return fail(VQ_ERR_SHAPE, "%s: K = %lld exceeds what the decode GEMV takes for %s", fn, (long long)K,
                    vq_type_name(w));
    return hip_status(e, fn);
}

vq_status vq_mfma_probe(int64_t iters, void* sink, size_t sink_bytes, int64_t* ops_out, hipStream_t stream) {
    const char* fn = "vq_mfma_probe";
    if (iters < 1 || iters > ((int64_t)1 << 24))
        return fail(VQ_ERR_INVALID_ARG, "%s: iters = %lld outside [1, 2^24]", fn, (long long)iters);
    if (!sink) return fail(VQ_ERR_INVALID_ARG, "%s: null sink", fn);
    if (!aligned(sink, 4)) return fail(VQ_ERR_INVALID_ARG, "%s: sink must be 4-byte aligned", fn);
    if (sink_bytes < 4) return fail(VQ_ERR_WORKSPACE, "%s: sink of %zu bytes, 4 needed", fn, sink_bytes);
    return hip_status(vqk::launch_mfma_probe(iters, (uint32_t*)sink, ops_out, stream), fn);
}

vq_status vq_set_debug(int flags, int64_t wait_polls) {
    if (flags & ~(VQ_DEBUG_SYNC | VQ_DEBUG_CHECK_IDS))
        return fail(VQ_ERR_INVALID_ARG, "vq_set_debug: unknown flags 0x%x", flags);
    if (wait_polls < 0 || wait_polls > (1 << 30))
        return fail(VQ_ERR_INVALID_ARG, "vq_set_debug: wait_polls = %lld outside [0, 2^30]", (long long)wait_polls);
    g_debug_flags = flags;
    vqk::g_dbg.wait_polls = wait_polls == 0 ? (1 << 20) : (int)wait_polls;
    return VQ_OK;
}

vq_status vq_device_status(hipStream_t stream) { return read_device_status("vq_device_status", stream); }

size_t vq_gemm_workspace(int w, int64_t M, int64_t N, int64_t K) {
    if (!is_weight(w) || w == VQ_Q8_0 || M <= 0 || N <= 0 || K <= 0 || K % 256 != 0 || M > kMaxDim ||
        N > kMaxDim || K > kMaxK)
        return 0;
    if (vqk::gemm_skinny_ok(w, N, K, M, g_small_max[widx(w)])) return 0;
    return vqk::gemm_kq_call_ws_bytes(w, M, N, K);
}

vq_status vq_gemm(int w, const void* W, int64_t N, int64_t K, int act, const void* Xq, int64_t M, float* Y,
                  int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "vq_gemm";
    VQ_TRY(check_weight(w, fn));
    VQ_TRY(check_pair(w, act, fn));
    VQ_TRY(check_k(w, K, fn));
    VQ_TRY(check_dim(N, "N", fn));
    VQ_TRY(check_dim(M, "M", fn));
    if (ldy < N) return fail(VQ_ERR_SHAPE, "%s: ldy = %lld < N = %lld", fn, (long long)ldy, (long long)N);
    if (M == 0 || N == 0) return VQ_OK;
    if (!W || !Xq || !Y) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(W, 16) || !aligned(Xq, 16) || !aligned(Y, 4) || (ws && !aligned(ws, 256)))
        return fail(VQ_ERR_INVALID_ARG, "%s: W and Xq must be 16-byte, Y 4-byte, ws 256-byte aligned", fn);
    if (!ws) ws_bytes = 0;
    const size_t wb = vq_weight_bytes(w, N, K), ab = vq_act_bytes(act, M, K);
    const size_t yb = ((size_t)(M - 1) * (size_t)ldy + (size_t)N) * 4;
    if (overlap(Y, yb, W, wb) || overlap(Y, yb, Xq, ab)) return fail(VQ_ERR_ALIAS, "%s: Y overlaps an input", fn);
    if (overlap(ws, ws_bytes, W, wb) || overlap(ws, ws_bytes, Xq, ab) || overlap(ws, ws_bytes, Y, yb))
        return fail(VQ_ERR_ALIAS, "%s: the workspace overlaps an input or Y", fn);
    const uint8_t* base = (const uint8_t*)Xq;
    const void* qs = base;
    const void* d = base + vq_act_d_offset(act, M, K);
    const void* aux = base + vq_act_aux_offset(act, M, K);
    if (w == VQ_Q4_K) g_stats.gemm_q4k++;
    else if (w == VQ_Q6_K) g_stats.gemm_q6k++;
    else if (w == VQ_Q5_K) g_stats.gemm_q5k++;
    else g_stats.gemm_q8_0++;
    VQ_TRY(prepare_launch(fn));
    hipError_t e;
    if (vqk::gemm_skinny_ok(w, N, K, M, g_small_max[widx(w)])) {
        // small batch: the weights streamed once through the GEMV kernel for all M rows
        g_stats.gemm_skinny++;
        e = vqk::launch_gemm_skinny(w, (const uint8_t*)W, N, K, base, M, (int64_t)vq_act_d_offset(act, M, K),
                                    (int64_t)vq_act_aux_offset(act, M, K), Y, ldy, stream);
    } else if (w != VQ_Q8_0) {
        e = vqk::launch_gemm_kq(w, (const uint8_t*)W, N, K, qs, d, aux, M, Y, ldy, ws, ws_bytes, stream);
    } else {
        e = vqk::launch_gemm(w, (const uint8_t*)W, N, K, qs, d, aux, M, Y, ldy, stream);
    }
    return finish_launch(fn, hip_status(e, fn), stream);
}

vq_status vq_set_small_batch_max(int w, int64_t max_m) {
    const char* fn = "vq_set_small_batch_max";
    VQ_TRY(check_weight(w, fn));
    if (max_m < -1 || max_m > vqk::kSkinnyMaxM)
        return fail(VQ_ERR_INVALID_ARG, "%s: max_m = %lld outside [-1, %d]", fn, (long long)max_m,
                    vqk::kSkinnyMaxM);
    const int i = widx(w);
    g_small_max[i] = (max_m < 0) ? kSmallMaxDefault[i] : max_m;
    return VQ_OK;
}

int64_t vq_small_batch_max(int w) {
    if (!is_weight(w)) return -1;
    return g_small_max[widx(w)];
}

vq_status vq_set_gemm_row_block(int64_t rows) {
    if (rows < 0)
        return fail(VQ_ERR_INVALID_ARG, "vq_set_gemm_row_block: rows = %lld < 0", (long long)rows);
    vqk::set_gemm_row_block(rows);
    return VQ_OK;
}

size_t vq_grouped_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
    if (E <= 0 || T < 0 || top_k <= 0) return 0;
    return vqk::route_ws_layout(E, T, top_k, nullptr, nullptr);
}

// Both arms of the routed-expert GEMM: the broadcast arm reads activation row
// t for pair (t, s); the per-row arm reads row t*top_k + s.  static_ws: take
// the routing workspace from the static scratch array instead of ws.
static vq_status gemm_grouped_impl(const char* fn, int per_row, int w, const void* W, int64_t E, int64_t N,
                                   int64_t K, int act, const void* Xq, int64_t T, const int32_t* ids, int64_t top_k,
                                   const float* route_w, float* Y, float* Ysum, void* ws, size_t ws_bytes,
                                   hipStream_t stream, bool static_ws = false) {
    VQ_TRY(check_weight(w, fn));
    VQ_TRY(check_pair(w, act, fn));
    VQ_TRY(check_k(w, K, fn));
    VQ_TRY(check_dim(N, "N", fn));
    VQ_TRY(check_dim(T, "T", fn));
    if (E < 1 || E > 1024) return fail(VQ_ERR_SHAPE, "%s: E = %lld outside [1, 1024]", fn, (long long)E);
    if (top_k < 1 || top_k > 16 || top_k > E)
        return fail(VQ_ERR_SHAPE, "%s: top_k = %lld outside [1, min(16, E)]", fn, (long long)top_k);
    if (N % 16 != 0) return fail(VQ_ERR_SHAPE, "%s: N = %lld is not a multiple of 16", fn, (long long)N);
    if (T * top_k > ((int64_t)1 << 30)) return fail(VQ_ERR_SHAPE, "%s: T*top_k too large", fn);
    if (T == 0 || N == 0) return VQ_OK;
    if (!W || !Xq || !ids || !Y) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (Ysum && !route_w) return fail(VQ_ERR_INVALID_ARG, "%s: Ysum requested without route_w", fn);
    const size_t need = vq_grouped_workspace_bytes(E, T, top_k);
    if (static_ws) {
        if (need > kScratchBytes)
            return fail(VQ_ERR_WORKSPACE,
                        "%s: routing workspace of %zu bytes (E = %lld, T*top_k = %lld) exceeds the static %zu-byte "
                        "scratch array; use vq_gemm_grouped with a workspace",
                        fn, need, (long long)E, (long long)(T * top_k), kScratchBytes);
        VQ_TRY(scratch_ptr(fn, &ws));
        ws_bytes = kScratchBytes;
    }
    if (!ws || ws_bytes < need)
        return fail(VQ_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
    if (!aligned(W, 16) || !aligned(Xq, 16) || !aligned(ids, 4) || !aligned(Y, 16) || !aligned(ws, 256) ||
        (Ysum && (!aligned(Ysum, 16) || !aligned(route_w, 4))))
        return fail(VQ_ERR_INVALID_ARG, "%s: misaligned pointer (W, Xq, Y, Ysum: 16 B; ws: 256 B)", fn);
    const int64_t arows = per_row ? T * top_k : T;
    const size_t wb = vq_weight_bytes(w, E * N, K), ab = vq_act_bytes(act, arows, K);
    const size_t yb = (size_t)T * (size_t)top_k * (size_t)N * 4, ib = (size_t)T * (size_t)top_k * 4;
    const size_t sb = (size_t)T * (size_t)N * 4;
    if (overlap(Y, yb, W, wb) || overlap(Y, yb, Xq, ab) || overlap(Y, yb, ids, ib) || overlap(Y, yb, ws, need) ||
        (route_w && overlap(Y, yb, route_w, ib)))
        return fail(VQ_ERR_ALIAS, "%s: Y overlaps another buffer", fn);
    if (Ysum && (overlap(Ysum, sb, Y, yb) || overlap(Ysum, sb, W, wb) || overlap(Ysum, sb, Xq, ab) ||
                 overlap(Ysum, sb, ids, ib) || overlap(Ysum, sb, route_w, ib) || overlap(Ysum, sb, ws, need)))
        return fail(VQ_ERR_ALIAS, "%s: Ysum overlaps another buffer", fn);
    if (overlap(ws, need, W, wb) || overlap(ws, need, Xq, ab) || overlap(ws, need, ids, ib))
        return fail(VQ_ERR_ALIAS, "%s: workspace overlaps an input", fn);
    vqk::RouteWs rws;
    vqk::route_ws_layout(E, T, top_k, &rws, (uint8_t*)ws);
    VQ_TRY(prepare_launch(fn));
    if (g_debug_flags & VQ_DEBUG_CHECK_IDS)
        VQ_TRY(hip_status(vqk::launch_check_ids(ids, T, top_k, E, vqk::g_dbg.err_word, stream), fn));
    g_stats.route++;
    const int tile_rows = vqk::grouped_tile_rows(w, E, T, top_k, K, per_row);
    vq_status s = hip_status(vqk::launch_route(ids, T, top_k, E, tile_rows, rws, stream), fn);
    if (s != VQ_OK) return s;
    if (w == VQ_Q4_K) g_stats.gemm_grouped_q4k++;
    else if (w == VQ_Q6_K) g_stats.gemm_grouped_q6k++;
    else if (w == VQ_Q5_K) g_stats.gemm_grouped_q5k++;
    else g_stats.gemm_grouped_q8_0++;
    if (per_row) g_stats.gemm_grouped_rows++;
    hipError_t e;
    if (act == VQ_Q8_K) {
        const vqk::ActQ8K a = act_q8k((void*)Xq, arows, K);
        e = vqk::launch_gemm_grouped(w, (const uint8_t*)W, E, N, K, a.qs, a.d, a.bsums, T, top_k, per_row, tile_rows, rws, Y,
                                     stream);
    } else {
        const vqk::ActQ81 a = act_q81((void*)Xq, arows, K);
        e = vqk::launch_gemm_grouped(w, (const uint8_t*)W, E, N, K, a.qs, a.d, nullptr, T, top_k, per_row, tile_rows, rws, Y,
                                     stream);
    }
    s = hip_status(e, fn);
    if (s != VQ_OK || !Ysum) return finish_launch(fn, s, stream);
    g_stats.weighted_sum++;
    return finish_launch(fn, hip_status(vqk::launch_weighted_sum(Y, route_w, T, top_k, N, Ysum, stream), fn),
                         stream);
}

vq_status vq_gemm_grouped(int w, const void* W, int64_t E, int64_t N, int64_t K, int act, const void* Xq,
                          int64_t T, const int32_t* ids, int64_t top_k, const float* route_w, float* Y,
                          float* Ysum, void* ws, size_t ws_bytes, hipStream_t stream) {
    return gemm_grouped_impl("vq_gemm_grouped", 0, w, W, E, N, K, act, Xq, T, ids, top_k, route_w, Y, Ysum, ws,
                             ws_bytes, stream);
}

vq_status vq_gemm_grouped_noalloc(int w, const void* W, int64_t E, int64_t N, int64_t K, int act, const void* Xq,
                                  int64_t T, const int32_t* ids, int64_t top_k, const float* route_w, float* Y,
                                  float* Ysum, hipStream_t stream) {
    return gemm_grouped_impl("vq_gemm_grouped_noalloc", 0, w, W, E, N, K, act, Xq, T, ids, top_k, route_w, Y, Ysum,
                             nullptr, 0, stream, true);
}

vq_status vq_gemm_grouped_rows(int w, const void* W, int64_t E, int64_t N, int64_t K, int act, const void* Xq,
                               int64_t T, const int32_t* ids, int64_t top_k, const float* route_w, float* Y,
                               float* Ysum, void* ws, size_t ws_bytes, hipStream_t stream) {
    return gemm_grouped_impl("vq_gemm_grouped_rows", 1, w, W, E, N, K, act, Xq, T, ids, top_k, route_w, Y, Ysum,
                             ws, ws_bytes, stream);
}

vq_status vq_weighted_sum(const float* Y, const float* route_w, int64_t T, int64_t top_k, int64_t N, float* Ysum,
                          hipStream_t stream) {
    const char* fn = "vq_weighted_sum";
    VQ_TRY(check_dim(T, "T", fn));
    VQ_TRY(check_dim(N, "N", fn));
    if (top_k < 1 || top_k > 64) return fail(VQ_ERR_SHAPE, "%s: top_k = %lld outside [1, 64]", fn, (long long)top_k);
    if (N % 4 != 0) return fail(VQ_ERR_SHAPE, "%s: N = %lld is not a multiple of 4", fn, (long long)N);
    if (T == 0 || N == 0) return VQ_OK;
    if (!Y || !route_w || !Ysum) return fail(VQ_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(Y, 16) || !aligned(Ysum, 16) || !aligned(route_w, 4))
        return fail(VQ_ERR_INVALID_ARG, "%s: Y and Ysum must be 16-byte aligned", fn);
    const size_t yb = (size_t)T * (size_t)top_k * (size_t)N * 4, sb = (size_t)T * (size_t)N * 4;
    if (overlap(Ysum, sb, Y, yb) || overlap(Ysum, sb, route_w, (size_t)T * (size_t)top_k * 4))
        return fail(VQ_ERR_ALIAS, "%s: Ysum overlaps an input", fn);
    g_stats.weighted_sum++;
    return hip_status(vqk::launch_weighted_sum(Y, route_w, T, top_k, N, Ysum, stream), fn);
}

void vq_get_stats(vq_stats* out) {
    if (!out) return;
    out->quantize_q8k = g_stats.quantize_q8k.load();
    out->quantize_q8_1 = g_stats.quantize_q8_1.load();
    out->quantize_weights = g_stats.quantize_weights.load();
    out->gemv_q4k = g_stats.gemv_q4k.load();
    out->gemv_q6k = g_stats.gemv_q6k.load();
    out->gemv_q8_0 = g_stats.gemv_q8_0.load();
    out->gemm_q4k = g_stats.gemm_q4k.load();
    out->gemm_q6k = g_stats.gemm_q6k.load();
    out->gemm_q8_0 = g_stats.gemm_q8_0.load();
    out->route = g_stats.route.load();
    out->gemm_grouped_q4k = g_stats.gemm_grouped_q4k.load();
    out->weighted_sum = g_stats.weighted_sum.load();
    out->gemm_grouped_q6k = g_stats.gemm_grouped_q6k.load();
    out->gemm_grouped_q8_0 = g_stats.gemm_grouped_q8_0.load();
    out->gemm_grouped_rows = g_stats.gemm_grouped_rows.load();
    out->gemm_skinny = g_stats.gemm_skinny.load();
    out->gemv_q5k = g_stats.gemv_q5k.load();
    out->gemm_q5k = g_stats.gemm_q5k.load();
    out->gemm_grouped_q5k = g_stats.gemm_grouped_q5k.load();
    out->rmsnorm_quant = g_stats.rmsnorm_quant.load();
    out->silu_mul_quant = g_stats.silu_mul_quant.load();
}

void vq_reset_stats(void) {
    g_stats.quantize_q8k = 0;
    g_stats.quantize_q8_1 = 0;
    g_stats.quantize_weights = 0;
    g_stats.gemv_q4k = 0;
    g_stats.gemv_q6k = 0;
    g_stats.gemv_q8_0 = 0;
    g_stats.gemm_q4k = 0;
    g_stats.gemm_q6k = 0;
    g_stats.gemm_q8_0 = 0;
    g_stats.route = 0;
    g_stats.gemm_grouped_q4k = 0;
    g_stats.weighted_sum = 0;
    g_stats.gemm_grouped_q6k = 0;
    g_stats.gemm_grouped_q8_0 = 0;
    g_stats.gemm_grouped_rows = 0;
    g_stats.gemm_skinny = 0;
    g_stats.gemv_q5k = 0;
    g_stats.gemm_q5k = 0;
    g_stats.gemm_grouped_q5k = 0;
    g_stats.rmsnorm_quant = 0;
    g_stats.silu_mul_quant = 0;
}

const char* vq_version(void) { return "vq 0.1.0 (gfx950)"; }

}  // extern "C"
