// C-ABI front end of the SLiM compressed linear layer (declarations and the
// contract of every call are in include/slim.h).  Validates every argument
// before launching anything, maps HIP errors to status codes, and never
// aborts or throws across the ABI.
#include "slim.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "internal.hpp"

// Scratch of slim_linear_noalloc, for callers that cannot allocate: one copy
// per GPU, held until the process ends, in the code object's zero-filled
// uninitialised data, so the hand-off state in its first 16384 bytes starts at
// zero (a valid state); afterwards every call leaves that state valid for the
// next.  In host code `scratch` names a host-side stand-in, never device
// memory: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local std::string g_last_error;

slim_status fail(slim_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
slim_status fail(slim_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Cached "is the current device gfx950" per device ordinal.
constexpr int kMaxDevices = 64;
int g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::mutex g_arch_mutex;

slim_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SLIM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SLIM_EUNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_arch_mutex);
    if (g_arch_state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(SLIM_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        g_arch_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        if (g_arch_state[dev] == 2)
            return fail(SLIM_EUNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    }
    if (g_arch_state[dev] != 1) return fail(SLIM_EUNSUPPORTED, "device %d is not gfx950", dev);
    return SLIM_OK;
}

slim_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SLIM_EHIP, "%s: %s", what, hipGetErrorString(e));
    g_last_error.clear();
    return SLIM_OK;
}

// Largest sizes any call accepts: every product of two of them fits int64
// (the kernels' grid and offset math, and the size queries, stay exact).
constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxRank = 4096;
constexpr int64_t kMaxWeights = int64_t(1) << 40;   // N * K of one weight or factor
constexpr int64_t kMaxStride = int64_t(1) << 40;    // elements between batched problems

bool dims_ok(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= kMaxDim && b <= kMaxDim; }

// The shapes slim_linear and its variants accept (group 128).
bool linear_shape_ok(int64_t M, int64_t N, int64_t K, int64_t r) {
    return M >= 0 && M <= kMaxDim && dims_ok(N, K) && N % 16 == 0 && K % slim::kGroup == 0 && r >= 0 &&
           r <= kMaxRank && r % 32 == 0;
}

slim_status check_linear_shape(int64_t M, int64_t N, int64_t K, int64_t r, int64_t group) {
    if (group != slim::kGroup) return fail(SLIM_EUNSUPPORTED, "group must be 128 (got %lld)", (long long)group);
    if (M < 0) return fail(SLIM_EINVAL, "M must be >= 0 (got %lld)", (long long)M);
    if (N <= 0 || N % 16) return fail(SLIM_EINVAL, "N must be a positive multiple of 16 (got %lld)", (long long)N);
    if (K <= 0 || K % slim::kGroup) return fail(SLIM_EINVAL, "K must be a positive multiple of 128 (got %lld)", (long long)K);
    if (r < 0 || r % 32) return fail(SLIM_EINVAL, "r must be a non-negative multiple of 32 (got %lld)", (long long)r);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || r > kMaxRank)
        return fail(SLIM_EINVAL, "shape too large (M, N, K <= 2^24, r <= 4096)");
    return SLIM_OK;
}

constexpr int kDefaultWaitLimit = 1 << 18;
std::atomic<int> g_wait_limit{kDefaultWaitLimit};

// Arguments of slim_linear / slim_linear_batched other than the workspace.
// Sets *nothing when the call has no work (batch or M is 0).
slim_status check_linear_args(int64_t batch, int64_t M, int64_t N, int64_t K, int64_t r, int64_t group,
                              const uint16_t* X, int64_t stride_X, const uint8_t* values, int64_t stride_values,
                              const uint8_t* meta, int64_t stride_meta, const uint16_t* scales,
                              int64_t stride_scales, const uint16_t* Lt, int64_t stride_Lt, const uint16_t* Rt,
                              int64_t stride_Rt, const uint16_t* Y, int64_t stride_Y, bool* nothing) {
    slim_status st = check_linear_shape(M, N, K, r, group);
    if (st != SLIM_OK) return st;
    if (batch < 0) return fail(SLIM_EINVAL, "batch must be >= 0");
    if (batch > 65535) return fail(SLIM_EINVAL, "batch must be <= 65535");
    if (batch == 0 || M == 0) {
        g_last_error.clear();
        *nothing = true;
        return SLIM_OK;
    }
    if (!X || !values || !meta || !scales || !Y) return fail(SLIM_EINVAL, "NULL tensor pointer");
    if (r > 0 && (!Lt || !Rt)) return fail(SLIM_EINVAL, "Lt and Rt must be non-NULL when r > 0");
    if (!aligned16(X) || !aligned16(values) || !aligned16(meta) || !aligned16(scales) || !aligned16(Y) ||
        (r > 0 && (!aligned16(Lt) || !aligned16(Rt))))
        return fail(SLIM_EINVAL, "tensor pointers must be 16-byte aligned");
    if (stride_X < 0 || stride_values < 0 || stride_meta < 0 || stride_scales < 0 || stride_Lt < 0 ||
        stride_Rt < 0 || stride_Y < 0)
        return fail(SLIM_EINVAL, "strides must be >= 0");
    if (batch > 1) {
        // Strided problems must keep 16-byte alignment (8 fp16 elements, 16
        // bytes), stay within reach of 64-bit offsets, and Y blocks must not
        // overlap.
        if (stride_X % 8 || stride_values % 16 || stride_meta % 16 || stride_scales % 8 || stride_Lt % 8 ||
            stride_Rt % 8 || stride_Y % 8)
            return fail(SLIM_EINVAL, "strides must keep every problem 16-byte aligned");
        if (stride_X > kMaxStride || stride_values > kMaxStride || stride_meta > kMaxStride ||
            stride_scales > kMaxStride || stride_Lt > kMaxStride || stride_Rt > kMaxStride || stride_Y > kMaxStride)
            return fail(SLIM_EINVAL, "strides must be <= 2^40 elements");
        if (stride_Y < M * N) return fail(SLIM_EINVAL, "stride_Y must be >= M*N (outputs must not overlap)");
    }
    return SLIM_OK;
}

slim::LinearArgs linear_args(int64_t batch, int64_t M, int64_t N, int64_t K, int64_t r, const uint16_t* X,
                             int64_t stride_X, const uint8_t* values, int64_t stride_values, const uint8_t* meta,
                             int64_t stride_meta, const uint16_t* scales, int64_t stride_scales,
                             const uint16_t* Lt, int64_t stride_Lt, const uint16_t* Rt, int64_t stride_Rt,
                             uint16_t* Y, int64_t stride_Y, unsigned char* ws, size_t ws_per_problem) {
    slim::LinearArgs a;
    a.X = X; a.sX = stride_X;
    a.values = values; a.sV = stride_values;
    a.meta = meta; a.sMeta = stride_meta;
    a.scales = scales; a.sS = stride_scales;
    a.Lt = Lt; a.sLt = stride_Lt;
    a.Rt = Rt; a.sRt = stride_Rt;
    a.Y = Y; a.sY = stride_Y;
    a.batch = batch; a.M = M; a.N = N; a.K = K; a.r = r;
    a.ws = ws;
    a.ws_per_problem = ws_per_problem;
    a.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
    return a;
}

unsigned char* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once known
std::mutex g_scratch_mutex;

slim_status noalloc_scratch(unsigned char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SLIM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SLIM_EUNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SLIM_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return SLIM_OK;
}

}  // namespace

namespace slim {
int wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
}  // namespace slim

extern "C" {

const char* slim_status_string(int status) {
    switch (status) {
        case SLIM_OK: return "SLIM_OK";
        case SLIM_EINVAL: return "SLIM_EINVAL: invalid argument";
        case SLIM_EUNSUPPORTED: return "SLIM_EUNSUPPORTED: unsupported configuration or device";
        case SLIM_EHIP: return "SLIM_EHIP: HIP runtime error";
        default: return "unknown slim_status";
    }
}

const char* slim_last_error(void) { return g_last_error.c_str(); }

int slim_version(void) { return 1; }

size_t slim_values_bytes(int64_t N, int64_t K) {
    if (!dims_ok(N, K) || K % slim::kGroup) return 0;
    return (size_t)N * (size_t)K / 4;
}

size_t slim_meta_bytes(int64_t N, int64_t K) {
    if (!dims_ok(N, K) || K % slim::kGroup) return 0;
    return (size_t)N * (size_t)K / 8;
}

size_t slim_scales_bytes(int64_t N, int64_t K, int64_t group) {
    if (!dims_ok(N, K) || group != slim::kGroup || K % group) return 0;
    return (size_t)N * (size_t)(K / group) * 2;
}

slim_status slim_pack(const float* W, int64_t N, int64_t K, int64_t group, uint8_t* values,
                      uint8_t* meta, uint16_t* scales, hipStream_t stream) {
    if (group != slim::kGroup) return fail(SLIM_EUNSUPPORTED, "group must be 128 (got %lld)", (long long)group);
    if (!W || !values || !meta || !scales) return fail(SLIM_EINVAL, "slim_pack: NULL pointer");
    if (!aligned16(W) || !aligned16(values) || !aligned16(meta) || !aligned16(scales))
        return fail(SLIM_EINVAL, "slim_pack: pointers must be 16-byte aligned");
    if (N <= 0 || K <= 0 || K % slim::kGroup)
        return fail(SLIM_EINVAL, "slim_pack: need N > 0 and K a positive multiple of 128 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (!dims_ok(N, K) || N * K > kMaxWeights) return fail(SLIM_EINVAL, "slim_pack: W too large");
    slim_status st = check_device();
    if (st != SLIM_OK) return st;
    return launched(slim::launch_pack(W, N, K, values, meta, scales, stream), "slim_pack launch");
}

size_t slim_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    if (!linear_shape_ok(M, N, K, r)) return 0;
    return slim::linear_workspace_bytes(M, N, K, r);
}

slim_status slim_linear_batched(int64_t batch, int64_t M, int64_t N, int64_t K, int64_t r,
                                int64_t group, const uint16_t* X, int64_t stride_X,
                                const uint8_t* values, int64_t stride_values, const uint8_t* meta,
                                int64_t stride_meta, const uint16_t* scales, int64_t stride_scales,
                                const uint16_t* Lt, int64_t stride_Lt, const uint16_t* Rt,
                                int64_t stride_Rt, uint16_t* Y, int64_t stride_Y, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    bool nothing = false;
    slim_status st = check_linear_args(batch, M, N, K, r, group, X, stride_X, values, stride_values, meta,
                                       stride_meta, scales, stride_scales, Lt, stride_Lt, Rt, stride_Rt, Y,
                                       stride_Y, &nothing);
    if (st != SLIM_OK || nothing) return st;
    const size_t per = slim::linear_workspace_bytes(M, N, K, r);
    if (per > 0) {
        if (!workspace) return fail(SLIM_EINVAL, "workspace is NULL but %zu bytes are needed", per * (size_t)batch);
        if (!aligned16(workspace)) return fail(SLIM_EINVAL, "workspace must be 16-byte aligned");
        if (workspace_bytes < per * (size_t)batch)
            return fail(SLIM_EINVAL, "workspace too small: %zu < %zu bytes", workspace_bytes, per * (size_t)batch);
    }
    st = check_device();
    if (st != SLIM_OK) return st;
    const slim::LinearArgs a = linear_args(batch, M, N, K, r, X, stride_X, values, stride_values, meta, stride_meta,
                                           scales, stride_scales, Lt, stride_Lt, Rt, stride_Rt, Y, stride_Y,
                                           static_cast<unsigned char*>(workspace), per);
    return launched(slim::launch_linear(a, stream), "slim_linear launch");
}

slim_status slim_linear(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* values,
                        const uint8_t* meta, const uint16_t* scales, int64_t group, const uint16_t* Lt,
                        const uint16_t* Rt, int64_t r, uint16_t* Y, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    return slim_linear_batched(1, M, N, K, r, group, X, 0, values, 0, meta, 0, scales, 0, Lt, 0, Rt, 0, Y,
                               0, workspace, workspace_bytes, stream);
}

slim_status slim_linear_noalloc(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* values,
                                const uint8_t* meta, const uint16_t* scales, int64_t group, const uint16_t* Lt,
                                const uint16_t* Rt, int64_t r, uint16_t* Y, hipStream_t stream) {
    bool nothing = false;
    slim_status st = check_linear_args(1, M, N, K, r, group, X, 0, values, 0, meta, 0, scales, 0, Lt, 0, Rt, 0, Y,
                                       0, &nothing);
    if (st != SLIM_OK || nothing) return st;
    const size_t need = slim::linear_workspace_bytes(M, N, K, r);
    if (need > kNoallocScratchBytes)
        return fail(SLIM_EINVAL,
                    "slim_linear_noalloc: this shape needs %zu bytes of scratch, more than the %zu-byte maximum "
                    "(call slim_linear with a workspace)",
                    need, kNoallocScratchBytes);
    st = check_device();
    if (st != SLIM_OK) return st;
    unsigned char* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != SLIM_OK) return st;
    const slim::LinearArgs a = linear_args(1, M, N, K, r, X, 0, values, 0, meta, 0, scales, 0, Lt, 0, Rt, 0, Y, 0,
                                           ws, need);
    return launched(slim::launch_linear(a, stream), "slim_linear_noalloc launch");
}

size_t slim_adapter_codes_bytes(int64_t rows, int64_t cols) {
    if (!dims_ok(rows, cols) || cols % 8) return 0;
    return (size_t)rows * (size_t)cols / 2;
}

size_t slim_adapter_scales_bytes(int64_t rows, int64_t cols, int64_t group) {
    if (!dims_ok(rows, cols) || (group != slim::kAdapterGroupL && group != slim::kAdapterGroupR) || cols % group)
        return 0;
    return (size_t)rows * (size_t)(cols / group) * 2;
}

slim_status slim_pack_adapter(const float* A, int64_t rows, int64_t cols, int64_t group, uint8_t* codes,
                              uint16_t* scales, hipStream_t stream) {
    if (group != slim::kAdapterGroupL && group != slim::kAdapterGroupR)
        return fail(SLIM_EUNSUPPORTED, "slim_pack_adapter: group must be 32 or 128 (got %lld)", (long long)group);
    if (!A || !codes || !scales) return fail(SLIM_EINVAL, "slim_pack_adapter: NULL pointer");
    if (!aligned16(A) || !aligned16(codes) || !aligned16(scales))
        return fail(SLIM_EINVAL, "slim_pack_adapter: pointers must be 16-byte aligned");
    if (rows <= 0 || cols <= 0 || cols % group)
        return fail(SLIM_EINVAL, "slim_pack_adapter: need rows > 0 and cols a positive multiple of %lld (rows=%lld cols=%lld)",
                    (long long)group, (long long)rows, (long long)cols);
    if (!dims_ok(rows, cols) || rows * cols > kMaxWeights)
        return fail(SLIM_EINVAL, "slim_pack_adapter: factor too large");
    slim_status st = check_device();
    if (st != SLIM_OK) return st;
    return launched(slim::launch_adapter_pack(A, rows, cols, group, codes, scales, stream), "slim_pack_adapter launch");
}

size_t slim_transposed_values_bytes(int64_t N, int64_t K) {
    if (!dims_ok(N, K) || N % 16 || K % slim::kGroup) return 0;
    return (size_t)N * (size_t)K;
}

size_t slim_transposed_meta_bytes(int64_t N, int64_t K) {
    if (!dims_ok(N, K) || N % 16 || K % slim::kGroup) return 0;
    return (size_t)N * (size_t)K / 8;
}

slim_status slim_pack_transposed(const uint8_t* values, const uint8_t* meta, const uint16_t* scales, int64_t N,
                                 int64_t K, int64_t group, uint16_t* tvalues, uint16_t* tmeta, hipStream_t stream) {
    if (group != slim::kGroup) return fail(SLIM_EUNSUPPORTED, "group must be 128 (got %lld)", (long long)group);
    if (!values || !meta || !scales || !tvalues || !tmeta) return fail(SLIM_EINVAL, "slim_pack_transposed: NULL pointer");
    if (!aligned16(values) || !aligned16(meta) || !aligned16(scales) || !aligned16(tvalues) || !aligned16(tmeta))
        return fail(SLIM_EINVAL, "slim_pack_transposed: pointers must be 16-byte aligned");
    if (N <= 0 || K <= 0 || N % 16 || K % slim::kGroup)
        return fail(SLIM_EINVAL, "slim_pack_transposed: need N a positive multiple of 16 and K of 128 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (!dims_ok(N, K) || N * K > kMaxWeights)
        return fail(SLIM_EINVAL, "slim_pack_transposed: W too large (N=%lld K=%lld)", (long long)N, (long long)K);
    slim_status st = check_device();
    if (st != SLIM_OK) return st;
    return launched(slim::launch_pack_transposed(values, meta, scales, N, K, tvalues, tmeta, stream),
                    "slim_pack_transposed launch");
}

size_t slim_linear_qa_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    if (!linear_shape_ok(M, N, K, r) || r == 0) return 0;
    return slim::linear_qa_workspace_bytes(M, N, K, r);
}

slim_status slim_linear_qa(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* values,
                           const uint8_t* meta, const uint16_t* scales, int64_t group, const uint8_t* Lq,
                           const uint16_t* Ls, const uint8_t* Rq, const uint16_t* Rs, int64_t r, uint16_t* Y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    slim_status st = check_linear_shape(M, N, K, r, group);
    if (st != SLIM_OK) return st;
    if (r == 0) return fail(SLIM_EINVAL, "slim_linear_qa: r must be > 0 (use slim_linear without an adapter)");
    if (M == 0) { g_last_error.clear(); return SLIM_OK; }
    if (!X || !values || !meta || !scales || !Y || !Lq || !Ls || !Rq || !Rs)
        return fail(SLIM_EINVAL, "NULL tensor pointer");
    if (!aligned16(X) || !aligned16(values) || !aligned16(meta) || !aligned16(scales) || !aligned16(Y) ||
        !aligned16(Lq) || !aligned16(Ls) || !aligned16(Rq) || !aligned16(Rs))
        return fail(SLIM_EINVAL, "tensor pointers must be 16-byte aligned");
    const size_t need = slim::linear_qa_workspace_bytes(M, N, K, r);
    if (!workspace) return fail(SLIM_EINVAL, "workspace is NULL but %zu bytes are needed", need);
    if (!aligned16(workspace)) return fail(SLIM_EINVAL, "workspace must be 16-byte aligned");
    if (workspace_bytes < need) return fail(SLIM_EINVAL, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    st = check_device();
    if (st != SLIM_OK) return st;
    slim::LinearArgs a;
    a.X = X; a.sX = 0;
    a.values = values; a.sV = 0;
    a.meta = meta; a.sMeta = 0;
    a.scales = scales; a.sS = 0;
    a.Lt = nullptr; a.sLt = 0;
    a.Rt = nullptr; a.sRt = 0;
    a.Y = Y; a.sY = 0;
    a.batch = 1; a.M = M; a.N = N; a.K = K; a.r = r;
    a.ws = static_cast<unsigned char*>(workspace);
    a.ws_per_problem = need;
    a.Lq = Lq; a.Ls = Ls; a.Rq = Rq; a.Rs = Rs;
    a.wait_limit = slim::wait_limit();
    return launched(slim::launch_linear_qa(a, stream), "slim_linear_qa launch");
}

slim_status slim_quantize_input(const uint16_t* X, int64_t M, int64_t K, int8_t* q, uint16_t* s,
                                hipStream_t stream) {
    if (M < 0 || K <= 0 || K % 8) return fail(SLIM_EINVAL, "slim_quantize_input: need M >= 0 and K a positive multiple of 8");
    if (M > kMaxDim || K > kMaxDim) return fail(SLIM_EINVAL, "slim_quantize_input: shape too large");
    if (M == 0) { g_last_error.clear(); return SLIM_OK; }
    if (!X || !q || !s) return fail(SLIM_EINVAL, "slim_quantize_input: NULL pointer");
    if (!aligned16(X) || !aligned16(q) || !aligned16(s))
        return fail(SLIM_EINVAL, "slim_quantize_input: pointers must be 16-byte aligned");
    slim_status st = check_device();
    if (st != SLIM_OK) return st;
    return launched(slim::launch_quantize_input(X, M, K, q, s, stream), "slim_quantize_input launch");
}

size_t slim_linear_a8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    if (!linear_shape_ok(M, N, K, r)) return 0;
    return slim::linear_a8_workspace_bytes(M, N, K, r);
}

slim_status slim_linear_a8(const int8_t* qx, const uint16_t* sx, int64_t M, int64_t N, int64_t K,
                           const uint8_t* values, const uint8_t* meta, const uint16_t* scales, int64_t group,
                           const uint16_t* Lt, const uint16_t* Rt, int64_t r, uint16_t* Y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    bool nothing = false;
    // The fp16 input slot of the shared checks is the int8 input here.
    slim_status st = check_linear_args(1, M, N, K, r, group, reinterpret_cast<const uint16_t*>(qx), 0, values, 0,
                                       meta, 0, scales, 0, Lt, 0, Rt, 0, Y, 0, &nothing);
    if (st != SLIM_OK || nothing) return st;
    if (!sx) return fail(SLIM_EINVAL, "slim_linear_a8: NULL input scales");
    if (!aligned16(sx)) return fail(SLIM_EINVAL, "slim_linear_a8: input scales must be 16-byte aligned");
    const size_t need = slim::linear_a8_workspace_bytes(M, N, K, r);
    if (!workspace) return fail(SLIM_EINVAL, "workspace is NULL but %zu bytes are needed", need);
    if (!aligned16(workspace)) return fail(SLIM_EINVAL, "workspace must be 16-byte aligned");
    if (workspace_bytes < need) return fail(SLIM_EINVAL, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    st = check_device();
    if (st != SLIM_OK) return st;
    const slim::LinearArgs a = linear_args(1, M, N, K, r, nullptr, 0, values, 0, meta, 0, scales, 0, Lt, 0, Rt, 0, Y,
                                           0, static_cast<unsigned char*>(workspace), need);
    return launched(slim::launch_linear_a8(a, qx, sx, stream), "slim_linear_a8 launch");
}

slim_status slim_pack_hybrid(const float* W, int64_t N, int64_t K, int64_t group, const int32_t* dense,
                             uint8_t* values, uint8_t* meta, uint16_t* scales, uint8_t* dvalues, hipStream_t stream) {
    if (group != slim::kGroup) return fail(SLIM_EUNSUPPORTED, "group must be 128 (got %lld)", (long long)group);
    if (!W || !dense || !values || !meta || !scales || !dvalues) return fail(SLIM_EINVAL, "slim_pack_hybrid: NULL pointer");
    if (!aligned16(W) || !aligned16(dense) || !aligned16(values) || !aligned16(meta) || !aligned16(scales) ||
        !aligned16(dvalues))
        return fail(SLIM_EINVAL, "slim_pack_hybrid: pointers must be 16-byte aligned");
    if (N <= 0 || K <= 0 || K % slim::kGroup)
        return fail(SLIM_EINVAL, "slim_pack_hybrid: need N > 0 and K a positive multiple of 128 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (!dims_ok(N, K) || N * K > kMaxWeights) return fail(SLIM_EINVAL, "slim_pack_hybrid: W too large");
    slim_status st = check_device();
    if (st != SLIM_OK) return st;
    return launched(slim::launch_pack_hybrid(W, N, K, dense, values, meta, scales, dvalues, stream),
                    "slim_pack_hybrid launch");
}

slim_status slim_linear_hybrid(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* values,
                               const uint8_t* meta, const uint16_t* scales, const uint8_t* dvalues,
                               const int32_t* dense, int64_t group, const uint16_t* Lt, const uint16_t* Rt, int64_t r,
                               uint16_t* Y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    bool nothing = false;
    slim_status st = check_linear_args(1, M, N, K, r, group, X, 0, values, 0, meta, 0, scales, 0, Lt, 0, Rt, 0, Y, 0,
                                       &nothing);
    if (st != SLIM_OK || nothing) return st;
    if (!dvalues || !dense) return fail(SLIM_EINVAL, "slim_linear_hybrid: NULL dvalues or tile flags");
    if (!aligned16(dvalues) || !aligned16(dense))
        return fail(SLIM_EINVAL, "slim_linear_hybrid: dvalues and tile flags must be 16-byte aligned");
    const size_t need = slim::linear_workspace_bytes(M, N, K, r);
    if (need > 0) {
        if (!workspace) return fail(SLIM_EINVAL, "workspace is NULL but %zu bytes are needed", need);
        if (!aligned16(workspace)) return fail(SLIM_EINVAL, "workspace must be 16-byte aligned");
        if (workspace_bytes < need) return fail(SLIM_EINVAL, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    }
    st = check_device();
    if (st != SLIM_OK) return st;
    slim::LinearArgs a = linear_args(1, M, N, K, r, X, 0, values, 0, meta, 0, scales, 0, Lt, 0, Rt, 0, Y, 0,
                                     static_cast<unsigned char*>(workspace), need);
    a.dvalues = dvalues;
    a.dflags = reinterpret_cast<const uint8_t*>(dense);
    return launched(slim::launch_linear_hybrid(a, stream), "slim_linear_hybrid launch");
}

int64_t slim_set_wait_limit(int64_t limit) {
    const int v = limit < 0 ? kDefaultWaitLimit : (limit > (1 << 30) ? (1 << 30) : (int)limit);
    return g_wait_limit.exchange(v, std::memory_order_relaxed);
}

slim_status slim_linear_giveups(const void* workspace, int reset, uint64_t* count, hipStream_t stream) {
    if (!workspace || !count) return fail(SLIM_EINVAL, "slim_linear_giveups: NULL pointer");
    if (!aligned16(workspace)) return fail(SLIM_EINVAL, "slim_linear_giveups: workspace must be 16-byte aligned");
    const unsigned char* at = static_cast<const unsigned char*>(workspace) + slim::kGiveupOffset;
    uint64_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, at, sizeof v, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e == hipSuccess && reset) {
        static const uint64_t zero = 0;
        e = hipMemcpyAsync(const_cast<unsigned char*>(at), &zero, sizeof zero, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
    }
    if (e != hipSuccess) return fail(SLIM_EHIP, "slim_linear_giveups: %s", hipGetErrorString(e));
    *count = v;
    g_last_error.clear();
    return SLIM_OK;
}

}  // extern "C"
