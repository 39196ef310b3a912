// Internal interface between the C-ABI front end (slim_api.cpp) and the HIP
// kernels.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slim {

constexpr int kGroup = 128;

// One batched linear problem set: problem b reads base + b * stride for every
// tensor (strides in elements of the tensor's type).
struct LinearArgs {
    const uint16_t* X;      int64_t sX;
    const uint8_t*  values; int64_t sV;
    const uint8_t*  meta;   int64_t sMeta;
    const uint16_t* scales; int64_t sS;
    const uint16_t* Lt;     int64_t sLt;     // L^T [r][K]
    const uint16_t* Rt;     int64_t sRt;     // R^T [N][r]
    uint16_t*       Y;      int64_t sY;
    int64_t batch, M, N, K, r;
    unsigned char*  ws;            // workspace base
    size_t          ws_per_problem;
    // Quantised adapters (slim_linear_qa; then Lt and Rt are unused): int4
    // codes of Lt [r][K] (groups of 128) and Rt [N][r] (groups of 32), two per
    // byte, and their fp16 scales.  NULL for fp16 adapters.
    const uint8_t*  Lq = nullptr;  const uint16_t* Ls = nullptr;
    const uint8_t*  Rq = nullptr;  const uint16_t* Rs = nullptr;
    // Bounded waits of the one-launch decode forms: poll passes before a
    // workgroup gives up (slim_set_wait_limit; 0 gives up at once).
    int wait_limit = 1 << 18;
    // Hybrid dense / 2:4 tiles (slim_linear_hybrid; NULL otherwise): the
    // second pair of codes of dense tiles (positions 2 and 3 of each group of
    // 4), in the arrangement of `values`, and one int32 flag per tile of 16
    // rows x one 128-k group, [N/16][K/128], nonzero = dense.
    const uint8_t*  dvalues = nullptr;
    const uint8_t*  dflags = nullptr;
};

// Process-wide poll limit of the one-launch decode forms (slim_set_wait_limit).
int wait_limit();

// Workspace bytes one problem of this shape needs on the path the dispatcher
// picks for it.
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* values,
                       uint8_t* meta, uint16_t* scales, hipStream_t stream);
// Hybrid dense / 2:4 pack: flags int32 [ceil(N/16)][K/128] (nonzero = dense tile).
hipError_t launch_pack_hybrid(const float* W, int64_t N, int64_t K, const int32_t* flags, uint8_t* values,
                              uint8_t* meta, uint16_t* scales, uint8_t* dvalues, hipStream_t stream);
// Hybrid layer: a.dvalues and a.dflags set.
hipError_t launch_linear_hybrid(const LinearArgs& a, hipStream_t stream);

// Bytes [0, kCounterRegion) of every problem's workspace are reserved;
// scratch starts after them.  The first problem's reserved bytes hold the
// hand-off state of the one-launch decode path: a 64-bit epoch at byte 0, a
// 64-bit count of workgroups whose bounded wait gave up at byte 8, and T as
// tagged entries from byte kTagBase.  Zero before the workspace's first use;
// every call, completed or given up, leaves them valid for the next.  No
// other path touches them.
constexpr size_t kCounterRegion = 16384;
constexpr size_t kGiveupOffset = 8;
constexpr size_t kTagBase = 256;

// Plain one-thread-per-output kernels: correct for every legal shape.
hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t stream);

// Dispatch to the kernel family that fits the shape.
hipError_t launch_linear(const LinearArgs& a, hipStream_t stream);

// Quantised adapters: codes and scales of one factor stored output-major
// (rows x cols, groups of `group` along cols); dequantised fp16 copy.
constexpr int kAdapterGroupL = 128;
constexpr int kAdapterGroupR = 32;
// Double-pruned transpose of a packed weight (N % 16 == 0): tvalues fp16
// [K][N/2], tmeta uint16 [K][N/16].
hipError_t launch_pack_transposed(const uint8_t* values, const uint8_t* meta, const uint16_t* scales, int64_t N,
                                  int64_t K, uint16_t* tvalues, uint16_t* tmeta, hipStream_t stream);

hipError_t launch_adapter_pack(const float* A, int64_t rows, int64_t cols, int64_t group, uint8_t* q,
                               uint16_t* scales, hipStream_t stream);
// Both factors q0 [rows0][cols0] and q1 [rows1][cols1] to fp16 in one launch.
hipError_t launch_adapter_dequant2(const uint8_t* q0, const uint16_t* s0, int64_t rows0, int64_t cols0, int64_t group0,
                                   uint16_t* out0, const uint8_t* q1, const uint16_t* s1, int64_t rows1, int64_t cols1,
                                   int64_t group1, uint16_t* out1, hipStream_t stream);
size_t linear_qa_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
hipError_t launch_linear_qa(const LinearArgs& a, hipStream_t stream);

// 8-bit input: per-token int8 codes q [M][K] and fp16 scales s [M].
hipError_t launch_quantize_input(const uint16_t* X, int64_t M, int64_t K, int8_t* q, uint16_t* s,
                                 hipStream_t stream);
size_t linear_a8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
hipError_t launch_linear_a8(const LinearArgs& a, const int8_t* qx, const uint16_t* sx, hipStream_t stream);

}  // namespace slim
