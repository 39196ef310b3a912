// Chooses the kernel family for a slim_linear problem and sizes its workspace.
//
// Workspace layout of one problem (all paths): bytes [0, kCounterRegion) are
// reserved (the first problem's hold the one-launch decode path's hand-off
// state); the rest is scratch whose layout depends on the path.
#include "internal.hpp"

namespace slim {

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
bool decode_fits(const LinearArgs& a);
hipError_t launch_linear_decode(const LinearArgs& a, hipStream_t stream);
size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
bool prefill_fits(const LinearArgs& a);
hipError_t launch_linear_prefill(const LinearArgs& a, hipStream_t stream);

namespace {
constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    const size_t generic = kCounterRegion + align256((size_t)M * (size_t)r * sizeof(float));
    const size_t decode = decode_workspace_bytes(M, N, K, r);
    const size_t prefill = prefill_workspace_bytes(M, N, K, r);
    size_t w = generic > decode ? generic : decode;
    return w > prefill ? w : prefill;
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) {
    if (decode_fits(a)) return launch_linear_decode(a, stream);
    if (prefill_fits(a)) return launch_linear_prefill(a, stream);
    return launch_linear_generic(a, stream);
}

}  // namespace slim
