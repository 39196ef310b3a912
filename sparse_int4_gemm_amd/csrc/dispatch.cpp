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
size_t prefill_kx_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
bool prefill_kx_fits(const LinearArgs& a);
hipError_t launch_linear_prefill_kx(const LinearArgs& a, hipStream_t stream);

namespace {
constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    const size_t generic = kCounterRegion + align256((size_t)M * (size_t)r * sizeof(float));
    const size_t decode = decode_workspace_bytes(M, N, K, r);
    const size_t prefill = prefill_workspace_bytes(M, N, K, r);
    const size_t kx = prefill_kx_workspace_bytes(M, N, K, r);
    size_t w = generic > decode ? generic : decode;
    w = w > prefill ? w : prefill;
    return w > kx ? w : kx;
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) {
    if (decode_fits(a)) return launch_linear_decode(a, stream);
    if (prefill_kx_fits(a)) return launch_linear_prefill_kx(a, stream);
    if (prefill_fits(a)) return launch_linear_prefill(a, stream);
    return launch_linear_generic(a, stream);
}

bool decode_hybrid_fits(const LinearArgs& a);
hipError_t launch_linear_decode_hybrid(const LinearArgs& a, hipStream_t stream);

// Hybrid dense / 2:4 tiles: 1 to 16 tokens on the two-launch decode kernel,
// prefill shapes on the prefill kernel (both read the second pair of codes of
// dense tiles only), the plain kernels elsewhere.
hipError_t launch_linear_hybrid(const LinearArgs& a, hipStream_t stream) {
    if (decode_hybrid_fits(a)) return launch_linear_decode_hybrid(a, stream);
    if (prefill_fits(a)) return launch_linear_prefill(a, stream);
    return launch_linear_generic(a, stream);
}

bool decode_qa_fits(const LinearArgs& a);
hipError_t launch_linear_decode_qa(const LinearArgs& a, hipStream_t stream);
bool decode_qa2_fits(const LinearArgs& a);
hipError_t launch_linear_decode_qa2(const LinearArgs& a, hipStream_t stream);
bool split_fits(const LinearArgs& a);
hipError_t launch_linear_split(const LinearArgs& a, hipStream_t stream);

// Quantised adapters.  Decode shapes read the int4 factors directly: one or
// two tokens in one launch when its workgroups can all be resident, else in
// two; 3 to 16 tokens on the K-split path.  Every other shape dequantises
// them into fp16 copies after the workspace of the fp16 path and runs that
// path.
size_t linear_qa_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    return align256(linear_workspace_bytes(M, N, K, r)) + align256((size_t)r * K * 2) + align256((size_t)N * r * 2);
}

hipError_t launch_linear_qa(const LinearArgs& a, hipStream_t stream) {
    if (decode_qa_fits(a)) return launch_linear_decode_qa(a, stream);
    if (decode_qa2_fits(a)) return launch_linear_decode_qa2(a, stream);
    if (a.M > 2 && a.batch == 1 && split_fits(a)) return launch_linear_split(a, stream);
    const size_t base = align256(linear_workspace_bytes(a.M, a.N, a.K, a.r));
    uint16_t* lt = reinterpret_cast<uint16_t*>(a.ws + base);
    uint16_t* rt = reinterpret_cast<uint16_t*>(a.ws + base + align256((size_t)a.r * a.K * 2));
    const hipError_t e = launch_adapter_dequant2(a.Lq, a.Ls, a.r, a.K, kAdapterGroupL, lt, a.Rq, a.Rs, a.N, a.r,
                                                 kAdapterGroupR, rt, stream);
    if (e != hipSuccess) return e;
    LinearArgs b = a;
    b.Lt = lt; b.Rt = rt;
    b.Lq = nullptr; b.Ls = nullptr; b.Rq = nullptr; b.Rs = nullptr;
    return launch_linear(b, stream);
}

}  // namespace slim
