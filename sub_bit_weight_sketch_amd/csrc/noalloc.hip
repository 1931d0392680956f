// noalloc.hip -- sketch_matmul for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// sketch_matmul needs a workspace only when Z = P^T x is staged once per call
// (stacks of many row blocks, several tokens, the float32 fallback); the
// multi-row prefill product can also use one to split K (optional: with a
// workspace too small it runs unsplit).  Here
// that workspace is a file-scope device array of fixed size, `scratch`: each
// GPU the library runs on holds its own copy until the process ends.  Its
// host-side name is only a stand-in for the symbol, so the device address of
// each GPU's copy is looked up once per device with hipGetSymbolAddress and
// only that address is handed to the kernels.  The scratch holds nothing
// between calls that a call relies on (Z, its maxima and the parts of a K
// split are written before they are read, on the call's stream), but every
// call on one GPU uses the
// same copy: calls that overlap in time on one GPU race.
#include <mutex>

#include "common.h"

namespace sketch {
namespace {

constexpr size_t kScratchBytes = SKETCH_NOALLOC_SCRATCH_BYTES;

static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of this device's scratch, looked up on the first call that
// has work to do with that device current; nullptr if the lookup fails.
void* scratch_address() {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

}  // namespace
}  // namespace sketch

extern "C" sketch_status sketch_matmul_noalloc(const sketch_params* p, const void* proj, const uint16_t* tables,
                                               const void* X, sketch_dtype x_dtype, int64_t batch, float* Y,
                                               void* stream) {
    // the workspace the product cannot do without must fit the scratch; the
    // scratch is then offered whole, so optional workspace that fits it is
    // used too
    size_t need = 0, want = 0;
    sketch_status rc = sketch::required_workspace_bytes(p, batch, x_dtype, &need);
    if (rc != SKETCH_OK) return rc;
    if (need > sketch::kScratchBytes) return SKETCH_ENOSPACE;
    rc = sketch_workspace_bytes(p, batch, x_dtype, &want);
    if (rc != SKETCH_OK) return rc;
    if (batch == 0 || p->M == 0)   // no-op, validated like sketch_matmul; touches no device
        return sketch_matmul(p, proj, tables, X, x_dtype, batch, Y, nullptr, 0, stream);
    if (want == 0) return sketch_matmul(p, proj, tables, X, x_dtype, batch, Y, nullptr, 0, stream);
    void* ws = sketch::scratch_address();
    if (!ws) return SKETCH_EDEVICE;
    return sketch_matmul(p, proj, tables, X, x_dtype, batch, Y, ws, sketch::kScratchBytes, stream);
}
