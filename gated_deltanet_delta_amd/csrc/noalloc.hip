// noalloc.hip -- gdn_chunk_fwd_noalloc: the chunked prefill with its scratch in a static device array,
// for callers that cannot allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The bf16 chunked prefill needs scratch between its two phases (per-chunk decay sums, M = T diag(beta)
// and N = K K_prev^T, per chunk).  gdn_chunk_fwd takes it from the caller's workspace; this variant
// takes it from `scratch`, a file-scope device array of kScratchBytes that every GPU the library runs
// on holds (one copy per device, at its own address) until the process ends.  The array's device
// address is looked up once per device with hipGetSymbolAddress, with that device current, and that
// address -- never the array's host-side name -- is what the kernels receive.  Nothing here allocates.
//
// Every call on one GPU shares that GPU's array and finds the previous call's contents in it; the
// prefill reads only what its own first phase wrote in the same call, so nothing needs clearing.
// Two calls that overlap in time on one GPU (different streams or threads) race on the array.

#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // GDN_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` on device d, null until looked up

// Device address of `scratch` on device `dev`, which is current on the calling thread.
hipError_t scratch_on(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                                 int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                 gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o, float* final_state,
                                 hipStream_t stream) {
    // the size query returns 0 for calls that need no scratch (fp32 inputs) and for rejected sizes,
    // which gdn_chunk_fwd then reports as such
    const size_t need = gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv_dtype);
    if (need > kScratchBytes) return GDN_ERROR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERROR_LAUNCH_FAILURE;
        if (stream) {   // the array is looked up on the current device: the stream must run there
            int sdev = -1;
            if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GDN_ERROR_INVALID_VALUE;
            if (sdev != dev) return GDN_ERROR_INVALID_VALUE;
        }
        if (scratch_on(dev, &ws) != hipSuccess) return GDN_ERROR_LAUNCH_FAILURE;
    }
    return gdn_chunk_fwd(q, k, v, g, beta, initial_state, cu_seqlens, B, T, Hk, Hv, dk, dv, N, qkv_dtype,
                         gate_dtype, o, final_state, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
