// engram_forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops): the forward's workspace is a
// fixed array of the library's own in device memory instead of a buffer the
// caller passes.
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never uses the array's name as an address (on the host it only names the
// symbol); the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Each call on a
// GPU uses that GPU's copy, so calls that overlap on one GPU race on it.
// The forward needs nothing in its workspace on entry (every region is
// written before it is read), so nothing is cleared between calls.
#include <mutex>

#include "internal.h"

static __device__ __align__(256) uint8_t scratch[ENGRAM_FIXED_SCRATCH_BYTES];

namespace {

constexpr size_t kFixedScratchBytes = (size_t)ENGRAM_FIXED_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device ordinal

// The current device's copy of `scratch`; the stream must belong to that
// device.
engram_status fixed_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ENGRAM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ENGRAM_ERR_UNSUPPORTED;
    if (stream != nullptr) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ENGRAM_ERR_HIP;
        if (sdev != dev) return ENGRAM_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return ENGRAM_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ENGRAM_OK;
}

}  // namespace

extern "C" {

size_t engram_fixed_scratch_bytes(void) { return kFixedScratchBytes; }

engram_status engram_forward_noalloc(const engram_geometry* g, const engram_hash_tables* t,
                                     const uint8_t* table, const uint8_t* scales,
                                     const uint16_t* w, const uint16_t* q, const uint16_t* k,
                                     int32_t* state, const uint16_t* x, const int32_t* ids,
                                     const uint8_t* mask, int32_t B, int32_t T, uint16_t* out,
                                     float* gate, uint32_t* err, void* stream) {
    const engram_status st =
        engram::forward_check(g, t, table, scales, w, q, k, x, ids, B, T, out);
    if (st != ENGRAM_OK || (int64_t)B * T == 0) return st;
    // sizes beyond the fixed array are refused before anything touches the GPU
    if (engram_forward_workspace_size(g, (int64_t)B * T) > kFixedScratchBytes)
        return ENGRAM_ERR_TOO_LARGE;
    void* ws = nullptr;
    const engram_status sst = fixed_scratch((hipStream_t)stream, &ws);
    if (sst != ENGRAM_OK) return sst;
    return engram::forward_launch(g, t, table, scales, w, q, k, state, x, ids, mask, B, T, out,
                                  gate, ws, err, stream);
}

}  // extern "C"
