// mp_loss_mse_noalloc: the scaled MSE loss of mp_loss_mse for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). Its per-block partials live in `scratch`, a file-scope device array of the
// library that each GPU holds until the process ends, instead of a caller workspace. The loss
// kernels never use more partials than the array holds (their grid is capped at 1024 blocks).
//
// `scratch` names a host-side stand-in in host code, not a device address: the address of
// each GPU's copy is looked up once per device (hipGetSymbolAddress, with that device current)
// on the entry point's first call there, kept per device, and only that address is passed to
// the kernels. Every call on one GPU shares its array; each launch overwrites every partial it
// later reads, so nothing needs clearing, but calls that overlap on one GPU race.
#include <mutex>

#include "mp_loss.h"

namespace {

constexpr int kScratchFloats = 1024;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_scratch_mutex;
float* g_scratch_addr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up on the first call on the device).
mp_status scratch_for_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return mp::hip_status(e, "mp_loss_mse_noalloc/hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return MP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return mp::hip_status(e, "mp_loss_mse_noalloc/hipGetSymbolAddress");
        if (!p) return MP_ERR_HIP;
        g_scratch_addr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_addr[dev];
    return MP_OK;
}

}  // namespace

extern "C" mp_status mp_loss_mse_noalloc(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, float c,
                                         const mp_scaler* scaler, float* loss, uint16_t* dy, mp_stream stream) {
    if (mp_status st = mp::loss_mse_args(y, t, M, N, scaler, loss, dy)) return st;
    if (M == 0 || N == 0) return MP_OK;
    if (mp::loss_mse_partials(M, N) > size_t(kScratchFloats)) return MP_ERR_INVALID_ARGUMENT;
    float* partials = nullptr;
    if (mp_status st = scratch_for_current_device(&partials)) return st;
    return mp::loss_mse_into(y, t, M, N, c, scaler, loss, dy, partials, mp::as_stream(stream));
}
