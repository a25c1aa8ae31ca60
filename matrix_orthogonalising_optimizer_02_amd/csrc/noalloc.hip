// rownorm_update_noalloc: the Periodic variant's RowNorm step ("Scaling Muon for
// Diffusion Transformers", Periodic Row-wise paragraphs) for callers that cannot
// allocate device memory: code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc. Its workspace is a fixed-size array in device memory that the
// library holds (one copy per GPU, for the life of the process); the caller passes only
// the matrices, the optional monitor array and the stream. Declared in
// include/muon_rocm.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "abi_internal.hpp"

#define MUON_API extern "C" __attribute__((visibility("default")))

namespace muon {

constexpr size_t kNoAllocScratchBytes = MUON_NOALLOC_SCRATCH_BYTES;

// The scratch array. In host code `scratch` names a host-side stand-in, not the device
// array: host code uses only the address hipGetSymbolAddress returns for the current
// device (scratch_for_current_device below).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t status = hipSuccess;
};

DeviceScratch g_dev[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device with that device
// current. NULL with *error set when there is no device or the lookup fails.
void* scratch_for_current_device(std::string* error) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *error = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *error = "device index " + std::to_string(dev) + " out of range";
        return nullptr;
    }
    DeviceScratch& d = g_dev[dev];
    std::call_once(d.once, [&d] {
        void* p = nullptr;
        d.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.status == hipSuccess) d.ptr = p;
    });
    if (d.status != hipSuccess || d.ptr == nullptr) {
        *error = std::string("hipGetSymbolAddress: ") + hipGetErrorString(d.status);
        return nullptr;
    }
    return d.ptr;
}

}  // namespace
}  // namespace muon

MUON_API int rownorm_update_noalloc(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                                    float* update_rms, void* stream) {
    return muon::rownorm_noalloc_impl(mats, count, hp, update_rms, stream, muon::kNoAllocScratchBytes,
                                      &muon::scratch_for_current_device);
}
