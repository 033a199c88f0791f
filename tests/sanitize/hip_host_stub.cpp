// Host-only stand-in for the few HIP runtime calls the library's host code makes, and for its
// device launch tables, so that the host code (encoders, import validation, handle life cycle,
// argument checks) can be built with AddressSanitizer / UndefinedBehaviorSanitizer and run on
// a machine without a GPU.  "Device" memory is host memory here; every launch reports an
// error, as a missing GPU would.  Test infrastructure only.
#include <stdlib.h>
#include <string.h>

#include "lscd_internal.h"

extern "C" {

hipError_t hipGetDevice(int* device) {
    if (!device) return hipErrorInvalidValue;
    *device = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
    if (!value || device != 0) return hipErrorInvalidValue;
    *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

hipError_t hipMalloc(void** ptr, size_t size) {
    if (!ptr) return hipErrorInvalidValue;
    *ptr = malloc(size ? size : 1);
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipFree(void* ptr) {
    free(ptr);
    return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
    if (n && (!dst || !src)) return hipErrorInvalidValue;
    if (n) memcpy(dst, src, n);
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t) {
    return hipMemcpy(dst, src, n, kind);
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

}  // extern "C"

namespace lscd {

hipError_t launch_spmm(int, int, int, const SpmmArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_reduce(const float*, uint16_t*, int, int, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(int, const DecodeArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_bitmap(const DecodeArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_three_level(const DecodeArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stream_read(const void*, int64_t, int, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t encode_device(const uint16_t*, const uint8_t*, const Grid&, uint32_t*, uint32_t*, unsigned long long*,
                         hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t encode_device_fill(const uint16_t*, const uint8_t*, const Grid&, const uint32_t*, uint32_t*, bool,
                              hipStream_t) {
    return hipErrorNoDevice;
}
int spmm_blocks_per_cu(int, int, int, int, int) { return 2; }
hipError_t scratch_partials(int, float**) { return hipErrorNoDevice; }
void release_dense(struct ::lscd_handle_s*) {}

}  // namespace lscd
