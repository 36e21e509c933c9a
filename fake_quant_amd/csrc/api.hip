// api.hip -- ABI-level helpers of libfq.so: version, status strings, sizes.
#include <atomic>

#include "fq_host.h"

namespace fqh {

namespace {
// Per-device cache of one device attribute (fallback when the query fails).
int cached_attr(std::atomic<int>* cache, hipDeviceAttribute_t attr, int fallback) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) v = fallback;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}
}  // namespace

int num_cus() {
    static std::atomic<int> cache[kMaxDevices];
    return cached_attr(cache, hipDeviceAttributeMultiprocessorCount, 256);
}

int lds_per_cu() {
    static std::atomic<int> cache[kMaxDevices];
    return cached_attr(cache, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, 160 * 1024);
}

int lds_per_block() {
    static std::atomic<int> cache[kMaxDevices];
    return cached_attr(cache, hipDeviceAttributeMaxSharedMemoryPerBlock, 64 * 1024);
}

}  // namespace fqh

extern "C" {

int fq_version(void) { return FQ_ABI_VERSION; }

const char* fq_status_string(int status) {
    switch (status) {
        case FQ_OK: return "ok";
        case FQ_E_INVALID: return "invalid argument";
        case FQ_E_UNSUPPORTED: return "unsupported width, scheme, format or dtype";
        case FQ_E_DIM: return "dimension mismatch";
        case FQ_E_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

size_t fq_workspace_bytes(int64_t n) {
    if (n < 1) return 0;
    return (size_t)fqh::reduce_blocks(n) * 4 * sizeof(float);
}

int fq_q4dq_sizes(int64_t n, int64_t* packed_bytes, int64_t* num_blocks, int64_t* num_super) {
    if (n < 1 || !packed_bytes || !num_blocks || !num_super) return FQ_E_INVALID;
    int64_t nb = (n + 63) / 64;
    *packed_bytes = (n + 1) / 2;
    *num_blocks = nb;
    *num_super = (nb + 255) / 256;
    return FQ_OK;
}

}  // extern "C"
