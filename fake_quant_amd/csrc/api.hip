// api.hip -- ABI-level helpers of libfq.so: version, status strings, sizes.
#include <atomic>

#include "fq_host.h"

namespace fqh {

int num_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev >= 64) dev = 63;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
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
