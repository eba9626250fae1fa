// hqq_noalloc.hip -- hqq_quantize_noalloc: hqq_quantize for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its scratch is one file-scope device array of fixed size; each GPU the library
// runs on holds its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "hqq.h"
#include "hqq_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device

// In host code this name is a stand-in, not a device address: kernels receive the address
// hipGetSymbolAddress returns for the current device, never the name itself.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

}  // namespace

extern "C" hqq_status hqq_quantize_noalloc(const void *W, int64_t rows, int64_t cols, int nbits,
                                           int group_size, int axis, float p, float beta,
                                           float kappa, int iters, int early_stop, int zero_bits,
                                           void *packed, void *scale, void *zero,
                                           void *zero_meta, uint8_t *passes, void *stream)
{
    hqq_job j;
    j.W = W;
    j.rows = rows;
    j.cols = cols;
    j.nbits = nbits;
    j.group_size = group_size;
    j.axis = axis;
    j.p = p;
    j.beta = beta;
    j.kappa = kappa;
    j.iters = iters;
    j.early_stop = early_stop;
    j.zero_bits = zero_bits;
    j.packed = packed;
    j.scale = scale;
    j.zero = zero;
    j.zero_meta = zero_meta;
    j.passes = passes;
    const size_t need = hqq_workspace_bytes(&j, 1);
    if (need == SIZE_MAX || need == 0)      // invalid arguments (reported), or no scratch needed
        return hqq_quantize_batch(&j, 1, nullptr, 0, stream);
    if (need > kScratchBytes) {
        const std::string msg = "this tensor needs " + std::to_string(need) +
                                " bytes of scratch; the static scratch holds " +
                                std::to_string(kScratchBytes) + " (use hqq_quantize)";
        return (hqq_status)hqq::report_error(HQQ_ERR_WORKSPACE, msg.c_str());
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (hqq_status)hqq::report_error(HQQ_ERR_DEVICE, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return (hqq_status)hqq::report_error(HQQ_ERR_UNSUPPORTED, "device index above 63");
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_scratch[dev]) {             // first call on this device: look the copy up
            void *p_dev = nullptr;
            e = hipGetSymbolAddress(&p_dev, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p_dev) {
                const std::string msg = std::string("scratch lookup: ") + hipGetErrorString(e);
                return (hqq_status)hqq::report_error(HQQ_ERR_DEVICE, msg.c_str());
            }
            g_scratch[dev] = p_dev;
        }
        ptr = g_scratch[dev];
    }
    return hqq_quantize_batch(&j, 1, ptr, kScratchBytes, stream);
}
