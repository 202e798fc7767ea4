// spec_verify_sample_noalloc: spec_verify_sample for callers that cannot
// allocate (code under stream capture, tight serving loops): its scratch, the
// exit counter and the group mailbox, is a fixed array of the library instead
// of a caller's workspace.
//
// The array is a file-scope device variable, so every device that loads the
// library holds its own copy, at its own address, until the process ends. On
// the host its name is only a stand-in; the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept. The sampler's kernels leave the mailbox zero-filled at the end of
// every call, which is what the next call needs; the array is zero from load
// and is cleared once more, by a fill kernel, when its address is first
// looked up. Calls on one device share the array, so calls that overlap in
// time on one device race (keep them on one stream).

#include <mutex>

#include "common.h"

namespace tav {
namespace {

constexpr size_t kScratchBytes = 256 * 1024;   // exit counter + mailbox; 64 KB covers any plan
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_fill_kernel(uint64_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

std::mutex g_mu;
void *g_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// This device's scratch address (NULL on failure). The first call for a
// device looks it up and queues the clearing fill on `stream`, ahead of the
// caller's kernel.
void *device_scratch(hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return nullptr;
        hipLaunchKernelGGL(zero_fill_kernel, dim3(64), dim3(256), 0, stream,
                           static_cast<uint64_t *>(ptr), (int64_t)(kScratchBytes / 8));
        if (hipGetLastError() != hipSuccess)
            return nullptr;
        g_ptr[dev] = ptr;
    }
    return g_ptr[dev];
}

} // namespace
} // namespace tav

extern "C" tav_status spec_verify_sample_noalloc(const float *target_logits,
                                                 const float *draft_logits,
                                                 const int32_t *parent, const int32_t *token,
                                                 int32_t B, int32_t N, int32_t V,
                                                 double temperature, uint64_t seed,
                                                 uint64_t offset, int32_t *path,
                                                 int32_t *n_accepted, int32_t *out_tokens,
                                                 uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    // argument errors first, exactly as spec_verify_sample reports them (its
    // checks come before its workspace check; a NULL workspace fails that)
    const tav_status pre = sv_launch(target_logits, draft_logits, parent, token, B, N, V,
                                     temperature, seed, offset, path, n_accepted, out_tokens,
                                     nullptr, 0, dev_flags, stream, false, nullptr, nullptr,
                                     nullptr);
    if (pre != TAV_ERR_WORKSPACE)
        return pre;   // an argument or shape error (nothing was launched)
    const size_t need = spec_verify_workspace_bytes(B, N, V);
    if (need == 0)
        return TAV_ERR_LAUNCH;
    if (need > kScratchBytes)
        return TAV_ERR_WORKSPACE;   // the plan's mailbox does not fit the fixed array
    void *ws = device_scratch(as_stream(stream));
    if (!ws)
        return TAV_ERR_LAUNCH;
    return sv_launch(target_logits, draft_logits, parent, token, B, N, V, temperature, seed,
                     offset, path, n_accepted, out_tokens, ws, kScratchBytes, dev_flags, stream,
                     false, nullptr, nullptr, nullptr);
}
