// la_noalloc.hip -- lightning_attn_fwd_noalloc: the forward pass for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// It runs exactly the kernels of lightning_attn_fwd, with their scratch (the
// chunk and sub-chunk tables and the per-sub-chunk fp32 states of the scan)
// in a file-scope static device array instead of a caller's workspace.  Each
// GPU the library runs on holds its own copy of the array until the process
// ends.  Its device address is looked up once per device, with that device
// current, and only that address is ever handed to a kernel: the array's
// name in host code is a host-side stand-in, not a device address.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/lightning_attn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// Device address of the current device's copy of `scratch`, looked up on the
// device's first call; nullptr (with the HIP error cleared) on failure.
void *scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    scratch_ptr[dev].store(addr, std::memory_order_release);
    return addr;
}

}  // namespace

extern "C" int lightning_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o,
                                          int batch, int heads, int64_t seq_len, int head_dim,
                                          int block_size, const int32_t *cu_seqlens, int dtype,
                                          void *stream) {
    const size_t need = lightning_attn_fwd_workspace_size(batch, heads, seq_len, head_dim, block_size,
                                                          cu_seqlens != nullptr, dtype);
    if (need == 0)   // rejected arguments, or no tokens: lightning_attn_fwd gives the status
        return lightning_attn_fwd(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens,
                                  dtype, nullptr, 0, stream);
    if (need > kScratchBytes) return LA_ESCRATCH;
    void *ws = scratch_of_current_device();
    if (!ws) return LA_EHIP;
    // the kernels write every table and state they read: nothing to clear
    return lightning_attn_fwd(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                              ws, kScratchBytes, stream);
}
