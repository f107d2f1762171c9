// Streaming device copy: the measured HBM ceiling that the WKV7 kernels are
// reported against next to the nominal 8 TB/s.  The decode step moves each
// state from HBM through registers and back once, which is what a copy does,
// so a copy tuned the same way (whole 1 KiB wave accesses, non-temporal loads
// and stores, every byte read and written once) measures what that traffic
// pattern can reach on this machine.
#include <stdint.h>

#include "wkv7_internal.h"

namespace wkv7 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16-byte piece per thread, 8 KiB per workgroup.  A sweep of 64..1024
// threads and 1..16 pieces per thread found this the fastest shape; several
// pieces per thread with 16-32 KiB per workgroup lost up to a third.
constexpr int kCopyThreads = 512;
constexpr int kCopyPerThread = 1;

// Workgroup g copies pieces [g*512, g*512+512), one KiB per wave instruction.
__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const f32x4 *src, f32x4 *dst,
                                                                   size_t n16) {
    const size_t base = (size_t)blockIdx.x * (kCopyThreads * kCopyPerThread) + threadIdx.x;
    f32x4 x[kCopyPerThread];
#pragma unroll
    for (int i = 0; i < kCopyPerThread; ++i) {
        const size_t e = base + (size_t)i * kCopyThreads;
        if (e < n16) x[i] = __builtin_nontemporal_load(src + e);
    }
#pragma unroll
    for (int i = 0; i < kCopyPerThread; ++i) {
        const size_t e = base + (size_t)i * kCopyThreads;
        if (e < n16) __builtin_nontemporal_store(x[i], dst + e);
    }
}

}  // namespace
}  // namespace wkv7

using namespace wkv7;

extern "C" rwkv7_status rwkv7_stream_copy(const void *src, void *dst, size_t bytes,
                                          void *stream) {
    if (bytes == 0) return RWKV7_OK;
    if (!src || !dst) return RWKV7_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
        return RWKV7_ERR_ALIGN;
    if (bytes % 16 != 0) return RWKV7_ERR_SHAPE;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return RWKV7_ERR_ALIAS;
    const size_t n16 = bytes / 16;
    const size_t per_group = (size_t)kCopyThreads * kCopyPerThread;
    const size_t groups = (n16 + per_group - 1) / per_group;
    if (groups > 0x7fffffffu) return RWKV7_ERR_SHAPE;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)groups), dim3(kCopyThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const f32x4 *>(src),
                       static_cast<f32x4 *>(dst), n16);
    return hipGetLastError() == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}
