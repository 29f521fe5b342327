// vox_host.h - host-side helpers of libvox (status codes, error text, launch checks).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "../../include/vox.h"

namespace vox {

// Records a message for vox_last_error() on this thread and returns `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread's message; returns VOX_OK.
int ok();
// Checks hipGetLastError() after enqueuing; maps a failure to VOX_E_HIP.
int check_launch(const char *what);
int check_hip(hipError_t e, const char *what);

// Number of compute units of the current device (cached per device).
int cu_count();

// Resident workgroups of `threads` threads per compute unit for `kernel`, computed on first use
// and kept in `cache` (at least 1).  Safe to call from several threads.
template <class K>
int resident_per_cu(std::atomic<int> &cache, K kernel, int threads)
{
    int v = cache.load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, 0) != hipSuccess || v < 1)
            v = 1;
        cache.store(v, std::memory_order_relaxed);
    }
    return v;
}

inline bool overlaps(const void *a, size_t an, const void *b, size_t bn)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return an && bn && a0 < b0 + bn && b0 < a0 + an;
}

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace vox
