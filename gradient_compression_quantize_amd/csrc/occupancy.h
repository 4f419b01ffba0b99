// occupancy.h -- an LDS reservation that caps the resident workgroups of a
// launch per CU (host code; used by libgcq.so and the benchmark's ceiling
// kernels).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <mutex>
#include <unordered_map>

namespace gcq {

// Dynamic LDS, in bytes, that holds a workgroup declaring `own` bytes of LDS
// of its own to `per_cu` resident workgroups on a CU with `lds_per_cu` bytes
// of LDS and at most `lds_per_block` per workgroup; 0 (no limit) when
// per_cu < 1 or those sizes cannot express that cap.
//
// The CU hands out LDS in units coarser than 512 bytes: 27,136 bytes per
// workgroup left room for 5 of them in 160 KB, not 6. A workgroup's LDS (its
// own plus the reservation) is made 256 bytes short of a multiple of 2560
// bytes, which rounds up to that multiple in any unit from 512 to 2560 bytes
// that divides it; at 256-byte units it is taken as is, and one more
// workgroup still does not fit.
constexpr size_t lds_reservation(size_t lds_per_cu, size_t lds_per_block, int per_cu,
                                 size_t own)
{
    constexpr size_t kUnit = 2560, kSlack = 256;
    if (per_cu < 1)
        return 0;
    const size_t whole = lds_per_cu / size_t(per_cu) / kUnit * kUnit;
    if (whole <= kSlack + own || whole > lds_per_block)
        return 0;
    const size_t total = whole - kSlack;  // own + reservation
    // per_cu fit (each takes at most `whole`); one more does not
    if (size_t(per_cu + 1) * total <= lds_per_cu)
        return 0;
    return total - own;
}

// lds_reservation for the current device (its LDS sizes read once per
// device). The kernel never touches the reservation. Some streaming kernels
// move HBM faster with fewer waves in flight per CU than their registers
// allow.
inline size_t lds_for_wg_per_cu(int per_cu, size_t own = 0)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> lds_per_cu[kMaxDevices] = {};
    static std::atomic<int> lds_per_block[kMaxDevices] = {};
    int dev = 0;
    if (per_cu < 1)
        return 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();  // the launch that follows reports its own status
        return 0;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return 0;
    int cu = lds_per_cu[dev].load(std::memory_order_relaxed);
    int blk = lds_per_block[dev].load(std::memory_order_relaxed);
    if (cu <= 0 || blk <= 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            hipDeviceGetAttribute(&blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            cu <= 0 || blk <= 0) {
            (void)hipGetLastError();  // the launch that follows reports its own status
            return 0;
        }
        lds_per_cu[dev].store(cu, std::memory_order_relaxed);
        lds_per_block[dev].store(blk, std::memory_order_relaxed);
    }
    return lds_reservation(size_t(cu), size_t(blk), per_cu, own);
}

// LDS a kernel declares itself (hipFuncGetAttributes), cached per kernel;
// false if the runtime cannot say.
inline bool kernel_own_lds(const void* fn, size_t* own)
{
    static std::mutex mu;
    static std::unordered_map<const void*, long long> cache;  // -1: unknown
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(fn);
    if (it == cache.end()) {
        hipFuncAttributes a{};
        long long v = -1;
        if (hipFuncGetAttributes(&a, fn) == hipSuccess)
            v = (long long)a.sharedSizeBytes;
        else
            (void)hipGetLastError();  // the launch that follows reports its own status
        it = cache.emplace(fn, v).first;
    }
    if (it->second < 0)
        return false;
    *own = size_t(it->second);
    return true;
}

// The reservation for `kernel` at `per_cu` resident workgroups per CU, its
// own LDS accounted for; 0 (no limit) for per_cu < 1 or when that LDS is
// unknown.
template <typename Kernel>
size_t lds_cap(Kernel kernel, int per_cu)
{
    size_t own = 0;
    if (per_cu < 1 || !kernel_own_lds(reinterpret_cast<const void*>(kernel), &own))
        return 0;
    return lds_for_wg_per_cu(per_cu, own);
}

}  // namespace gcq
