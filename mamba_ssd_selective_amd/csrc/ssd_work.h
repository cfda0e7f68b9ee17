// ssd_work.h -- workgroup -> work-item mapping shared by the scan kernels.
// Internal to libssd.so.
#pragma once

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// Consecutive workgroup ids are dealt round-robin to the 8 XCDs of an MI355X,
// each with its own L2.  Remap so that one XCD receives a contiguous range of
// work items (workgroups sharing B/C data then share that XCD's L2).
__device__ __forceinline__ int64_t xcd_work_index(int64_t bid, int64_t nblocks) {
    constexpr int kXcd = 8;
    if (nblocks % kXcd != 0) return bid;
    return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

struct WorkItem {
    int64_t b;
    int seg, h, g;
};

// Work order (fastest first): head within its group, group, segment, row.
// Grids stay below 2^31 workgroups, so the index arithmetic is 32-bit.
__device__ __forceinline__ WorkItem decode_work(const ScanArgs& a, int nseg_grid) {
    uint32_t w = static_cast<uint32_t>(xcd_work_index(blockIdx.x, gridDim.x));
    const uint32_t hpg = static_cast<uint32_t>(a.H / a.G);
    WorkItem it;
    const int hh = static_cast<int>(w % hpg);
    w /= hpg;
    it.g = static_cast<int>(w % static_cast<uint32_t>(a.G));
    w /= static_cast<uint32_t>(a.G);
    it.seg = static_cast<int>(w % static_cast<uint32_t>(nseg_grid));
    it.b = static_cast<int64_t>(w / static_cast<uint32_t>(nseg_grid));
    it.h = it.g * static_cast<int>(hpg) + hh;
    return it;
}

// Offset of chunk c of (row b, head h) from each of the metadata pointers
// (cs, dtv, wgt): blocks of 3Q floats.
__device__ __forceinline__ int64_t meta_offset(const ScanArgs& a, int64_t b, int h, int c, int Q) {
    return ((b * a.H + h) * a.nc + c) * static_cast<int64_t>(3 * Q);
}

}  // namespace ssd
