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

// Work item w in the order (fastest first): head within its group, group,
// segment, row.  Work counts stay below 2^31, so the arithmetic is 32-bit.
__device__ __forceinline__ WorkItem decode_work_at(const ScanArgs& a, int nseg_grid, uint32_t w) {
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
// The work item of this workgroup (one per workgroup, XCD-aware order).
__device__ __forceinline__ WorkItem decode_work(const ScanArgs& a, int nseg_grid) {
    return decode_work_at(a, nseg_grid, static_cast<uint32_t>(xcd_work_index(blockIdx.x, gridDim.x)));
}

// The tokens of row b: the first one's index in x, dt, B, C, y and seq_idx
// (counted in tokens) and how many there are.  Chunk c of the row is tokens
// [c Q, min(c Q + Q, len)) from there; chunks at or past len are not part of
// it (no kernel reads or writes their data).
struct RowSpan {
    int64_t t0;
    int64_t len;    // <= L
    int64_t state;  // the row's initial / final state: row b, or its slot
    bool live;      // false: a row of no slot (nothing of it is read or written)
};
__device__ __forceinline__ RowSpan row_span(const ScanArgs& a, int64_t b) {
    RowSpan r;
    r.state = b;
    r.live = true;
    if (a.slot) {
        const int64_t s = a.slot[b];
        r.live = s >= 0 && s < a.slots;
        r.state = r.live ? s : 0;
        r.t0 = r.state * a.L;
        r.len = 0;
        if (r.live) {
            r.len = a.L;
            if (a.pos) {
                const int64_t i = a.pos[b];
                r.len = i >= 0 && i < a.L ? i + 1 : 0;
            } else if (a.row_len) {
                const int64_t rl = a.row_len[b];
                r.len = rl < 0 ? 0 : (rl < a.L ? rl : a.L);
            }
        }
    } else if (a.cu) {
        int64_t lo = a.cu[b], hi = a.cu[b + 1];
        lo = lo < 0 ? 0 : (lo > a.T ? a.T : lo);
        hi = hi < lo ? lo : (hi > a.T ? a.T : hi);
        r.t0 = lo;
        r.len = hi - lo < a.L ? hi - lo : a.L;
    } else {
        r.t0 = b * a.L;
        r.len = a.L;
        if (a.row_len) {
            const int64_t rl = a.row_len[b];
            r.len = rl < 0 ? 0 : (rl < a.L ? rl : a.L);
        }
    }
    return r;
}

// Offset of chunk c of (row b, head h) from each of the metadata pointers
// (cs, dtv, wgt): blocks of 3Q floats.
__device__ __forceinline__ int64_t meta_offset(const ScanArgs& a, int64_t b, int h, int c, int Q) {
    return ((b * a.H + h) * a.nc + c) * static_cast<int64_t>(3 * Q);
}

}  // namespace ssd
