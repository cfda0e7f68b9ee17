// ssd_varlen.hip -- packed variable-length prefill on gfx950: the copies
// between the packed token layout (sequences back to back, cu_seqlens
// offsets) and one row per sequence, so that every sequence is chunked from
// its own first token and has its own initial and final state (RL-Kernel RFC
// "Nemotron-3-Nano-30B-A3B", section 8, open question 4: cu_seqlens-aware
// chunking, against 128-aligned pack offsets).
//
//   varlen_pack_kernel    row r, token j < len_r: x, dt, B, C of packed token
//                         cu[r] + j; zeros from len_r to the row's end; and
//                         len_r itself;
//   varlen_unpack_kernel  y of row r, token j < len_r, to packed token cu[r] + j.
// Lengths and offsets are clamped so that every access stays inside the
// packed buffers (total tokens T) and the rows (max_seqlen) whatever
// cu_seqlens holds.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kVarThreads = 256;

// Row r's packed offset and length (clamped to [0, T] and [0, Lmax]).
__device__ __forceinline__ void varlen_row(const VarlenArgs& a, int64_t r, int64_t& off,
                                           int64_t& len) {
    int64_t lo = a.cu[r], hi = a.cu[r + 1];
    lo = lo < 0 ? 0 : (lo > a.T ? a.T : lo);
    hi = hi < lo ? lo : (hi > a.T ? a.T : hi);
    len = hi - lo < a.Lmax ? hi - lo : a.Lmax;
    off = lo;
}

template <typename Word>
__global__ __launch_bounds__(kVarThreads) void varlen_pack_kernel(VarlenArgs a) {
    const int64_t r = blockIdx.y;
    int64_t off, len;
    varlen_row(a, r, off, len);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.row_len[r] = static_cast<int32_t>(len);
    // one token per block step, its words over the threads (no division)
    const int wx = static_cast<int>(a.wx), wd = static_cast<int>(a.wd), wb = static_cast<int>(a.wb);
    const int W = wx + wd + 2 * wb;
    for (int64_t j = blockIdx.x; j < a.Lmax; j += gridDim.x) {
        const bool real = j < len;
        const int64_t src_t = off + j, dst_t = r * a.Lmax + j;
        for (int o = threadIdx.x; o < W; o += kVarThreads) {
            const Word* src;
            Word* dst;
            int e = o, width;
            if (e < wx) {
                src = static_cast<const Word*>(a.x);
                dst = static_cast<Word*>(a.xw);
                width = wx;
            } else if ((e -= wx) < wd) {
                src = reinterpret_cast<const Word*>(a.dt);
                dst = reinterpret_cast<Word*>(a.dtw);
                width = wd;
            } else if ((e -= wd) < wb) {
                src = static_cast<const Word*>(a.B);
                dst = static_cast<Word*>(a.bw);
                width = wb;
            } else {
                e -= wb;
                src = static_cast<const Word*>(a.C);
                dst = static_cast<Word*>(a.cw);
                width = wb;
            }
            Word v = Word{};
            if (real) v = src[src_t * width + e];
            dst[dst_t * width + e] = v;
        }
    }
}

template <typename Word>
__global__ __launch_bounds__(kVarThreads) void varlen_unpack_kernel(VarlenArgs a) {
    const int64_t r = blockIdx.y;
    int64_t off, len;
    varlen_row(a, r, off, len);
    const int wx = static_cast<int>(a.wx);
    for (int64_t j = blockIdx.x; j < len; j += gridDim.x) {
        const Word* src = static_cast<const Word*>(a.yw) + (r * a.Lmax + j) * wx;
        Word* dst = static_cast<Word*>(a.y) + (off + j) * wx;
        for (int o = threadIdx.x; o < wx; o += kVarThreads) dst[o] = src[o];
    }
}

}  // namespace

hipError_t launch_varlen_pack(const VarlenArgs& a, bool wide, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.Lmax < 512 ? a.Lmax : 512), static_cast<unsigned>(a.nseq));
    if (wide) return dispatch(varlen_pack_kernel<uint4>, grid, dim3(kVarThreads), st, a);
    return dispatch(varlen_pack_kernel<uint32_t>, grid, dim3(kVarThreads), st, a);
}

hipError_t launch_varlen_unpack(const VarlenArgs& a, bool wide, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.Lmax < 512 ? a.Lmax : 512), static_cast<unsigned>(a.nseq));
    if (wide) return dispatch(varlen_unpack_kernel<uint4>, grid, dim3(kVarThreads), st, a);
    return dispatch(varlen_unpack_kernel<uint32_t>, grid, dim3(kVarThreads), st, a);
}

}  // namespace ssd
