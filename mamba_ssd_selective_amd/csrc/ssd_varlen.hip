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
    const int64_t wx = a.wx, wd = a.wd, wb = a.wb;
    const int64_t W = wx + wd + 2 * wb;
    const int64_t total = a.Lmax * W;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kVarThreads;
    for (int64_t w = static_cast<int64_t>(blockIdx.x) * kVarThreads + threadIdx.x; w < total;
         w += stride) {
        const int64_t j = w / W;
        int64_t o = w % W;
        const Word* src;
        Word* dst;
        int64_t width;
        if (o < wx) {
            src = static_cast<const Word*>(a.x);
            dst = static_cast<Word*>(a.xw);
            width = wx;
        } else if ((o -= wx) < wd) {
            src = reinterpret_cast<const Word*>(a.dt);
            dst = reinterpret_cast<Word*>(a.dtw);
            width = wd;
        } else if ((o -= wd) < wb) {
            src = static_cast<const Word*>(a.B);
            dst = static_cast<Word*>(a.bw);
            width = wb;
        } else {
            o -= wb;
            src = static_cast<const Word*>(a.C);
            dst = static_cast<Word*>(a.cw);
            width = wb;
        }
        Word v = Word{};
        if (j < len) v = src[(off + j) * width + o];
        dst[(r * a.Lmax + j) * width + o] = v;
    }
}

template <typename Word>
__global__ __launch_bounds__(kVarThreads) void varlen_unpack_kernel(VarlenArgs a) {
    const int64_t r = blockIdx.y;
    int64_t off, len;
    varlen_row(a, r, off, len);
    const int64_t total = len * a.wx;
    const Word* src = static_cast<const Word*>(a.yw) + r * a.Lmax * a.wx;
    Word* dst = static_cast<Word*>(a.y) + off * a.wx;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kVarThreads;
    for (int64_t w = static_cast<int64_t>(blockIdx.x) * kVarThreads + threadIdx.x; w < total;
         w += stride)
        dst[w] = src[w];
}

}  // namespace

hipError_t launch_varlen_pack(const VarlenArgs& a, bool wide, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    const dim3 grid(64, static_cast<unsigned>(a.nseq));
    if (wide) return dispatch(varlen_pack_kernel<uint4>, grid, dim3(kVarThreads), st, a);
    return dispatch(varlen_pack_kernel<uint32_t>, grid, dim3(kVarThreads), st, a);
}

hipError_t launch_varlen_unpack(const VarlenArgs& a, bool wide, hipStream_t st) {
    if (a.nseq == 0) return hipSuccess;
    const dim3 grid(64, static_cast<unsigned>(a.nseq));
    if (wide) return dispatch(varlen_unpack_kernel<uint4>, grid, dim3(kVarThreads), st, a);
    return dispatch(varlen_unpack_kernel<uint32_t>, grid, dim3(kVarThreads), st, a);
}

}  // namespace ssd
