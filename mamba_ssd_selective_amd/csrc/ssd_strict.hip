// ssd_strict.hip -- chunk-emulating decode on gfx950 (RL-Kernel RFC
// "Nemotron-3-Nano-30B-A3B", section 1, operator family 1, and section 3,
// Figure 2, box [F2]: the SSD scan runs train, prefill and "chunk-emulating
// decode" with one arithmetic, so that how a sequence is split into prefill
// and decode steps does not change a bit of its outputs).
//
// A decode token at offset i of its chunk is not folded into a running state.
// Each slot keeps the state at its current chunk's start and that chunk's
// tokens so far.  A step appends the new token to its slot's chunk buffers
// (emul_stage_kernel, which also records the row's length i + 1), then runs
// the chunked scan kernels on the slots in place (each row reads its slot's
// chunk buffers and chunk-start state) in their decode-output form: only the
// row block of offset i is computed and only y at offset i is written, which
// is the value the chunked prefill computes for that token.  When the chunk is
// complete (i = Q - 1) the scan's state at its end replaces the slot's
// chunk-start state.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kEmulThreads = 256;

__device__ __forceinline__ bool emul_row(const EmulArgs& a, int64_t r, int64_t& s, int& i) {
    s = a.state_idx[r];
    i = a.pos[r];
    return s >= 0 && s < a.cache_rows && i >= 0 && i < a.Q;
}

// The new token of row r into offset i of its slot's chunk buffers, and the
// row's length (0 for a padding row).  Word = uint4 when every width is a
// multiple of 16 bytes (the host then passes the widths in 16-byte words),
// else uint32_t.
template <typename Word>
__global__ __launch_bounds__(kEmulThreads) void emul_stage_kernel(EmulArgs a) {
    const int64_t r = blockIdx.x;
    int64_t s;
    int i;
    const bool live = emul_row(a, r, s, i);
    if (threadIdx.x == 0) a.row_len[r] = live ? i + 1 : 0;
    if (!live) return;
    const int wx = static_cast<int>(a.wx), wd = static_cast<int>(a.wd), wb = static_cast<int>(a.wb);
    const int W = wx + wd + 2 * wb;
    for (int o = threadIdx.x; o < W; o += kEmulThreads) {
        const Word* tok;  // the new token's row
        Word* buf;        // the slot's chunk buffer, token 0
        int e = o, width;
        if (e < wx) {
            tok = static_cast<const Word*>(a.x) + r * wx;
            buf = static_cast<Word*>(a.x_buf);
            width = wx;
        } else if ((e -= wx) < wd) {
            tok = reinterpret_cast<const Word*>(a.dt) + r * wd;
            buf = reinterpret_cast<Word*>(a.dt_buf);
            width = wd;
        } else if ((e -= wd) < wb) {
            tok = static_cast<const Word*>(a.B) + r * wb;
            buf = static_cast<Word*>(a.b_buf);
            width = wb;
        } else {
            e -= wb;
            tok = static_cast<const Word*>(a.C) + r * wb;
            buf = static_cast<Word*>(a.c_buf);
            width = wb;
        }
        buf[(s * a.Q + i) * width + e] = tok[e];
    }
}

}  // namespace

hipError_t launch_emul_stage(const EmulArgs& a, bool wide, int64_t b, hipStream_t st) {
    if (b == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(b));
    if (wide) return dispatch(emul_stage_kernel<uint4>, grid, dim3(kEmulThreads), st, a);
    return dispatch(emul_stage_kernel<uint32_t>, grid, dim3(kEmulThreads), st, a);
}

}  // namespace ssd
