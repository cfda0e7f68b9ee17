// ssd_strict.hip -- chunk-emulating decode on gfx950 (RL-Kernel RFC
// "Nemotron-3-Nano-30B-A3B", section 1, operator family 1, and section 3,
// Figure 2, box [F2]: the SSD scan runs train, prefill and "chunk-emulating
// decode" with one arithmetic, so that how a sequence is split into prefill
// and decode steps does not change a bit of its outputs).
//
// A decode token at offset i of its chunk is not folded into a running state.
// Each slot keeps the state at its current chunk's start and that chunk's
// tokens so far; a step appends the new token and runs the chunked scan over
// the chunk (offsets 0..i real, the rest padding with dt 0) from the
// chunk-start state, and returns y at offset i: the value the chunked prefill
// computes for that token.  When the chunk is complete (i = Q - 1) the scan's
// final state becomes the slot's new chunk-start state.
//
// Two small copy kernels around the scan:
//   emul_stage_kernel   writes the new token into its slot's chunk buffers and
//                       copies the slot's chunk (new token included, zeros past
//                       it) into batch-ordered scan inputs; row lengths i + 1;
//   emul_finish_kernel  copies y at offset i out, and commits the final state
//                       of a completed chunk to the slot.
// They move 16-byte words where every width allows (else 4-byte words).
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

// Word = uint4 when every width is a multiple of 16 bytes (the host then
// passes the widths in 16-byte words), else uint32_t.
template <typename Word>
__global__ __launch_bounds__(kEmulThreads) void emul_stage_kernel(EmulArgs a) {
    const int64_t r = blockIdx.y;
    int64_t s;
    int i;
    const bool live = emul_row(a, r, s, i);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.row_len[r] = live ? i + 1 : 0;
    // one token per block step, its words (x, dt, B, C) over the threads
    const int wx = static_cast<int>(a.wx), wd = static_cast<int>(a.wd), wb = static_cast<int>(a.wb);
    const int W = wx + wd + 2 * wb;
    for (int j = blockIdx.x; j < a.Q; j += gridDim.x) {
        for (int o = threadIdx.x; o < W; o += kEmulThreads) {
            const Word* tok;   // the new token's row
            Word* buf;         // the slot's chunk buffer, token 0
            Word* ws;          // the batch-ordered scan input, token 0
            int e = o, width;
            if (e < wx) {
                tok = static_cast<const Word*>(a.x) + r * wx;
                buf = static_cast<Word*>(a.x_buf);
                ws = static_cast<Word*>(a.xw);
                width = wx;
            } else if ((e -= wx) < wd) {
                tok = reinterpret_cast<const Word*>(a.dt) + r * wd;
                buf = reinterpret_cast<Word*>(a.dt_buf);
                ws = reinterpret_cast<Word*>(a.dtw);
                width = wd;
            } else if ((e -= wd) < wb) {
                tok = static_cast<const Word*>(a.B) + r * wb;
                buf = static_cast<Word*>(a.b_buf);
                ws = static_cast<Word*>(a.bw);
                width = wb;
            } else {
                e -= wb;
                tok = static_cast<const Word*>(a.C) + r * wb;
                buf = static_cast<Word*>(a.c_buf);
                ws = static_cast<Word*>(a.cw);
                width = wb;
            }
            Word v = Word{};
            if (live) {
                Word* slot = buf + (s * a.Q + j) * width + e;
                if (j == i) {
                    v = tok[e];
                    *slot = v;
                } else if (j < i) {
                    v = *slot;
                }
            }
            ws[(r * a.Q + j) * width + e] = v;
        }
    }
}

__global__ __launch_bounds__(kEmulThreads) void emul_finish_kernel(EmulArgs a) {
    const int64_t r = blockIdx.y;
    int64_t s;
    int i;
    if (!emul_row(a, r, s, i)) return;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kEmulThreads;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kEmulThreads + threadIdx.x;
    const uint32_t* yw = static_cast<const uint32_t*>(a.yw) + (r * a.Q + i) * a.wx;
    uint32_t* y = static_cast<uint32_t*>(a.y) + r * a.wx;
    for (int64_t w = t0; w < a.wx; w += stride) y[w] = yw[w];
    if (i == a.Q - 1) {
        const float4* src = reinterpret_cast<const float4*>(a.states + r * a.hpn);
        float4* dst = reinterpret_cast<float4*>(a.state_cache + s * a.hpn);
        for (int64_t w = t0; w < a.hpn / 4; w += stride) dst[w] = src[w];
    }
}

}  // namespace

hipError_t launch_emul_stage(const EmulArgs& a, bool wide, int64_t b, hipStream_t st) {
    if (b == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.Q), static_cast<unsigned>(b));
    if (wide) return dispatch(emul_stage_kernel<uint4>, grid, dim3(kEmulThreads), st, a);
    return dispatch(emul_stage_kernel<uint32_t>, grid, dim3(kEmulThreads), st, a);
}

hipError_t launch_emul_finish(const EmulArgs& a, int64_t b, hipStream_t st) {
    if (b == 0) return hipSuccess;
    return dispatch(emul_finish_kernel, dim3(64, static_cast<unsigned>(b)), dim3(kEmulThreads), st, a);
}

}  // namespace ssd
