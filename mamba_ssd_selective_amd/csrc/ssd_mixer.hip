// ssd_mixer.hip -- the steps beside the scan in the Mamba-2 mixer on gfx950
// (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 3, Figure 2, box [F2]):
//   * causal depthwise conv1d, width 4, + bias + SiLU over the xBC channels,
//     with the conv-state cache, written straight into the scan's separate
//     x (b, L, nx), B and C (b, L, nb) buffers (no split copy);
//   * its one-token decode update;
//   * gated group RMSNorm of the scan's output: v = y * silu(z), per group of
//     channels v / sqrt(mean(v^2) + eps) * weight.
// With w[c][k] the taps (k = 3 the current token):
//   out_t[c] = silu(bias[c] + sum_k w[c][k] in_{t-3+k}[c]),
// inputs before token 0 from the conv state (oldest first) or zero, and with
// packed sequences an input of another sequence counts as zero (the state
// belongs to the sequence of token 0).  The new conv state holds the last three
// inputs, zero where they belong to another sequence than the last token's.
// All three kernels are bandwidth-bound elementwise / stencil passes: each
// thread moves 16-byte vectors of 8 channels (bf16) and keeps its weights and
// the sliding window in registers.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kConvW = 4;        // taps (the pages' mamba_d_conv)
constexpr int kConvTile = 32;    // tokens per thread of the prefill kernel
constexpr int kConvStep = 8;     // tokens whose loads are in flight together
constexpr int kMixThreads = 256;

template <typename T> struct V8;
template <> struct V8<uint16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = u; }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
        return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
    __device__ __forceinline__ void set(const float (&v)[8]) {
        u = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
    }
};
template <> struct V8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void store(float* p) const {
        *reinterpret_cast<float4*>(p) = a;
        *reinterpret_cast<float4*>(p + 4) = b;
    }
    __device__ __forceinline__ float get(int e) const {
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        return v[e];
    }
    __device__ __forceinline__ void set(const float (&v)[8]) {
        a = make_float4(v[0], v[1], v[2], v[3]);
        b = make_float4(v[4], v[5], v[6], v[7]);
    }
};

// v * sigmoid(v) with the reciprocal instruction (these kernels are bound by
// their VALU work, and an IEEE divide costs several times more)
__device__ __forceinline__ float silu_f32(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// Destination of channels c0 .. c0+7 of token row `row` (row = b * L + t).
template <typename T>
__device__ __forceinline__ T* conv_dst(const ConvArgs& a, int64_t row, int c0) {
    if (c0 < a.nx) return static_cast<T*>(a.x_out) + row * a.nx + c0;
    if (c0 < a.nx + a.nb) return static_cast<T*>(a.b_out) + row * a.nb + (c0 - a.nx);
    return static_cast<T*>(a.c_out) + row * a.nb + (c0 - a.nx - a.nb);
}

// One thread: 8 channels, kConvTile consecutive tokens of one row.  kSeq: the
// row packs sequences (the masks are compiled only into that form).
template <typename T, bool kSeq>
__global__ __launch_bounds__(kMixThreads) void conv1d_fwd_kernel(ConvArgs a) {
    const int cg = static_cast<int>(blockIdx.x) * kMixThreads + static_cast<int>(threadIdx.x);
    const int c0 = 8 * cg;
    if (c0 >= a.dim) return;
    const int64_t b = blockIdx.z;
    const int64_t L = a.L;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kConvTile;
    const T* src = static_cast<const T*>(a.xbc);
    const int64_t rowb = b * L;
    const int32_t* seq = kSeq ? a.seq_idx + rowb : nullptr;
    float w[8][kConvW], bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float4 wv = *reinterpret_cast<const float4*>(a.weight + (c0 + e) * kConvW);
        w[e][0] = wv.x; w[e][1] = wv.y; w[e][2] = wv.z; w[e][3] = wv.w;
        bias[e] = a.bias ? a.bias[c0 + e] : 0.0f;
    }
    // window of the three inputs before token t: values and sequence ids
    // (state inputs carry the sequence of token 0)
    float win[3][8];
    int wseq[3];
    const int seq0 = seq ? seq[0] : 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int64_t j = t0 - 3 + k;
        if (j >= 0) {
            V8<T> v;
            v.load(src + (rowb + j) * a.dim + c0);
#pragma unroll
            for (int e = 0; e < 8; ++e) win[k][e] = v.get(e);
            wseq[k] = seq ? seq[j] : 0;
        } else {
            const int slot = static_cast<int>(j + 3);  // state slot, oldest first
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float sv = 0.0f;
                if (a.state_in) {
                    const T* sp = static_cast<const T*>(a.state_in) + (b * a.dim + c0 + e) * 3 + slot;
                    if constexpr (sizeof(T) == 2) sv = bf16_to_f32(*sp);
                    else sv = *reinterpret_cast<const float*>(sp);
                }
                win[k][e] = sv;
            }
            wseq[k] = seq0;
        }
    }
    // the new conv state: read here, before any thread writes it (the first
    // tile's block reads the old state, so the two may be the same buffer)
    if (a.state_out && t0 == 0) {
        const int seq_last = seq ? seq[L - 1] : 0;
        float ns[3][8];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int64_t j = L - 3 + k;  // token of slot k (negative: old state slot j + 3)
            bool keep = true;
            if (j >= 0) {
                V8<T> v;
                v.load(src + (rowb + j) * a.dim + c0);
#pragma unroll
                for (int e = 0; e < 8; ++e) ns[k][e] = v.get(e);
                keep = !seq || seq[j] == seq_last;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float sv = 0.0f;
                    if (a.state_in) {
                        const T* sp = static_cast<const T*>(a.state_in) + (b * a.dim + c0 + e) * 3 + (j + 3);
                        if constexpr (sizeof(T) == 2) sv = bf16_to_f32(*sp);
                        else sv = *reinterpret_cast<const float*>(sp);
                    }
                    ns[k][e] = sv;
                }
                keep = !seq || seq0 == seq_last;
            }
            if (!keep)
#pragma unroll
                for (int e = 0; e < 8; ++e) ns[k][e] = 0.0f;
        }
        // every read of the old state by this thread is above; other blocks
        // read only the inputs
        T* so = static_cast<T*>(a.state_out);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                T* d = so + (b * a.dim + c0 + e) * 3 + k;
                if constexpr (sizeof(T) == 2) *d = f32_to_bf16(ns[k][e]);
                else *reinterpret_cast<float*>(d) = ns[k][e];
            }
    }
    const int64_t tend = t0 + kConvTile < L ? t0 + kConvTile : L;
    T* const dst0 = conv_dst<T>(a, rowb, c0);
    const int64_t dstride = c0 < a.nx ? a.nx : a.nb;  // elements between token rows of the output
    // kConvStep tokens at a time: their loads are issued together
#pragma unroll
    for (int64_t tb = t0; tb < t0 + kConvTile; tb += kConvStep) {
        V8<T> cur[kConvStep];
        int sq[kConvStep];
#pragma unroll
        for (int u = 0; u < kConvStep; ++u) {
            const int64_t t = tb + u < tend ? tb + u : tend - 1;
            cur[u].load(src + (rowb + t) * a.dim + c0);
            sq[u] = seq ? seq[t] : 0;
        }
#pragma unroll
        for (int u = 0; u < kConvStep; ++u) {
            if (tb + u < tend) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // the same fused order as the decode update: bias, current
                    // token, then the three earlier inputs oldest first
                    // (another sequence's count as 0)
                    float acc = fmaf(w[e][3], cur[u].get(e), bias[e]);
#pragma unroll
                    for (int k = 0; k < 3; ++k)
                        acc = fmaf(w[e][k], (!kSeq || wseq[k] == sq[u]) ? win[k][e] : 0.0f, acc);
                    o[e] = silu_f32(acc);
                }
                V8<T> ov;
                ov.set(o);
                ov.store(dst0 + (tb + u) * dstride);
            }
            // slide the window
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                win[0][e] = win[1][e];
                win[1][e] = win[2][e];
                win[2][e] = cur[u].get(e);
            }
            wseq[0] = wseq[1];
            wseq[1] = wseq[2];
            wseq[2] = sq[u];
        }
    }
}

// One decode token per row: xbc (b, dim), conv_state (b, dim, 3) updated in place.
template <typename T>
__global__ __launch_bounds__(kMixThreads) void conv1d_update_kernel(ConvArgs a) {
    const int cg = static_cast<int>(blockIdx.x) * kMixThreads + static_cast<int>(threadIdx.x);
    const int c0 = 8 * cg;
    if (c0 >= a.dim) return;
    const int64_t b = blockIdx.y;
    int64_t sb = b;  // the conv-state cache row of batch row b (padding rows: skipped)
    if (a.state_idx) {
        sb = a.state_idx[b];
        if (sb < 0 || sb >= a.cache_rows) return;
    }
    V8<T> cur;
    cur.load(static_cast<const T*>(a.xbc) + b * a.dim + c0);
    T* st = static_cast<T*>(a.state_out) + sb * a.dim * 3;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float4 wv = *reinterpret_cast<const float4*>(a.weight + (c0 + e) * kConvW);
        T* sp = st + (c0 + e) * 3;
        float s[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if constexpr (sizeof(T) == 2) s[k] = bf16_to_f32(sp[k]);
            else s[k] = reinterpret_cast<const float*>(sp)[k];
        }
        const float x = cur.get(e);
        float acc = fmaf(wv.w, x, a.bias ? a.bias[c0 + e] : 0.0f);
        acc = fmaf(wv.x, s[0], acc);
        acc = fmaf(wv.y, s[1], acc);
        acc = fmaf(wv.z, s[2], acc);
        o[e] = silu_f32(acc);
        const float ns[3] = {s[1], s[2], x};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if constexpr (sizeof(T) == 2) sp[k] = f32_to_bf16(ns[k]);
            else reinterpret_cast<float*>(sp)[k] = ns[k];
        }
    }
    V8<T> ov;
    ov.set(o);
    ov.store(conv_dst<T>(a, b, c0));
}

// Groups of 512 channels: one wave per kNormUnits consecutive (row, group)
// units, all their loads issued before any arithmetic; each unit as below.
constexpr int kNormUnits = 2;
template <typename T>
__global__ __launch_bounds__(kMixThreads) void gated_rmsnorm512_kernel(NormArgs a) {
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int64_t groups = a.dim / 512;
    const int64_t total = a.rows * groups;
    const int64_t unit0 = (static_cast<int64_t>(blockIdx.x) * (kMixThreads / kWave) +
                           static_cast<int64_t>(threadIdx.x) / kWave) * kNormUnits;
    if (unit0 >= total) return;
    V8<T> y[kNormUnits], z[kNormUnits];
#pragma unroll
    for (int u = 0; u < kNormUnits; ++u) {
        const int64_t unit = unit0 + u < total ? unit0 + u : total - 1;
        const int64_t base = (unit / groups) * a.dim + (unit % groups) * 512 + 8 * lane;
        y[u].load(static_cast<const T*>(a.y) + base);
        z[u].load(static_cast<const T*>(a.z) + base);
    }
#pragma unroll
    for (int u = 0; u < kNormUnits; ++u) {
        const int64_t unit = unit0 + u;
        if (unit >= total) break;
        const int gq = static_cast<int>(unit % groups);
        const int64_t base = (unit / groups) * a.dim + static_cast<int64_t>(gq) * 512 + 8 * lane;
        float v[8];
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = y[u].get(e) * silu_f32(z[u].get(e));
            ss += v[e] * v[e];
        }
        ss = wave_sum(ss);
        const float rstd = rsqrtf(ss / 512.0f + a.eps);
        const int64_t ch = static_cast<int64_t>(gq) * 512 + 8 * lane;
        const float4 w0 = *reinterpret_cast<const float4*>(a.weight + ch);
        const float4 w1 = *reinterpret_cast<const float4*>(a.weight + ch + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[e] * rstd * wv[e];
        V8<T> ov;
        ov.set(o);
        ov.store(static_cast<T*>(a.out) + base);
    }
}

// One wave per (row, group of channels); a lane holds 8 channels per 512.
template <typename T>
__global__ __launch_bounds__(kMixThreads) void gated_rmsnorm_kernel(NormArgs a) {
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int64_t unit = static_cast<int64_t>(blockIdx.x) * (kMixThreads / kWave) +
                         static_cast<int64_t>(threadIdx.x) / kWave;
    const int64_t groups = a.dim / a.group;
    if (unit >= a.rows * groups) return;
    const int64_t row = unit / groups;
    const int gq = static_cast<int>(unit % groups);
    const int64_t base = row * a.dim + static_cast<int64_t>(gq) * a.group;
    constexpr int kMaxPass = 8;  // groups of up to 4096 channels
    float v[kMaxPass][8];
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxPass; ++q) {
        const int c = 512 * q + 8 * lane;
        if (c < a.group) {
            V8<T> y, z;
            y.load(static_cast<const T*>(a.y) + base + c);
            z.load(static_cast<const T*>(a.z) + base + c);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[q][e] = y.get(e) * silu_f32(z.get(e));
                ss += v[q][e] * v[q][e];
            }
        }
    }
    ss = wave_sum(ss);
    const float rstd = rsqrtf(ss / static_cast<float>(a.group) + a.eps);
#pragma unroll
    for (int q = 0; q < kMaxPass; ++q) {
        const int c = 512 * q + 8 * lane;
        if (c < a.group) {
            const int64_t ch = static_cast<int64_t>(gq) * a.group + c;
            const float4 w0 = *reinterpret_cast<const float4*>(a.weight + ch);
            const float4 w1 = *reinterpret_cast<const float4*>(a.weight + ch + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = v[q][e] * rstd * wv[e];
            V8<T> ov;
            ov.set(o);
            ov.store(static_cast<T*>(a.out) + base + c);
        }
    }
}

}  // namespace

hipError_t launch_conv1d_fwd(int io, const ConvArgs& a, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((a.dim / 8 + kMixThreads - 1) / kMixThreads),
                    static_cast<unsigned>((a.L + kConvTile - 1) / kConvTile), static_cast<unsigned>(a.batch));
    if (io == 1) {
        if (a.seq_idx) return dispatch(conv1d_fwd_kernel<uint16_t, true>, grid, dim3(kMixThreads), st, a);
        return dispatch(conv1d_fwd_kernel<uint16_t, false>, grid, dim3(kMixThreads), st, a);
    }
    if (a.seq_idx) return dispatch(conv1d_fwd_kernel<float, true>, grid, dim3(kMixThreads), st, a);
    return dispatch(conv1d_fwd_kernel<float, false>, grid, dim3(kMixThreads), st, a);
}

hipError_t launch_conv1d_update(int io, const ConvArgs& a, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((a.dim / 8 + kMixThreads - 1) / kMixThreads),
                    static_cast<unsigned>(a.batch));
    if (io == 1) return dispatch(conv1d_update_kernel<uint16_t>, grid, dim3(kMixThreads), st, a);
    return dispatch(conv1d_update_kernel<float>, grid, dim3(kMixThreads), st, a);
}

hipError_t launch_gated_rmsnorm(int io, const NormArgs& a, hipStream_t st) {
    const int64_t units = a.rows * (a.dim / a.group);
    const int per_block = kMixThreads / kWave;
    if (a.group == 512) {
        const int64_t per = static_cast<int64_t>(per_block) * kNormUnits;
        const dim3 g512(static_cast<unsigned>((units + per - 1) / per));
        if (io == 1) return dispatch(gated_rmsnorm512_kernel<uint16_t>, g512, dim3(kMixThreads), st, a);
        return dispatch(gated_rmsnorm512_kernel<float>, g512, dim3(kMixThreads), st, a);
    }
    const dim3 grid(static_cast<unsigned>((units + per_block - 1) / per_block));
    if (io == 1) return dispatch(gated_rmsnorm_kernel<uint16_t>, grid, dim3(kMixThreads), st, a);
    return dispatch(gated_rmsnorm_kernel<float>, grid, dim3(kMixThreads), st, a);
}

}  // namespace ssd
