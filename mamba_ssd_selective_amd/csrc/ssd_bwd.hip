// ssd_bwd.hip -- gradients of the chunked SSD scan on gfx950 (bf16 x, B, C and
// dy; fp32 dt, A, D and states; P = 64, N = 128, chunk Q = 128).
//
// Operation: the scan of ssd_kernels.hip (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B",
// section 1 operator families 1-2 and section 3 Figure 2 box [F2]: the chunked
// scan serves training, which needs its backward pass).  For chunk c of one
// (row, head), with cs the segmented chunk cumsum of a = dt*A, V the tokens of
// the chunk inside the sequence, seq_prev the sequence id of the token before
// the chunk and seq_last that of its last token:
//   kappa_i = [seq_i = seq_prev] exp(cs_i)             decay carried into token i
//   omega_j = [seq_j = seq_last] exp(cs_last - cs_j)   decay from token j to the end
//   e_c     = [seq_last = seq_prev] exp(cs_last)
//   L_ij    = [j <= i][seq_i = seq_j] exp(cs_i - cs_j)
// the forward pass is
//   y_i   = sum_j (C_i.B_j) L_ij dt_j x_j + kappa_i h_in C_i + D x_i
//   h_out = e_c h_in + sum_j omega_j dt_j x_j (outer) B_j.
// With g_out the gradient of the loss with respect to h_out (from later chunks,
// or the final-state gradient) and dy the gradient with respect to y:
//   g_in    = e_c g_out + sum_i kappa_i dy_i (outer) C_i            (into h_in)
//   u_j     = sum_i (C_i.B_j) L_ij dy_i + omega_j g_out B_j          (= g_j B_j)
//   dx_j    = dt_j u_j + D dy_j
//   dB_j    = sum over the group's heads of dt_j [sum_i L_ij (dy_i.x_j) C_i + omega_j g_out^T x_j]
//   dC_i    = sum over the group's heads of sum_j L_ij dt_j (dy_i.x_j) B_j + kappa_i h_in^T dy_i
//   d(dt_j) = x_j.u_j + A d(a_j),  d(a_k) = sum of dcs_i over i >= k in k's sequence run
//   dcs_i   = sum_j M_ij - sum_j M_ji + kappa_i dy_i.(h_in C_i) - T_i
//             (+ sum_j T_j + e_c <g_out, h_in> at the last token of the chunk)
//   with M_ij = (C_i.B_j) L_ij dt_j (dy_i.x_j) and T_j = omega_j dt_j x_j.(g_out B_j);
//   dA = sum dt_k d(a_k), dD = sum dy.x, d(h_init) = g_in of chunk 0, and
//   d(dt_raw) = d(dt) [not clamped] (sigmoid(dt_raw + dt_bias) with softplus).
// Every term is local to its chunk once h_in and g_out are known.
//
// Kernels (one backward call):
//   bwd_states_kernel   the two chains of states, both directions in one
//        launch: forward, the states h_in of every chunk in chunk order
//        (h <- e_c h + sum_j omega_j dt_j x_j B_j^T); backward, g_out of every
//        chunk (g <- e_c g + sum_i kappa_i dy_i C_i^T), whose last state is
//        d(h_init); each walk loads the next chunk during the current one.
//        With few rows x heads the walks are cut into segments, as the
//        forward scan's: bwd_seg_ends_kernel walks every segment but the last
//        from zero to its end state, a pass over segments (state_pass_kernel)
//        turns those into each segment's incoming state, and
//        bwd_states_kernel walks the segments from there, one workgroup per
//        (direction, row, head, segment);
//   bwd_chunk_kernel          one workgroup per (row, chunk, group), the group's
//        heads in turn: every gradient above on bf16 MFMA, dB and dC summed over
//        the heads in registers (no atomics: deterministic);
//   bwd_reduce_kernel         dA, dD, d(dt_bias) from per-chunk partial sums in a
//        fixed order.
// The per-token metadata (cs, dt, weights) comes from chunk_prep_kernel.
//
// Operand conventions are those of ssd_scan_tr.hip: MFMA 16x16x32 bf16, lane
// (r16, g = lane / 16); k over tokens (transposing reads) in the order element
// e < 4: token 32s + 4g + e, e >= 4: token 32s + 16 + 4g + (e - 4); k over a
// contiguous dimension read plainly: element e is 32s + 8g + e.  Products whose
// operands are both read with k over tokens use the token order on both sides.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_lds.h"
#include "ssd_work.h"

namespace ssd {
namespace {

// Compiled shapes: P = 64, Q = 128, N (the state size) a template parameter
// of the kernels, 128 or 64.
constexpr int kBP = 64, kBQ = 128;
constexpr int kBWaves = 8;
constexpr int kBThreads = kBWaves * kWave;
constexpr int kRowX = 2 * kBP;   // bytes of a token row of an x / dy tile
constexpr int kRowT = 2 * kBQ;   // bytes of a row of a Q x Q matrix
// bytes of a token row of a B / C tile, and of a state row, for state size N
template <int N>
struct BwdN {
    static_assert(N == 64 || N == 128, "compiled state sizes");
    static constexpr int RB = 2 * N;
    static constexpr int NNB = N / 16;        // 16-wide n blocks
    static constexpr int SP = N / 8;          // 16-byte pieces of a state row
    static constexpr int GP = kBP * SP / kBThreads;  // a state's pieces per thread
    static_assert(kBP * SP % kBThreads == 0, "whole rounds");
};

// ------------------------------------------------------------------ helpers

// 16-byte pieces of a [rows][ROW bytes] bf16 tile from global rows (stride
// gstride bytes, `valid` rows inside the sequence, the rest zero) into LDS in
// the swizzled layout of tr_off; all threads of the workgroup take part.
template <int ROW, int ROWS>
__device__ __forceinline__ void stage_rows(char* lds, const char* src, int64_t gstride, int valid) {
    constexpr int SPR = ROW / 16;
    constexpr int PIECES = ROWS * SPR;
#pragma unroll
    for (int k = 0; k < (PIECES + kBThreads - 1) / kBThreads; ++k) {
        const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
        if (q < PIECES) {
            const int r = q / SPR, slot = q % SPR;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r < valid) v = *reinterpret_cast<const uint4*>(src + r * gstride + slot * 16);
            lds_st<uint4>(lds, lds_addr(lds) + tr_off<ROW>(r, slot * 16), v);
        }
    }
}

// The same in two steps, so that several tiles' loads are in flight together:
// the 16-byte pieces of this thread (zeros past `valid` rows), then their LDS
// stores.
template <int ROW, int ROWS>
struct RowPieces {
    static constexpr int SPR = ROW / 16;
    static constexpr int K = ROWS * SPR / kBThreads;
    static_assert(ROWS * SPR % kBThreads == 0, "whole rounds");
    uint4 v[K];
};
template <int ROW, int ROWS>
__device__ __forceinline__ void load_rows(RowPieces<ROW, ROWS>& rp, const char* src, int64_t gstride,
                                          int valid) {
#pragma unroll
    for (int k = 0; k < RowPieces<ROW, ROWS>::K; ++k) {
        const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
        const int r = q / RowPieces<ROW, ROWS>::SPR, slot = q % RowPieces<ROW, ROWS>::SPR;
        rp.v[k] = make_uint4(0u, 0u, 0u, 0u);
        if (r < valid) rp.v[k] = *reinterpret_cast<const uint4*>(src + r * gstride + slot * 16);
    }
}
template <int ROW, int ROWS>
__device__ __forceinline__ void store_rows(char* lds, const RowPieces<ROW, ROWS>& rp) {
#pragma unroll
    for (int k = 0; k < RowPieces<ROW, ROWS>::K; ++k) {
        const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
        const int r = q / RowPieces<ROW, ROWS>::SPR, slot = q % RowPieces<ROW, ROWS>::SPR;
        lds_st<uint4>(lds, lds_addr(lds) + tr_off<ROW>(r, slot * 16), rp.v[k]);
    }
}

// Plain fragment: row R of a tile, k = 32s + 8g + e (16 contiguous bytes).
// `base` is the tile's LDS address; the chunk kernel passes it opaque (formed
// again for every head), so that no lane address is hoisted out of its loop.
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> row_frag(const char* tile, uint32_t base, int R, int s, int g) {
    return frag_of(lds_ld<uint4>(tile, base + tr_off<ROW>(R, 64 * s + 16 * g)));
}
// Row R of a tile with k over its columns in the token order (two 8-byte reads).
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> row_frag_tk(const char* tile, uint32_t base, int R, int s, int g) {
    const uint2 lo = lds_ld<uint2>(tile, base + tr_off<ROW>(R, 64 * s + 8 * g));
    const uint2 hi = lds_ld<uint2>(tile, base + tr_off<ROW>(R, 64 * s + 32 + 8 * g));
    return frag_of(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Column block mb of a tile whose rows are the k index (token order).
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> col_frag(const char* tile, uint32_t base, int mb, int s, int lane) {
    return tr_frag<ROW>(tile, base + tr_lane_off<ROW>(mb, lane), s);
}
// Lane bases for the read patterns above, so that a block or k step costs one
// XOR and an immediate offset (the swizzle of rows r, r + 16 and r + 32 is the
// same, and tile bases are 1 KB aligned):
//   col_base: transposing read of column block mb -> base ^ (mb << 5);
//   row_base: row 16 blk + r16, k step s -> (base ^ (s << 6)) + 16 blk ROW;
//   tk_base:  row R in token order, k step s -> halves base ^ (2s << 5) and
//             base ^ ((2s + 1) << 5); 8 bytes at column 32 m + 8g -> base ^ (m << 5).
template <int ROW>
__device__ __forceinline__ uint32_t col_base(uint32_t tile, int lane) {
    return tile + static_cast<uint32_t>(tr_lane_off<ROW>(0, lane));
}
template <int ROW>
__device__ __forceinline__ uint32_t row_base(uint32_t tile, int r16, int g) {
    return tile + static_cast<uint32_t>(tr_off<ROW>(r16, 16 * g));
}
template <int ROW>
__device__ __forceinline__ uint32_t tk_base(uint32_t tile, int R, int g) {
    return tile + static_cast<uint32_t>(tr_off<ROW>(R, 8 * g));
}
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> col_at(const char* tile, uint32_t cb, int mb, int s) {
    return tr_frag<ROW>(tile, cb ^ static_cast<uint32_t>(mb << 5), s);
}
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> row_at(const char* tile, uint32_t rb, int blk, int s) {
    return frag_of(lds_ld<uint4>(tile, (rb ^ static_cast<uint32_t>(s << 6)) + 16 * blk * ROW));
}
__device__ __forceinline__ Frag<uint16_t> tk_at(const char* tile, uint32_t tb, int s) {
    const uint2 lo = lds_ld<uint2>(tile, tb ^ static_cast<uint32_t>(s << 6));
    const uint2 hi = lds_ld<uint2>(tile, tb ^ static_cast<uint32_t>((2 * s + 1) << 5));
    return frag_of(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Token-order fragment elements scaled by per-token factors f[32s + ...].
__device__ __forceinline__ Frag<uint16_t> scale_tk(const Frag<uint16_t>& f, const float* fv, int s, int g) {
    const float4 w0 = *reinterpret_cast<const float4*>(fv + 32 * s + 4 * g);
    const float4 w1 = *reinterpret_cast<const float4*>(fv + 32 * s + 16 + 4 * g);
    return scale_frag(f, w0, w1);
}

// Four bf16 values (one accumulator) as 8 bytes.
__device__ __forceinline__ uint2 pack4(const f32x4_t& v) {
    return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Metadata block [cs Q | dt Q | w Q] of (row b, head h, chunk c) from a.cs.
__device__ __forceinline__ int64_t meta_offset_bwd(const BwdArgs& a, int64_t b, int h, int c) {
    return ((b * a.H + h) * a.nc + c) * static_cast<int64_t>(3 * kBQ);
}

__device__ __forceinline__ int seq_at(const int32_t* seq, int64_t row_base, int64_t t, int64_t L) {
    return seq ? seq[row_base + (t < L ? t : L - 1)] : 0;
}

// ------------------------------------------------------------ chain of states

// The state before every chunk (forward: h_in, chunk order) or the gradient
// after every chunk (backward: g_out, reverse chunk order), fp32 [p][n] in
// `states` at (row, head, chunk).  Wave w owns state rows n = 16w + 4g + r,
// column p = 16pb + r16 (the MFMA accumulator layout); with N = 64 waves
// 4-7 own no n block and only help with the copies.
// One walk covers the chunks k in [k_begin, k_end) of the walk order (chunk
// k, or nc - 1 - k backwards), starting from `init` (P x N, or zero):
//  kChunks = true:  the state before each of them is written to `states`;
//                   the walk that ends the chain writes d(h_init);
//  kChunks = false: only the state at the end is written, to `end`, and the
//                   product of the chunks' decays to *mult (a segment's part
//                   of the chain, for a pass over segments).
template <int N, bool kRev, bool kChunks>
__device__ __forceinline__ void bwd_states_walk(const BwdArgs& a, int64_t bh, int k_begin, int k_end,
                                                const float* init, float* end, float* mult,
                                                char* sV, char* sK, float* sW) {
    constexpr int kRowB = BwdN<N>::RB;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int r16 = lane & 15, g = lane >> 4;
    const bool owner = wave < BwdN<N>::NNB;  // owns n block `wave`
    const int64_t b = bh / a.H;
    const int h = static_cast<int>(bh % a.H);
    const int grp = h / (a.H / a.G);
    const int64_t L = a.L;
    const int64_t srow = b * L;

    f32x4_t st[kBP / 16];
#pragma unroll
    for (int pb = 0; pb < kBP / 16; ++pb) {
        st[pb] = acc_zero();
        if (init && owner) {
            const float4 v = *reinterpret_cast<const float4*>(init + (16 * pb + r16) * N +
                                                              16 * wave + 4 * g);
            st[pb] = f32x4_t{v.x, v.y, v.z, v.w};
        }
    }
    float prod = 1.0f;  // product of the decays (kChunks = false)
    const char* vsrc = static_cast<const char*>(kRev ? a.dy : a.x);
    const char* ksrc = static_cast<const char*>(kRev ? a.C : a.B);
    const int64_t vstride = static_cast<int64_t>(a.H) * kRowX;
    const int64_t kstride = static_cast<int64_t>(a.G) * kRowB;
    // chunk k of the walk: its tiles, this thread's token weight and the decay
    // e_c, all loaded into registers one chunk ahead
    struct Next {
        RowPieces<kRowX, kBQ> v;
        RowPieces<kRowB, kBQ> kr;
        float w, e;
    };
    auto fetch = [&](int k, Next& nx) {
        const int c = kRev ? a.nc - 1 - k : k;
        const int64_t t0 = static_cast<int64_t>(c) * kBQ;
        const int valid = static_cast<int>(L - t0 < kBQ ? L - t0 : kBQ);
        const float* meta = a.cs + meta_offset_bwd(a, b, h, c);
        const int seq_prev = seq_at(a.seq_idx, srow, t0 == 0 ? 0 : t0 - 1, L);
        const int seq_last = seq_at(a.seq_idx, srow, t0 + valid - 1, L);
        load_rows(nx.v, vsrc + ((srow + t0) * a.H + h) * kRowX, vstride, valid);
        load_rows(nx.kr, ksrc + ((srow + t0) * a.G + grp) * kRowB, kstride, valid);
        const int t = static_cast<int>(threadIdx.x);
        nx.w = 0.0f;
        if (t < valid) {
            if (kRev) {
                nx.w = seq_at(a.seq_idx, srow, t0 + t, L) == seq_prev ? decay_exp(meta[t]) : 0.0f;
            } else {
                nx.w = meta[2 * kBQ + t];  // omega_t dt_t from chunk_prep_kernel
            }
        }
        const float cs_last = meta[valid - 1];
        nx.e = seq_last == seq_prev ? decay_exp(cs_last) : 0.0f;
    };
    Next nx;
    if (k_begin < k_end) fetch(k_begin, nx);
    for (int k = k_begin; k < k_end; ++k) {
        const int c = kRev ? a.nc - 1 - k : k;
        if (kChunks && owner) {
            // the state before this chunk's update, as bf16 [p][n]
            uint16_t* dst = (kRev ? a.gstates : a.states) + (bh * a.nc + c) * kBP * N;
#pragma unroll
            for (int pb = 0; pb < kBP / 16; ++pb)
                *reinterpret_cast<uint2*>(dst + (16 * pb + r16) * N + 16 * wave + 4 * g) =
                    make_uint2(pack_bf16x2(st[pb][0], st[pb][1]), pack_bf16x2(st[pb][2], st[pb][3]));
        }
        store_rows(sV, nx.v);
        store_rows(sK, nx.kr);
        if (threadIdx.x < kBQ) sW[threadIdx.x] = nx.w;
        const float e = nx.e;
        prod *= e;
        __syncthreads();
        if (k + 1 < k_end) fetch(k + 1, nx);  // in flight during this chunk's products
        const uint32_t bsK = lds_keep(lds_addr(sK)), bsV = lds_keep(lds_addr(sV));
        if (owner) {
#pragma unroll
            for (int pb = 0; pb < kBP / 16; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[pb][r] *= e;
#pragma unroll
            for (int s = 0; s < kBQ / 32; ++s) {
                const Frag<uint16_t> kf = scale_tk(col_frag<kRowB>(sK, bsK, wave, s, lane), sW, s, g);
#pragma unroll
                for (int pb = 0; pb < kBP / 16; ++pb) mma(st[pb], kf, col_frag<kRowX>(sV, bsV, pb, s, lane));
            }
        }
        __syncthreads();
    }
    if (end && owner) {
#pragma unroll
        for (int pb = 0; pb < kBP / 16; ++pb)
            *reinterpret_cast<float4*>(end + (16 * pb + r16) * N + 16 * wave + 4 * g) =
                make_float4(st[pb][0], st[pb][1], st[pb][2], st[pb][3]);
    }
    if (!kChunks && mult && threadIdx.x == 0) *mult = prod;
}

// Work item of a walk workgroup: (direction, row, head, segment) with the
// heads of a B/C group fastest, then the group, the segment, the row and the
// direction; the XCD-aware order then gives the workgroups that share a
// group's B (or C) rows the same L2.
struct WalkItem {
    int dir, seg;
    int64_t bh;
};
__device__ __forceinline__ WalkItem walk_item(const BwdArgs& a, int nseg_grid) {
    uint32_t w = static_cast<uint32_t>(xcd_work_index(blockIdx.x, gridDim.x));
    const uint32_t hpg = static_cast<uint32_t>(a.H / a.G);
    const uint32_t hh = w % hpg;
    w /= hpg;
    const uint32_t g = w % static_cast<uint32_t>(a.G);
    w /= static_cast<uint32_t>(a.G);
    WalkItem it;
    it.seg = static_cast<int>(w % static_cast<uint32_t>(nseg_grid));
    w /= static_cast<uint32_t>(nseg_grid);
    const int64_t b = w % static_cast<uint32_t>(a.batch);
    it.dir = static_cast<int>(w / static_cast<uint32_t>(a.batch));
    it.bh = b * a.H + g * hpg + hh;
    return it;
}

// Segment ends of the walks (nseg > 1): one workgroup per (direction, row,
// head, segment s < nseg - 1); each segment from a zero state.
template <int N>
__global__ __launch_bounds__(kBThreads) void bwd_seg_ends_kernel(BwdArgs a) {
    constexpr int kRowB = BwdN<N>::RB;
    __shared__ __attribute__((aligned(1024))) char sV[kBQ * kRowX];
    __shared__ __attribute__((aligned(1024))) char sK[kBQ * kRowB];
    __shared__ __attribute__((aligned(16))) float sW[kBQ];
    const int64_t nbh = static_cast<int64_t>(a.batch) * a.H;
    const WalkItem it = walk_item(a, a.nseg - 1);
    const int dir = it.dir, seg = it.seg;
    const int64_t bh = it.bh;
    const int k0 = seg * a.cps, k1 = min(k0 + a.cps, a.nc);
    const int64_t slot = (dir * nbh + bh) * a.nseg + seg;
    float* end = a.seg_end + slot * kBP * N;
    float* mult = a.seg_mult + slot;
    if (dir == 0) bwd_states_walk<N, false, false>(a, bh, k0, k1, nullptr, end, mult, sV, sK, sW);
    else bwd_states_walk<N, true, false>(a, bh, k0, k1, nullptr, end, mult, sV, sK, sW);
}

// Both walks in one launch (they are independent): one workgroup per
// (direction, row, head, segment), ordered as walk_item says.  A segment starts
// from its incoming state (after the pass over segment ends), the first from
// h_init (forward) or d(final states) (backward); the backward walk's last
// segment ends in d(h_init).
template <int N>
__global__ __launch_bounds__(kBThreads) void bwd_states_kernel(BwdArgs a) {
    constexpr int kRowB = BwdN<N>::RB;
    __shared__ __attribute__((aligned(1024))) char sV[kBQ * kRowX];   // x or dy rows
    __shared__ __attribute__((aligned(1024))) char sK[kBQ * kRowB];   // B or C rows
    __shared__ __attribute__((aligned(16))) float sW[kBQ];            // per-token weights
    const int64_t nbh = static_cast<int64_t>(a.batch) * a.H;
    const WalkItem it = walk_item(a, a.nseg);
    const int dir = it.dir, seg = it.seg;
    const int64_t bh = it.bh;
    const int k0 = seg * a.cps, k1 = min(k0 + a.cps, a.nc);
    const float* first = dir == 0 ? a.h_init : a.dh_final;
    const float* init = a.nseg > 1 ? a.seg_end + ((dir * nbh + bh) * a.nseg + seg) * kBP * N
                                   : (first ? first + bh * kBP * N : nullptr);
    float* dh0 = dir == 1 && seg == a.nseg - 1 && a.dh_init ? a.dh_init + bh * kBP * N : nullptr;
    if (dir == 0) bwd_states_walk<N, false, true>(a, bh, k0, k1, init, nullptr, nullptr, sV, sK, sW);
    else bwd_states_walk<N, true, true>(a, bh, k0, k1, init, dh0, nullptr, sV, sK, sW);
}

// --------------------------------------------------------- per-chunk gradients

// Sum over the 16 lanes of a 16-lane row (same g).
__device__ __forceinline__ float sum16(float v) { return row16_sum(v); }
// Sum over the 4 lane groups g with the same r16.
__device__ __forceinline__ float sum_g(float v) { return add_lane_xor32(add_lane_xor16(v)); }
__device__ __forceinline__ float sum64(float v) { return wave_sum(v); }
// Workgroup sum (fixed order); every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = sum64(v);
    const int wave = static_cast<int>(threadIdx.x) / kWave;
    if ((threadIdx.x % kWave) == 0) red[wave] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kBWaves; ++w) t += red[w];
    __syncthreads();
    return t;
}

// One head's inputs of the gradient kernel, held in registers from their
// loads to their LDS stores: x and dy rows, g_out (bf16), and this thread's
// token of the metadata and of dt_raw.
template <int N>
struct HeadInputs {
    RowPieces<kRowX, kBQ> px, pdy;
    uint4 gq[BwdN<N>::GP];
    float m_cs, m_dt, m_raw;
};

template <int N>
__global__ __launch_bounds__(kBThreads) void bwd_chunk_kernel(BwdArgs a) {
    constexpr int kRowB = BwdN<N>::RB;
    constexpr int NNB = BwdN<N>::NNB;  // n blocks of dB, dC and the states
    constexpr int SP = BwdN<N>::SP;    // 16-byte pieces of a state row
    constexpr int GP = BwdN<N>::GP;    // a state's pieces per thread
    __shared__ __attribute__((aligned(1024))) char sB[kBQ * kRowB];
    __shared__ __attribute__((aligned(1024))) char sC[kBQ * kRowB];
    __shared__ __attribute__((aligned(1024))) char sX[kBQ * kRowX];
    __shared__ __attribute__((aligned(1024))) char sDY[kBQ * kRowX];
    __shared__ __attribute__((aligned(1024))) char sT[kBQ * kRowT];
    __shared__ __attribute__((aligned(1024))) char sH[kBP * kRowB];
    // per-token values of the current head: chunk cumsum, dt, omega, kappa,
    // row sums of M (then dcs), per-row-block column sums of M, x.u, T_j,
    // kappa_i dy_i.(h_in C_i); sequence ids; block reductions
    __shared__ __attribute__((aligned(16))) float sCs[kBQ];
    __shared__ __attribute__((aligned(16))) float sDt[kBQ];
    __shared__ __attribute__((aligned(16))) float sOm[kBQ];
    __shared__ __attribute__((aligned(16))) float sKa[kBQ];
    __shared__ __attribute__((aligned(16))) float sRows[kBQ];
    __shared__ __attribute__((aligned(16))) float sCols[kBWaves * kBQ];
    __shared__ __attribute__((aligned(16))) float sDin[kBQ];
    __shared__ __attribute__((aligned(16))) float sTj[kBQ];
    __shared__ __attribute__((aligned(16))) float sCar[kBQ];
    __shared__ __attribute__((aligned(16))) float sRaw[kBQ];  // dt_raw of the head's tokens
    __shared__ __attribute__((aligned(16))) int sSeq[kBQ];
    __shared__ float sRed[kBWaves];

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int r16 = lane & 15, g = lane >> 4;
    // work item: group fastest, then chunk, then row
    int64_t w = blockIdx.x;
    const int grp = static_cast<int>(w % a.G);
    w /= a.G;
    const int c = static_cast<int>(w % a.nc);
    const int64_t b = w / a.nc;
    const int hpg = a.H / a.G;
    const int64_t L = a.L;
    const int64_t srow = b * L;
    const int64_t t0 = static_cast<int64_t>(c) * kBQ;
    const int valid = static_cast<int>(L - t0 < kBQ ? L - t0 : kBQ);
    const int seq_prev = seq_at(a.seq_idx, srow, t0 == 0 ? 0 : t0 - 1, L);
    const int seq_last = seq_at(a.seq_idx, srow, t0 + valid - 1, L);
    const int I = wave;  // row block (P1, P4) / column block (P2, P3) of this wave

    // ---- the group's B and C rows, and C.B^T (tiles (I, J <= I) of this wave)
    const int64_t bcstride = static_cast<int64_t>(a.G) * kRowB;
    stage_rows<kRowB, kBQ>(sB, static_cast<const char*>(a.B) + ((srow + t0) * a.G + grp) * kRowB, bcstride, valid);
    stage_rows<kRowB, kBQ>(sC, static_cast<const char*>(a.C) + ((srow + t0) * a.G + grp) * kRowB, bcstride, valid);
    for (int t = static_cast<int>(threadIdx.x); t < kBQ; t += kBThreads)
        sSeq[t] = seq_at(a.seq_idx, srow, t0 + t, L);
    __syncthreads();
    f32x4_t dBacc[NNB], dCacc[NNB];  // dB^T tiles (nb, J = wave), dC^T tiles (nb, I = wave)
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
        dBacc[nb] = acc_zero();
        dCacc[nb] = acc_zero();
    }

    // loads of head hh's inputs, issued during the previous head's last
    // phases (an earlier issue keeps them in registers through the heaviest
    // phases, which then spill)
    auto load_head = [&](int hh, HeadInputs<N>& in) {
        const int h = grp * hpg + hh;
        const int64_t bh = b * a.H + h;
        const int64_t xstride = static_cast<int64_t>(a.H) * kRowX;
        load_rows(in.px, static_cast<const char*>(a.x) + ((srow + t0) * a.H + h) * kRowX, xstride, valid);
        load_rows(in.pdy, static_cast<const char*>(a.dy) + ((srow + t0) * a.H + h) * kRowX, xstride, valid);
        const uint16_t* gsrc = a.gstates + (bh * a.nc + c) * kBP * N;
#pragma unroll
        for (int k = 0; k < GP; ++k) {
            const int q = static_cast<int>(threadIdx.x) + kBThreads * k;  // 16-byte bf16 piece
            in.gq[k] = *reinterpret_cast<const uint4*>(gsrc + (q / SP) * N + 8 * (q % SP));
        }
        const float* meta = a.cs + meta_offset_bwd(a, b, h, c);
        const int tt = static_cast<int>(threadIdx.x);
        in.m_cs = in.m_dt = in.m_raw = 0.0f;
        if (tt < kBQ) {
            in.m_cs = meta[tt];
            in.m_dt = meta[kBQ + tt];
            if (tt < valid) in.m_raw = a.dt_raw[(srow + t0 + tt) * a.H + h];
        }
    };
    HeadInputs<N> nx;
    load_head(0, nx);

    for (int hh = 0; hh < hpg; ++hh) {
        // lane bases of this head's accesses (opaque: formed again per head)
        const uint32_t bsT = lds_keep(lds_addr(sT)), bsH = lds_keep(lds_addr(sH));
        const uint32_t rbX = lds_keep(row_base<kRowX>(lds_addr(sX), r16, g));
        const uint32_t rbDY = lds_keep(row_base<kRowX>(lds_addr(sDY), r16, g));
        const uint32_t rbB = lds_keep(row_base<kRowB>(lds_addr(sB), r16, g));
        const uint32_t rbC = lds_keep(row_base<kRowB>(lds_addr(sC), r16, g));
        const uint32_t rbH = lds_keep(row_base<kRowB>(lds_addr(sH), r16, g));
        const uint32_t cbDY = lds_keep(col_base<kRowX>(lds_addr(sDY), lane));
        const uint32_t cbB = lds_keep(col_base<kRowB>(lds_addr(sB), lane));
        const uint32_t cbC = lds_keep(col_base<kRowB>(lds_addr(sC), lane));
        const uint32_t cbH = lds_keep(col_base<kRowB>(lds_addr(sH), lane));
        const uint32_t cbT = lds_keep(col_base<kRowT>(lds_addr(sT), lane));
        // row 16 * wave + r16 (the j of P2, P3 and the i of P4) in token order
        const int rw = 16 * wave + r16;
        const uint32_t tkT = lds_keep(tk_base<kRowT>(lds_addr(sT), rw, g));
        const uint32_t tkX = lds_keep(tk_base<kRowX>(lds_addr(sX), rw, g));
        const uint32_t tkDY = lds_keep(tk_base<kRowX>(lds_addr(sDY), rw, g));
        const uint32_t tkC = lds_keep(tk_base<kRowB>(lds_addr(sC), rw, g));
        // S^T / W^T writes: row 16 J + r16, columns 16 I + 4g .. +3
        const uint32_t wT = lds_keep(tk_base<kRowT>(lds_addr(sT), r16, g) ^ static_cast<uint32_t>(I << 5));
        const int h = grp * hpg + hh;
        const int64_t bh = b * a.H + h;
        const float Ah = a.A[h];
        const float Dh = a.D ? a.D[h] : 0.0f;
        const float* meta = a.cs + meta_offset_bwd(a, b, h, c);
        const float cs_last = meta[valid - 1];
        const float e = seq_last == seq_prev ? decay_exp(cs_last) : 0.0f;
        // ---- head inputs (loaded during the previous head)
        const uint16_t* hsrc = a.states + (bh * a.nc + c) * kBP * N;
        const int tt = static_cast<int>(threadIdx.x);
        const float m_cs = nx.m_cs;
        store_rows(sX, nx.px);
        store_rows(sDY, nx.pdy);
        if (tt < kBQ) {
            sCs[tt] = m_cs;
            sDt[tt] = nx.m_dt;
            sRaw[tt] = nx.m_raw;
            const bool in = tt < valid;
            sOm[tt] = in && sSeq[tt] == seq_last ? decay_exp(cs_last - m_cs) : 0.0f;
            sKa[tt] = in && sSeq[tt] == seq_prev ? decay_exp(m_cs) : 0.0f;
        }
        // g_out as the bf16 operand
#pragma unroll
        for (int k = 0; k < GP; ++k) {
            const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
            lds_st<uint4>(sH, bsH + tr_off<kRowB>(q / SP, 16 * (q % SP)), nx.gq[k]);
        }
        __syncthreads();

        // ---- P1: tiles (I, J <= I) of M1 = dY X^T and C.B^T (rows i of block I);
        // S = CB L, M = S dt_j M1; row sums of M, column-sum partials, S^T to LDS
        float rsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float cs_i[4];
        int sq_i[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            cs_i[r] = sCs[16 * I + 4 * g + r];
            sq_i[r] = sSeq[16 * I + 4 * g + r];
        }
        // L_ij of this lane's rows and column j
        auto decay_l = [&](int J, int r) {
            const int i = 16 * I + 4 * g + r, j = 16 * J + r16;
            return (j <= i && sq_i[r] == sSeq[j]) ? decay_exp(cs_i[r] - sCs[j]) : 0.0f;
        };
        auto m1_tile = [&](int J) {
            f32x4_t m1 = acc_zero();
#pragma unroll
            for (int ks = 0; ks < kBP / 32; ++ks)
                mma(m1, row_at<kRowX>(sDY, rbDY, I, ks), row_at<kRowX>(sX, rbX, J, ks));
            return m1;
        };
        for (int J = 0; J < 8; ++J) {
            f32x4_t sv = acc_zero();
            float csum = 0.0f;
            if (J <= I) {
                const f32x4_t m1 = m1_tile(J);
                f32x4_t cbt = acc_zero();
#pragma unroll
                for (int ks = 0; ks < N / 32; ++ks)
                    mma(cbt, row_at<kRowB>(sC, rbC, I, ks), row_at<kRowB>(sB, rbB, J, ks));
                const float dt_j = sDt[16 * J + r16];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[r] = cbt[r] * decay_l(J, r);
                    const float mv = sv[r] * dt_j * m1[r];
                    rsum[r] += mv;
                    csum += mv;
                }
            }
            // S^T row j, columns i = 16I + 4g .. +3 (zeros right of the diagonal block)
            lds_st<uint2>(sT, wT + 16 * J * kRowT, pack4(sv));
            csum = sum_g(csum);
            if (g == 0) sCols[I * kBQ + 16 * J + r16] = csum;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = sum16(rsum[r]);
            if (r16 == 0) sRows[16 * I + 4 * g + r] = v;
        }
        __syncthreads();

        // ---- P2: u^T = (S^T dY)^T + omega (g_out B^T), columns j of block J = wave
        {
            const int J = wave;
            const int j = 16 * J + r16;
            f32x4_t ut[4], vt[4];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                ut[pb] = acc_zero();
                vt[pb] = acc_zero();
            }
#pragma unroll
            for (int ks = 0; ks < kBQ / 32; ++ks) {
                if (2 * ks + 1 >= J) {
                    const Frag<uint16_t> sf = tk_at(sT, tkT, ks);
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) mma(ut[pb], col_at<kRowX>(sDY, cbDY, pb, ks), sf);
                }
            }
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) {
                const Frag<uint16_t> bf = row_at<kRowB>(sB, rbB, J, ks);
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) mma(vt[pb], row_at<kRowB>(sH, rbH, pb, ks), bf);
            }
            const float om_j = sOm[j], dt_j = sDt[j];
            float din = 0.0f, tsum = 0.0f, dd = 0.0f;
            uint2 dxw[4];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                // row j, p = 16pb + 4g .. +3
                const uint2 xr = lds_ld<uint2>(sX, tkX ^ static_cast<uint32_t>(pb << 5));
                const uint2 yr = lds_ld<uint2>(sDY, tkDY ^ static_cast<uint32_t>(pb << 5));
                const float xv[4] = {bf_lo(xr.x), bf_hi(xr.x), bf_lo(xr.y), bf_hi(xr.y)};
                const float yv[4] = {bf_lo(yr.x), bf_hi(yr.x), bf_lo(yr.y), bf_hi(yr.y)};
                float dxv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float u = ut[pb][r] + om_j * vt[pb][r];
                    dxv[r] = dt_j * u + Dh * yv[r];
                    din += xv[r] * u;
                    tsum += xv[r] * vt[pb][r];
                    dd += xv[r] * yv[r];
                }
                dxw[pb] = make_uint2(pack_bf16x2(dxv[0], dxv[1]), pack_bf16x2(dxv[2], dxv[3]));
            }
            if (j < valid) {
                uint16_t* dxp = static_cast<uint16_t*>(a.dx) + ((srow + t0 + j) * a.H + h) * kBP + 4 * g;
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) *reinterpret_cast<uint2*>(dxp + 16 * pb) = dxw[pb];
            }
            din = sum_g(din);
            tsum = sum_g(tsum);
            if (g == 0) {
                sDin[j] = din;
                sTj[j] = om_j * dt_j * tsum;
            }
            dd = sum64(dd);
            if (lane == 0) sRed[wave] = dd;
        }
        __syncthreads();
        float dD_part = 0.0f;
#pragma unroll
        for (int q = 0; q < kBWaves; ++q) dD_part += sRed[q];

        // ---- W'^T over S^T: W'_ij = M1_ij L_ij dt_j (M1 formed again); both of
        // its products need W scaled by dt of its column
        for (int J = 0; J < 8; ++J) {
            f32x4_t wv = acc_zero();
            if (J <= I) {
                const f32x4_t m1 = m1_tile(J);
                const float dt_j = sDt[16 * J + r16];
#pragma unroll
                for (int r = 0; r < 4; ++r) wv[r] = m1[r] * decay_l(J, r) * dt_j;
            }
            lds_st<uint2>(sT, wT + 16 * J * kRowT, pack4(wv));
        }
        __syncthreads();

        // h_in's loads, in flight during P3 (its first use is after P3)
        uint4 hq[GP];
#pragma unroll
        for (int k = 0; k < GP; ++k) {
            const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
            hq[k] = *reinterpret_cast<const uint4*>(hsrc + (q / SP) * N + 8 * (q % SP));
        }
        // ---- P3: dB^T += C^T W' + dt_j omega_j g_out^T X^T, columns j of block J = wave
        {
            const int J = wave;
            const int j = 16 * J + r16;
            const float dt_j = sDt[j], om_j = sOm[j];
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                f32x4_t a1 = acc_zero(), a2 = acc_zero();
#pragma unroll
                for (int ks = 0; ks < kBQ / 32; ++ks)
                    if (2 * ks + 1 >= J) mma(a1, col_at<kRowB>(sC, cbC, nb, ks), tk_at(sT, tkT, ks));
#pragma unroll
                for (int ks = 0; ks < kBP / 32; ++ks)
                    mma(a2, col_at<kRowB>(sH, cbH, nb, ks), tk_at(sX, tkX, ks));
#pragma unroll
                for (int r = 0; r < 4; ++r) dBacc[nb][r] += a1[r] + dt_j * om_j * a2[r];
                __builtin_amdgcn_sched_barrier(0);  // one n block's operands live at a time
            }
        }
        // <g_out, h_in> over their bf16 values (fp32 sums; g_out from its LDS
        // operand); then h_in replaces g_out as the bf16 operand
        float ghp = 0.0f;
#pragma unroll
        for (int k = 0; k < GP; ++k) {
            const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
            const int p = q / SP, slot = q % SP;
            const uint4 gv = lds_ld<uint4>(sH, bsH + tr_off<kRowB>(p, 16 * slot));
            const uint32_t hw[4] = {hq[k].x, hq[k].y, hq[k].z, hq[k].w};
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ghp += bf_lo(gw[e]) * bf_lo(hw[e]) + bf_hi(gw[e]) * bf_hi(hw[e]);
        }
        const float gh = block_sum(ghp, sRed);  // its barriers also end P3's reads of g_out
#pragma unroll
        for (int k = 0; k < GP; ++k) {
            const int q = static_cast<int>(threadIdx.x) + kBThreads * k;
            lds_st<uint4>(sH, bsH + tr_off<kRowB>(q / SP, 16 * (q % SP)), hq[k]);
        }
        __syncthreads();

        // the next head's inputs, in flight during P4 and the dcs pass
        if (hh + 1 < hpg) load_head(hh + 1, nx);
        // ---- P4: dC^T += B^T W'^T + kappa_i h_in^T dY^T, columns i of block I = wave
        {
            const int i = 16 * I + r16;
            const float ka_i = sKa[i];
            float car = 0.0f;
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                f32x4_t cw = acc_zero(), cc = acc_zero();
#pragma unroll
                for (int ks = 0; ks < kBQ / 32; ++ks)
                    if (2 * ks <= I)
                        mma(cw, col_at<kRowB>(sB, cbB, nb, ks), col_at<kRowT>(sT, cbT, I, ks));
#pragma unroll
                for (int ks = 0; ks < kBP / 32; ++ks)
                    mma(cc, col_at<kRowB>(sH, cbH, nb, ks), tk_at(sDY, tkDY, ks));
                const uint2 cr = lds_ld<uint2>(sC, tkC ^ static_cast<uint32_t>(nb << 5));
                const float cv[4] = {bf_lo(cr.x), bf_hi(cr.x), bf_lo(cr.y), bf_hi(cr.y)};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dCacc[nb][r] += cw[r] + ka_i * cc[r];
                    car += cv[r] * cc[r];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            car = sum_g(car);
            if (g == 0) sCar[i] = ka_i * car;
        }
        __syncthreads();

        // ---- dcs, d(a) by a reverse segmented sum over each sequence run, d(dt)
        if (wave == 0) {
            // column sums of M over the row blocks
            float tsum = 0.0f;
            for (int t = lane; t < kBQ; t += kWave) tsum += sTj[t];
            tsum = sum64(tsum);
            // lane q holds tokens t1 = 2(63 - q) + 1 then t0 = 2(63 - q) (reverse order)
            const int tA = 2 * (kWave - 1 - lane) + 1, tB = tA - 1;
            auto dcs_of = [&](int t) {
                if (t >= valid) return 0.0f;
                float cols = 0.0f;
#pragma unroll
                for (int q = 0; q < kBWaves; ++q) cols += (t < 16 * q + 16) ? sCols[q * kBQ + t] : 0.0f;
                float v = sRows[t] - cols + sCar[t] - sTj[t];
                if (t == valid - 1) v += tsum + e * gh;
                return v;
            };
            // a token ends its run (starts a segment in reverse order) at the
            // last real token or before a sequence change
            auto run_end = [&](int t) {
                return t >= valid - 1 || sSeq[t + 1] != sSeq[t];
            };
            const float dA0 = dcs_of(tA), dB0 = dcs_of(tB);
            const bool hA = run_end(tA), hB = run_end(tB);
            const float agg = hB ? dB0 : dA0 + dB0;
            const float incl = wave_segmented_scan(agg, (hA || hB) ? 1 : 0);
            float carry = __shfl_up(incl, 1, kWave);
            if (lane == 0) carry = 0.0f;
            const float rA = hA ? dA0 : carry + dA0;
            const float rB = hB ? dB0 : rA + dB0;
            // d(dt), d(dt_raw), the per-chunk sums
            float dA_part = 0.0f, dbias_part = 0.0f;
            const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = u == 0 ? tA : tB;
                const float da = u == 0 ? rA : rB;
                if (t < valid) {
                    const float dtv = sDt[t];
                    dA_part += dtv * da;
                    const float ddt = sDin[t] + Ah * da;
                    const int64_t ti = (srow + t0 + t) * a.H + h;
                    const float v = sRaw[t] + bias;
                    const float sp = a.softplus ? softplus_f32(v) : v;
                    float draw = 0.0f;
                    if (sp >= a.dt_min && sp <= a.dt_max) draw = a.softplus ? ddt / (1.0f + __expf(-v)) : ddt;
                    a.ddt[ti] = draw;
                    dbias_part += draw;
                }
            }
            dA_part = sum64(dA_part);
            dbias_part = sum64(dbias_part);
            if (lane == 0) {
                float* part = a.partials + ((b * a.nc + c) * a.H + h) * 3;
                part[0] = dA_part;
                part[1] = dD_part;
                part[2] = dbias_part;
            }
        }
        __syncthreads();  // LDS is reused by the next head
    }

    // ---- dB, dC of the group: lane holds n = 16nb + 4g .. +3 of row 16 * wave + r16
    const int jr = 16 * wave + r16;
    if (jr < valid) {
        uint16_t* dbp = static_cast<uint16_t*>(a.dB) + ((srow + t0 + jr) * a.G + grp) * N + 4 * g;
        uint16_t* dcp = static_cast<uint16_t*>(a.dC) + ((srow + t0 + jr) * a.G + grp) * N + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
            *reinterpret_cast<uint2*>(dbp + 16 * nb) = pack4(dBacc[nb]);
            *reinterpret_cast<uint2*>(dcp + 16 * nb) = pack4(dCacc[nb]);
        }
    }
}

// dA, dD, d(dt_bias) of head blockIdx.x: sums of the per-(row, chunk) partials
// in a fixed order.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a, int64_t rows_chunks) {
    __shared__ float red[3][256];
    const int h = blockIdx.x;
    float acc[3] = {0.0f, 0.0f, 0.0f};
    for (int64_t k = threadIdx.x; k < rows_chunks; k += 256) {
        const float* part = a.partials + (k * a.H + h) * 3;
        acc[0] += part[0];
        acc[1] += part[1];
        acc[2] += part[2];
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) red[q][threadIdx.x] = acc[q];
    __syncthreads();
    for (int d = 128; d > 0; d >>= 1) {
        if (static_cast<int>(threadIdx.x) < d)
#pragma unroll
            for (int q = 0; q < 3; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + d];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.dA[h] = red[0][0];
        if (a.dD) a.dD[h] = red[1][0];
        if (a.ddt_bias) a.ddt_bias[h] = red[2][0];
    }
}

// Gradients when there are no tokens: d(h_init) = dh_final (or zero) and
// zero dA, dD, d(dt_bias).
__global__ __launch_bounds__(256) void bwd_empty_kernel(BwdArgs a, int64_t nstate) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (a.dh_init && i < nstate) a.dh_init[i] = a.dh_final ? a.dh_final[i] : 0.0f;
    if (i < a.H) {
        a.dA[i] = 0.0f;
        if (a.dD) a.dD[i] = 0.0f;
        if (a.ddt_bias) a.ddt_bias[i] = 0.0f;
    }
}

}  // namespace

hipError_t launch_bwd_empty(const BwdArgs& a, int64_t nstate, hipStream_t st) {
    const int64_t n = nstate > a.H ? nstate : a.H;
    return dispatch(bwd_empty_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), st, a,
                    nstate);
}

hipError_t launch_bwd_seg_ends(const BwdArgs& a, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(2 * static_cast<int64_t>(a.batch) * a.H * (a.nseg - 1)));
    if (a.N == 64) return dispatch(bwd_seg_ends_kernel<64>, grid, dim3(kBThreads), st, a);
    return dispatch(bwd_seg_ends_kernel<128>, grid, dim3(kBThreads), st, a);
}

hipError_t launch_bwd_states(const BwdArgs& a, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(2 * static_cast<int64_t>(a.batch) * a.H * a.nseg));
    if (a.N == 64) return dispatch(bwd_states_kernel<64>, grid, dim3(kBThreads), st, a);
    return dispatch(bwd_states_kernel<128>, grid, dim3(kBThreads), st, a);
}

hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.nc * a.G));
    if (a.N == 64) return dispatch(bwd_chunk_kernel<64>, grid, dim3(kBThreads), st, a);
    return dispatch(bwd_chunk_kernel<128>, grid, dim3(kBThreads), st, a);
}

hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t st) {
    return dispatch(bwd_reduce_kernel, dim3(static_cast<unsigned>(a.H)), dim3(256), st, a,
                    static_cast<int64_t>(a.batch) * a.nc);
}

}  // namespace ssd
