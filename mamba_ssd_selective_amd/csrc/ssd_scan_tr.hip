// ssd_scan_tr.hip -- bf16 chunk-scan kernels for gfx950 built on direct-to-LDS
// staging and transposing LDS reads (P = 64, N in {64, 128}, Q in {64, 128}).
//
// Same operation, chunk decomposition and work split as chunk_scan_kernel in
// ssd_kernels.hip (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 3
// Figure 2 box [F2]; the chunked form is written out at the top of that file),
// which keeps serving the fp32 and the other bf16 shapes.  What differs is how
// operands reach the matrix cores:
//  * the x (token x p) and B (token x n) tiles of a chunk and its per-token
//    metadata are copied into LDS unchanged by loads that write LDS directly
//    (no registers, no VALU).  Rows past the end of a ragged last chunk come
//    back as zeros from the buffer range check.  Tiles are double-buffered:
//    the next chunk's copy is in flight during the current chunk's math;
//  * operands that need the token index as their MFMA k dimension (x^T for
//    the output product, x and B^T for the state product) are read with
//    ds_read_b64_tr_b16, which transposes 16-bit elements across lanes;
//  * 16-byte LDS slots are XOR-swizzled per row so that those reads and the
//    state-operand reads hit distinct banks;
//  * C rows (k = n, contiguous in memory) and the precomputed C.B^T tiles go
//    from global memory into registers one chunk ahead;
//  * outputs of chunk c are stored at the start of chunk c+1, so no wait on
//    store completion sits on the chunk loop's critical path.
//
// Lane conventions (wave of 64, g = lane / 16, r16 = lane % 16):
//  * MFMA v_mfma_f32_16x16x32_bf16 operands: lane holds row/column r16 and
//    eight k values; the accumulator holds rows 4g + r (r < 4), column r16.
//  * k over tokens (transposing reads): element e < 4 is token 32s + 4g + e,
//    element e >= 4 is token 32s + 16 + 4g + (e - 4).  The C.B^T tiles written
//    by chunk_prep_kernel use the same token order.
//  * k over n (state operand, C rows): element e is n = 32s + 8g + e.
#include <atomic>

#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_lds.h"
#include "ssd_work.h"

namespace ssd {
namespace {

// Row blocks and state n-blocks are at most 8 per chunk.  The segment-state
// kernel runs 8 waves, each owning one state n-block; the output kernel runs
// 12: waves 0-7 own one output row block each, waves 8-11 two state n-blocks
// each, so that the state chain and the output products of a chunk proceed on
// different waves of each SIMD (three waves per SIMD).
// Decode-output forms (kDec: rows of one chunk, one output row block per
// row, single buffers), 4 waves, each computing one 16-wide p block of that
// row block.  Each wave reads its rows of the chunk-start state straight
// into the bf16 operand registers of the carried-state term (the values the
// state waves would have written to LDS); every output element takes the
// same products in the same order as in the prefill forms.
//  kDec = 1: for rows whose chunk does not complete (no B tile).
//  kDec = 2: for rows whose chunk completes: each wave also updates its 16
//            rows of the chunk's state from the fp32 chunk-start state, in
//            the products and order of the prefill forms' state waves.
constexpr int kTrWaves = 8;
template <bool kOut, int kDec = 0>
struct TrWaves {
    static constexpr int W = kDec ? 4 : (kOut ? 12 : 8);
    static constexpr int kThreads = W * kWave;
    static constexpr int NBW = kOut ? 2 : 1;  // state n-blocks per state wave
    static constexpr int first_state = kDec ? W : (kOut ? 8 : 0);
};
template <int P, int N, int Q>
struct TrGeo {
    static_assert(P == 64 && (N == 64 || N == 128) && (Q == 64 || Q == 128), "compiled shapes");
    static constexpr int PB = P / 16;     // 16-wide p blocks
    static constexpr int NNB = N / 16;    // 16-wide n blocks (one per state wave)
    static constexpr int NB = Q / 16;     // 16-token row blocks (one per output wave)
    static constexpr int KQ = Q / 32;     // MFMA k steps over tokens
    static constexpr int KN = N / 32;     // MFMA k steps over n
    static constexpr int NCB = NB / 2;    // C.B^T k steps of the last row block
    static constexpr int XROW = 2 * P;    // bytes of one token row of the x tile
    static constexpr int BROW = 2 * N;    // bytes of one token row of the B tile
    static constexpr int HROW = 2 * N;    // bytes of one p row of the state operand
    static constexpr int XBYTES = Q * XROW;
    static constexpr int BBYTES = Q * BROW;
    static constexpr int HBYTES = P * HROW;
    static_assert(NNB <= kTrWaves && NB <= kTrWaves, "one block per wave");
};

// Per-token metadata of one chunk (written by chunk_prep_kernel; cs, dt, w are
// contiguous as in the workspace block).
template <int Q>
struct TrMeta {
    float cs[Q];  // segmented chunk cumsum of dt*A
    float dt[Q];  // transformed dt (0 past L)
    float w[Q];   // chunk-state weights
    int seq[Q];   // sequence ids (0 past L)
};

// State operand sH[p][n]: 16-byte slot s of row p is stored at slot s ^ x(p);
// sixteen consecutive rows read one slot each in a ds_read_b128.
template <int HROW>
__device__ __forceinline__ int h_off(int p, int slot) {
    constexpr int S = HROW / 16;
    const int x = S == 16 ? (p & 15) : ((p & 7) ^ ((p >> 3) & 1));
    return p * HROW + ((slot ^ x) << 4);
}

// ---------------------------------------------------------- global -> LDS

// Copies of a swizzled [token][ROW bytes] tile: wave instruction k = wave +
// 8 kk writes LDS bytes [1024 k, 1024 k + 1024), 16 per lane.  dma_voff is the
// lane's source byte offset for instruction kk (chunk independent); rows past
// the resource's range read as zeros.
template <int ROW, int W>
__device__ __forceinline__ uint32_t dma_voff(int kk, int wave, int lane, int gstride) {
    constexpr int RPI = 1024 / ROW;  // rows per wave instruction (64 lanes x 16 bytes)
    constexpr int SPR = ROW / 16;    // 16-byte slots per row
    static_assert(1024 % ROW == 0, "whole rows per instruction");
    const int k = wave + W * kk;
    const int row = k * RPI + lane / SPR;
    const int slot = (lane % SPR) ^ (2 * tr_swz<ROW>(row));
    return static_cast<uint32_t>(row * gstride + slot * 16);
}
template <int W>
__device__ __forceinline__ void dma_one(char* lds_tile, __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                        int kk, int wave) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (SSD_LDS void*)(lds_tile + (s_opaque(wave) + W * kk) * 1024), 16, voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows, int stride) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, rows * stride,
                                             kRawBufferWord3);
}

// -------------------------------------------------------------- the kernel

// Output row block of an output wave; for Q = 128 the two waves sharing a
// SIMD (w, w + 4) get rows (k, 7 - k).
template <int NB>
__device__ __forceinline__ int tr_row_block(int wave) {
    if constexpr (NB == 8) return wave < 4 ? wave : 11 - wave;
    else return wave;
}

template <int P, int N, int Q, bool kOut, bool kSeq, int kDec = 0>
struct TrScan {
    using G_ = TrGeo<P, N, Q>;
    static constexpr int W = TrWaves<kOut, kDec>::W;
    static constexpr int NBW = TrWaves<kOut, kDec>::NBW;
    static constexpr int NXI = G_::XBYTES / 1024;   // 1 KB copy instructions of an x tile
    static constexpr int NBI = G_::BBYTES / 1024;   // ... of a B tile
    static constexpr int XI = (NXI + W - 1) / W;    // per wave (the last round may be partial)
    static constexpr int BI = (NBI + W - 1) / W;
    // p blocks of an output wave: all of them, or (kDec) the wave's own
    static constexpr int OPB = kDec ? 1 : G_::PB;
    static_assert(!kDec || W == G_::PB, "one p block per wave");
    static_assert(G_::XBYTES % 1024 == 0 && G_::BBYTES % 1024 == 0, "whole copy instructions");
    // A row block's intra-chunk decays are factored when the decay across its
    // 16 tokens is at most this (the column factors then stay below e^64).
    static constexpr float kDiagSpan = 64.0f;

    const ScanArgs& a;
    int wave, lane, r16, g;
    int c_begin, c_end, L, nc;
    bool want_final;
    bool st_wave_, out_wave_;
    // with 8 waves and 8 n-blocks every wave owns a state n-block
    __device__ __forceinline__ bool st() const { return (!kOut && G_::NNB == W) || st_wave_; }
    __device__ __forceinline__ bool ow() const { return kOut && out_wave_; }
    int I;                  // output row block of an output wave
    int nb;                 // first state n-block of a state wave (it owns NBW)
    int pb0;                // kDec: this wave's p block
    bool commit_;           // kDec = 2: the row's chunk completes (its state is updated)
    int64_t row_state_;     // the row's state index (row, or slot)
    int head_;
    __device__ __forceinline__ int pbase() const { return kDec ? pb0 : 0; }
    float Dh, Ah;           // D[h], A[h]
    int seq_prev;           // sequence id of the token before the current chunk
    float mult;             // decay of the segment (chunk-state kernel)
    // per-(row, head) / per-(row, group) bases; chunk c adds c times the chunk stride
    const uint16_t* xg;  int xstride;   // x[b][.][h][0], token stride in bytes
    const uint16_t* bg;  int bstride;   // B[b][.][g][0]
    const uint16_t* cmg;                // C rows in operand order at (b, chunk 0, g)
    int64_t cm_cstride;                 // elements between chunks of that copy
    uint16_t* yg;                       // y[b][.][h][0]
    uint16_t* ylg;                      // decode output y_last[b][h][0], or null
    const float* mg;                    // metadata block (b, h, chunk 0): [cs | dt | w]
    const int32_t* sqg;                 // seq_idx[b][0]
    const uint16_t* cbg;                // C.B^T tiles at (b, chunk 0, g)
    int64_t cb_cstride;                 // elements between chunks of the tile buffer

    // LDS objects and lane addresses per buffer parity (opaque, see lds_keep)
    char* xo[2];
    char* bo[2];
    TrMeta<Q>* mo[2];
    char* ho[2];
    float* cjo;
    uint32_t xa[2];          // x tile, transposing read of p block 0, k step 0 (block pb: ^ 32 pb)
    uint32_t ba[2][NBW];     // B tile, transposing read of this wave's n blocks
    uint32_t ha[2];          // state operand, rows p = r16 (+16 pb), slot g (k step 0)
    uint32_t hw[2][NBW];     // state operand, this state wave's write positions
    uint32_t ma[2];          // metadata + 16 g (reads at tokens 32 s + 4 g)
    uint32_t mbase[2];       // metadata
    uint32_t cja;            // column factors of this wave + 16 g
    uint32_t cjw;            // column factors of this wave + 4 lane
    // chunk-independent source offsets of this wave's copies
    uint32_t xv[XI], bv[BI];
    uint32_t cv;             // C rows: byte offset of piece (I, 0), lane's 16 bytes

    f32x4_t h[NBW][G_::PB];     // state rows n = 16 (nb + t) + 4g + r, column p = 16pb + r16
    uint4 cr[G_::KN];           // C rows of a chunk (k over n), loaded a chunk ahead
    uint4 cb[G_::NCB];          // C.B^T tile pairs of a chunk, loaded a chunk ahead
    // kDec: the state operand of the carried-state term, fragment (s, pb0)
    uint4 hreg[kDec ? G_::KN : 1];
    // kDec = 2: the fp32 state rows p = 16 pb0 + r16 of n-block nb, n = 16 nb + 4g + r
    f32x4_t hs[kDec == 2 ? G_::NNB : 1];

    __device__ __forceinline__ TrScan(const ScanArgs& args) : a(args) {}

    // rows of chunk c inside the sequence (c * Q < L < 2^31)
    __device__ __forceinline__ int rows_in(int c) const {
        const int rem = L - c * Q;
        return rem < Q ? rem : Q;
    }

    // C rows of row block I (k over n) from chunk_prep's operand-order copy:
    // 1 KB contiguous per k step
    __device__ __forceinline__ void load_c(int c) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(cmg + static_cast<int64_t>(c) * cm_cstride), 0, Q * N * 2, kRawBufferWord3);
#pragma unroll
        for (int s = 0; s < G_::KN; ++s) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, cv + 1024 * s, 0, 0);
            cr[s] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }

    // The (I >> 1) + 1 tile pairs of row block I.
    __device__ __forceinline__ void load_cb(int c) {
        const uint4* tiles = reinterpret_cast<const uint4*>(cbg + static_cast<int64_t>(c) * cb_cstride) +
                             cb_pair_base(I) * 64 + lane;
#pragma unroll
        for (int u = 0; u < G_::NCB; ++u)
            if (u <= (I >> 1)) cb[u] = tiles[64 * u];
    }

    // Copies of chunk c+1, split so that they spread over the chunk's math.
    __device__ __forceinline__ void dma_x(char* sX, int c) const {
        const __amdgpu_buffer_rsrc_t rs =
            rows_rsrc(xg + static_cast<int64_t>(c) * Q * (xstride / 2), rows_in(c), xstride);
#pragma unroll
        for (int kk = 0; kk < XI; ++kk)
            if (NXI % W == 0 || s_opaque(wave) + W * kk < NXI) dma_one<W>(sX, rs, xv[kk], kk, wave);
    }
    __device__ __forceinline__ void dma_b(char* sB, int c, int k0, int k1) const {
        if (k0 < k1) {
            const __amdgpu_buffer_rsrc_t rs =
                rows_rsrc(bg + static_cast<int64_t>(c) * Q * (bstride / 2), rows_in(c), bstride);
#pragma unroll
            for (int kk = 0; kk < BI; ++kk)
                if (kk >= k0 && kk < k1 && (NBI % W == 0 || s_opaque(wave) + W * kk < NBI))
                    dma_one<W>(sB, rs, bv[kk], kk, wave);
        }
    }
    // [cs | dt | w] of a chunk is one contiguous block of 3Q floats (Q * 3/4
    // pieces of 16 bytes) in the workspace and in TrMeta.
    __device__ __forceinline__ void dma_meta(TrMeta<Q>* sM, int c) const {
        constexpr int NPC = 3 * Q / 4;       // 16-byte pieces
        const int mw = W - 1 - wave;  // from the last waves
        // a lane past the block would write LDS past [cs | dt | w] (the sequence ids)
        if (kWave * mw + lane < NPC) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(mg + static_cast<int64_t>(c) * (3 * Q)), 0, 3 * Q * 4,
                kRawBufferWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (SSD_LDS void*)(reinterpret_cast<char*>(sM) + 1024 * mw), 16,
                16 * (kWave * mw + lane), 0, 0, 0);
        }
        if constexpr (kSeq) {
            if (mw == (NPC + kWave - 1) / kWave && lane < Q / 4) {
                const __amdgpu_buffer_rsrc_t rs = rows_rsrc(sqg + static_cast<int64_t>(c) * Q, rows_in(c), 4);
                // destination formed from its 32-bit LDS address (a generic-pointer
                // form of it can hit an instruction-selection fault)
                const uint32_t dst = lds_addr(sM) + static_cast<uint32_t>(offsetof(TrMeta<Q>, seq));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (SSD_LDS void*)(uintptr_t)dst, 16, 16 * lane, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void dma_all(char* sX, char* sB, TrMeta<Q>* sM, int c) const {
        dma_x(sX, c);
        // the decode forms update a state only when the row's chunk completes
        if constexpr (!kDec) dma_b(sB, c, 0, BI);
        else if constexpr (kDec == 2) {
            if (commit_) dma_b(sB, c, 0, BI);
        }
        dma_meta(sM, c);
    }

    // kDec = 2: the fp32 chunk-start state rows of this wave (accumulator layout)
    __device__ __forceinline__ void load_state_f32(const float* __restrict__ src) {
#pragma unroll
        for (int nbk = 0; nbk < G_::NNB; ++nbk) {
            if (src) {
                const float4 v = *reinterpret_cast<const float4*>(src + (16 * pb0 + r16) * N + 16 * nbk + 4 * g);
                hs[nbk] = f32x4_t{v.x, v.y, v.z, v.w};
            } else {
                hs[nbk] = acc_zero();
            }
        }
    }

    // kDec = 2: the state update of a completed chunk for this wave's rows,
    // h = exp(cs_last) h + (B w)^T x, stored as [p][n]
    template <int K>
    __device__ __forceinline__ void commit_state(float* __restrict__ dst) {
        const TrMeta<Q>* M = mo[K];
        const char* X = xo[K];
        const char* Bt = bo[K];
        const float e = decay_exp(lds_ld<float>(M, mbase[K] + offsetof(TrMeta<Q>, cs) + 4 * (Q - 1)));
#pragma unroll
        for (int nbk = 0; nbk < G_::NNB; ++nbk)
#pragma unroll
            for (int r = 0; r < 4; ++r) hs[nbk][r] *= e;
#pragma unroll
        for (int s = 0; s < G_::KQ; ++s) {
            const Frag<uint16_t> xf = tr_frag<G_::XROW>(X, xa[K] ^ (32 * pb0), s);
            const float4 w0 = lds_ld<float4>(M, ma[K] + offsetof(TrMeta<Q>, w) + 128 * s);
            const float4 w1 = lds_ld<float4>(M, ma[K] + offsetof(TrMeta<Q>, w) + 128 * s + 64);
#pragma unroll
            for (int nbk = 0; nbk < G_::NNB; ++nbk) {
                // (n-block nbk's lane base: that of block 0 with its 32-byte unit moved)
                const Frag<uint16_t> braw = tr_frag<G_::BROW>(Bt, ba[K][0] ^ static_cast<uint32_t>(nbk << 5), s);
                mma(hs[nbk], scale_frag(braw, w0, w1), xf);
            }
        }
#pragma unroll
        for (int nbk = 0; nbk < G_::NNB; ++nbk)
            *reinterpret_cast<float4*>(dst + (16 * pb0 + r16) * N + 16 * nbk + 4 * g) =
                make_float4(hs[nbk][0], hs[nbk][1], hs[nbk][2], hs[nbk][3]);
    }

    // kDec: the chunk-start state, row p = 16 pb0 + r16, n = 32 s + 8 g .. +7,
    // as the bf16 pairs the state waves' operand copy holds
    __device__ __forceinline__ void load_state_operand(const float* __restrict__ src) {
#pragma unroll
        for (int s = 0; s < G_::KN; ++s) {
            if (src) {
                const float* q = src + (16 * pb0 + r16) * N + 32 * s + 8 * g;
                const float4 v0 = *reinterpret_cast<const float4*>(q);
                const float4 v1 = *reinterpret_cast<const float4*>(q + 4);
                hreg[s] = make_uint4(pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w),
                                     pack_bf16x2(v1.x, v1.y), pack_bf16x2(v1.z, v1.w));
            } else {
                hreg[s] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }

    // Factors of the G^T fragment of k step u (tiles J = 2u, 2u+1; element e
    // is token j_e in the k order above) for lane column i = 16I + r16, in
    // the exact form: f_e = [j_e <= i] [seq_j = seq_i] exp(cs_i - cs_j) dt_j,
    // so that G[i][j_e] = (C_i . B_j) f_e.
    // sigma: the sequence a pass serves (rows of other sequences get zero
    // factors; callers without one pass seq_i).
    __device__ __forceinline__ void exact_factors(float (&f)[8], const void* mobj, uint32_t mq, int u,
                                                  float cs_i, int seq_i, int sigma) const {
        // token 16J + 4g + r of tile J is kept when r <= lim: all of a tile left
        // of the diagonal, r <= r16 - 4g on it, none right of it
        int tdiag = r16 - 4 * g;
        int Iv = I;
        // opaque to the optimizer: keeps the per-element compares here instead
        // of hoisting them out of the chunk loop as 64-bit lane masks
        asm volatile("" : "+v"(tdiag), "+v"(Iv));
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            const int J = 2 * u + hp;
            const int off = 128 * u + 64 * hp;
            const float4 cs4 = lds_ld<float4>(mobj, mq + off + offsetof(TrMeta<Q>, cs));
            const float4 dt4 = lds_ld<float4>(mobj, mq + off + offsetof(TrMeta<Q>, dt));
            int4 sq4 = make_int4(0, 0, 0, 0);
            if constexpr (kSeq) sq4 = lds_ld<int4>(mobj, mq + off + offsetof(TrMeta<Q>, seq));
            const float csv[4] = {cs4.x, cs4.y, cs4.z, cs4.w};
            const float dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
            const int sqv[4] = {sq4.x, sq4.y, sq4.z, sq4.w};
            const int lim = J < Iv ? 3 : (J == Iv ? tdiag : -1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bool keep = r <= lim;
                if constexpr (kSeq) keep = keep && sqv[r] == seq_i && seq_i == sigma;
                // masked elements may overflow here; the select drops them
                f[4 * hp + r] = keep ? decay_exp(cs_i - csv[r]) * dtv[r] : 0.0f;
            }
            // one half at a time (bounds the registers of this rarely taken path)
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Packed sequences: 16-bit masks of k step s's tokens (the fragment
    // element order above) that belong to sequence sigma, one word per bf16
    // pair.  ANDing a fragment with them zeroes every other sequence's values
    // (NaN and Inf included), where a product with a zero weight would not.
    __device__ __forceinline__ uint4 seq_keep_mask(const void* mobj, uint32_t mq, int s,
                                                   int sigma) const {
        const int4 q0 = lds_ld<int4>(mobj, mq + 128 * s + offsetof(TrMeta<Q>, seq));
        const int4 q1 = lds_ld<int4>(mobj, mq + 128 * s + 64 + offsetof(TrMeta<Q>, seq));
        auto m2 = [](bool lo, bool hi) { return (lo ? 0x0000FFFFu : 0u) | (hi ? 0xFFFF0000u : 0u); };
        return make_uint4(m2(q0.x == sigma, q0.y == sigma), m2(q0.z == sigma, q0.w == sigma),
                          m2(q1.x == sigma, q1.y == sigma), m2(q1.z == sigma, q1.w == sigma));
    }
    static __device__ __forceinline__ Frag<uint16_t> frag_and(const Frag<uint16_t>& f, const uint4& m) {
        uint4 u = __builtin_bit_cast(uint4, f.v);
        u.x &= m.x;
        u.y &= m.y;
        u.z &= m.z;
        u.w &= m.w;
        return frag_of(u);
    }

    // G^T fragment from a C.B^T tile pair and per-element factors f (both
    // forms).  Factored form, k steps left of the diagonal one:
    // G[i][j] = r_i (C_i . B_j) c_j with c_j = [seq_j = seq_m] exp(cs_m - cs_j) dt_j
    // (m = 16I) and the row factor r_i applied to the accumulator at the end.
    // On the diagonal step (u = I/2) the tile right of the diagonal is zero,
    // the diagonal tile keeps j <= i, and dd is added on the diagonal element:
    // D[h] / r_i in the factored form (r_i then restores D[h]), D[h] in the
    // exact form (whose factors already hold the masks).
    // kMasked: zero factors mark another sequence's pairs, kept zero by a
    // select whatever the tile holds.
    __device__ __forceinline__ Frag<uint16_t> g_apply(const uint4& t, const float (&f)[8], bool diag,
                                                      float dd, bool kMasked) const {
        const uint32_t d[4] = {t.x, t.y, t.z, t.w};
        float out[8];
        if (!diag) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = ((e & 1) ? bf_hi(d[e >> 1]) : bf_lo(d[e >> 1])) * f[e];
                // a masked pair (zero factor) stays zero whatever its tile value
                out[e] = (kSeq && kMasked && f[e] == 0.0f) ? 0.0f : v;
            }
        } else {
            int tdiag = r16 - 4 * g;
            asm volatile("" : "+v"(tdiag));
            const bool odd = I & 1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = e & 3;
                const float cbv = (e & 1) ? bf_hi(d[e >> 1]) : bf_lo(d[e >> 1]);
                // tile 2u is the diagonal one for even I (and left of it for odd I);
                // tile 2u+1 is the diagonal one for odd I (and right of it for even I)
                const bool on_diag = (e < 4) ? !odd : odd;
                bool keep = (e < 4) ? (odd || r <= tdiag) : (odd && r <= tdiag);
                if (kSeq && kMasked) keep = keep && f[e] != 0.0f;  // another sequence's pair
                const float v = keep ? cbv * f[e] : 0.0f;
                out[e] = (on_diag && r == tdiag) ? v + dd : v;
            }
        }
        return frag_from_f32<uint16_t>(out);
    }

    // Copies of chunk c+1 that are this wave's share, interleaved with the k
    // steps (s = -1: before them).
    __device__ __forceinline__ void copies(int s, int c, char* Xn, char* Bn, TrMeta<Q>* Mn) const {
        if (s < 0) {
            dma_x(Xn, c + 1);
        } else {
            dma_b(Bn, c + 1, BI * s / G_::KQ, BI * (s + 1) / G_::KQ);
            if (s == 0) dma_meta(Mn, c + 1);
        }
    }

    // Row i of y (lane column i, p = 16 pb + 4 g + r in the accumulators) as
    // bf16, scaled by fin.  Lanes of 16-lane rows g and g ^ 1 swap p blocks
    // (q, q + 1) so that each lane holds 8 consecutive p: p0 = 16 (g & 1) +
    // 8 (g >> 1) and p0 + 32; a store then writes 64 contiguous bytes of each
    // of 16 rows.  y is not read again, so the stores are non-temporal.  All
    // lanes take part in the swap; only rows inside the sequence are stored.
    static constexpr int kYStores = G_::PB / 2;  // store instructions per row block
    __device__ __forceinline__ void store_y(const f32x4_t (&y)[OPB], float fin, int c, int i, int valid) const {
        if constexpr (kDec) {
            // the row's last token: the lanes of column i = valid - 1 hold
            // p = 16 pb0 + 4 g + r
            if (i == valid - 1)
                *reinterpret_cast<uint2*>(ylg + 16 * pb0 + 4 * g) =
                    make_uint2(pack_bf16x2(y[0][0] * fin, y[0][1] * fin),
                               pack_bf16x2(y[0][2] * fin, y[0][3] * fin));
        } else {
            store_rows(y, fin, c, i, valid);
        }
    }
    __device__ __forceinline__ void store_rows(const f32x4_t (&y)[G_::PB], float fin, int c, int i,
                                               int valid) const {
        static_assert(G_::PB == 4, "two swapped block pairs");
        typedef unsigned int u4 __attribute__((ext_vector_type(4)));
        uint32_t yw[G_::PB][2];
#pragma unroll
        for (int pb = 0; pb < G_::PB; ++pb) {
            yw[pb][0] = pack_bf16x2(y[pb][0] * fin, y[pb][1] * fin);
            yw[pb][1] = pack_bf16x2(y[pb][2] * fin, y[pb][3] * fin);
        }
        // odd rows of the first operand trade places with even rows of the second
#pragma unroll
        for (int q = 0; q < G_::PB; q += 2)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const auto r = __builtin_amdgcn_permlane16_swap(yw[q][w], yw[q + 1][w], false, false);
                yw[q][w] = r[0];
                yw[q + 1][w] = r[1];
            }
        // decode output: the row's last token alone
        const bool keep = ylg ? i == valid - 1 : i < valid;
        if (keep) {
            uint16_t* yp = (ylg ? ylg : yg + (static_cast<int64_t>(c) * Q + i) * (xstride / 2)) +
                           16 * (g & 1) + 8 * (g >> 1);
#pragma unroll
            for (int q = 0; q < G_::PB; q += 2) {
                const u4 v = {yw[q][0], yw[q][1], yw[q + 1][0], yw[q + 1][1]};
                __builtin_nontemporal_store(v, reinterpret_cast<u4*>(yp + 16 * q));
            }
        }
    }

    // One chunk on an output wave (row block I).  On entry chunk c's tiles and
    // metadata are in buffer K, the state before it in H[K] (bf16 operand
    // copy), and its C rows and C.B^T tiles in cr, cb.  Issues this wave's
    // share of chunk c+1's copies into buffer K^1 and leaves after the barrier
    // that ends the chunk.
    // Whether chunk c (in buffer K) holds more than one packed sequence among
    // its tokens.  Such chunks take the kMixed code (masks and passes), which
    // the others never execute.
    template <int K>
    __device__ __forceinline__ bool chunk_mixed(int c) const {
        if constexpr (!kSeq) {
            return false;
        } else {
            const TrMeta<Q>* M = mo[K];
            const uint32_t mb = mbase[K];
            return lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq)) !=
                   lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * (rows_in(c) - 1));
        }
    }
    // A row block that holds more than one packed sequence: the main k-step
    // loop served its first sequence (seq_m).  Rows of later sequences have no
    // carried-state term (their sequence starts inside this chunk), so they
    // restart from zero and take one pass per sequence: x masked to the
    // sequence, exact factors for its rows only, and each k step's product
    // added to its rows with a select.  Rare: only where a sequence boundary
    // falls inside a 16-row block.
    template <int K>
    __device__ __forceinline__ void span_passes(f32x4_t (&y)[OPB], int c, int valid, int i,
                                                         int sd, float cs_i, int seq_i, int seq_m,
                                                         float dr) const {
        static_assert(OPB == G_::PB, "packed sequences take forms with every p block per wave");
        const TrMeta<Q>* M = mo[K];
        const char* X = xo[K];
#pragma unroll
        for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r) y[pb][r] = seq_i == seq_m ? y[pb][r] : 0.0f;
        int sigma = seq_m;
        for (int pass = 0; pass < 16; ++pass) {
            // the next sequence among this block's rows (the ids rise along
            // lanes 0..15; at most 16 passes whatever the ids)
            const uint64_t nxt = __builtin_amdgcn_ballot_w64(g == 0 && i < valid && seq_i > sigma);
            if (nxt == 0) break;
            sigma = __builtin_amdgcn_readlane(seq_i, static_cast<int>(__builtin_ctzll(nxt)));
            const bool mine = seq_i == sigma;
#pragma unroll
            for (int s = 0; s < G_::KQ; ++s) {
                if (s <= sd) {
                    Frag<uint16_t> xf[G_::PB];
                    float f[8];
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) xf[pb] = tr_frag<G_::XROW>(X, xa[K] ^ (32 * pb), s);
                    exact_factors(f, M, ma[K], s, cs_i, seq_i, sigma);
                    const uint4 km = seq_keep_mask(M, ma[K], s, sigma);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) xf[pb] = frag_and(xf[pb], km);
                    const Frag<uint16_t> gf = g_apply(cb[s], f, s == sd, dr, true);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) {
                        f32x4_t t = acc_zero();
                        mma(t, xf[pb], gf);
#pragma unroll
                        for (int r = 0; r < 4; ++r) y[pb][r] += mine ? t[r] : 0.0f;
                    }
                }
            }
        }
    }

    template <int K>
    __device__ __forceinline__ void chunk_out(int c, char* Xn, char* Bn, TrMeta<Q>* Mn) {
        const bool has_next = c + 1 < c_end;
        const int valid = rows_in(c);
        // decode output (rows of one chunk): only the row block of the last token
        if (ylg && I != ((valid - 1) >> 4)) {
            __syncthreads();
            return;
        }
        const uint32_t mb = mbase[K];
        const char* X = xo[K];
        const TrMeta<Q>* M = mo[K];
        const char* H = ho[K];

        // chunk c+1's x copy first (its source is the one input no earlier
        // kernel has read, so it may come from HBM)
        if (has_next) copies(-1, c, Xn, Bn, Mn);
        const int i = 16 * I + r16;
        const int m0 = 16 * I;
        const float cs_i = lds_ld<float>(M, mb + offsetof(TrMeta<Q>, cs) + 4 * i);
        const float cs_m = lds_ld<float>(M, mb + offsetof(TrMeta<Q>, cs) + 4 * m0);
        // last real token of the row block (ids past L read as 0)
        const int me = min(m0 + 15, max(valid - 1, m0));
        const float cs_e = lds_ld<float>(M, mb + offsetof(TrMeta<Q>, cs) + 4 * me);
        int seq_i = 0, seq_m = 0, seq_e = 0;
        // packed sequences: the chunk holds more than one of them ("mixed"),
        // and this row block does ("spanning")
        bool mixed = false, spanning = false;
        if constexpr (kSeq) {
            seq_i = lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * i);
            seq_m = lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * m0);
            seq_e = lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * me);
            mixed = chunk_mixed<K>(c);
            spanning = mixed && seq_m != seq_e;
        }
        // carried-state term y^T[p][i] = h . C_i, scaled below; each k step's
        // operand reads are issued before its products
        f32x4_t y[OPB];
#pragma unroll
        for (int q = 0; q < OPB; ++q) y[q] = acc_zero();
#pragma unroll
        for (int s = 0; s < G_::KN; ++s) {
            Frag<uint16_t> hf[OPB];
#pragma unroll
            for (int q = 0; q < OPB; ++q) {
                if constexpr (kDec) hf[q] = frag_of(hreg[s]);
                else hf[q] = frag_of(lds_ld<uint4>(H, (ha[K] ^ (s << 6)) + 16 * q * G_::HROW));
            }
            __builtin_amdgcn_sched_barrier(0);
            const Frag<uint16_t> cf = frag_of(cr[s]);
#pragma unroll
            for (int q = 0; q < OPB; ++q) mma(y[q], hf[q], cf);
        }
        // column factors c_j = [seq_j = seq_m] exp(cs_m - cs_j) dt_j of the
        // tokens j < m0 + 16, and whether any of them has dt_j * A > 0
        bool rising = false;
#pragma unroll
        for (int k = 0; k < (Q + kWave - 1) / kWave; ++k) {
            const int j = lane + kWave * k;
            if (j < m0 + 16) {
                bool keep = true;
                if constexpr (kSeq)
                    keep = lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * j) == seq_m;
                const float csj = lds_ld<float>(M, mb + offsetof(TrMeta<Q>, cs) + 4 * j);
                const float dtj = lds_ld<float>(M, mb + offsetof(TrMeta<Q>, dt) + 4 * j);
                // (other sequences' tokens have no say in the form this block takes)
                rising = rising || (keep && dtj * Ah > 0.0f);
                // overflows only where the factored form is not taken
                lds_st<float>(cjo, cjw + 256 * k, keep ? decay_exp(cs_m - csj) * dtj : 0.0f);
            }
        }
        // factored when cs never rises over these tokens (every factor is then
        // at most dt_j, and r_i at most 1), the row block holds one sequence and
        // decays by at most kDiagSpan (r_i >= e^-kDiagSpan), and the strict
        // mode is off (the choice depends on the row block's later tokens);
        // else the exact form
        const bool wfast = !__builtin_amdgcn_ballot_w64(rising) && (!kSeq || seq_m == seq_e) &&
                           cs_m - cs_e <= kDiagSpan && !a.exact_decay;
        float sc, fin = 1.0f, dr = Dh;
        bool carry = true;  // the carried state reaches this row (select, not a product)
        if (wfast) {
            fin = decay_exp(cs_i - cs_m);  // r_i
            dr = Dh / fin;
            sc = decay_exp(cs_m);
            if constexpr (kSeq) carry = seq_m == seq_prev;
        } else {
            sc = decay_exp(cs_i);
            if constexpr (kSeq) carry = seq_i == seq_prev;
        }
#pragma unroll
        for (int q = 0; q < OPB; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) y[q][r] = carry ? y[q][r] * sc : 0.0f;
        if (has_next) load_c(c + 1);  // this chunk's C rows are consumed

        // intra-chunk outputs y^T += x^T G^T over the k steps up to the
        // diagonal one.  In a chunk that holds several sequences the x
        // operand is masked to the row block's first sequence with a select
        // and masked pairs of G stay zero whatever their tile holds, so a
        // non-finite value of another sequence never meets a zero weight.
        const int sd = I >> 1;
#pragma unroll
        for (int s = 0; s < G_::KQ; ++s) {
            if (s <= sd) {
                Frag<uint16_t> xf[OPB];
                float f[8];
#pragma unroll
                for (int q = 0; q < OPB; ++q) xf[q] = tr_frag<G_::XROW>(X, xa[K] ^ (32 * (pbase() + q)), s);
                if (wfast) {
                    const float4 c0 = lds_ld<float4>(cjo, cja + 128 * s);
                    const float4 c1 = lds_ld<float4>(cjo, cja + 128 * s + 64);
                    f[0] = c0.x; f[1] = c0.y; f[2] = c0.z; f[3] = c0.w;
                    f[4] = c1.x; f[5] = c1.y; f[6] = c1.z; f[7] = c1.w;
                } else {
                    exact_factors(f, M, ma[K], s, cs_i, seq_i, kSeq ? seq_m : seq_i);
                }
                if (kSeq && mixed) {
                    const uint4 km = seq_keep_mask(M, ma[K], s, seq_m);
#pragma unroll
                    for (int q = 0; q < OPB; ++q) xf[q] = frag_and(xf[q], km);
                }
                __builtin_amdgcn_sched_barrier(0);
                const Frag<uint16_t> gf = g_apply(cb[s], f, s == sd, dr, kSeq && mixed);
#pragma unroll
                for (int q = 0; q < OPB; ++q) mma(y[q], xf[q], gf);
            }
            if (has_next) copies(s, c, Xn, Bn, Mn);
        }
        if constexpr (kSeq) {
            if (spanning) span_passes<K>(y, c, valid, i, sd, cs_i, seq_i, seq_m, dr);
        }
        if (has_next) load_cb(c + 1);  // after the last use
        store_y(y, fin, c, i, valid);
        if constexpr (kDec == 2) {
            if (commit_) commit_state<K>(a.final_states + (row_state_ * a.H + head_) * P * N);
        }
        if constexpr (kSeq) seq_prev = lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * (Q - 1));
        // this wave's copies of chunk c+1 have landed; the C.B^T tiles and y
        // stores issued after them may still be in flight (the first use of the
        // tiles waits for them)
        static_assert(G_::NCB + kYStores < 16, "vmcnt immediate");
        if (has_next) {
            const int nt = (I >> 1) + 1;  // tile loads of this row block
            if (nt == 1) wait_vmcnt<1 + kYStores>();
            else if (G_::NCB > 2 && nt == 2) wait_vmcnt<2 + kYStores>();
            else if (G_::NCB > 3 && nt == 3) wait_vmcnt<3 + kYStores>();
            else wait_vmcnt<G_::NCB + kYStores>();
        }
        __syncthreads();
    }

    // One chunk on a state wave (n-block nb; waves owning neither an n-block
    // nor a row block only copy): h_c = [no reset in c] exp(cs_last) h_{c-1} + S_c
    // with S_c = (B w)^T x, then (output kernel) the bf16 operand copy of h_c in
    // H[K^1] for the next chunk's carried-state term.
    template <int K>
    __device__ __forceinline__ void chunk_st(int c, char* Xn, char* Bn, TrMeta<Q>* Mn) {
        if (chunk_mixed<K>(c)) chunk_st_t<K, true>(c, Xn, Bn, Mn);
        else chunk_st_t<K, false>(c, Xn, Bn, Mn);
    }
    template <int K, bool kMixed>
    __device__ __forceinline__ void chunk_st_t(int c, char* Xn, char* Bn, TrMeta<Q>* Mn) {
        const bool has_next = c + 1 < c_end;
        const int valid = rows_in(c);
        // decode output (rows of one chunk): the state is needed at the chunk's end only
        if (kOut && a.y_last && valid != Q) {
            __syncthreads();
            return;
        }
        const uint32_t mb = mbase[K];
        const char* X = xo[K];
        const char* Bt = bo[K];
        const TrMeta<Q>* M = mo[K];

        const float cs_last = lds_ld<float>(M, mb + offsetof(TrMeta<Q>, cs) + 4 * (Q - 1));
        const int seq_last = kSeq ? lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * (valid - 1)) : 0;
        if (has_next) copies(-1, c, Xn, Bn, Mn);
        // at a sequence change the state restarts: selects, so that a
        // non-finite state of the previous sequence does not survive a zero
        // factor
        const bool keep_h = !kSeq || seq_last == seq_prev;
        const float e = decay_exp(cs_last);
        if (st()) {
#pragma unroll
            for (int t = 0; t < NBW; ++t)
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) h[t][pb][r] = keep_h ? h[t][pb][r] * e : 0.0f;
        }
        if constexpr (!kOut) mult = keep_h ? mult * e : 0.0f;
#pragma unroll
        for (int s = 0; s < G_::KQ; ++s) {
            if (st()) {
                Frag<uint16_t> xf[G_::PB], braw[NBW];
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb) xf[pb] = tr_frag<G_::XROW>(X, xa[K] ^ (32 * pb), s);
#pragma unroll
                for (int t = 0; t < NBW; ++t) braw[t] = tr_frag<G_::BROW>(Bt, ba[K][t], s);
                const float4 w0 = lds_ld<float4>(M, ma[K] + offsetof(TrMeta<Q>, w) + 128 * s);
                const float4 w1 = lds_ld<float4>(M, ma[K] + offsetof(TrMeta<Q>, w) + 128 * s + 64);
                if constexpr (kMixed) {
                    // only the last sequence's tokens enter the chunk's state
                    const uint4 km = seq_keep_mask(M, ma[K], s, seq_last);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) xf[pb] = frag_and(xf[pb], km);
#pragma unroll
                    for (int t = 0; t < NBW; ++t) braw[t] = frag_and(braw[t], km);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < NBW; ++t) {
                    const Frag<uint16_t> bw = scale_frag(braw[t], w0, w1);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) mma(h[t][pb], bw, xf[pb]);
                }
            }
            if (has_next) copies(s, c, Xn, Bn, Mn);
        }
        if constexpr (kOut) {
            if (has_next && st()) {
#pragma unroll
                for (int t = 0; t < NBW; ++t)
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb)
                        lds_st<uint2>(ho[K ^ 1], hw[K ^ 1][t] + 16 * pb * G_::HROW,
                                      make_uint2(pack_bf16x2(h[t][pb][0], h[t][pb][1]),
                                                 pack_bf16x2(h[t][pb][2], h[t][pb][3])));
            }
        }
        if constexpr (kSeq) seq_prev = lds_ld<int>(M, mb + offsetof(TrMeta<Q>, seq) + 4 * (Q - 1));
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's copies of chunk c+1 have landed
        __syncthreads();
    }

    __device__ __forceinline__ void state_load(const float* __restrict__ src) {
#pragma unroll
        for (int t = 0; t < NBW; ++t)
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb) {
                if (src && st()) {
                    const float4 v = *reinterpret_cast<const float4*>(
                        src + (16 * pb + r16) * N + 16 * (nb + t) + 4 * g);
                    h[t][pb] = f32x4_t{v.x, v.y, v.z, v.w};
                } else {
                    h[t][pb] = acc_zero();
                }
            }
    }

    // Offset of this lane's four values of state block (n-block nb, p-block
    // pb) in the register-order layout of the segment states: blocks
    // [nb][pb] of 64 lanes x 4 floats, so that a wave moves 1 KB contiguous.
    __device__ __forceinline__ int reg_order(int nbk, int pb) const {
        return ((nbk * G_::PB + pb) * kWave + lane) * 4;
    }

    // h = m_s h + S_s over the segments s < count in order (m_s = 0 at a
    // sequence reset: h = S_s); mult[s] and the P x N states[s] (register
    // order) as written by the segment-state kernel.  The loads of kCarryBatch segments are issued
    // before any of them is combined.
    static constexpr int kCarryBatch = 2;
    __device__ __forceinline__ void state_carry(const float* __restrict__ mult,
                                                const float* __restrict__ states, int count) {
        for (int s0 = 0; s0 < count; s0 += kCarryBatch) {
            float4 v[kCarryBatch][NBW][G_::PB];
            float m[kCarryBatch];
#pragma unroll
            for (int u = 0; u < kCarryBatch; ++u) {
                if (s0 + u < count) {
                    m[u] = mult[s0 + u];
                    const float* src = states + static_cast<int64_t>(s0 + u) * P * N;
#pragma unroll
                    for (int t = 0; t < NBW; ++t)
#pragma unroll
                        for (int pb = 0; pb < G_::PB; ++pb)
                            v[u][t][pb] = *reinterpret_cast<const float4*>(src + reg_order(nb + t, pb));
                }
            }
#pragma unroll
            for (int u = 0; u < kCarryBatch; ++u) {
                if (s0 + u < count) {
#pragma unroll
                    for (int t = 0; t < NBW; ++t)
#pragma unroll
                        for (int pb = 0; pb < G_::PB; ++pb) {
                            const float vv[4] = {v[u][t][pb].x, v[u][t][pb].y, v[u][t][pb].z, v[u][t][pb].w};
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                h[t][pb][r] = m[u] != 0.0f ? fmaf(m[u], h[t][pb][r], vv[r]) : vv[r];
                        }
                }
            }
        }
    }

    // the state in register order (segment states)
    __device__ __forceinline__ void state_store_reg(float* __restrict__ dst) const {
        if (!st()) return;
#pragma unroll
        for (int t = 0; t < NBW; ++t)
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb)
                *reinterpret_cast<float4*>(dst + reg_order(nb + t, pb)) =
                    make_float4(h[t][pb][0], h[t][pb][1], h[t][pb][2], h[t][pb][3]);
    }

    // the state as [p][n] (final states)
    __device__ __forceinline__ void state_store(float* __restrict__ dst) const {
        if (!st()) return;
#pragma unroll
        for (int t = 0; t < NBW; ++t)
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb)
                *reinterpret_cast<float4*>(dst + (16 * pb + r16) * N + 16 * (nb + t) + 4 * g) =
                    make_float4(h[t][pb][0], h[t][pb][1], h[t][pb][2], h[t][pb][3]);
    }
};

// LDS of one workgroup (separate objects per buffer: the compiler then knows
// that reads of one buffer do not wait for copies into the other).
template <int P, int N, int Q, bool kOut>
struct TrLds {
    char* x[2];
    char* b[2];
    TrMeta<Q>* m[2];
    char* h[2];
    float* cj;
};

// One (row, head, segment) from set-up to the final stores.
template <int P, int N, int Q, bool kOut, bool kSeq, int kDec>
__device__ __forceinline__ void scan_tr_run(const ScanArgs& a, const TrLds<P, N, Q, kOut>& s, uint32_t widx) {
    using G_ = TrGeo<P, N, Q>;
    using S_ = TrScan<P, N, Q, kOut, kSeq, kDec>;
    S_ k(a);
    const WorkItem it = decode_work_at(a, kOut ? a.nseg : a.nseg - 1, widx);
    k.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    k.lane = static_cast<int>(threadIdx.x) % kWave;
    k.r16 = k.lane & 15;
    k.g = k.lane >> 4;
    k.nb = (k.wave - TrWaves<kOut, kDec>::first_state) * S_::NBW;
    k.st_wave_ = k.nb >= 0 && k.nb < G_::NNB;
    const int64_t bh = it.b * a.H + it.h;
    const RowSpan rs = row_span(a, it.b);
    k.L = static_cast<int>(rs.len);
    k.nc = a.nc;
    k.c_begin = it.seg * a.cps;
    // no chunks when the row ends before this segment
    k.c_end = min(k.c_begin + a.cps, static_cast<int>((rs.len + Q - 1) / Q));
    const bool any = k.c_begin < k.c_end;
    // decode output in two passes: kDec = 1 takes the rows whose chunk does
    // not complete, kDec = 2 those whose chunk does
    if constexpr (kDec == 1) {
        if (!any || rs.len == a.L) return;
    } else if constexpr (kDec == 2) {
        if (rs.len != a.L) return;
    }
    // (decode output: a slot's state moves on at chunk ends only)
    k.want_final = kOut && it.seg == a.nseg - 1 && a.final_states != nullptr && rs.live &&
                   (a.y_last == nullptr || rs.len == a.L);
    k.out_wave_ = kDec || (kOut && k.wave < G_::NB);
    k.pb0 = kDec ? k.wave : 0;
    k.commit_ = kDec == 2 && k.want_final;
    k.row_state_ = rs.state;
    k.head_ = it.h;
    if constexpr (kDec) {
        // the row block of the row's last token (rows of one chunk)
        k.I = rs.len > 0 ? static_cast<int>((rs.len - 1) >> 4) : 0;
    } else {
        k.I = kOut && k.wave < kTrWaves ? tr_row_block<G_::NB>(k.wave) : 0;
    }
    k.Dh = (kOut && a.D) ? a.D[it.h] : 0.0f;
    k.Ah = a.A[it.h];
    k.mult = 1.0f;
    k.xstride = a.H * P * 2;
    k.bstride = a.G * N * 2;
    k.xg = static_cast<const uint16_t*>(a.x) + (rs.t0 * a.H + it.h) * P;
    k.bg = static_cast<const uint16_t*>(a.B) + (rs.t0 * a.G + it.g) * N;
    k.cm_cstride = static_cast<int64_t>(a.G) * Q * N;
    k.cmg = static_cast<const uint16_t*>(a.cmf) + (it.b * a.nc * a.G + it.g) * static_cast<int64_t>(Q) * N;
    k.yg = static_cast<uint16_t*>(a.y) + (rs.t0 * a.H + it.h) * P;
    k.ylg = kOut && a.y_last ? static_cast<uint16_t*>(a.y_last) + bh * P : nullptr;
    k.mg = a.cs + meta_offset(a, it.b, it.h, 0, Q);
    k.sqg = a.seq_idx ? a.seq_idx + rs.t0 : nullptr;
    k.cb_cstride = static_cast<int64_t>(a.G) * cbt_elems_per_chunk_group(Q);
    k.cbg = static_cast<const uint16_t*>(a.cbt) + (it.b * a.nc * a.G + it.g) * (k.cb_cstride / a.G);
    k.seq_prev = 0;
    if constexpr (kSeq) {
        const int64_t tp = k.c_begin == 0 ? 0 : static_cast<int64_t>(k.c_begin) * Q - 1;
        if (any) k.seq_prev = a.seq_idx[rs.t0 + tp];
    }

    // lane addresses and copy offsets, fixed for the whole segment
    const int st_nb = k.st() ? k.nb : 0;
    const int hx = G_::HROW == 256 ? k.r16 : ((k.r16 & 7) ^ ((k.r16 >> 3) & 1));  // h_off's swizzle
#pragma unroll
    for (int K = 0; K < 2; ++K) {
        k.xo[K] = s.x[K];
        k.bo[K] = s.b[K];
        k.mo[K] = s.m[K];
        k.ho[K] = s.h[K];
        k.xa[K] = lds_keep(lds_addr(s.x[K]) + tr_lane_off<G_::XROW>(0, k.lane));
#pragma unroll
        for (int t = 0; t < S_::NBW; ++t) {
            k.ba[K][t] = lds_keep(lds_addr(s.b[K]) + tr_lane_off<G_::BROW>(st_nb + t, k.lane));
            k.hw[K][t] = lds_keep(lds_addr(s.h[K]) + k.r16 * G_::HROW +
                                  (((2 * (st_nb + t) + (k.g >> 1)) ^ hx) << 4) + 8 * (k.g & 1));
        }
        k.ha[K] = lds_keep(lds_addr(s.h[K]) + k.r16 * G_::HROW + ((k.g ^ hx) << 4));
        k.ma[K] = lds_keep(lds_addr(s.m[K]) + 16 * k.g);
        k.mbase[K] = lds_addr(s.m[K]);
    }
    k.cjo = s.cj;
    const int cw = k.ow() ? k.wave : 0;  // output waves own a column-factor row each
    k.cja = lds_keep(lds_addr(s.cj) + 4 * Q * cw + 16 * k.g);
    k.cjw = lds_keep(lds_addr(s.cj) + 4 * Q * cw + 4 * k.lane);
#pragma unroll
    for (int kk = 0; kk < S_::XI; ++kk)
        k.xv[kk] = lds_keep(dma_voff<G_::XROW, S_::W>(kk, k.wave, k.lane, k.xstride));
#pragma unroll
    for (int kk = 0; kk < S_::BI; ++kk)
        k.bv[kk] = lds_keep(dma_voff<G_::BROW, S_::W>(kk, k.wave, k.lane, k.bstride));
    k.cv = lds_keep(static_cast<uint32_t>(k.I * G_::KN * 1024 + 16 * k.lane));

    // Role set-up, chunk loop and final stores per role, so that each role's
    // registers are live only in its own code; both roles pass the same number
    // of barriers (one after the first copies, one per chunk).
    if (k.ow()) {
        if (any) {
            k.load_c(k.c_begin);
            k.load_cb(k.c_begin);
            k.dma_all(s.x[0], s.b[0], s.m[0], k.c_begin);
        }
        if constexpr (kDec)
            k.load_state_operand(a.init && rs.live ? a.init + (rs.state * a.H + it.h) * P * N : nullptr);
        if constexpr (kDec == 2) {
            if (k.commit_) k.load_state_f32(a.init && rs.live ? a.init + (rs.state * a.H + it.h) * P * N : nullptr);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        for (int c = k.c_begin; c < k.c_end; c += 2) {
            k.template chunk_out<0>(c, s.x[1], s.b[1], s.m[1]);
            if (c + 1 < k.c_end) k.template chunk_out<1>(c + 1, s.x[0], s.b[0], s.m[0]);
        }
    } else {
        // the first chunk's copies, then (in flight together with them) the
        // incoming state.  Output kernel: the initial state (or zero) carried
        // through the end states of the earlier segments, and its bf16 operand
        // copy in H[0].
        if (any) k.dma_all(s.x[0], s.b[0], s.m[0], k.c_begin);
        // the initial state of the row (or of its slot)
        const int64_t sh = rs.state * a.H + it.h;
        k.state_load(kOut && a.init && rs.live ? a.init + sh * P * N : nullptr);
        if constexpr (kOut) {
            if (k.st()) k.state_carry(a.seg_mult + bh * a.nseg, a.seg_state + bh * a.nseg * P * N, it.seg);
            if (k.st()) {
#pragma unroll
                for (int t = 0; t < S_::NBW; ++t)
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb)
                        lds_st<uint2>(k.ho[0], k.hw[0][t] + 16 * pb * G_::HROW,
                                      make_uint2(pack_bf16x2(k.h[t][pb][0], k.h[t][pb][1]),
                                                 pack_bf16x2(k.h[t][pb][2], k.h[t][pb][3])));
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        for (int c = k.c_begin; c < k.c_end; c += 2) {
            k.template chunk_st<0>(c, s.x[1], s.b[1], s.m[1]);
            if (c + 1 < k.c_end) k.template chunk_st<1>(c + 1, s.x[0], s.b[0], s.m[0]);
        }
        if constexpr (kOut) {
            if (k.want_final) k.state_store(a.final_states + sh * P * N);
        } else {
            const int64_t slot = bh * a.nseg + it.seg;
            k.state_store_reg(a.seg_state + slot * P * N);
            if (threadIdx.x == 0) a.seg_mult[slot] = k.mult;
        }
    }
}

// The chunked scan over one (row, head, segment), as chunk_scan_kernel:
//   kOut = false: end states of segments 0 .. nseg-2 (from a zero state) and
//                 their decay multipliers, written to the workspace;
//   kOut = true:  outputs of every segment from its incoming state; final
//                 states from the last segment.
// kDec: the decode-output forms (one chunk per row, so the second buffers are
// never used and take no LDS; one column-factor row per output wave).
template <int P, int N, int Q, bool kOut, bool kSeq, int kDec>
__global__ __launch_bounds__((TrWaves<kOut, kDec>::kThreads)) void scan_tr_kernel(ScanArgs a) {
    using G_ = TrGeo<P, N, Q>;
    // sizes and alignments of the tiles, or of 16-byte stubs where a form has
    // no such tile (kDec: no second buffers and no state operand; kDec = 1:
    // no B tile)
    constexpr bool kB = kDec != 1, kX1 = !kDec, kH0 = kOut && !kDec, kH1 = kOut && !kDec;
    __shared__ __attribute__((aligned(1024))) char sX0[G_::XBYTES];
    __shared__ __attribute__((aligned(kX1 ? 1024 : 16))) char sX1[kX1 ? G_::XBYTES : 16];
    __shared__ __attribute__((aligned(kB ? 1024 : 16))) char sB0[kB ? G_::BBYTES : 16];
    __shared__ __attribute__((aligned(kX1 ? 1024 : 16))) char sB1[kX1 ? G_::BBYTES : 16];
    __shared__ __attribute__((aligned(16))) TrMeta<Q> sM0;
    __shared__ __attribute__((aligned(16))) char sM1[kX1 ? sizeof(TrMeta<Q>) : 16];
    __shared__ __attribute__((aligned(kH0 ? 1024 : 16))) char sH0[kH0 ? G_::HBYTES : 16];
    __shared__ __attribute__((aligned(kH1 ? 1024 : 16))) char sH1[kH1 ? G_::HBYTES : 16];
    // column factors: one row per output wave
    constexpr int kCj = kDec ? G_::PB * Q : (kOut ? kTrWaves * Q : 4);
    __shared__ __attribute__((aligned(16))) float sCj[kCj];
    const TrLds<P, N, Q, kOut> lds{{sX0, sX1}, {sB0, sB1},
                                   {&sM0, reinterpret_cast<TrMeta<Q>*>(sM1)}, {sH0, sH1}, sCj};

    if constexpr (kDec == 2) {
        // rows whose chunk completes, among this workgroup's work items
        // blockIdx.x + k gridDim.x: every wave checks 64 of them at a time
        // (one per lane) and the workgroup runs the ones that qualify
        const uint32_t n = static_cast<uint32_t>(a.dec_items), step = gridDim.x;
        const uint32_t lane = threadIdx.x % kWave;
        for (uint32_t k0 = 0; blockIdx.x + k0 * step < n; k0 += kWave) {
            const uint32_t w = blockIdx.x + (k0 + lane) * step;
            const bool run = w < n && row_span(a, decode_work_at(a, a.nseg, w).b).len == a.L;
            uint64_t m = __builtin_amdgcn_ballot_w64(run);
            while (m != 0) {
                const uint32_t j = static_cast<uint32_t>(__builtin_ctzll(m));
                m &= m - 1;
                scan_tr_run<P, N, Q, kOut, kSeq, kDec>(a, lds, blockIdx.x + (k0 + j) * step);
                __syncthreads();  // the next item's copies overwrite the tiles
            }
        }
    } else {
        scan_tr_run<P, N, Q, kOut, kSeq, kDec>(
            a, lds, static_cast<uint32_t>(xcd_work_index(blockIdx.x, gridDim.x)));
    }
}

// Compute units of the current device (queried once per device).
int device_cus() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cus[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 1;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            return 1;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int P, int N, int Q, bool kOut>
hipError_t launch_scan_tr(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(nblocks));
    if constexpr (kOut) {
        // decode output (rows of one chunk, no seq_idx): pass 1, the rows
        // whose chunk does not complete (kDec = 1, one workgroup each); pass
        // 2, the others (kDec = 2) on as many workgroups as the device holds
        // at once, each walking its share of the work items (so that a pass
        // with no such row costs one round of workgroups)
        if (a.y_last && !a.seq_idx) {
            if (a.dec_pass == 1)
                return dispatch(scan_tr_kernel<P, N, Q, true, false, 1>, grid,
                                dim3(TrWaves<true, 1>::kThreads), st, a);
            if (a.dec_pass != 2) return hipErrorInvalidValue;
            constexpr int kThreads = TrWaves<true, 2>::kThreads;
            static const int per_cu = [] {
                int n = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &n, scan_tr_kernel<P, N, Q, true, false, 2>, kThreads, 0) != hipSuccess)
                    n = 1;
                return n < 1 ? 1 : n;
            }();
            ScanArgs c = a;
            c.dec_items = nblocks;
            const int64_t cap = static_cast<int64_t>(per_cu) * device_cus();
            return dispatch(scan_tr_kernel<P, N, Q, true, false, 2>,
                            dim3(static_cast<unsigned>(nblocks < cap ? nblocks : cap)),
                            dim3(kThreads), st, c);
        }
    }
    const dim3 block(TrWaves<kOut>::kThreads);
    if (a.seq_idx) return dispatch(scan_tr_kernel<P, N, Q, kOut, true, 0>, grid, block, st, a);
    return dispatch(scan_tr_kernel<P, N, Q, kOut, false, 0>, grid, block, st, a);
}

}  // namespace

#define SSD_SCAN_TR(P, N, Q)                                                                  \
    hipError_t scan_tr_state_##P##_##N##_##Q(const ScanArgs& a, int64_t nb, hipStream_t st) { \
        return launch_scan_tr<P, N, Q, false>(a, nb, st);                                     \
    }                                                                                         \
    hipError_t scan_tr_output_##P##_##N##_##Q(const ScanArgs& a, int64_t nb, hipStream_t st) { \
        return launch_scan_tr<P, N, Q, true>(a, nb, st);                                      \
    }

SSD_SCAN_TR(64, 64, 64)
SSD_SCAN_TR(64, 64, 128)
SSD_SCAN_TR(64, 128, 64)
SSD_SCAN_TR(64, 128, 128)

}  // namespace ssd
