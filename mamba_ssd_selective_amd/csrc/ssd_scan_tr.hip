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
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_work.h"

#define SSD_LDS __attribute__((address_space(3)))
#define SSD_GLOBAL __attribute__((address_space(1)))

namespace ssd {
namespace {

constexpr int kTrThreads = 512;
constexpr int kTrWaves = kTrThreads / kWave;
// Word 3 of a raw (unswizzled, untyped) buffer resource on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maximum.
constexpr int kWaitVmcnt0 = 0x0F70;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------- LDS layout

// Tiles read by transposing reads: 32-byte unit u of row r is stored at unit
// u ^ tr_swz(r).  Sixteen lanes of one such read cover four consecutive rows
// (32 bytes each), 32 lanes eight rows; the swizzle puts them on distinct
// banks for either phase width.
template <int ROW>
__device__ __forceinline__ int tr_swz(int r) {
    if constexpr (ROW == 128) return (r & 3) ^ ((r >> 2) & 1);
    else return r & 7;
}
template <int ROW>
__device__ __forceinline__ int tr_off(int r, int byte_col) {
    return r * ROW + (((byte_col >> 5) ^ tr_swz<ROW>(r)) << 5) + (byte_col & 31);
}

// State operand sH[p][n]: 16-byte slot s of row p is stored at slot s ^ x(p);
// sixteen consecutive rows read one slot each in a ds_read_b128.
template <int HROW>
__device__ __forceinline__ int h_off(int p, int slot) {
    constexpr int S = HROW / 16;
    const int x = S == 16 ? (p & 15) : ((p & 7) ^ ((p >> 3) & 1));
    return p * HROW + ((slot ^ x) << 4);
}

__device__ __forceinline__ uint2 ds_tr16(const char* p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSD_LDS i16x4_t*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Lane byte offset of the transposing read of column block mb at k step 0.
// A ds_read_b64_tr_b16 returns to lane i of a 16-lane group element k of the
// 4-element read of lane i/4 + 4k in that group, position i % 4; so lane jj
// of group g reads row 4g + jj/4, columns 16mb + 4(jj % 4) .. +3, and lane i
// receives column 16mb + i of rows 4g .. 4g + 3.
template <int ROW>
__device__ __forceinline__ int tr_lane_off(int mb, int lane) {
    const int g = lane >> 4, jj = lane & 15;
    return tr_off<ROW>(4 * g + (jj >> 2), 32 * mb + 8 * (jj & 3));
}

// Operand fragment of k step s from a [token][column] tile.  The swizzle of
// rows r, r + 16 and r + 32s is the same, so steps are plain row offsets.
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> tr_frag(const char* tile, int off, int s) {
    const uint2 lo = ds_tr16(tile + off + 32 * s * ROW);
    const uint2 hi = ds_tr16(tile + off + (32 * s + 16) * ROW);
    Frag<uint16_t> f;
    f.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
    return f;
}

__device__ __forceinline__ float bf_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Fragment elements (token order above) scaled by per-token weights.
__device__ __forceinline__ Frag<uint16_t> scale_frag(const Frag<uint16_t>& f, const float4& w0,
                                                     const float4& w1) {
    const uint4 u = __builtin_bit_cast(uint4, f.v);
    const float v[8] = {bf_lo(u.x) * w0.x, bf_hi(u.x) * w0.y, bf_lo(u.y) * w0.z,
                        bf_hi(u.y) * w0.w, bf_lo(u.z) * w1.x, bf_hi(u.z) * w1.y,
                        bf_lo(u.w) * w1.z, bf_hi(u.w) * w1.w};
    return frag_from_f32<uint16_t>(v);
}

__device__ __forceinline__ Frag<uint16_t> frag_of(const uint4& u) {
    Frag<uint16_t> f;
    f.v = __builtin_bit_cast(bf16x8_t, u);
    return f;
}

// ---------------------------------------------------------- global -> LDS

// Copy instructions kk in [k0, k1) (kk < KMAX) of this wave (instruction
// k = wave + 8 kk covers 1024 bytes) of a swizzled [token][ROW bytes] tile; row
// r comes from byte r * gstride of the resource, and rows past its range read
// as zeros.  The loop unrolls fully, so constant bounds fold away.
template <int ROW, int KMAX>
__device__ __forceinline__ void dma_rows(char* lds, __amdgpu_buffer_rsrc_t rs, int gstride,
                                         int k0, int k1, int wave, int lane) {
    constexpr int RPI = 1024 / ROW;  // rows per wave instruction (64 lanes x 16 bytes)
    constexpr int SPR = ROW / 16;    // 16-byte slots per row
    static_assert(1024 % ROW == 0, "whole rows per instruction");
#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk) {
        if (kk >= k0 && kk < k1) {
            const int k = wave + kTrWaves * kk;
            const int row = k * RPI + lane / SPR;
            const int slot = (lane % SPR) ^ (2 * tr_swz<ROW>(row));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (SSD_LDS void*)(lds + k * 1024), 16,
                                                     row * gstride + slot * 16, 0, 0, 0);
        }
    }
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

template <int P, int N, int Q, bool kOut, bool kSeq>
struct TrScan {
    using G_ = TrGeo<P, N, Q>;
    static constexpr int XI = G_::XBYTES / 1024 / kTrWaves;  // x-tile copy instructions per wave
    static constexpr int BI = G_::BBYTES / 1024 / kTrWaves;  // B-tile copy instructions per wave
    static_assert(XI >= 1 && BI >= 1 && G_::XBYTES % (1024 * kTrWaves) == 0 &&
                      G_::BBYTES % (1024 * kTrWaves) == 0, "tile copy split");

    const ScanArgs& a;
    int wave, lane, r16, g;
    int c_begin, c_end, L, nc;
    bool last_seg, want_final;
    bool fast_;             // factored intra-chunk decays (every dt * A <= 0 in the segment)
    bool st_wave_, out_wave_;
    // every wave owns a state n-block / an output row block when there are 8
    __device__ __forceinline__ bool st() const { return G_::NNB == kTrWaves || st_wave_; }
    __device__ __forceinline__ bool ow() const { return kOut && (G_::NB == kTrWaves || out_wave_); }
    int I;                  // output row block of this wave
    float Dh, Ah;           // D[h], A[h]
    int xoff[G_::PB], boff; // transposing-read lane offsets (x per p block, B of n block `wave`)
    int seq_prev;           // sequence id of the token before the current chunk
    float mult;             // decay of the segment (chunk-state kernel)
    // per-(row, head) / per-(row, group) bases; chunk c adds c times the chunk stride
    const uint16_t* xg;  int xstride;   // x[b][.][h][0], token stride in bytes
    const uint16_t* bg;  int bstride;   // B[b][.][g][0]
    const uint16_t* cg;                 // C[b][.][g][0] (stride bstride)
    uint16_t* yg;                       // y[b][.][h][0]
    const float* mg;                    // metadata block (b, h, chunk 0): [cs | dt | w]
    const int32_t* sqg;                 // seq_idx[b][0]
    const uint16_t* cbg;                // C.B^T tiles at (b, chunk 0, g)
    int64_t cb_cstride;                 // elements between chunks of the tile buffer

    f32x4_t h[G_::PB];          // state rows n = 16 wave + 4g + r, column p = 16pb + r16
    uint4 cr[G_::KN];           // C rows of a chunk (k over n), loaded a chunk ahead
    uint4 cb[G_::NCB];          // C.B^T tile pairs of a chunk, loaded a chunk ahead
    uint2 ypk[G_::PB];          // packed outputs awaiting their store
    uint16_t* ypos;
    bool ypend;

    __device__ __forceinline__ TrScan(const ScanArgs& args) : a(args) {}

    __device__ __forceinline__ int rows_in(int c) const {
        const int64_t rem = static_cast<int64_t>(L) - static_cast<int64_t>(c) * Q;
        return rem < Q ? static_cast<int>(rem) : Q;
    }

    __device__ __forceinline__ void load_c(int c) {
        const __amdgpu_buffer_rsrc_t rs =
            rows_rsrc(cg + static_cast<int64_t>(c) * Q * (bstride / 2), rows_in(c), bstride);
#pragma unroll
        for (int s = 0; s < G_::KN; ++s) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (16 * I + r16) * bstride + (32 * s + 8 * g) * 2, 0, 0);
            cr[s] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }

    __device__ __forceinline__ void load_cb(int c) {
        const uint16_t* tiles = cbg + static_cast<int64_t>(c) * cb_cstride;
        const int first = cb_pair_base(I);
#pragma unroll
        for (int u = 0; u < G_::NCB; ++u)
            if (2 * u <= I) cb[u] = *reinterpret_cast<const uint4*>(tiles + ((first + u) * 64 + lane) * 8);
    }

    // Copies of chunk c+1, split so that they spread over the chunk's math.
    __device__ __forceinline__ void dma_x(char* sX, int c) const {
        const __amdgpu_buffer_rsrc_t rs =
            rows_rsrc(xg + static_cast<int64_t>(c) * Q * (xstride / 2), rows_in(c), xstride);
        dma_rows<G_::XROW, XI>(sX, rs, xstride, 0, XI, wave, lane);
    }
    __device__ __forceinline__ void dma_b(char* sB, int c, int k0, int k1) const {
        if (k0 < k1) {
            const __amdgpu_buffer_rsrc_t rs =
                rows_rsrc(bg + static_cast<int64_t>(c) * Q * (bstride / 2), rows_in(c), bstride);
            dma_rows<G_::BROW, BI>(sB, rs, bstride, k0, k1, wave, lane);
        }
    }
    // [cs | dt | w] of a chunk is one contiguous block of 3Q floats (Q * 3/4
    // pieces of 16 bytes) in the workspace and in TrMeta.
    __device__ __forceinline__ void dma_meta(TrMeta<Q>* sM, int c) const {
        constexpr int NPC = 3 * Q / 4;       // 16-byte pieces
        const int mw = kTrWaves - 1 - wave;  // from the last waves
        const int piece = kWave * mw + lane;
        if (kWave * mw < NPC && piece < NPC) {
            const float* src = mg + static_cast<int64_t>(c) * (3 * Q) + 4 * piece;
            float* dst = reinterpret_cast<float*>(sM) + 4 * kWave * mw;  // [cs | dt | w] in order
            __builtin_amdgcn_global_load_lds((SSD_GLOBAL void*)(src), (SSD_LDS void*)(dst), 16, 0, 0);
        }
        if constexpr (kSeq) {
            if (mw == (NPC + kWave - 1) / kWave && lane < Q / 4) {
                const __amdgpu_buffer_rsrc_t rs = rows_rsrc(sqg + static_cast<int64_t>(c) * Q, rows_in(c), 4);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (SSD_LDS void*)(sM->seq), 16, 16 * lane, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void dma_all(char* sX, char* sB, TrMeta<Q>* sM, int c) const {
        dma_x(sX, c);
        dma_b(sB, c, 0, BI);
        dma_meta(sM, c);
    }

    // G^T fragment of k step u, exact form: lane column i = 16I + r16, tokens
    // j in the k order above; G[i][j] = (C_i . B_j) exp(cs_i - cs_j) dt_j,
    // masked to j <= i and (with sequence ids) seq_j = seq_i; D[h] is added on
    // the diagonal (the D x skip rides on the same MFMA).
    __device__ __forceinline__ Frag<uint16_t> g_exact(const uint4& t, const TrMeta<Q>& m, int u,
                                                      float cs_i, int seq_i) const {
        // token 16J + 4g + r of tile J is kept when r <= lim: all of a tile left
        // of the diagonal, r <= r16 - 4g on it, none right of it
        int tdiag = r16 - 4 * g;
        // opaque to the optimizer: keeps the per-element compares here instead
        // of hoisting them out of the chunk loop as 64-bit lane masks
        asm volatile("" : "+v"(tdiag));
        float out[8];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            const int J = 2 * u + hp;
            const int jb = 32 * u + 16 * hp + 4 * g;
            const float4 cs4 = *reinterpret_cast<const float4*>(&m.cs[jb]);
            const float4 dt4 = *reinterpret_cast<const float4*>(&m.dt[jb]);
            int4 sq4 = make_int4(0, 0, 0, 0);
            if constexpr (kSeq) sq4 = *reinterpret_cast<const int4*>(&m.seq[jb]);
            const uint32_t d0 = hp ? t.z : t.x, d1 = hp ? t.w : t.y;
            const float cbv[4] = {bf_lo(d0), bf_hi(d0), bf_lo(d1), bf_hi(d1)};
            const float csv[4] = {cs4.x, cs4.y, cs4.z, cs4.w};
            const float dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
            const int sqv[4] = {sq4.x, sq4.y, sq4.z, sq4.w};
            const int lim = J < I ? 3 : (J == I ? tdiag : -1);
            const int dlim = J == I ? tdiag : -1;  // D on the diagonal element
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bool keep = r <= lim;
                if constexpr (kSeq) keep = keep && sqv[r] == seq_i;
                // masked elements may overflow here; the select drops them
                const float v = cbv[r] * decay_exp(cs_i - csv[r]) * dtv[r];
                out[4 * hp + r] = (keep ? v : 0.0f) + (r == dlim ? Dh : 0.0f);
            }
        }
        return frag_from_f32<uint16_t>(out);
    }

    // Factored form for k steps strictly left of row block I (all j < 16I):
    // G[i][j] = r_i * (C_i . B_j) c_j with c_j = [seq_j = seq_m] exp(cs_m - cs_j) dt_j
    // (m = 16I, from this wave's scratch) and the row factor r_i applied to the
    // accumulator later.
    __device__ __forceinline__ Frag<uint16_t> g_factored(const uint4& t, const float* cj, int u) const {
        const float4 c0 = *reinterpret_cast<const float4*>(&cj[32 * u + 4 * g]);
        const float4 c1 = *reinterpret_cast<const float4*>(&cj[32 * u + 16 + 4 * g]);
        const float v[8] = {bf_lo(t.x) * c0.x, bf_hi(t.x) * c0.y, bf_lo(t.y) * c0.z,
                            bf_hi(t.y) * c0.w, bf_lo(t.z) * c1.x, bf_hi(t.z) * c1.y,
                            bf_lo(t.w) * c1.z, bf_hi(t.w) * c1.w};
        return frag_from_f32<uint16_t>(v);
    }

    __device__ __forceinline__ void store_y() {
        if (ypend) {
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb) *reinterpret_cast<uint2*>(ypos + 16 * pb) = ypk[pb];
        }
        ypend = false;
    }

    // One chunk.  On entry chunk c's tiles and metadata are in (X, Bt, M), the
    // state before it in H (bf16 operand copy) and h (fp32, state waves), and
    // its C rows and C.B^T tiles in cr, cb.  Issues chunk c+1's loads
    // into the other buffers while it works, and leaves after a barrier with
    // them complete.
    template <int K>
    __device__ __forceinline__ void chunk(int c, const char* X, const char* Bt, const TrMeta<Q>* M,
                                          const char* H, char* Xn, char* Bn, TrMeta<Q>* Mn,
                                          char* Hn, float* cj) {
        const bool has_next = c + 1 < c_end;
        const int valid = rows_in(c);
        const TrMeta<Q>& m = *M;

        if constexpr (kOut) store_y();  // previous chunk's outputs
        const float cs_last = m.cs[Q - 1];
        const int seq_last = kSeq ? m.seq[valid - 1] : 0;

        const bool fast = kOut && fast_;
        f32x4_t y[G_::PB];
        int i = 0;
        float cs_i = 0.0f, r_i = 1.0f;
        int seq_i = 0;
        if constexpr (kOut) {
            if (ow()) {
                // carried-state term: y^T[p][i] = exp(cs_i) [seq_i = seq_prev] h.C_i,
                // with exp(cs_i) = r_i exp(cs_m) in the factored form
                i = 16 * I + r16;
                const int m0 = 16 * I;
                cs_i = m.cs[i];
                const float cs_m = m.cs[m0];
                int seq_m = 0;
                if constexpr (kSeq) {
                    seq_i = m.seq[i];
                    seq_m = m.seq[m0];
                }
                Frag<uint16_t> hf[2][G_::PB];
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb) {
                    y[pb] = acc_zero();
                    hf[0][pb] = frag_of(*reinterpret_cast<const uint4*>(H + h_off<G_::HROW>(16 * pb + r16, g)));
                }
#pragma unroll
                for (int s = 0; s < G_::KN; ++s) {
                    if (s + 1 < G_::KN) {
#pragma unroll
                        for (int pb = 0; pb < G_::PB; ++pb)
                            hf[(s + 1) & 1][pb] = frag_of(*reinterpret_cast<const uint4*>(
                                H + h_off<G_::HROW>(16 * pb + r16, 4 * (s + 1) + g)));
                    }
                    const Frag<uint16_t> cf = frag_of(cr[s]);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) mma(y[pb], hf[s & 1][pb], cf);
                }
                // fast: exp(cs_i) = r_i exp(cs_m); r_i is applied at the diagonal step
                float sc = (!kSeq || seq_i == seq_prev) ? decay_exp(cs_i) : 0.0f;
                r_i = 1.0f;
                if (fast) {
                    r_i = (!kSeq || seq_i == seq_m) ? decay_exp(cs_i - cs_m) : 0.0f;
                    sc = (!kSeq || seq_m == seq_prev) ? decay_exp(cs_m) : 0.0f;
                    // column factors of the steps left of the row block
#pragma unroll
                    for (int k = 0; k < (Q + kWave - 1) / kWave; ++k) {
                        const int j = lane + kWave * k;
                        if (j < m0) {
                            bool keep = true;
                            if constexpr (kSeq) keep = m.seq[j] == seq_m;
                            cj[j] = keep ? decay_exp(cs_m - m.cs[j]) * m.dt[j] : 0.0f;
                        }
                    }
                }
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) y[pb][r] *= sc;
            }
        }
        if (has_next) {
            if constexpr (kOut) {
                if (ow()) load_c(c + 1);  // this chunk's C rows are consumed
            }
            dma_x(Xn, c + 1);
        }

        // h_c = [no reset in c] exp(cs_last) h_{c-1} + S_c
        {
            const float e = (!kSeq || seq_last == seq_prev) ? decay_exp(cs_last) : 0.0f;
            if (st()) {
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) h[pb][r] *= e;
            }
            if constexpr (!kOut) mult *= e;
        }

        // k steps over the chunk's tokens: S_c += (B w)^T x and the
        // intra-chunk outputs y^T += x^T G^T, sharing the x fragments
#pragma unroll
        for (int s = 0; s < G_::KQ; ++s) {
            const bool do_state = st();
            const bool do_out = kOut && ow() && 2 * s <= I;
            if (do_state || do_out) {
                Frag<uint16_t> xf[G_::PB];
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb) xf[pb] = tr_frag<G_::XROW>(X, xoff[pb], s);
                if (do_state) {
                    const float4 w0 = *reinterpret_cast<const float4*>(&m.w[32 * s + 4 * g]);
                    const float4 w1 = *reinterpret_cast<const float4*>(&m.w[32 * s + 16 + 4 * g]);
                    const Frag<uint16_t> bw = scale_frag(tr_frag<G_::BROW>(Bt, boff, s), w0, w1);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) mma(h[pb], bw, xf[pb]);
                }
                if constexpr (kOut) {
                    if (do_out) {
                        Frag<uint16_t> gf;
                        if (fast && 2 * s + 1 < I) {
                            gf = g_factored(cb[s], cj, s);
                        } else {
                            if (2 * s + 2 > I) {
                                // the diagonal step (last): apply the row factor first
#pragma unroll
                                for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
                                    for (int r = 0; r < 4; ++r) y[pb][r] *= r_i;
                            }
                            gf = g_exact(cb[s], m, s, cs_i, seq_i);
                        }
#pragma unroll
                        for (int pb = 0; pb < G_::PB; ++pb) mma(y[pb], xf[pb], gf);
                    }
                }
            }
            // spread the next chunk's copies over the steps
            if (has_next) {
                dma_b(Bn, c + 1, BI * s / G_::KQ, BI * (s + 1) / G_::KQ);
                if (s == 0) dma_meta(Mn, c + 1);
                if constexpr (kOut) {
                    if (s == G_::KQ - 1 && ow()) load_cb(c + 1);  // after the last use
                }
            }
        }

        if constexpr (kOut) {
            if (ow()) {
                ypk[0] = make_uint2(0, 0);
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb)
                    ypk[pb] = make_uint2(pack_bf16x2(y[pb][0], y[pb][1]), pack_bf16x2(y[pb][2], y[pb][3]));
                ypos = yg + (static_cast<int64_t>(c) * Q + i) * (xstride / 2) + 4 * g;
                ypend = i < valid;
            }
            // bf16 operand copy of h_c for the next chunk's carried-state term
            if (has_next && st()) {
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb) {
                    const int p = 16 * pb + r16;
                    *reinterpret_cast<uint2*>(Hn + h_off<G_::HROW>(p, 2 * wave + (g >> 1)) +
                                              8 * (g & 1)) =
                        make_uint2(pack_bf16x2(h[pb][0], h[pb][1]), pack_bf16x2(h[pb][2], h[pb][3]));
                }
            }
        }
        if constexpr (kSeq) seq_prev = m.seq[Q - 1];
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's copies of chunk c+1 have landed
        __syncthreads();
    }

    template <bool kFast>
    __device__ __forceinline__ void loop(char* sX0, char* sB0, TrMeta<Q>* sM0, char* sH0,
                                         char* sX1, char* sB1, TrMeta<Q>* sM1, char* sH1,
                                         float* cj) {
        for (int c = c_begin; c < c_end; c += 2) {
            chunk<0, kFast>(c, sX0, sB0, sM0, sH0, sX1, sB1, sM1, sH1, cj);
            if (c + 1 < c_end) chunk<1, kFast>(c + 1, sX1, sB1, sM1, sH1, sX0, sB0, sM0, sH0, cj);
        }
    }
    __device__ __forceinline__ void state_load(const float* __restrict__ src) {
#pragma unroll
        for (int pb = 0; pb < G_::PB; ++pb) {
            if (src && st()) {
                const float4 v = *reinterpret_cast<const float4*>(src + (16 * pb + r16) * N +
                                                                  16 * wave + 4 * g);
                h[pb] = f32x4_t{v.x, v.y, v.z, v.w};
            } else {
                h[pb] = acc_zero();
            }
        }
    }

    __device__ __forceinline__ void state_store(float* __restrict__ dst) const {
        if (!st()) return;
#pragma unroll
        for (int pb = 0; pb < G_::PB; ++pb)
            *reinterpret_cast<float4*>(dst + (16 * pb + r16) * N + 16 * wave + 4 * g) =
                make_float4(h[pb][0], h[pb][1], h[pb][2], h[pb][3]);
    }
};

// LDS of one workgroup (separate objects per buffer: the compiler then knows
// that reads of one buffer do not wait for copies into the other).
template <int P, int N, int Q, bool kOut>
struct TrLds {
    using G_ = TrGeo<P, N, Q>;
    char* x[2];
    char* b[2];
    TrMeta<Q>* m[2];
    char* h[2];
    float* cj;
};

// One (row, head, segment) from set-up to the final stores.  fast: every
// dt * A of the segment is <= 0 (see the kernel).
template <int P, int N, int Q, bool kOut, bool kSeq>
__device__ __forceinline__ void scan_tr_run(const ScanArgs& a, const TrLds<P, N, Q, kOut>& s,
                                            bool fast) {
    using G_ = TrGeo<P, N, Q>;
    TrScan<P, N, Q, kOut, kSeq> k(a);
    k.fast_ = fast;
    const WorkItem it = decode_work(a, kOut ? a.nseg : a.nseg - 1);
    k.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    k.lane = static_cast<int>(threadIdx.x) % kWave;
    k.r16 = k.lane & 15;
    k.g = k.lane >> 4;
    k.L = static_cast<int>(a.L);
    k.nc = a.nc;
    k.c_begin = it.seg * a.cps;
    k.c_end = min(k.c_begin + a.cps, a.nc);
    k.last_seg = kOut && it.seg == a.nseg - 1;
    k.want_final = k.last_seg && a.final_states != nullptr;
    k.st_wave_ = k.wave < G_::NNB;
    k.out_wave_ = kOut && k.wave < G_::NB;
    k.I = tr_row_block<G_::NB>(k.wave);
    k.Dh = (kOut && a.D) ? a.D[it.h] : 0.0f;
    k.Ah = a.A[it.h];
#pragma unroll
    for (int pb = 0; pb < G_::PB; ++pb) k.xoff[pb] = tr_lane_off<G_::XROW>(pb, k.lane);
    k.boff = tr_lane_off<G_::BROW>(k.st() ? k.wave : 0, k.lane);
    k.mult = 1.0f;
    k.ypend = false;
    k.ypos = nullptr;
    k.xstride = a.H * P * 2;
    k.bstride = a.G * N * 2;
    k.xg = static_cast<const uint16_t*>(a.x) + (it.b * a.L * a.H + it.h) * P;
    k.bg = static_cast<const uint16_t*>(a.B) + (it.b * a.L * a.G + it.g) * N;
    k.cg = static_cast<const uint16_t*>(a.C) + (it.b * a.L * a.G + it.g) * N;
    k.yg = static_cast<uint16_t*>(a.y) + (it.b * a.L * a.H + it.h) * P;
    k.mg = a.cs + meta_offset(a, it.b, it.h, 0, Q);
    k.sqg = a.seq_idx ? a.seq_idx + it.b * a.L : nullptr;
    k.cb_cstride = static_cast<int64_t>(a.G) * cbt_elems_per_chunk_group(Q);
    k.cbg = static_cast<const uint16_t*>(a.cbt) + (it.b * a.nc * a.G + it.g) * (k.cb_cstride / a.G);
    const int64_t bh = it.b * a.H + it.h;
    if constexpr (kSeq) {
        const int64_t tp = k.c_begin == 0 ? 0 : static_cast<int64_t>(k.c_begin) * Q - 1;
        k.seq_prev = a.seq_idx[it.b * a.L + tp];
    } else {
        k.seq_prev = 0;
    }
    float* cj = s.cj + (kOut ? k.wave * Q : 0);

    // incoming state: fp32 in registers, bf16 operand copy in h[0]
    if constexpr (kOut) {
        if (a.nseg == 1) k.state_load(a.init ? a.init + bh * P * N : nullptr);
        else k.state_load(a.seg_state + (bh * a.nseg + it.seg) * P * N);
        if (k.st()) {
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb) {
                const int p = 16 * pb + k.r16;
                *reinterpret_cast<uint2*>(s.h[0] + h_off<G_::HROW>(p, 2 * k.wave + (k.g >> 1)) +
                                          8 * (k.g & 1)) =
                    make_uint2(pack_bf16x2(k.h[pb][0], k.h[pb][1]), pack_bf16x2(k.h[pb][2], k.h[pb][3]));
            }
        }
        if (k.ow()) {
            k.load_c(k.c_begin);
            k.load_cb(k.c_begin);
        }
    } else {
        k.state_load(nullptr);
    }
    k.dma_all(s.x[0], s.b[0], s.m[0], k.c_begin);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    for (int c = k.c_begin; c < k.c_end; c += 2) {
        k.template chunk<0>(c, s.x[0], s.b[0], s.m[0], s.h[0], s.x[1], s.b[1], s.m[1], s.h[1], cj);
        if (c + 1 < k.c_end)
            k.template chunk<1>(c + 1, s.x[1], s.b[1], s.m[1], s.h[1], s.x[0], s.b[0], s.m[0],
                                       s.h[0], cj);
    }

    if constexpr (kOut) {
        k.store_y();
        if (k.want_final) k.state_store(a.final_states + bh * P * N);
    } else {
        const int64_t slot = bh * a.nseg + it.seg;
        k.state_store(a.seg_state + slot * P * N);
        if (threadIdx.x == 0) a.seg_mult[slot] = k.mult;
    }
}

// The chunked scan over one (row, head, segment), as chunk_scan_kernel:
//   kOut = false: end states of segments 0 .. nseg-2 (from a zero state) and
//                 their decay multipliers, written to the workspace;
//   kOut = true:  outputs of every segment from its incoming state; final
//                 states from the last segment.
template <int P, int N, int Q, bool kOut, bool kSeq>
__global__ __launch_bounds__(kTrThreads) void scan_tr_kernel(ScanArgs a) {
    using G_ = TrGeo<P, N, Q>;
    __shared__ __attribute__((aligned(16))) char sX0[G_::XBYTES];
    __shared__ __attribute__((aligned(16))) char sX1[G_::XBYTES];
    __shared__ __attribute__((aligned(16))) char sB0[G_::BBYTES];
    __shared__ __attribute__((aligned(16))) char sB1[G_::BBYTES];
    __shared__ __attribute__((aligned(16))) TrMeta<Q> sM0;
    __shared__ __attribute__((aligned(16))) TrMeta<Q> sM1;
    __shared__ __attribute__((aligned(16))) char sH0[kOut ? G_::HBYTES : 16];
    __shared__ __attribute__((aligned(16))) char sH1[kOut ? G_::HBYTES : 16];
    __shared__ __attribute__((aligned(16))) float sCj[kOut ? kTrWaves * Q : 4];
    const TrLds<P, N, Q, kOut> lds{{sX0, sX1}, {sB0, sB1}, {&sM0, &sM1}, {sH0, sH1}, sCj};

    if constexpr (kOut) {
        // The factored form of the intra-chunk decays needs dt_j * A <= 0 for
        // every token of the segment (cs then never increases inside a
        // sequence and every factor is at most 1); otherwise every k step takes
        // the exact form.
        const WorkItem it = decode_work(a, a.nseg);
        const int c0 = it.seg * a.cps, c1 = min(c0 + a.cps, a.nc);
        const float Ah = a.A[it.h];
        const float* blk = a.cs + meta_offset(a, it.b, it.h, c0, Q);
        const int n = (c1 - c0) * Q;
        int up = 0;
        for (int j = static_cast<int>(threadIdx.x); j < n; j += kTrThreads)
            up |= blk[(j / Q) * (3 * Q) + Q + j % Q] * Ah > 0.0f;  // dt of token j
        scan_tr_run<P, N, Q, true, kSeq>(a, lds, __syncthreads_or(up) == 0);
    } else {
        scan_tr_run<P, N, Q, false, kSeq>(a, lds, false);
    }
}

template <int P, int N, int Q, bool kOut>
hipError_t launch_scan_tr(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(nblocks));
    if (a.seq_idx)
        hipLaunchKernelGGL((scan_tr_kernel<P, N, Q, kOut, true>), grid, dim3(kTrThreads), 0, st, a);
    else
        hipLaunchKernelGGL((scan_tr_kernel<P, N, Q, kOut, false>), grid, dim3(kTrThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

#define SSD_SCAN_TR(P, N, Q)                                                                  \
    hipError_t scan_tr_state_##P##_##N##_##Q(const ScanArgs& a, int64_t nb, hipStream_t st) { \
        return launch_scan_tr<P, N, Q, false>(a, nb, st);                                     \
    }                                                                                         \
    hipError_t scan_tr_output_##P##_##N##_##Q(const ScanArgs& a, int64_t nb, hipStream_t st) { \
        return launch_scan_tr<P, N, Q, true>(a, nb, st);                                      \
    }

SSD_SCAN_TR(64, 64, 128)
SSD_SCAN_TR(64, 128, 64)
SSD_SCAN_TR(64, 128, 128)

}  // namespace ssd
