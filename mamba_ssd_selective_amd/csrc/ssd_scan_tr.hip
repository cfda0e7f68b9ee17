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

// Per-token metadata of one chunk (written by chunk_prep_kernel).
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

// Copy `rows` token rows of ROW bytes (row r at byte r * gstride from gbase)
// into a swizzled tile; rows at or past `rows_valid` read as zeros.
template <int ROW, int rows>
__device__ __forceinline__ void dma_tile(char* lds, const void* gbase, int gstride, int rows_valid,
                                         int wave, int lane) {
    constexpr int RPI = 1024 / ROW;  // rows per wave instruction (64 lanes x 16 bytes)
    constexpr int SPR = ROW / 16;    // 16-byte slots per row
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(gbase), 0, rows_valid * gstride, kRawBufferWord3);
    constexpr int ninstr = rows / RPI;
    static_assert(1024 % ROW == 0 && ninstr % kTrWaves == 0, "whole rows per wave");
#pragma unroll
    for (int kk = 0; kk < ninstr / kTrWaves; ++kk) {
        const int k = wave + kTrWaves * kk;
        const int row = k * RPI + lane / SPR;
        const int slot = (lane % SPR) ^ (2 * tr_swz<ROW>(row));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (SSD_LDS void*)(lds + k * 1024), 16,
                                                 row * gstride + slot * 16, 0, 0, 0);
    }
}

// Copy chunk c's x and B tiles and its metadata (cs, dt, w from the prep
// workspaces; sequence ids from seq_idx, zeros past L).
template <int P, int N, int Q, bool kSeq>
__device__ __forceinline__ void dma_chunk(char* sX, char* sB, TrMeta<Q>* sM, const ScanArgs& a,
                                          const WorkItem& it, int c, int wave, int lane) {
    using G_ = TrGeo<P, N, Q>;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const int64_t rem = a.L - t0;
    const int valid = rem < Q ? static_cast<int>(rem) : Q;
    const uint16_t* xb = static_cast<const uint16_t*>(a.x) + ((it.b * a.L + t0) * a.H + it.h) * P;
    const uint16_t* bb = static_cast<const uint16_t*>(a.B) + ((it.b * a.L + t0) * a.G + it.g) * N;
    dma_tile<G_::XROW, Q>(sX, xb, a.H * P * 2, valid, wave, lane);
    dma_tile<G_::BROW, Q>(sB, bb, a.G * N * 2, valid, wave, lane);
    constexpr int ML = Q / 4;  // lanes per metadata array (16 bytes each)
    const int mw = kTrWaves - 1 - wave;  // metadata from the last waves (fewest tile rows)
    if (mw < 4 && lane < ML) {
        const int64_t mo = meta_offset(a, it.b, it.h, c, Q) + 4 * lane;
        if (mw == 0) {
            __builtin_amdgcn_global_load_lds((SSD_GLOBAL void*)(a.cs + mo), (SSD_LDS void*)(sM->cs),
                                             16, 0, 0);
        } else if (mw == 1) {
            __builtin_amdgcn_global_load_lds((SSD_GLOBAL void*)(a.dtv + mo),
                                             (SSD_LDS void*)(sM->dt), 16, 0, 0);
        } else if (mw == 2) {
            __builtin_amdgcn_global_load_lds((SSD_GLOBAL void*)(a.wgt + mo), (SSD_LDS void*)(sM->w),
                                             16, 0, 0);
        } else if (kSeq) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<int32_t*>(a.seq_idx + it.b * a.L + t0), 0, valid * 4, kRawBufferWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (SSD_LDS void*)(sM->seq), 16, 16 * lane, 0,
                                                     0, 0);
        }
    }
}

// -------------------------------------------------------------- the kernel

// Output row block of an output wave; for Q = 128 the two waves sharing a
// SIMD (w, w + 4) get rows (k, 7 - k): equal triangular work per SIMD.
template <int NB>
__device__ __forceinline__ int tr_row_block(int wave) {
    if constexpr (NB == 8) return wave < 4 ? wave : 11 - wave;
    else return wave;
}

template <int P, int N, int Q, bool kOut, bool kSeq>
struct TrScan {
    using G_ = TrGeo<P, N, Q>;

    const ScanArgs& a;
    WorkItem it;
    int wave, lane, r16, g;
    int c_begin, c_end;
    bool last_seg, st_wave, out_wave;
    int I;                  // output row block of this wave
    float Dh;               // skip weight D[h]
    int xoff[G_::PB], boff; // transposing-read lane offsets (x per p block, B of n block `wave`)
    int seq_prev;           // sequence id of the token before the current chunk
    float mult;             // decay of the segment (chunk-state kernel)

    f32x4_t h[G_::PB];          // state rows n = 16 wave + 4g + r, column p = 16pb + r16
    uint4 cr[2][G_::KN];        // C rows of the current / next chunk (k over n)
    uint4 cb[2][G_::NCB];       // C.B^T tile pairs of the current / next chunk
    uint2 ypk[G_::PB];          // packed outputs awaiting their store
    int64_t ypos;               // element offset of ypk[0]
    bool ypend;

    __device__ __forceinline__ TrScan(const ScanArgs& args) : a(args) {}

    __device__ __forceinline__ void load_c(int k, int c) {
        const int64_t t0 = static_cast<int64_t>(c) * Q;
        const int64_t rem = a.L - t0;
        const int valid = rem < Q ? static_cast<int>(rem) : Q;
        const int stride = a.G * N * 2;
        const uint16_t* base = static_cast<const uint16_t*>(a.C) + ((it.b * a.L + t0) * a.G + it.g) * N;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base), 0, valid * stride, kRawBufferWord3);
#pragma unroll
        for (int s = 0; s < G_::KN; ++s) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (16 * I + r16) * stride + (32 * s + 8 * g) * 2, 0, 0);
            cr[k][s] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }

    __device__ __forceinline__ void load_cb(int k, int c) {
        constexpr int NT = G_::NB * (G_::NB + 1) / 2;
        const uint16_t* tiles = static_cast<const uint16_t*>(a.cbt) +
                                ((it.b * a.nc + c) * a.G + it.g) * static_cast<int64_t>(NT) * 256;
        const int first = I * (I + 1) / 2;
#pragma unroll
        for (int u = 0; u < G_::NCB; ++u) {
            if (2 * u <= I) {
                const int j1 = 2 * u + 1 <= I ? 2 * u + 1 : I;
                const uint2 v0 = *reinterpret_cast<const uint2*>(
                    tiles + (static_cast<int64_t>(first + 2 * u) * 64 + lane) * 4);
                const uint2 v1 = *reinterpret_cast<const uint2*>(
                    tiles + (static_cast<int64_t>(first + j1) * 64 + lane) * 4);
                cb[k][u] = make_uint4(v0.x, v0.y, v1.x, v1.y);
            }
        }
    }

    // G^T fragment of k step u: lane column i = 16I + r16, tokens j in the
    // k order above; G[i][j] = (C_i . B_j) exp(cs_i - cs_j) dt_j, masked to
    // j <= i and (with sequence ids) seq_j = seq_i.
    __device__ __forceinline__ Frag<uint16_t> g_frag(const uint4& t, const TrMeta<Q>& m, int u,
                                                     int i, float cs_i, int seq_i) const {
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
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bool keep = J < I || (J == I && 4 * g + r <= r16);
                if constexpr (kSeq) keep = keep && sqv[r] == seq_i;
                const float v = cbv[r] * decay_exp(keep ? cs_i - csv[r] : 0.0f) * dtv[r];
                out[4 * hp + r] = keep ? v : 0.0f;
            }
        }
        return frag_from_f32<uint16_t>(out);
    }

    __device__ __forceinline__ void store_y() {
        if (ypend) {
            uint16_t* y = static_cast<uint16_t*>(a.y) + ypos;
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb) *reinterpret_cast<uint2*>(y + 16 * pb) = ypk[pb];
        }
        ypend = false;
    }

    // One chunk.  On entry chunk c's tiles and metadata are in (X, Bt, M), the
    // state before it in H (bf16 operand copy) and h (fp32, state waves), and
    // its C rows and C.B^T tiles in cr[K], cb[K].  Issues chunk c+1's loads
    // into the other buffers, and leaves after a barrier with them complete.
    template <int K>
    __device__ __forceinline__ void chunk(int c, const char* X, const char* Bt, const TrMeta<Q>* M,
                                          const char* H, char* Xn, char* Bn, TrMeta<Q>* Mn,
                                          char* Hn) {
        const bool has_next = c + 1 < c_end;
        const int64_t t0 = static_cast<int64_t>(c) * Q;
        const int64_t rem = a.L - t0;
        const int valid = rem < Q ? static_cast<int>(rem) : Q;
        const bool need_state = !kOut || has_next || (last_seg && a.final_states != nullptr);

        if constexpr (kOut) store_y();  // previous chunk's outputs
        if (has_next) {
            if constexpr (kOut) {
                if (out_wave) {
                    load_c(K ^ 1, c + 1);
                    load_cb(K ^ 1, c + 1);
                }
            }
            dma_chunk<P, N, Q, kSeq>(Xn, Bn, Mn, a, it, c + 1, wave, lane);
        }
        const TrMeta<Q>& m = *M;
        const float cs_last = m.cs[Q - 1];
        const int seq_last = kSeq ? m.seq[valid - 1] : 0;

        // carried-state term of the outputs: y^T[p][i] = exp(cs_i) [seq_i = seq_prev] h.C_i
        f32x4_t y[G_::PB];
        int i = 0;
        float cs_i = 0.0f;
        int seq_i = 0;
        if constexpr (kOut) {
            if (out_wave) {
                i = 16 * I + r16;
                cs_i = m.cs[i];
                if constexpr (kSeq) seq_i = m.seq[i];
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb) y[pb] = acc_zero();
#pragma unroll
                for (int s = 0; s < G_::KN; ++s) {
                    const Frag<uint16_t> cf = frag_of(cr[K][s]);
#pragma unroll
                    for (int pb = 0; pb < G_::PB; ++pb) {
                        const Frag<uint16_t> hf = frag_of(*reinterpret_cast<const uint4*>(
                            H + h_off<G_::HROW>(16 * pb + r16, 4 * s + g)));
                        mma(y[pb], hf, cf);
                    }
                }
                const bool keep = !kSeq || seq_i == seq_prev;
                const float e = decay_exp(cs_i);
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = y[pb][r] * e;
                        y[pb][r] = keep ? v : 0.0f;
                    }
            }
        }

        // h_c = [no reset in c] exp(cs_last) h_{c-1} + S_c
        {
            const bool keep = !kSeq || seq_last == seq_prev;
            const float e = decay_exp(cs_last);
            if (need_state && st_wave) {
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = h[pb][r] * e;
                        h[pb][r] = keep ? v : 0.0f;
                    }
            }
            if constexpr (!kOut) mult = keep ? mult * e : 0.0f;
        }

        // k steps over the chunk's tokens: S_c += (B w)^T x, and the
        // intra-chunk outputs y^T += x^T G^T, sharing the x fragments
#pragma unroll
        for (int s = 0; s < G_::KQ; ++s) {
            const bool do_state = need_state && st_wave;
            const bool do_out = kOut && out_wave && 2 * s <= I;
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
                        const Frag<uint16_t> gf = g_frag(cb[K][s], m, s, i, cs_i, seq_i);
#pragma unroll
                        for (int pb = 0; pb < G_::PB; ++pb) mma(y[pb], xf[pb], gf);
                    }
                }
            }
        }

        if constexpr (kOut) {
            if (out_wave) {
                // D x skip, then pack; the store waits for the next chunk
#pragma unroll
                for (int pb = 0; pb < G_::PB; ++pb) {
                    const uint2 xv = *reinterpret_cast<const uint2*>(
                        X + tr_off<G_::XROW>(i, 32 * pb + 8 * g));
                    const float x0 = bf_lo(xv.x), x1 = bf_hi(xv.x);
                    const float x2 = bf_lo(xv.y), x3 = bf_hi(xv.y);
                    ypk[pb] = make_uint2(pack_bf16x2(fmaf(Dh, x0, y[pb][0]), fmaf(Dh, x1, y[pb][1])),
                                         pack_bf16x2(fmaf(Dh, x2, y[pb][2]), fmaf(Dh, x3, y[pb][3])));
                }
                ypos = ((it.b * a.L + t0 + i) * a.H + it.h) * P + 4 * g;
                ypend = i < valid;
            }
            // bf16 operand copy of h_c for the next chunk's carried-state term
            if (has_next && st_wave) {
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

    __device__ __forceinline__ void state_load(const float* __restrict__ src) {
#pragma unroll
        for (int pb = 0; pb < G_::PB; ++pb) {
            if (src && st_wave) {
                const float4 v = *reinterpret_cast<const float4*>(src + (16 * pb + r16) * N +
                                                                  16 * wave + 4 * g);
                h[pb] = f32x4_t{v.x, v.y, v.z, v.w};
            } else {
                h[pb] = acc_zero();
            }
        }
    }

    __device__ __forceinline__ void state_store(float* __restrict__ dst) const {
        if (!st_wave) return;
#pragma unroll
        for (int pb = 0; pb < G_::PB; ++pb)
            *reinterpret_cast<float4*>(dst + (16 * pb + r16) * N + 16 * wave + 4 * g) =
                make_float4(h[pb][0], h[pb][1], h[pb][2], h[pb][3]);
    }
};

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

    TrScan<P, N, Q, kOut, kSeq> k(a);
    k.it = decode_work(a, kOut ? a.nseg : a.nseg - 1);
    k.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    k.lane = static_cast<int>(threadIdx.x) % kWave;
    k.r16 = k.lane & 15;
    k.g = k.lane >> 4;
    k.c_begin = k.it.seg * a.cps;
    k.c_end = min(k.c_begin + a.cps, a.nc);
    k.last_seg = kOut && k.it.seg == a.nseg - 1;
    k.st_wave = k.wave < G_::NNB;
    k.out_wave = kOut && k.wave < G_::NB;
    k.I = tr_row_block<G_::NB>(k.wave);
    k.Dh = (kOut && a.D) ? a.D[k.it.h] : 0.0f;
#pragma unroll
    for (int pb = 0; pb < G_::PB; ++pb) k.xoff[pb] = tr_lane_off<G_::XROW>(pb, k.lane);
    k.boff = tr_lane_off<G_::BROW>(k.st_wave ? k.wave : 0, k.lane);
    k.mult = 1.0f;
    k.ypend = false;
    k.ypos = 0;
    const int64_t bh = k.it.b * a.H + k.it.h;
    if constexpr (kSeq) {
        const int64_t tp = k.c_begin == 0 ? 0 : static_cast<int64_t>(k.c_begin) * Q - 1;
        k.seq_prev = a.seq_idx[k.it.b * a.L + tp];
    } else {
        k.seq_prev = 0;
    }

    // incoming state: fp32 in registers, bf16 operand copy in sH0
    if constexpr (kOut) {
        if (a.nseg == 1) k.state_load(a.init ? a.init + bh * P * N : nullptr);
        else k.state_load(a.seg_state + (bh * a.nseg + k.it.seg) * P * N);
        if (k.st_wave) {
#pragma unroll
            for (int pb = 0; pb < G_::PB; ++pb) {
                const int p = 16 * pb + k.r16;
                *reinterpret_cast<uint2*>(sH0 + h_off<G_::HROW>(p, 2 * k.wave + (k.g >> 1)) +
                                          8 * (k.g & 1)) =
                    make_uint2(pack_bf16x2(k.h[pb][0], k.h[pb][1]), pack_bf16x2(k.h[pb][2], k.h[pb][3]));
            }
        }
        if (k.out_wave) {
            k.load_c(0, k.c_begin);
            k.load_cb(0, k.c_begin);
        }
    } else {
        k.state_load(nullptr);
    }
    dma_chunk<P, N, Q, kSeq>(sX0, sB0, &sM0, a, k.it, k.c_begin, k.wave, k.lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    for (int c = k.c_begin; c < k.c_end; c += 2) {
        k.template chunk<0>(c, sX0, sB0, &sM0, sH0, sX1, sB1, &sM1, sH1);
        if (c + 1 < k.c_end) k.template chunk<1>(c + 1, sX1, sB1, &sM1, sH1, sX0, sB0, &sM0, sH0);
    }

    if constexpr (kOut) {
        k.store_y();
        if (k.last_seg && a.final_states) k.state_store(a.final_states + bh * P * N);
    } else {
        const int64_t slot = bh * a.nseg + k.it.seg;
        k.state_store(a.seg_state + slot * P * N);
        if (threadIdx.x == 0) a.seg_mult[slot] = k.mult;
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
