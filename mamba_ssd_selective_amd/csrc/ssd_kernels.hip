// ssd_kernels.hip -- gfx950 kernels of the chunked SSD scan and the decode update.
//
// Operation (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1 operator
// families 1-2, section 3 Figure 2 box [F2]; "Nemotron 3 Nano - JAX
// Implementation", Key Components item 1):
//   h_t = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t,   y_t = h_t . C_t + D x_t
//
// Chunked form used for prefill (chunk Q, token i of a chunk, cs = running sum
// of a = dt*A inside the chunk, restarted at the chunk start and at every
// sequence change):
//   S_c   = sum_{j in c, seq_j = seq_last} exp(cs_last - cs_j) dt_j x_j (outer) B_j
//   h_c   = [no reset in c] exp(cs_last) h_{c-1} + S_c
//   y_i   = sum_{j <= i, seq_j = seq_i} (C_i . B_j) exp(cs_i - cs_j) dt_j x_j
//           + [seq_i = seq of the previous chunk's last token] exp(cs_i) h_{c-1} . C_i
//           + D x_i
//
// Kernels of one ssd_chunk_scan_fwd call (one process, one GPU), each
// workgroup owning one (row, head, segment of consecutive chunks):
//   chunk_scan_kernel<kOut = false>  "chunk state": per chunk, the dt transform
//        and segmented chunk cumsum (wave-level scan), then S_c on bf16 MFMA from
//        LDS-staged transposed B and x tiles, chained through the segment in
//        registers; writes the segment's end state and decay multiplier.
//   state_pass_kernel                fp32 pass over segments: each segment's
//        incoming state (segment multipliers are wave-uniform scalars).
//   chunk_scan_kernel<kOut = true>   "chunk output": the same per-chunk state
//        chain plus the outputs: C.B^T masked-decay intra-chunk product, the
//        C.h_prev carried-state term and the D skip, on MFMA.
// The first two run only when the rows are cut into more than one segment
// (few rows x heads); with one segment per row the state is carried through
// the whole row inside one workgroup.
// Decode:
//   state_update_kernel              one token: coalesced in-place fp32 update.
//
// Inside a workgroup (8 waves) the chunk loop is software-pipelined: the
// global loads of chunk c+1 (x, B, C rows, raw dt, seq ids) are issued into
// registers before chunk c's MFMA work, and wave 0 runs chunk c+1's dt scan
// while the other waves finish chunk c; two barriers per chunk.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Work-index mapping: consecutive workgroup ids are dealt round-robin to the
// 8 XCDs of an MI355X, each with its own L2.  Remap so that one XCD receives a
// contiguous range of work items (the heads sharing one B/C group and the same
// chunks then share that XCD's L2).
__device__ __forceinline__ int64_t xcd_work_index(int64_t bid, int64_t nblocks) {
    constexpr int kXcd = 8;
    if (nblocks % kXcd != 0) return bid;
    return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsBytes = 160 * 1024;

// ===========================================================================
// Tile configuration.
template <typename T, int P, int N, int Q>
struct Cfg {
    static_assert(P % 16 == 0 && N % 16 == 0 && Q % 32 == 0 && Q <= 256, "tile shape");
    static constexpr int kVec = Io<T>::kVec;
    static constexpr int NP = (N + 31) / 32 * 32;  // n padded to the MFMA k step
    static constexpr int PAD = kVec;               // 16 bytes of row padding in LDS
    static constexpr int SB = NP + PAD;            // natural B rows   [Q][SB]
    static constexpr int SBW = Q + PAD;            // B^T*w rows       [N][SBW]
    static constexpr int SX = Q + PAD;             // x^T rows         [P][SX]
    static constexpr int SH = NP + PAD;            // h (operand) rows [P][SH]
    static constexpr int NB = Q / 16;              // 16-row output blocks
    static constexpr int PB = P / 16;              // 16-column blocks of P
    static constexpr int NNB = N / 16;             // 16-row blocks of the state's n
    static constexpr int KN = NP / 32;             // k steps over n
    static constexpr int KQ = Q / 32;              // k steps over tokens
    static constexpr int MT = (NNB + kWaves - 1) / kWaves;  // state n-blocks per wave
    static constexpr int RB = NB >= 16 ? NB / 8 : 1;        // output row blocks per wave
    // C fragments are prefetched a chunk ahead when a wave owns one row block;
    // with two, they are loaded at the start of each row block (register budget).
    static constexpr bool kPrefetchC = RB == 1;
    static constexpr int RBC = kPrefetchC ? RB : 1;
    static constexpr int CBX = P / kVec, XB = (Q / 4) * CBX;  // x staging blocks
    static constexpr int CBB = N / kVec, BBK = (Q / 4) * CBB; // B staging blocks
    static constexpr int XPT = (XB + kThreads - 1) / kThreads;
    static constexpr int BPT = (BBK + kThreads - 1) / kThreads;
    static constexpr int E = (Q + kWave - 1) / kWave;       // tokens per lane in the dt scan
    static constexpr int META = 3 * Q * 4 + 16;
    static constexpr int LDS_SEPARATE =
        (Q * SB + N * SBW + P * SX + P * SH) * static_cast<int>(sizeof(T)) + 2 * META;
    // When natural B and B^T*w do not both fit, B^T*w is written over natural B
    // after the outputs of the chunk are done.
    static constexpr bool kInPlace = LDS_SEPARATE > kLdsBytes;
    static constexpr int B_ELEMS =
        kInPlace ? (Q * SB > N * SBW ? Q * SB : N * SBW) : Q * SB;
    // the zero padding columns [N, NP) of natural B are written once per kernel
    static_assert(!(kInPlace && NP > N), "in-place B^T*w would overwrite B's zero padding");
};

// Row block r (< RB) of wave w, chosen so that the two waves sharing a SIMD
// (w and w+4) get equal triangular work.
template <int NB>
__device__ __forceinline__ int row_block(int wave, int r) {
    if constexpr (NB >= 16) {
        const int k = wave + 8 * (r / 2);
        return (r % 2 == 0) ? k : NB - 1 - k;
    } else if constexpr (NB == 8) {
        return wave < 4 ? wave : 11 - wave;
    } else {
        return wave;  // valid only for wave < NB
    }
}

// The fp32 state tiles a wave keeps in registers: n-block nb = wave + 8m,
// p-block pb; lane (r16, q) holds h[16pb + r16][16nb + 4q + i], i = 0..3.
template <typename T, int P, int N, int Q>
struct StateRegs {
    f32x4_t v[Cfg<T, P, N, Q>::MT][Cfg<T, P, N, Q>::PB];
};

// Per-chunk token metadata in LDS: transformed dt, segmented cumsum of dt*A,
// sequence ids (padded tokens repeat the last real token's id), and the id of
// the token before the chunk (token 0 for the first chunk: the initial state
// belongs to the sequence holding token 0).
template <int Q>
struct ChunkMeta {
    float cs[Q];
    float dt[Q];
    int seq[Q];
    int seq_prev;
    int pad_[3];
};

// Global data of one chunk, held in registers between its prefetch and its
// staging into LDS.
template <typename T, int P, int N, int Q, bool kOut>
struct Prefetch {
    using C_ = Cfg<T, P, N, Q>;
    uint4 xr[C_::XPT][4];                      // x rows (raw)
    uint4 br[C_::BPT][4];                      // B rows (raw)
    RawFrag<T> cf[kOut ? C_::RBC : 1][C_::KN]; // C fragments (raw)
    float dt[C_::E];                           // raw dt (wave 0)
    int seq[C_::E];                            // sequence ids (wave 0)
    int seq_prev;
};

struct WorkItem {
    int64_t b;
    int seg, h, g;
};
__device__ __forceinline__ WorkItem decode_work(const ScanArgs& a, int nseg_grid) {
    const int64_t nblocks = static_cast<int64_t>(gridDim.x);
    int64_t w = xcd_work_index(blockIdx.x, nblocks);
    const int hpg = a.H / a.G;
    WorkItem it;
    const int hh = static_cast<int>(w % hpg);
    w /= hpg;
    it.g = static_cast<int>(w % a.G);
    w /= a.G;
    it.seg = static_cast<int>(w % nseg_grid);
    it.b = w / nseg_grid;
    it.h = it.g * hpg + hh;
    return it;
}

// C_i fragments of row block r of this wave (operand of C.B^T and C.h):
// lane (r16, q) holds C[16I + r16][32s + 8q .. +7] for every k step s.  The
// loads are unconditional (row and column clamped into the tensor); rows past
// L and columns past N are zeroed where the fragments are used (c_frag_keep).
template <typename T, int P, int N, int Q>
using CRaw = RawFrag<T>[Cfg<T, P, N, Q>::KN];

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void load_c_frags(CRaw<T, P, N, Q>& cf, const ScanArgs& a,
                                             const WorkItem& it, int c, int r, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const T* __restrict__ Cp = static_cast<const T*>(a.C);
    const int r16 = lane & 15, q = lane >> 4;
    const int I = row_block<C_::NB>(wave, r);
    int64_t ti = static_cast<int64_t>(c) * Q + 16 * I + r16;
    ti = ti < a.L ? ti : a.L - 1;
#pragma unroll
    for (int s = 0; s < C_::KN; ++s) {
        int n0 = 32 * s + 8 * q;
        n0 = n0 < N ? n0 : N - 8;
        cf[s] = raw_frag_load8(Cp + ((it.b * a.L + ti) * a.G + it.g) * N + n0);
    }
}

// Whether C fragment s of row block r holds real data (row < L, column < N).
template <typename T, int P, int N, int Q>
__device__ __forceinline__ bool c_frag_keep(const ScanArgs& a, int c, int r, int s, int wave,
                                            int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int I = row_block<C_::NB>(wave, r);
    const int64_t ti = static_cast<int64_t>(c) * Q + 16 * I + (lane & 15);
    return (C_::NB >= 8 || wave < C_::NB) && ti < a.L && 32 * s + 8 * (lane >> 4) < N;
}

// Issue the global loads of chunk c without waiting for them: every address
// is clamped into its tensor (token index to L-1), and the values of tokens
// past L are replaced by zeros at staging time.
template <typename T, int P, int N, int Q, bool kOut>
__device__ __forceinline__ void prefetch_chunk(Prefetch<T, P, N, Q, kOut>& pf, const ScanArgs& a,
                                               const WorkItem& it, int c, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    constexpr int kV = C_::kVec;
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const int64_t tl = a.L - 1;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const T* __restrict__ Bp = static_cast<const T*>(a.B);
#pragma unroll
    for (int k = 0; k < C_::XPT; ++k) {
        int blk = tid + kThreads * k;
        blk = blk < C_::XB ? blk : C_::XB - 1;
        const int j0 = (blk / C_::CBX) * 4, p0 = (blk % C_::CBX) * kV;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int64_t t = t0 + j0 + r;
            t = t < tl ? t : tl;
            pf.xr[k][r] = ld_raw16(x + ((it.b * a.L + t) * a.H + it.h) * P + p0);
        }
    }
#pragma unroll
    for (int k = 0; k < C_::BPT; ++k) {
        int blk = tid + kThreads * k;
        blk = blk < C_::BBK ? blk : C_::BBK - 1;
        const int j0 = (blk / C_::CBB) * 4, n0 = (blk % C_::CBB) * kV;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int64_t t = t0 + j0 + r;
            t = t < tl ? t : tl;
            pf.br[k][r] = ld_raw16(Bp + ((it.b * a.L + t) * a.G + it.g) * N + n0);
        }
    }
    if constexpr (kOut && C_::kPrefetchC) load_c_frags<T, P, N, Q>(pf.cf[0], a, it, c, 0, wave, lane);
    if (wave == 0) {
        // without seq_idx the id loads read dt_raw (at least b*L elements of 4
        // bytes) and the values are replaced by 0 where they are used, so that
        // no load here depends on a branch
        const int32_t* __restrict__ sq =
            a.seq_idx ? a.seq_idx : reinterpret_cast<const int32_t*>(a.dt_raw);
#pragma unroll
        for (int k = 0; k < C_::E; ++k) {
            int64_t t = t0 + lane * C_::E + k;
            t = t < tl ? t : tl;
            pf.dt[k] = a.dt_raw[(it.b * a.L + t) * a.H + it.h];
            pf.seq[k] = sq[it.b * a.L + t];
        }
        pf.seq_prev = sq[it.b * a.L + (c == 0 ? 0 : t0 - 1)];
    }
}

// Wave 0: dt transform and segmented inclusive cumsum of dt*A over the chunk
// (restarted at the chunk start and at every sequence change), into LDS.
template <typename T, int P, int N, int Q, bool kOut>
__device__ __forceinline__ void chunk_meta_scan(ChunkMeta<Q>& m,
                                                const Prefetch<T, P, N, Q, kOut>& pf,
                                                const ScanArgs& a, int h, int c, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    constexpr int E = C_::E;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Ah = a.A[h];
    const bool has_seq = a.seq_idx != nullptr;
    int sq[E];
#pragma unroll
    for (int k = 0; k < E; ++k) sq[k] = has_seq ? pf.seq[k] : 0;
    // id of the token just before this lane's first token (within the chunk)
    const int prev_lane_last = __shfl_up(sq[E - 1], 1, kWave);
    float dtv[E], loc[E];
    int first_head = E;
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int t = lane * E + k;
        float d = 0.0f;
        bool head = false;
        if (t < Q) {
            if (t0 + t < a.L) d = dt_transform(pf.dt[k], bias, a.softplus, a.dt_min, a.dt_max);
            const int before = (k == 0) ? prev_lane_last : sq[k - 1];
            head = (t == 0) || (sq[k] != before);
        }
        dtv[k] = d;
        const float av = d * Ah;
        run = (k == 0 || head) ? av : run + av;
        if (head && first_head == E) first_head = k;
        loc[k] = run;
    }
    const float incl = wave_segmented_scan(loc[E - 1], first_head < E);
    float excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int t = lane * E + k;
        if (t < Q) {
            m.cs[t] = (k < first_head) ? excl + loc[k] : loc[k];
            m.dt[t] = dtv[k];
            m.seq[t] = sq[k];
        }
    }
    if (lane == 0) m.seq_prev = has_seq ? pf.seq_prev : 0;
}

// Per-token weight of the chunk-state sum: w_j = exp(cs_last - cs_j) dt_j for
// tokens of the chunk's last sequence, exactly 0 (by select) otherwise.
template <int Q>
__device__ __forceinline__ float state_weight(const ChunkMeta<Q>& m, int j, float cs_last,
                                              int seq_last) {
    const bool keep = m.seq[j] == seq_last;
    const float w = decay_exp(cs_last - m.cs[j]) * m.dt[j];
    return keep ? w : 0.0f;
}

// B^T * w: column E of one 4-token x kVec block of B, scaled by w_j and
// stored transposed into sBw[n0 + E][j0 .. j0+3]; then the next column.
template <typename T, int P, int N, int Q, int E = 0>
__device__ __forceinline__ void store_bw_cols(T* sBw, const uint4 (&rows)[4], const float (&w)[4],
                                              int j0, int n0) {
    using C_ = Cfg<T, P, N, Q>;
    if constexpr (E < C_::kVec) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float t = raw_elem_f32<T, E>(rows[r]) * w[r];
            v[r] = w[r] != 0.0f ? t : 0.0f;
        }
        store4_f32(sBw + (n0 + E) * C_::SBW + j0, v[0], v[1], v[2], v[3]);
        store_bw_cols<T, P, N, Q, E + 1>(sBw, rows, w, j0, n0);
    }
}

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void store_bw_block(T* sBw, const uint4 (&rows)[4],
                                               const ChunkMeta<Q>& m, int j0, int n0) {
    const float cs_last = m.cs[Q - 1];
    const int seq_last = m.seq[Q - 1];
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = state_weight<Q>(m, j0 + r, cs_last, seq_last);
    store_bw_cols<T, P, N, Q>(sBw, rows, w, j0, n0);
}

// x^T: column E of one 4-token x kVec block of x into sX[p0 + E][j0 .. j0+3].
template <typename T, int P, int N, int Q, int E = 0>
__device__ __forceinline__ void store_x_cols(T* sX, const uint4 (&rows)[4], int j0, int p0) {
    using C_ = Cfg<T, P, N, Q>;
    if constexpr (E < C_::kVec) {
        store_col4<T, E>(sX + (p0 + E) * C_::SX + j0, rows);
        store_x_cols<T, P, N, Q, E + 1>(sX, rows, j0, p0);
    }
}

// Stage a prefetched chunk into LDS: x^T always; natural B when outputs are
// computed; B^T*w unless it is written later over natural B.  Tokens past L
// are zeroed here.
template <typename T, int P, int N, int Q, bool kOut>
__device__ __forceinline__ void stage_chunk(const Prefetch<T, P, N, Q, kOut>& pf,
                                            const ChunkMeta<Q>& m, T* sX, T* sB, T* sBw,
                                            int64_t valid) {
    using C_ = Cfg<T, P, N, Q>;
    constexpr int kV = C_::kVec;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < C_::XPT; ++k) {
        const int blk = tid + kThreads * k;
        if (blk < C_::XB) {
            const int j0 = (blk / C_::CBX) * 4, p0 = (blk % C_::CBX) * kV;
            uint4 rows[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) rows[r] = raw_keep(j0 + r < valid, pf.xr[k][r]);
            store_x_cols<T, P, N, Q>(sX, rows, j0, p0);
        }
    }
#pragma unroll
    for (int k = 0; k < C_::BPT; ++k) {
        const int blk = tid + kThreads * k;
        if (blk < C_::BBK) {
            const int j0 = (blk / C_::CBB) * 4, n0 = (blk % C_::CBB) * kV;
            uint4 rows[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) rows[r] = raw_keep(j0 + r < valid, pf.br[k][r]);
            if constexpr (kOut) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<uint4*>(sB + (j0 + r) * C_::SB + n0) = rows[r];
            }
            if constexpr (!kOut || !C_::kInPlace) store_bw_block<T, P, N, Q>(sBw, rows, m, j0, n0);
        }
    }
}

// Chunk-state MFMA:  hreg[m][pb] += sum_j Bw^T[n][j] x[j][p]  (n-block wave + 8m)
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void chunk_state_mma(StateRegs<T, P, N, Q>& hreg, const T* sBw,
                                                const T* sX, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m) {
        const int nb = wave + kWaves * m;
        if (nb < C_::NNB) {
#pragma unroll
            for (int s = 0; s < C_::KQ; ++s) {
                const Frag<T> af = frag_load8(sBw + (16 * nb + r16) * C_::SBW + 32 * s + 8 * q);
#pragma unroll
                for (int pb = 0; pb < C_::PB; ++pb) {
                    const Frag<T> xb = frag_load8(sX + (16 * pb + r16) * C_::SX + 32 * s + 8 * q);
                    mma(hreg.v[m][pb], af, xb);
                }
            }
        }
    }
}

// h_c = [no reset] exp(cs_last) h_{c-1} (+ S_c afterwards); select, not multiply.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void decay_state(StateRegs<T, P, N, Q>& hreg, bool keep, float e) {
    using C_ = Cfg<T, P, N, Q>;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m)
#pragma unroll
        for (int pb = 0; pb < C_::PB; ++pb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = hreg.v[m][pb][i] * e;
                hreg.v[m][pb][i] = keep ? v : 0.0f;
            }
}

// fp32 state in global memory (P x N, n fastest) <-> register tiles.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void state_load(StateRegs<T, P, N, Q>& hreg,
                                           const float* __restrict__ src, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m) {
        const int nb = wave + kWaves * m;
#pragma unroll
        for (int pb = 0; pb < C_::PB; ++pb) {
            if (nb < C_::NNB && src) {
                const float4 v = *reinterpret_cast<const float4*>(
                    src + (16 * pb + r16) * N + 16 * nb + 4 * q);
                hreg.v[m][pb] = f32x4_t{v.x, v.y, v.z, v.w};
            } else {
                hreg.v[m][pb] = acc_zero();
            }
        }
    }
}

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void state_store(const StateRegs<T, P, N, Q>& hreg,
                                            float* __restrict__ dst, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m) {
        const int nb = wave + kWaves * m;
        if (nb < C_::NNB) {
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) {
                const f32x4_t v = hreg.v[m][pb];
                *reinterpret_cast<float4*>(dst + (16 * pb + r16) * N + 16 * nb + 4 * q) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// Register state -> operand copy in LDS, sH[p][n] in the io type.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void state_to_lds(const StateRegs<T, P, N, Q>& hreg, T* sH, int wave,
                                             int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m) {
        const int nb = wave + kWaves * m;
        if (nb < C_::NNB) {
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) {
                const f32x4_t v = hreg.v[m][pb];
                store4_f32(sH + (16 * pb + r16) * C_::SH + 16 * nb + 4 * q, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// Outputs of the wave's row blocks of one chunk:
//   y^T[p][i] = exp(cs_i) [seq_i = seq_prev] sum_n h[p][n] C_i[n]
//             + sum_{j <= i} x^T[p][j] G[i][j] + D x[i][p],
//   G[i][j]   = (C_i . B_j) exp(cs_i - cs_j) dt_j [seq_j = seq_i].
// C.B^T tiles come out of the MFMA with lane (r16, q) holding
// C_i . B_{16J+4q+r} for i = 16I + r16, which is exactly an operand fragment
// with k = j (two runs of four), so G never goes through LDS.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void chunk_outputs(
    const ChunkMeta<Q>& m, const RawFrag<T> (&cfp)[Cfg<T, P, N, Q>::RBC][Cfg<T, P, N, Q>::KN],
    const T* sB, const T* sX, const T* sH, const ScanArgs& a, const WorkItem& it, int c,
    float Dh, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    T* __restrict__ y = static_cast<T*>(a.y);
    const bool has_seq = a.seq_idx != nullptr;
#pragma unroll 1
    for (int rb = 0; rb < C_::RB; ++rb) {
        const int I = row_block<C_::NB>(wave, rb);
        if (C_::NB < 8 && wave >= C_::NB) continue;
        const int i = 16 * I + r16;
        const int64_t ti = t0 + i;
        Frag<T> cf[C_::KN];
        {
            RawFrag<T> raw[C_::KN];
            if constexpr (C_::kPrefetchC) {
#pragma unroll
                for (int s = 0; s < C_::KN; ++s) raw[s] = cfp[rb][s];
            } else {
                load_c_frags<T, P, N, Q>(raw, a, it, c, rb, wave, lane);
            }
#pragma unroll
            for (int s = 0; s < C_::KN; ++s)
                cf[s] = frag_from_raw(raw[s], c_frag_keep<T, P, N, Q>(a, c, rb, s, wave, lane));
        }
        f32x4_t acc[C_::PB];
#pragma unroll
        for (int pb = 0; pb < C_::PB; ++pb) acc[pb] = acc_zero();
#pragma unroll
        for (int s = 0; s < C_::KN; ++s)
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) {
                const Frag<T> hf = frag_load8(sH + (16 * pb + r16) * C_::SH + 32 * s + 8 * q);
                mma(acc[pb], hf, cf[s]);
            }
        const float cs_i = m.cs[i];
        const int seq_i = m.seq[i];
        {
            const bool keep = seq_i == m.seq_prev;
            const float e = decay_exp(cs_i);
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = acc[pb][r] * e;
                    acc[pb][r] = keep ? v : 0.0f;
                }
        }
        for (int u = 0; u <= I / 2; ++u) {
            float g[8];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const int J = 2 * u + hp;
                if (J <= I) {
                    f32x4_t t = acc_zero();
#pragma unroll
                    for (int s = 0; s < C_::KN; ++s) {
                        const Frag<T> bf = frag_load8(sB + (16 * J + r16) * C_::SB + 32 * s + 8 * q);
                        mma(t, bf, cf[s]);
                    }
                    const int jb = 16 * J + 4 * q;
                    const float4 csj = *reinterpret_cast<const float4*>(&m.cs[jb]);
                    const float4 dtj = *reinterpret_cast<const float4*>(&m.dt[jb]);
                    const float csv[4] = {csj.x, csj.y, csj.z, csj.w};
                    const float dtv[4] = {dtj.x, dtj.y, dtj.z, dtj.w};
                    int sqv[4] = {seq_i, seq_i, seq_i, seq_i};
                    if (has_seq) {
                        const int4 sqj = *reinterpret_cast<const int4*>(&m.seq[jb]);
                        sqv[0] = sqj.x; sqv[1] = sqj.y; sqv[2] = sqj.z; sqv[3] = sqj.w;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool keep = (J < I || jb + r <= i) && (sqv[r] == seq_i);
                        const float v = t[r] * decay_exp(keep ? cs_i - csv[r] : 0.0f) * dtv[r];
                        g[4 * hp + r] = keep ? v : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) g[4 * hp + r] = 0.0f;
                }
            }
            const Frag<T> gf = frag_from_f32<T>(g);
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) {
                const T* row = sX + (16 * pb + r16) * C_::SX;
                const Frag<T> xf = frag_load4x2(row + 32 * u + 4 * q, row + 32 * u + 16 + 4 * q);
                mma(acc[pb], xf, gf);
            }
        }
        if (ti < a.L) {
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) {
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float xv = Io<T>::to_f32(sX[(16 * pb + 4 * q + r) * C_::SX + i]);
                    o[r] = acc[pb][r] + Dh * xv;
                }
                store4_f32(y + ((it.b * a.L + ti) * a.H + it.h) * P + 16 * pb + 4 * q, o[0], o[1],
                           o[2], o[3]);
            }
        }
    }
}

// ===========================================================================
// The chunked scan over one (row, head, segment):
//   kOut = false: chunk states of segments 0 .. nseg-2, written to the
//                 workspace with each segment's decay multiplier;
//   kOut = true:  outputs of every segment, starting from the segment's
//                 incoming state; final states from the last segment.
template <typename T, int P, int N, int Q, bool kOut>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(ScanArgs a) {
    using C_ = Cfg<T, P, N, Q>;
    constexpr bool kSepBw = !kOut || !C_::kInPlace;
    __shared__ __attribute__((aligned(16))) T sB[kOut ? C_::B_ELEMS : 1];
    __shared__ __attribute__((aligned(16))) T sBwBuf[kSepBw ? N * C_::SBW : 1];
    __shared__ __attribute__((aligned(16))) T sX[P * C_::SX];
    __shared__ __attribute__((aligned(16))) T sH[kOut ? P * C_::SH : 1];
    __shared__ __attribute__((aligned(16))) ChunkMeta<Q> meta[2];
    T* sBw = kSepBw ? sBwBuf : sB;

    const WorkItem it = decode_work(a, kOut ? a.nseg : a.nseg - 1);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t bh = it.b * a.H + it.h;
    const float Dh = (kOut && a.D) ? a.D[it.h] : 0.0f;
    const int c_begin = it.seg * a.cps;
    const int c_end = min(c_begin + a.cps, a.nc);
    const bool last_seg = kOut && it.seg == a.nseg - 1;

    StateRegs<T, P, N, Q> hreg;
    if constexpr (kOut) {
        if (a.nseg == 1)
            state_load<T, P, N, Q>(hreg, a.init ? a.init + bh * P * N : nullptr, wave, lane);
        else
            state_load<T, P, N, Q>(hreg, a.seg_state + (bh * a.nseg + it.seg) * P * N, wave,
                                   lane);
        if (C_::NP > N) {  // zero the operand padding columns [N, NP) once
            constexpr int W = C_::NP - N;
            for (int idx = threadIdx.x; idx < P * W; idx += kThreads)
                sH[(idx / W) * C_::SH + N + idx % W] = Io<T>::from_f32(0.0f);
            for (int idx = threadIdx.x; idx < Q * W; idx += kThreads)
                sB[(idx / W) * C_::SB + N + idx % W] = Io<T>::from_f32(0.0f);
        }
        state_to_lds<T, P, N, Q>(hreg, sH, wave, lane);
    } else {
        state_load<T, P, N, Q>(hreg, nullptr, wave, lane);
    }
    float mult = 1.0f;

    Prefetch<T, P, N, Q, kOut> pf;
    prefetch_chunk<T, P, N, Q, kOut>(pf, a, it, c_begin, wave, lane);
    if (wave == 0) chunk_meta_scan<T, P, N, Q, kOut>(meta[0], pf, a, it.h, c_begin, lane);
    __syncthreads();
    stage_chunk<T, P, N, Q, kOut>(pf, meta[0], sX, sB, sBw,
                                  a.L - static_cast<int64_t>(c_begin) * Q);
    RawFrag<T> cf[kOut ? C_::RBC : 1][C_::KN];
    if constexpr (kOut && C_::kPrefetchC) {
#pragma unroll
        for (int r = 0; r < C_::RBC; ++r)
#pragma unroll
            for (int s = 0; s < C_::KN; ++s) cf[r][s] = pf.cf[r][s];
    }
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        const int cur = (c - c_begin) & 1;
        const bool has_next = c + 1 < c_end;
        const ChunkMeta<Q>& m = meta[cur];
        if (has_next) prefetch_chunk<T, P, N, Q, kOut>(pf, a, it, c + 1, wave, lane);
        const bool need_state = !kOut || has_next || (last_seg && a.final_states);
        if constexpr (kOut) {
            chunk_outputs<T, P, N, Q>(m, cf, sB, sX, sH, a, it, c, Dh, wave, lane);
            if constexpr (!kSepBw) {
                // natural B is dead after the outputs: rewrite it as B^T*w in place
                __syncthreads();
                if (need_state) {
                    uint4 rows[C_::BPT][4];
#pragma unroll
                    for (int k = 0; k < C_::BPT; ++k) {
                        const int blk = threadIdx.x + kThreads * k;
                        if (blk < C_::BBK) {
                            const int j0 = (blk / C_::CBB) * 4, n0 = (blk % C_::CBB) * C_::kVec;
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                rows[k][r] = ld_raw16(sB + (j0 + r) * C_::SB + n0);
                        }
                    }
                    __syncthreads();
#pragma unroll
                    for (int k = 0; k < C_::BPT; ++k) {
                        const int blk = threadIdx.x + kThreads * k;
                        if (blk < C_::BBK) {
                            const int j0 = (blk / C_::CBB) * 4, n0 = (blk % C_::CBB) * C_::kVec;
                            store_bw_block<T, P, N, Q>(sBw, rows[k], m, j0, n0);
                        }
                    }
                }
                __syncthreads();
            }
        }
        if (need_state) {
            const bool keep = m.seq[Q - 1] == m.seq_prev;
            const float e = decay_exp(m.cs[Q - 1]);
            decay_state<T, P, N, Q>(hreg, keep, e);
            mult = keep ? mult * e : 0.0f;
            chunk_state_mma<T, P, N, Q>(hreg, sBw, sX, wave, lane);
        }
        if (has_next && wave == 0)
            chunk_meta_scan<T, P, N, Q, kOut>(meta[cur ^ 1], pf, a, it.h, c + 1, lane);
        __syncthreads();  // every read of this chunk's LDS tiles is done
        if (has_next) {
            if constexpr (kOut) state_to_lds<T, P, N, Q>(hreg, sH, wave, lane);
            stage_chunk<T, P, N, Q, kOut>(pf, meta[cur ^ 1], sX, sB, sBw,
                                          a.L - static_cast<int64_t>(c + 1) * Q);
            if constexpr (kOut && C_::kPrefetchC) {
#pragma unroll
                for (int r = 0; r < C_::RBC; ++r)
#pragma unroll
                    for (int s = 0; s < C_::KN; ++s) cf[r][s] = pf.cf[r][s];
            }
            __syncthreads();
        }
    }
    if constexpr (kOut) {
        if (last_seg && a.final_states)
            state_store<T, P, N, Q>(hreg, a.final_states + bh * P * N, wave, lane);
    } else {
        const int64_t slot = bh * a.nseg + it.seg;
        state_store<T, P, N, Q>(hreg, a.seg_state + slot * P * N, wave, lane);
        if (threadIdx.x == 0) a.seg_mult[slot] = mult;
    }
}

// ===========================================================================
// fp32 pass over segments.  grid (ceil(P*N/1024), batch*H), 256 threads,
// four state elements per thread.  In place: slot s holds segment s's end
// state on entry and its incoming state on exit.
__global__ __launch_bounds__(256) void state_pass_kernel(PassArgs a) {
    const int64_t bh = blockIdx.y;
    const int64_t e4 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (e4 >= a.PN) return;
    float4 carry = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.init) carry = *reinterpret_cast<const float4*>(a.init + bh * a.PN + e4);
    for (int s = 0; s < a.nseg; ++s) {
        float* slot = a.seg_state + (bh * a.nseg + s) * a.PN + e4;
        float4 loc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (s < a.nseg - 1) loc = *reinterpret_cast<const float4*>(slot);
        *reinterpret_cast<float4*>(slot) = carry;
        if (s < a.nseg - 1) {
            // the segment multiplier is uniform across the wave
            const float m = __int_as_float(
                __builtin_amdgcn_readfirstlane(__float_as_int(a.seg_mult[bh * a.nseg + s])));
            if (m != 0.0f) {
                carry.x = fmaf(m, carry.x, loc.x);
                carry.y = fmaf(m, carry.y, loc.y);
                carry.z = fmaf(m, carry.z, loc.z);
                carry.w = fmaf(m, carry.w, loc.w);
            } else {
                carry = loc;
            }
        }
    }
}

// Copy (or zero) the initial state into final_states: the L = 0 case.
__global__ __launch_bounds__(256) void copy_state_kernel(const float* __restrict__ src,
                                                         float* __restrict__ dst, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// ===========================================================================
// One decode token.  grid = batch*H, 256 threads; N/4 lanes per state row
// (one float4 each), 256/(N/4) rows per pass.  Uses the same dt transform and
// decay functions as the chunked path.
template <typename T, int N>
__global__ __launch_bounds__(256) void state_update_kernel(StepArgs a) {
    constexpr int TPR = N / 4;
    constexpr int RP = 256 / TPR;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = static_cast<int>(bh % a.H);
    const int g = group_of_head(h, a.H / a.G);
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const T* __restrict__ Bp = static_cast<const T*>(a.B);
    const T* __restrict__ Cp = static_cast<const T*>(a.C);
    T* __restrict__ y = static_cast<T*>(a.y);
    const int rr = threadIdx.x / TPR, cc = threadIdx.x % TPR;
    const float dtv = dt_transform(a.dt[bh], a.dt_bias ? a.dt_bias[h] : 0.0f, a.softplus,
                                   a.dt_min, a.dt_max);
    const float dA = decay_exp(dtv * a.A[h]);
    const float Dh = a.D ? a.D[h] : 0.0f;
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bv[k] = Io<T>::to_f32(Bp[(b * a.G + g) * N + 4 * cc + k]);
        cv[k] = Io<T>::to_f32(Cp[(b * a.G + g) * N + 4 * cc + k]);
    }
    for (int p0 = 0; p0 < a.P; p0 += RP) {
        const int p = p0 + rr;
        float part = 0.0f;
        float xv = 0.0f;
        if (p < a.P) {
            xv = Io<T>::to_f32(x[bh * a.P + p]);
            float4* sp = reinterpret_cast<float4*>(a.state + (bh * a.P + p) * N + 4 * cc);
            float4 s = *sp;
            const float u = dtv * xv;
            s.x = fmaf(dA, s.x, u * bv[0]);
            s.y = fmaf(dA, s.y, u * bv[1]);
            s.z = fmaf(dA, s.z, u * bv[2]);
            s.w = fmaf(dA, s.w, u * bv[3]);
            *sp = s;
            part = s.x * cv[0] + s.y * cv[1] + s.z * cv[2] + s.w * cv[3];
        }
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
        if (p < a.P && cc == 0) y[bh * a.P + p] = Io<T>::from_f32(part + Dh * xv);
    }
}

// ===========================================================================
// Launchers.

hipError_t launch_state_pass(const PassArgs& a, int64_t bh, hipStream_t st) {
    dim3 grid(static_cast<unsigned>((a.PN / 4 + 255) / 256), static_cast<unsigned>(bh));
    hipLaunchKernelGGL(state_pass_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* src, float* dst, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, st, src, dst, n);
    return hipGetLastError();
}

template <typename T, int P, int N, int Q, bool kOut>
static hipError_t launch_chunk_scan_t(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    hipLaunchKernelGGL((chunk_scan_kernel<T, P, N, Q, kOut>),
                       dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T, int N>
static hipError_t launch_state_update_t(const StepArgs& a, int64_t nblocks, hipStream_t st) {
    hipLaunchKernelGGL((state_update_kernel<T, N>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

// The compiled (io, P, N, Q) set of the chunked scan.
#define SSD_SCAN_VARIANT(IO, T, P, N, Q)                   \
    {IO, P, N, Q, &launch_chunk_scan_t<T, P, N, Q, false>, \
     &launch_chunk_scan_t<T, P, N, Q, true>},

static const ScanVariant kScanVariants[] = {
    SSD_SCAN_VARIANT(0, float, 16, 16, 32)
    SSD_SCAN_VARIANT(0, float, 16, 16, 64)
    SSD_SCAN_VARIANT(0, float, 16, 16, 128)
    SSD_SCAN_VARIANT(0, float, 64, 128, 64)
    SSD_SCAN_VARIANT(0, float, 64, 128, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 16, 16, 64)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 64, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 128, 64)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 128, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 128, 256)
};

const ScanVariant* find_scan_variant(int io, int64_t P, int64_t N, int64_t Q) {
    for (const ScanVariant& v : kScanVariants)
        if (v.io == io && v.P == P && v.N == N && v.Q == Q) return &v;
    return nullptr;
}

int scan_variant_count() {
    return static_cast<int>(sizeof(kScanVariants) / sizeof(kScanVariants[0]));
}

const ScanVariant* scan_variant_at(int i) { return &kScanVariants[i]; }

hipError_t launch_state_update(int io, int64_t N, const StepArgs& a, int64_t nblocks,
                               hipStream_t st) {
    if (io == 0) {
        switch (N) {
            case 16: return launch_state_update_t<float, 16>(a, nblocks, st);
            case 32: return launch_state_update_t<float, 32>(a, nblocks, st);
            case 64: return launch_state_update_t<float, 64>(a, nblocks, st);
            case 128: return launch_state_update_t<float, 128>(a, nblocks, st);
            case 256: return launch_state_update_t<float, 256>(a, nblocks, st);
        }
    } else {
        switch (N) {
            case 16: return launch_state_update_t<uint16_t, 16>(a, nblocks, st);
            case 32: return launch_state_update_t<uint16_t, 32>(a, nblocks, st);
            case 64: return launch_state_update_t<uint16_t, 64>(a, nblocks, st);
            case 128: return launch_state_update_t<uint16_t, 128>(a, nblocks, st);
            case 256: return launch_state_update_t<uint16_t, 256>(a, nblocks, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace ssd
