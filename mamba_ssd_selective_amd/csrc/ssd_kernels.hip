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
// Kernels of one ssd_chunk_scan_fwd call (one process, one GPU):
//   chunk_prep_kernel     one workgroup per (row, chunk, B/C group), all in
//        parallel: the dt transform and segmented chunk cumsum of dt*A (wave-level
//        scan) for the group's heads, the chunk-state weights
//        w_j = exp(cs_last - cs_j) dt_j, and the lower-triangular C.B^T tiles of
//        the chunk on MFMA (once per group instead of once per head), stored in
//        the register layout the output kernel consumes them in.
//   chunk_scan_kernel<kOut = false>  "chunk state", one workgroup per (row, head,
//        segment of consecutive chunks) for all but the last segment: S_c on
//        bf16 MFMA from LDS-staged transposed tiles (B^T scaled by w, x^T),
//        chained through the segment in registers; writes the segment's end state
//        and decay multiplier.
//   state_pass_kernel     fp32 pass over segments: each segment's incoming state
//        (the segment multipliers are wave-uniform scalars).
//   chunk_scan_kernel<kOut = true>   "chunk output": the same state chain plus
//        y = masked-decay (C.B^T) x, the C.h_prev carried-state term and D x.
// With enough rows x heads there is one segment per row and only the prep and
// output kernels run.
// Decode:
//   state_update_kernel   one token: coalesced in-place fp32 state update.
//
// The chunk loop of the scan kernels (8 waves per workgroup) issues
// the next chunk's global loads (x and B rows, chunk metadata) into registers
// before the current chunk's MFMA work and stages them into LDS after it.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_work.h"

namespace ssd {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;

// ===========================================================================
// Tile configuration.
template <typename T, int P, int N, int Q>
struct Cfg {
    static_assert(P % 16 == 0 && N % 16 == 0 && Q % 32 == 0 && Q <= 256, "tile shape");
    static constexpr int kVec = Io<T>::kVec;
    static constexpr int NP = (N + 31) / 32 * 32;  // n padded to the MFMA k step
    static constexpr int PAD = kVec;               // 16 bytes of row padding in LDS
    static constexpr int SB = NP + PAD;            // natural B / C rows (prep) [Q][SB]
    static constexpr int SBW = Q + PAD;            // B^T*w rows       [N][SBW]
    static constexpr int SX = Q + PAD;             // x^T rows         [P][SX]
    static constexpr int SH = NP + PAD;            // h (operand) rows [P][SH]
    static constexpr int NB = Q / 16;              // 16-token blocks
    static constexpr int PB = P / 16;              // 16-column blocks of P
    static constexpr int NNB = N / 16;             // 16-row blocks of the state's n
    static constexpr int KN = NP / 32;             // k steps over n
    static constexpr int KQ = Q / 32;              // k steps over tokens
    static constexpr int MT = (NNB + kWaves - 1) / kWaves;  // state n-blocks per wave
    static constexpr int RB = NB >= 16 ? NB / 8 : 1;        // output row blocks per wave
    static constexpr int CBX = P / kVec, XB = (Q / 4) * CBX;  // x staging blocks
    static constexpr int CBB = N / kVec, BBK = (Q / 4) * CBB; // B staging blocks
    static constexpr int XPT = (XB + kThreads - 1) / kThreads;
    static constexpr int BPT = (BBK + kThreads - 1) / kThreads;
    static constexpr int E = (Q + kWave - 1) / kWave;       // tokens per lane in the dt scan
};

// Row block r (< RB) of wave w, chosen so that the two waves sharing a SIMD
// (w and w+4) get equal triangular work: rows (k, NB-1-k) pair up.
template <int NB>
__device__ __forceinline__ int row_block(int wave, int r) {
    if constexpr (NB >= 16) {
        const int k = wave + kWaves * (r / 2);
        return (r % 2 == 0) ? k : NB - 1 - k;
    } else if constexpr (NB == 8) {
        return wave < 4 ? wave : 11 - wave;
    } else {
        return wave;  // valid only for wave < NB
    }
}
template <int NB>
__device__ __forceinline__ bool row_block_valid(int wave) {
    return NB >= 8 || wave < NB;
}

// The fp32 state tiles a wave keeps in registers: n-block nb = wave + 8m,
// p-block pb; lane (r16, q) holds h[16pb + r16][16nb + 4q + i], i = 0..3.
template <typename T, int P, int N, int Q>
struct StateRegs {
    f32x4_t v[Cfg<T, P, N, Q>::MT][Cfg<T, P, N, Q>::PB];
};

// ===========================================================================
// chunk_prep_kernel: one workgroup per (row, chunk, group), grid order
// (group fastest, then chunk, then row).
//  1. wave w handles heads w, w+8, ... of the group: dt transform, segmented
//     inclusive cumsum of dt*A over the chunk (restarted at the chunk start and
//     at every sequence change), weights w_j = [seq_j = seq_last]
//     exp(cs_last - cs_j) dt_j; written to the cs / dtv / wgt workspaces.
//  2. the chunk's B and C rows are staged in LDS; the lower-triangular tiles
//     T(I, J)[j][i] = B_j . C_i (i in block I, j in block J <= I) are computed
//     on MFMA and stored lane by lane: lane (r16, q) keeps C_{16I+r16} .
//     B_{16J+4q+r}, r = 0..3, exactly the operand fragment the output kernel
//     needs (k = j), so that kernel reads contiguous bytes per tile.
// kTiles = false: step 1 only (the gradient kernels need the metadata alone).
// Emulated decode (a.pos): the row's last token is read from the new-token
// arrays, and the workgroup of its chunk copies the group's share of that
// token (x and dt of its heads, its B and C rows) into the slot's chunk
// buffers, where the output kernel reads it.  No workgroup of this launch
// reads a token there that another one writes.
template <typename T, int P, int N, int Q, bool kTiles>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(ScanArgs a) {
    using C_ = Cfg<T, P, N, Q>;
    constexpr int kV = C_::kVec;
    constexpr int E = C_::E;
    __shared__ __attribute__((aligned(16))) T sB[kTiles ? Q * C_::SB : kV];
    __shared__ __attribute__((aligned(16))) T sC[kTiles ? Q * C_::SB : kV];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    int64_t w = xcd_work_index(blockIdx.x, gridDim.x);
    const int g = static_cast<int>(w % a.G);
    w /= a.G;
    const int c = static_cast<int>(w % a.nc);
    const int64_t b = w / a.nc;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const RowSpan rs = row_span(a, b);
    // a chunk past the row's end: the scan kernels never read its data
    if (t0 >= rs.len) return;
    const int64_t tl = rs.len - 1;  // loads past it are clamped to it (and masked)
    const int64_t t_end = rs.len;
    const int64_t r0 = rs.t0;
    const T* __restrict__ Bp = static_cast<const T*>(a.B);
    const T* __restrict__ Cp = static_cast<const T*>(a.C);
    const bool emul = a.pos != nullptr;
    // raw dt of head h at token t of the row
    auto dt_at = [&](int64_t t, int h) {
        return emul && t == tl ? a.tok_dt[b * a.H + h] : a.dt_raw[(r0 + t) * a.H + h];
    };

    // ---- the sequence ids and the first head's dt first: loads return in
    // order, and the dt scan should not wait behind the B / C rows
    const int hpg = a.H / a.G;
    const bool has_seq = a.seq_idx != nullptr;
    int sq[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        int64_t t = t0 + lane * E + k;
        t = t < tl ? t : tl;
        sq[k] = has_seq ? a.seq_idx[r0 + t] : 0;
    }
    float raw0[E];
    {
        const int h = g * hpg + (wave < hpg ? wave : 0);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            int64_t tt = t0 + lane * E + k;
            tt = tt < tl ? tt : tl;
            raw0[k] = dt_at(tt, h);
        }
    }

    // ---- then the B / C row loads (they overlap the dt scan)
    constexpr int CPR = C_::NP / kV;       // 16-byte pieces per padded row
    constexpr int PIECES = Q * CPR;
    constexpr int PPT = (PIECES + kThreads - 1) / kThreads;
    // decode output: the output kernels read the tiles and C rows of the row
    // block of the row's last token only, which need the B rows up to that
    // block's end and the C rows of that block
    const int I_only = a.y_last ? static_cast<int>((rs.len - 1 - t0) >> 4) : -1;
    auto needed = [&](int j, bool isB) {
        return I_only < 0 || (j < 16 * I_only + 16 && (isB || j >= 16 * I_only));
    };
    uint4 rb[PPT], rc[PPT];
#pragma unroll
    for (int k = 0; k < (kTiles ? PPT : 0); ++k) {
        int li = threadIdx.x + kThreads * k;
        li = li < PIECES ? li : PIECES - 1;
        const int j = li / CPR;
        int n0 = (li % CPR) * kV;
        n0 = n0 < N ? n0 : N - kV;
        int64_t t = t0 + j;
        t = t < tl ? t : tl;
        rb[k] = rc[k] = make_uint4(0u, 0u, 0u, 0u);
        if (!needed(j, true)) continue;  // (the C rows needed lie inside the B rows needed)
        const bool wantC = needed(j, false);
        if (emul && t == tl) {
            const int64_t o = (b * a.G + g) * N + n0;
            rb[k] = ld_words16(static_cast<const T*>(a.tok_B) + o);
            if (wantC) rc[k] = ld_words16(static_cast<const T*>(a.tok_C) + o);
        } else {
            rb[k] = ld_raw16(Bp + ((r0 + t) * a.G + g) * N + n0);
            if (wantC) rc[k] = ld_raw16(Cp + ((r0 + t) * a.G + g) * N + n0);
        }
    }
    if (emul && tl < t0 + Q) {
        // the new token into the slot's chunk buffers: this group's heads
        // (x, dt) and its B / C rows
        const int64_t dst = r0 + tl, h0 = static_cast<int64_t>(g) * hpg;
        T* xd = const_cast<T*>(static_cast<const T*>(a.x)) + (dst * a.H + h0) * P;
        const T* xs = static_cast<const T*>(a.tok_x) + (b * a.H + h0) * P;
        for (int e = threadIdx.x; e < hpg * P; e += kThreads) xd[e] = xs[e];
        float* dd = const_cast<float*>(a.dt_raw) + dst * a.H + h0;
        for (int e = threadIdx.x; e < hpg; e += kThreads) dd[e] = a.tok_dt[b * a.H + h0 + e];
        const int64_t gd = (dst * a.G + g) * N, gs = (b * a.G + g) * N;
        for (int e = threadIdx.x; e < 2 * N; e += kThreads) {
            if (e < N) const_cast<T*>(Bp)[gd + e] = static_cast<const T*>(a.tok_B)[gs + e];
            else const_cast<T*>(Cp)[gd + e - N] = static_cast<const T*>(a.tok_C)[gs + e - N];
        }
    }

    // ---- per-head chunk metadata
    const int prev_lane_last = __shfl_up(sq[E - 1], 1, kWave);
    constexpr int kLastLane = (Q - 1) / E, kLastK = (Q - 1) % E;
    // one head: dt transform, segmented cumsum, weights, written out; raw are
    // this lane's dt_raw values of the head
    auto head_meta = [&](int hh, const float (&raw)[E]) {
        const int h = g * hpg + hh;
        const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
        const float Ah = a.A[h];
        float dtv[E], loc[E];
        int first_head = E;
        float run = 0.0f;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int t = lane * E + k;
            const bool real = t < Q && t0 + t < t_end;
            const float d = real ? dt_transform(raw[k], bias, a.softplus, a.dt_min, a.dt_max) : 0.0f;
            const int before = (k == 0) ? prev_lane_last : sq[k - 1];
            const bool head = t < Q && ((t == 0) || (sq[k] != before));
            dtv[k] = d;
            const float av = d * Ah;
            run = (k == 0 || head) ? av : run + av;
            if (head && first_head == E) first_head = k;
            loc[k] = run;
        }
        const float incl = wave_segmented_scan(loc[E - 1], first_head < E);
        float excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0f;
        float csv[E];
#pragma unroll
        for (int k = 0; k < E; ++k) csv[k] = (k < first_head) ? excl + loc[k] : loc[k];
        const float cs_last = __shfl(csv[kLastK], kLastLane, kWave);
        const int seq_last = __shfl(sq[kLastK], kLastLane, kWave);
        const int64_t base = meta_offset(a, b, h, c, Q);
        float wgv[E];
#pragma unroll
        for (int k = 0; k < E; ++k)
            wgv[k] = (sq[k] == seq_last) ? decay_exp(cs_last - csv[k]) * dtv[k] : 0.0f;
        if constexpr (E == 2) {
            // this lane's two tokens are adjacent: one 8-byte store per array
            if (lane * E < Q) {
                *reinterpret_cast<float2*>(a.cs + base + lane * E) = make_float2(csv[0], csv[1]);
                *reinterpret_cast<float2*>(a.dtv + base + lane * E) = make_float2(dtv[0], dtv[1]);
                *reinterpret_cast<float2*>(a.wgt + base + lane * E) = make_float2(wgv[0], wgv[1]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int t = lane * E + k;
                if (t < Q) {
                    a.cs[base + t] = csv[k];
                    a.dtv[base + t] = dtv[k];
                    a.wgt[base + t] = wgv[k];
                }
            }
        }
    };
    if (wave < hpg) head_meta(wave, raw0);
    for (int hh = wave + kWaves; hh < hpg; hh += kWaves) {
        float raw[E];
#pragma unroll
        for (int k = 0; k < E; ++k) {
            int64_t tt = t0 + lane * E + k;
            tt = tt < tl ? tt : tl;
            raw[k] = dt_at(tt, g * hpg + hh);
        }
        head_meta(hh, raw);
    }

    if constexpr (kTiles) {
        // ---- stage B and C rows (tokens past L and columns past N are zero;
        // decode output: the needed rows only, the others are never read)
        const int64_t valid = rs.len - t0;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int li = threadIdx.x + kThreads * k;
            if (li < PIECES) {
                const int j = li / CPR, n0 = (li % CPR) * kV;
                const bool keep = j < valid && n0 < N;
                if (needed(j, true)) *reinterpret_cast<uint4*>(sB + j * C_::SB + n0) = raw_keep(keep, rb[k]);
                if (needed(j, false)) *reinterpret_cast<uint4*>(sC + j * C_::SB + n0) = raw_keep(keep, rc[k]);
            }
        }
        __syncthreads();

        const int r16 = lane & 15, q = lane >> 4;
        // ---- the chunk's C rows in the output kernel's operand order: piece
        // (I, s) holds, lane (r16, q), C[16I + r16][32s + 8q .. +7] (16 bytes)
        if constexpr (sizeof(T) == 2 && N % 32 == 0) {
            if (a.cmf != nullptr) {
                constexpr int KS = N / 32;
                T* __restrict__ cm = static_cast<T*>(a.cmf) + ((b * a.nc + c) * a.G + g) * static_cast<int64_t>(Q * N);
                for (int pc = wave; pc < C_::NB * KS; pc += kWaves) {
                    const int I = pc / KS, s = pc % KS;
                    if (I_only >= 0 && I != I_only) continue;
                    const uint4 v = *reinterpret_cast<const uint4*>(sC + (16 * I + r16) * C_::SB + 32 * s + 8 * q);
                    *reinterpret_cast<uint4*>(cm + (static_cast<int64_t>(pc) * 64 + lane) * 8) = v;
                }
            }
        }

        // ---- C.B^T tiles, in pairs (layout at cb_pair_base); half-tile k of pair
        // p is tile (I, 2u + k), zeros when 2u + k > I
        T* __restrict__ out = static_cast<T*>(a.cbt) +
                              ((b * a.nc + c) * a.G + g) * cbt_elems_per_chunk_group(Q);
        constexpr int NPAIR = C_::NB / 2 * (C_::NB / 2 + 1);
        // one pair per pass: both tiles share row block I (and its C rows), and
        // the pair's 8 elements per lane are stored contiguously
        auto tile_of = [](int pidx, int& I, int& J) {
            int rbk = 0;
#pragma unroll
            for (int r = 1; r < C_::NB; ++r) rbk += cb_pair_base(r) <= pidx ? 1 : 0;
            I = rbk;
            J = 2 * (pidx - cb_pair_base(rbk));
        };
        for (int pidx = wave; pidx < NPAIR; pidx += kWaves) {
            int I, J0;
            tile_of(pidx, I, J0);
            if (I_only >= 0 && I != I_only) continue;
            const bool on1 = J0 + 1 <= I;  // the pair's second tile is left of or on the diagonal
            f32x4_t acc0 = acc_zero(), acc1 = acc_zero();
#pragma unroll
            for (int s = 0; s < C_::KN; ++s) {
                const Frag<T> cf = frag_load8(sC + (16 * I + r16) * C_::SB + 32 * s + 8 * q);
                const Frag<T> bf0 = frag_load8(sB + (16 * J0 + r16) * C_::SB + 32 * s + 8 * q);
                mma(acc0, bf0, cf);
                if (on1) {
                    const Frag<T> bf1 = frag_load8(sB + (16 * (J0 + 1) + r16) * C_::SB + 32 * s + 8 * q);
                    mma(acc1, bf1, cf);
                }
            }
            T* o = out + (static_cast<int64_t>(pidx) * 64 + lane) * 8;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4*>(o) =
                    make_uint4(pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
                               pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3]));
            } else {
                store4_f32(o, acc0[0], acc0[1], acc0[2], acc0[3]);
                store4_f32(o + 4, acc1[0], acc1[1], acc1[2], acc1[3]);
            }
        }
    }
}

// ===========================================================================
// Scan kernels: per-chunk data.

// Token metadata of one chunk in LDS.
template <int Q>
struct ChunkMeta {
    float cs[Q];   // segmented chunk cumsum of dt*A
    float dt[Q];   // transformed dt (0 past L)
    float w[Q];    // chunk-state weights
    int seq[Q];    // sequence ids (padded tokens repeat the last real token's)
    int seq_prev;  // id of the token before the chunk (token 0 for chunk 0)
    int pad_[3];
};

// Global data of the next chunk, held in registers between issue and staging.
template <typename T, int P, int N, int Q>
struct Prefetch {
    using C_ = Cfg<T, P, N, Q>;
    static constexpr int MP = (3 * Q / 4 + kThreads - 1) / kThreads;  // cs/dt/w pieces
    static constexpr int SP = (Q + kThreads - 1) / kThreads;          // seq ids
    uint4 xr[C_::XPT][4];  // x rows (raw)
    uint4 br[C_::BPT][4];  // B rows (raw)
    uint4 mr[MP];          // metadata, 16 bytes per piece
    int sq[SP];
    int seq_prev;
};

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void prefetch_chunk(Prefetch<T, P, N, Q>& pf, const ScanArgs& a,
                                               const WorkItem& it, const RowSpan& rs, int c) {
    using C_ = Cfg<T, P, N, Q>;
    using PF = Prefetch<T, P, N, Q>;
    constexpr int kV = C_::kVec;
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const int64_t tl = rs.len - 1;  // c < the row's chunks: tl >= t0
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
            pf.xr[k][r] = ld_raw16(x + ((rs.t0 + t) * a.H + it.h) * P + p0);
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
            pf.br[k][r] = ld_raw16(Bp + ((rs.t0 + t) * a.G + it.g) * N + n0);
        }
    }
    const int64_t mo = meta_offset(a, it.b, it.h, c, Q);
#pragma unroll
    for (int k = 0; k < PF::MP; ++k) {
        int piece = tid + kThreads * k;
        piece = piece < 3 * Q / 4 ? piece : 3 * Q / 4 - 1;
        const int arr = piece / (Q / 4), off = (piece % (Q / 4)) * 4;
        const float* src = arr == 0 ? a.cs : (arr == 1 ? a.dtv : a.wgt);
        pf.mr[k] = ld_raw16(src + mo + off);
    }
    // without seq_idx the id loads read dt_raw (H >= 1 values per token)
    // and the values are replaced by 0 at staging, so no load here sits behind
    // a branch
    const int32_t* __restrict__ sqp =
        a.seq_idx ? a.seq_idx : reinterpret_cast<const int32_t*>(a.dt_raw);
#pragma unroll
    for (int k = 0; k < PF::SP; ++k) {
        int64_t t = t0 + tid + kThreads * k;
        t = t < tl ? t : tl;
        pf.sq[k] = sqp[rs.t0 + t];
    }
    pf.seq_prev = sqp[rs.t0 + (c == 0 ? 0 : t0 - 1)];
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

// x^T: column E of one 4-token x kVec block of x into sX[p0 + E][j0 .. j0+3].
template <typename T, int P, int N, int Q, int E = 0>
__device__ __forceinline__ void store_x_cols(T* sX, const uint4 (&rows)[4], int j0, int p0) {
    using C_ = Cfg<T, P, N, Q>;
    if constexpr (E < C_::kVec) {
        store_col4<T, E>(sX + (p0 + E) * C_::SX + j0, rows);
        store_x_cols<T, P, N, Q, E + 1>(sX, rows, j0, p0);
    }
}

// Stage the metadata of a prefetched chunk into LDS.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void stage_meta(const Prefetch<T, P, N, Q>& pf, ChunkMeta<Q>& m,
                                           bool has_seq) {
    using PF = Prefetch<T, P, N, Q>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < PF::MP; ++k) {
        const int piece = tid + kThreads * k;
        if (piece < 3 * Q / 4) {
            const int arr = piece / (Q / 4), off = (piece % (Q / 4)) * 4;
            float* dst = arr == 0 ? m.cs : (arr == 1 ? m.dt : m.w);
            *reinterpret_cast<uint4*>(dst + off) = pf.mr[k];
        }
    }
#pragma unroll
    for (int k = 0; k < PF::SP; ++k) {
        const int t = tid + kThreads * k;
        if (t < Q) m.seq[t] = has_seq ? pf.sq[k] : 0;
    }
    if (tid == 0) m.seq_prev = has_seq ? pf.seq_prev : 0;
}

// Stage x^T and B^T*w of a prefetched chunk (its metadata already in LDS).
// Tokens past L are zeroed here.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void stage_tiles(const Prefetch<T, P, N, Q>& pf, const ChunkMeta<Q>& m,
                                            T* sX, T* sBw, int64_t valid) {
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
            const float4 w4 = *reinterpret_cast<const float4*>(&m.w[j0]);
            const float w[4] = {w4.x, w4.y, w4.z, w4.w};
            store_bw_cols<T, P, N, Q>(sBw, rows, w, j0, n0);
        }
    }
}

// Chunk-state MFMA:  hreg[m][pb] += sum_j Bw^T[n][j] x[j][p]  (n-block wave + 8m).
// Software-pipelined: the operands of k step s+1 are read from LDS while the
// MFMAs of step s run.
template <typename T, int P, int N, int Q>
struct StateOps {
    Frag<T> a[Cfg<T, P, N, Q>::MT];
    Frag<T> b[Cfg<T, P, N, Q>::PB];
};

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void load_state_ops(StateOps<T, P, N, Q>& o, const T* sBw, const T* sX,
                                               int s, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m) {
        int nb = wave + kWaves * m;
        nb = nb < C_::NNB ? nb : C_::NNB - 1;
        o.a[m] = frag_load8(sBw + (16 * nb + r16) * C_::SBW + 32 * s + 8 * q);
    }
#pragma unroll
    for (int pb = 0; pb < C_::PB; ++pb)
        o.b[pb] = frag_load8(sX + (16 * pb + r16) * C_::SX + 32 * s + 8 * q);
}

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void chunk_state_mma(StateRegs<T, P, N, Q>& hreg, const T* sBw,
                                                const T* sX, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    StateOps<T, P, N, Q> ops[2];
    load_state_ops<T, P, N, Q>(ops[0], sBw, sX, 0, wave, lane);
#pragma unroll
    for (int s = 0; s < C_::KQ; ++s) {
        if (s + 1 < C_::KQ) load_state_ops<T, P, N, Q>(ops[(s + 1) & 1], sBw, sX, s + 1, wave, lane);
#pragma unroll
        for (int m = 0; m < C_::MT; ++m) {
            if (wave + kWaves * m < C_::NNB) {
#pragma unroll
                for (int pb = 0; pb < C_::PB; ++pb) mma(hreg.v[m][pb], ops[s & 1].a[m], ops[s & 1].b[pb]);
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

// Raw operand data of one output row block, loaded at the start of a chunk:
// C_i fragments (lane (r16, q): C[16I + r16][32s + 8q .. +7]) and the
// C.B^T tiles (I, J) for J <= I (lane: C_i . B_{16J+4q+r}, r = 0..3).
template <typename T, int P, int N, int Q>
struct RowOps {
    using C_ = Cfg<T, P, N, Q>;
    RawFrag<T> cf[C_::KN];
    uint4 cb[C_::NB / 2 + 1][sizeof(T) == 2 ? 1 : 2];  // pairs of tiles (2u, 2u+1)
    // x[i][16pb + 4q .. +3] for the D skip.
    std::conditional_t<sizeof(T) == 2, uint2, uint4> xd[C_::PB];
};

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void load_row_ops(RowOps<T, P, N, Q>& ro, const ScanArgs& a,
                                             const WorkItem& it, const RowSpan& rs, int c, int I,
                                             int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const T* __restrict__ Cp = static_cast<const T*>(a.C);
    const int r16 = lane & 15, q = lane >> 4;
    int64_t ti = static_cast<int64_t>(c) * Q + 16 * I + r16;
    ti = ti < rs.len ? ti : rs.len - 1;
#pragma unroll
    for (int s = 0; s < C_::KN; ++s) {
        int n0 = 32 * s + 8 * q;
        n0 = n0 < N ? n0 : N - 8;
        ro.cf[s] = raw_frag_load8(Cp + ((rs.t0 + ti) * a.G + it.g) * N + n0);
    }
    const T* __restrict__ x = static_cast<const T*>(a.x);
#pragma unroll
    for (int pb = 0; pb < C_::PB; ++pb) {
        const T* px = x + ((rs.t0 + ti) * a.H + it.h) * P + 16 * pb + 4 * q;
        if constexpr (sizeof(T) == 2) ro.xd[pb] = *reinterpret_cast<const uint2*>(px);
        else ro.xd[pb] = ld_raw16(px);
    }
    const T* __restrict__ tiles = static_cast<const T*>(a.cbt) +
                                  ((it.b * a.nc + c) * a.G + it.g) * cbt_elems_per_chunk_group(Q);
    const int first = cb_pair_base(I);  // pair (I, 0)
#pragma unroll
    for (int u = 0; u <= C_::NB / 2; ++u) {
        // tile pair (I, 2u), (I, 2u+1), clamped into this row's pairs
        const int uu = u <= I / 2 ? u : I / 2;
        const T* p0 = tiles + (static_cast<int64_t>(first + uu) * 64 + lane) * 8;
        ro.cb[u][0] = ld_raw16(p0);
        if constexpr (sizeof(T) == 4) ro.cb[u][1] = ld_raw16(p0 + 4);
    }
}

// Element R (0..7) of tile pair u as fp32: R < 4 from tile 2u, else 2u+1.
template <typename T, int P, int N, int Q, int R>
__device__ __forceinline__ float cb_elem(const RowOps<T, P, N, Q>& ro, int u) {
    if constexpr (sizeof(T) == 2) {
        return raw_elem_f32<T, R>(ro.cb[u][0]);
    } else {
        return raw_elem_f32<T, R % 4>(ro.cb[u][R / 4]);
    }
}

// Per-k-step LDS operands of the intra-chunk product: x^T fragments of every
// p-block for token pair (2u, 2u+1) and the metadata of those tokens.
template <typename T, int P, int N, int Q>
struct IntraX {
    Frag<T> xf[Cfg<T, P, N, Q>::PB];
};

template <typename T, int P, int N, int Q>
__device__ __forceinline__ void load_intra_x(IntraX<T, P, N, Q>& o, const T* sX, int u, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
    const int j0 = 32 * u, j1 = 32 * u + 16 < Q ? 32 * u + 16 : 0;  // j1 masked when out of range
#pragma unroll
    for (int pb = 0; pb < C_::PB; ++pb) {
        const T* row = sX + (16 * pb + r16) * C_::SX;
        o.xf[pb] = frag_load4x2(row + j0 + 4 * q, row + j1 + 4 * q);
    }
}

// Outputs of one row block I of one chunk (lane (r16, q): token i = 16I + r16):
//   y^T[p][i] = exp(cs_i) [seq_i = seq_prev] sum_n h[p][n] C_i[n]
//             + sum_{j <= i} x^T[p][j] G[i][j] + D x[i][p],
//   G[i][j]   = (C_i . B_j) exp(cs_i - cs_j) dt_j [seq_j = seq_i].
// LDS operands are read one k step ahead of the MFMAs that use them.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void row_block_outputs(const RowOps<T, P, N, Q>& ro, const ChunkMeta<Q>& m,
                                                  const T* sX, const T* sH, const ScanArgs& a,
                                                  const WorkItem& it, const RowSpan& rs, int c,
                                                  int I, float Dh, bool has_seq, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
    const int i = 16 * I + r16;
    const int64_t ti = static_cast<int64_t>(c) * Q + i;
    Frag<T> cf[C_::KN];
#pragma unroll
    for (int s = 0; s < C_::KN; ++s) cf[s] = frag_from_raw(ro.cf[s], ti < rs.len && 32 * s + 8 * q < N);
    f32x4_t acc[C_::PB];
#pragma unroll
    for (int pb = 0; pb < C_::PB; ++pb) acc[pb] = acc_zero();
    {
        Frag<T> hf[2][C_::PB];
#pragma unroll
        for (int pb = 0; pb < C_::PB; ++pb)
            hf[0][pb] = frag_load8(sH + (16 * pb + r16) * C_::SH + 8 * q);
#pragma unroll
        for (int s = 0; s < C_::KN; ++s) {
            if (s + 1 < C_::KN) {
#pragma unroll
                for (int pb = 0; pb < C_::PB; ++pb)
                    hf[(s + 1) & 1][pb] =
                        frag_load8(sH + (16 * pb + r16) * C_::SH + 32 * (s + 1) + 8 * q);
            }
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) mma(acc[pb], hf[s & 1][pb], cf[s]);
        }
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
    IntraX<T, P, N, Q> ix[2];
    load_intra_x<T, P, N, Q>(ix[0], sX, 0, lane);
#pragma unroll
    for (int u = 0; u <= C_::NB / 2; ++u) {
        if (2 * u <= I) {
            float4 csq[2], dtq[2];
            int4 sqq[2];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                int jb = 16 * (2 * u + hp) + 4 * q;
                jb = jb < Q ? jb : 0;
                csq[hp] = *reinterpret_cast<const float4*>(&m.cs[jb]);
                dtq[hp] = *reinterpret_cast<const float4*>(&m.dt[jb]);
                sqq[hp] = has_seq ? *reinterpret_cast<const int4*>(&m.seq[jb]) : make_int4(0, 0, 0, 0);
            }
            if (2 * u + 2 <= I) load_intra_x<T, P, N, Q>(ix[(u + 1) & 1], sX, u + 1, lane);
            const IntraX<T, P, N, Q>& cur = ix[u & 1];
            float g[8];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const int J = 2 * u + hp;
                const int jb = 16 * J + 4 * q;
                const float csv[4] = {csq[hp].x, csq[hp].y, csq[hp].z, csq[hp].w};
                const float dtv[4] = {dtq[hp].x, dtq[hp].y, dtq[hp].z, dtq[hp].w};
                const int sqv[4] = {has_seq ? sqq[hp].x : seq_i, has_seq ? sqq[hp].y : seq_i,
                                    has_seq ? sqq[hp].z : seq_i, has_seq ? sqq[hp].w : seq_i};
                float t[4];
                if (hp == 0) {
                    t[0] = cb_elem<T, P, N, Q, 0>(ro, u); t[1] = cb_elem<T, P, N, Q, 1>(ro, u);
                    t[2] = cb_elem<T, P, N, Q, 2>(ro, u); t[3] = cb_elem<T, P, N, Q, 3>(ro, u);
                } else {
                    t[0] = cb_elem<T, P, N, Q, 4>(ro, u); t[1] = cb_elem<T, P, N, Q, 5>(ro, u);
                    t[2] = cb_elem<T, P, N, Q, 6>(ro, u); t[3] = cb_elem<T, P, N, Q, 7>(ro, u);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = (J < I || (J == I && jb + r <= i)) && (sqv[r] == seq_i);
                    const float v = t[r] * decay_exp(keep ? cs_i - csv[r] : 0.0f) * dtv[r];
                    g[4 * hp + r] = keep ? v : 0.0f;
                }
            }
            const Frag<T> gf = frag_from_f32<T>(g);
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) mma(acc[pb], cur.xf[pb], gf);
        }
    }
    // decode output: the row's last token alone, into y_last[b]
    if (a.y_last ? ti == rs.len - 1 : ti < rs.len) {
        T* __restrict__ y = a.y_last ? static_cast<T*>(a.y_last) + (it.b * a.H + it.h) * P
                                     : static_cast<T*>(a.y) + ((rs.t0 + ti) * a.H + it.h) * P;
#pragma unroll
        for (int pb = 0; pb < C_::PB; ++pb) {
            const float x0 = raw_elem_f32<T, 0>(ro.xd[pb]), x1 = raw_elem_f32<T, 1>(ro.xd[pb]);
            const float x2 = raw_elem_f32<T, 2>(ro.xd[pb]), x3 = raw_elem_f32<T, 3>(ro.xd[pb]);
            store4_f32(y + 16 * pb + 4 * q,
                       acc[pb][0] + Dh * x0, acc[pb][1] + Dh * x1, acc[pb][2] + Dh * x2,
                       acc[pb][3] + Dh * x3);
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
    __shared__ __attribute__((aligned(16))) T sBw[N * C_::SBW];
    __shared__ __attribute__((aligned(16))) T sX[P * C_::SX];
    __shared__ __attribute__((aligned(16))) T sH[kOut ? P * C_::SH : 1];
    __shared__ __attribute__((aligned(16))) ChunkMeta<Q> meta;

    const WorkItem it = decode_work(a, kOut ? a.nseg : a.nseg - 1);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t bh = it.b * a.H + it.h;
    const float Dh = (kOut && a.D) ? a.D[it.h] : 0.0f;
    const RowSpan rs = row_span(a, it.b);
    const int nc_row = static_cast<int>((rs.len + Q - 1) / Q);
    const int c_begin = it.seg * a.cps;
    const int c_end = min(c_begin + a.cps, nc_row);  // none when the row ends earlier
    // the final state is written by the last segment; decode output: only for
    // rows that hold a whole chunk (a slot's state moves on at chunk ends)
    const bool last_seg = kOut && it.seg == a.nseg - 1 && rs.live &&
                          (a.y_last == nullptr || rs.len == a.L);
    // the row's initial / final state (its own, or its slot's)
    const int64_t sh = rs.state * a.H + it.h;
    // decode output: only the row block of the row's last token is computed
    const int I_last = a.y_last ? static_cast<int>(((rs.len - 1) % Q) / 16) : -1;
    const bool has_seq = a.seq_idx != nullptr;

    StateRegs<T, P, N, Q> hreg;
    if constexpr (kOut) {
        if (a.nseg == 1)
            state_load<T, P, N, Q>(hreg, a.init && rs.live ? a.init + sh * P * N : nullptr, wave,
                                   lane);
        else
            state_load<T, P, N, Q>(hreg, a.seg_state + (bh * a.nseg + it.seg) * P * N, wave,
                                   lane);
        if (C_::NP > N) {  // zero the operand padding columns [N, NP) once
            constexpr int W = C_::NP - N;
            for (int idx = threadIdx.x; idx < P * W; idx += kThreads)
                sH[(idx / W) * C_::SH + N + idx % W] = Io<T>::from_f32(0.0f);
        }
        state_to_lds<T, P, N, Q>(hreg, sH, wave, lane);
    } else {
        state_load<T, P, N, Q>(hreg, nullptr, wave, lane);
    }
    float mult = 1.0f;

    Prefetch<T, P, N, Q> pf;
    if (c_begin < c_end) {
        prefetch_chunk<T, P, N, Q>(pf, a, it, rs, c_begin);
        stage_meta<T, P, N, Q>(pf, meta, has_seq);
        __syncthreads();
        stage_tiles<T, P, N, Q>(pf, meta, sX, sBw, rs.len - static_cast<int64_t>(c_begin) * Q);
        __syncthreads();
    }

    for (int c = c_begin; c < c_end; ++c) {
        const bool has_next = c + 1 < c_end;
        const bool need_state = !kOut || has_next || (last_seg && a.final_states);
        // operands of this chunk's output rows first, then the next chunk's tiles
        RowOps<T, P, N, Q> ro[kOut ? C_::RB : 1];
        if constexpr (kOut) {
#pragma unroll
            for (int r = 0; r < C_::RB; ++r)
                if (row_block_valid<C_::NB>(wave) && (I_last < 0 || row_block<C_::NB>(wave, r) == I_last))
                    load_row_ops<T, P, N, Q>(ro[r], a, it, rs, c, row_block<C_::NB>(wave, r), lane);
        }
        if (has_next) prefetch_chunk<T, P, N, Q>(pf, a, it, rs, c + 1);
        if (need_state) {
            const bool keep = meta.seq[Q - 1] == meta.seq_prev;
            const float e = decay_exp(meta.cs[Q - 1]);
            decay_state<T, P, N, Q>(hreg, keep, e);
            mult = keep ? mult * e : 0.0f;
            chunk_state_mma<T, P, N, Q>(hreg, sBw, sX, wave, lane);
        }
        if constexpr (kOut) {
#pragma unroll
            for (int r = 0; r < C_::RB; ++r)
                if (row_block_valid<C_::NB>(wave) && (I_last < 0 || row_block<C_::NB>(wave, r) == I_last))
                    row_block_outputs<T, P, N, Q>(ro[r], meta, sX, sH, a, it, rs, c,
                                                  row_block<C_::NB>(wave, r), Dh, has_seq, lane);
        }
        __syncthreads();  // every read of this chunk's LDS data is done
        if (has_next) {
            if constexpr (kOut) state_to_lds<T, P, N, Q>(hreg, sH, wave, lane);
            stage_meta<T, P, N, Q>(pf, meta, has_seq);
            __syncthreads();
            stage_tiles<T, P, N, Q>(pf, meta, sX, sBw, rs.len - static_cast<int64_t>(c + 1) * Q);
            __syncthreads();
        }
    }
    if constexpr (kOut) {
        if (last_seg && a.final_states)
            state_store<T, P, N, Q>(hreg, a.final_states + sh * P * N, wave, lane);
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

__global__ __launch_bounds__(256) void gather_slots_kernel(const float* __restrict__ cache,
                                                          const int32_t* __restrict__ idx,
                                                          int64_t rows, float* __restrict__ dst,
                                                          int64_t per_row) {
    const int64_t r = blockIdx.y;
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i >= per_row) return;
    const int64_t s = idx[r];
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cache && s >= 0 && s < rows) v = *reinterpret_cast<const float4*>(cache + s * per_row + i);
    *reinterpret_cast<float4*>(dst + r * per_row + i) = v;
}

__global__ __launch_bounds__(256) void scatter_slots_kernel(const float* __restrict__ src,
                                                           const int32_t* __restrict__ idx,
                                                           int64_t rows, float* __restrict__ cache,
                                                           int64_t per_row) {
    const int64_t r = blockIdx.y;
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    const int64_t s = idx[r];
    if (i >= per_row || s < 0 || s >= rows) return;
    // no source: the slot is cleared (a row of no tokens that starts from zeros)
    *reinterpret_cast<float4*>(cache + s * per_row + i) =
        src ? *reinterpret_cast<const float4*>(src + r * per_row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// ===========================================================================
// One decode token.  256 threads; N/4 lanes per state row (one float4 each),
// so RP = 256/(N/4) rows per pass.  Two layouts of the grid:
//  kSplit = false: one block per (row, head), looping over its P rows 4 RP at
//    a time with the four passes' loads issued together, the state streamed
//    with nontemporal loads and stores (large batches);
//  kSplit = true: one block per (row, head) and 2 RP rows, whose loads are
//    all issued before any arithmetic (few rows x heads: the latency of one
//    block is the time of the step).
// Uses the same dt transform and decay functions as the chunked path.
template <typename T, int N, bool kSplit>
__global__ __launch_bounds__(256) void state_update_kernel(StepArgs a) {
    constexpr int TPR = N / 4;
    constexpr int RP = 256 / TPR;
    constexpr int U = kSplit ? 2 : 4;  // passes whose loads are issued together
    const int pblocks = kSplit ? (a.P + RP * U - 1) / (RP * U) : 1;
    const int64_t bh = blockIdx.x / pblocks;
    const int p_first = kSplit ? static_cast<int>(blockIdx.x % pblocks) * RP * U : 0;
    const int p_end = kSplit ? min(a.P, p_first + RP * U) : a.P;
    const int64_t b = bh / a.H;
    const int h = static_cast<int>(bh % a.H);
    const int g = group_of_head(h, a.H / a.G);
    // the state row of batch row b in the cache (a padding row touches nothing)
    int64_t sb = b;
    if (a.state_idx) {
        sb = a.state_idx[b];
        if (sb < 0 || sb >= a.cache_rows) return;
    }
    float* __restrict__ state = a.state + (sb * a.H + h) * static_cast<int64_t>(a.P) * N;
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
    for (int p0 = p_first; p0 < p_end; p0 += RP * U) {
        float4 st[U];
        float xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + RP * u + rr;
            st[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            xv[u] = 0.0f;
            if (p < p_end) {
                const float* sp = state + static_cast<int64_t>(p) * N + 4 * cc;
                if constexpr (kSplit) {
                    st[u] = *reinterpret_cast<const float4*>(sp);
                } else {
                    // large batches stream each state once: keep it out of the caches
                    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(sp));
                    st[u] = make_float4(v[0], v[1], v[2], v[3]);
                }
                xv[u] = Io<T>::to_f32(x[bh * a.P + p]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + RP * u + rr;
            float part = 0.0f;
            if (p < p_end) {
                float4 s = st[u];
                const float uu = dtv * xv[u];
                s.x = fmaf(dA, s.x, uu * bv[0]);
                s.y = fmaf(dA, s.y, uu * bv[1]);
                s.z = fmaf(dA, s.z, uu * bv[2]);
                s.w = fmaf(dA, s.w, uu * bv[3]);
                float* sp = state + static_cast<int64_t>(p) * N + 4 * cc;
                if constexpr (kSplit) {
                    *reinterpret_cast<float4*>(sp) = s;
                } else {
                    const f32x4_t v = {s.x, s.y, s.z, s.w};
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(sp));
                }
                part = s.x * cv[0] + s.y * cv[1] + s.z * cv[2] + s.w * cv[3];
            }
            part = group_sum_wide_first<TPR>(part);
            if (p < p_end && cc == 0) y[bh * a.P + p] = Io<T>::from_f32(part + Dh * xv[u]);
        }
    }
}

// Rows x heads below which a decode step splits each head's rows over blocks.
constexpr int64_t kDecodeSplitBelow = 1024;

// ===========================================================================
// Launchers.

hipError_t launch_state_pass(const PassArgs& a, int64_t bh, hipStream_t st) {
    dim3 grid(static_cast<unsigned>((a.PN / 4 + 255) / 256), static_cast<unsigned>(bh));
    return dispatch(state_pass_kernel, grid, dim3(256), st, a);
}

hipError_t launch_copy_state(const float* src, float* dst, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    return dispatch(copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                    st, src, dst, n);
}

hipError_t launch_gather_slots(const float* cache, const int32_t* idx, int64_t rows, float* dst,
                               int64_t b, int64_t per_row, hipStream_t st) {
    if (b == 0 || per_row == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((per_row / 4 + 255) / 256), static_cast<unsigned>(b));
    return dispatch(gather_slots_kernel, grid, dim3(256), st, cache, idx, rows, dst, per_row);
}

hipError_t launch_scatter_slots(const float* src, const int32_t* idx, int64_t rows, float* cache,
                                int64_t b, int64_t per_row, hipStream_t st) {
    if (b == 0 || per_row == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((per_row / 4 + 255) / 256), static_cast<unsigned>(b));
    return dispatch(scatter_slots_kernel, grid, dim3(256), st, src, idx, rows, cache, per_row);
}

template <typename T, int P, int N, int Q, bool kTiles = true>
static hipError_t launch_chunk_prep_t(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    return dispatch(chunk_prep_kernel<T, P, N, Q, kTiles>, dim3(static_cast<unsigned>(nblocks)),
                    dim3(kThreads), st, a);
}

template <typename T, int P, int N, int Q, bool kOut>
static hipError_t launch_chunk_scan_t(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    return dispatch(chunk_scan_kernel<T, P, N, Q, kOut>, dim3(static_cast<unsigned>(nblocks)),
                    dim3(kThreads), st, a);
}

template <typename T, int N>
static hipError_t launch_state_update_t(const StepArgs& a, int64_t nblocks, hipStream_t st) {
    if (nblocks < kDecodeSplitBelow) {
        const int64_t rows = 2 * (256 / (N / 4));
        return dispatch(state_update_kernel<T, N, true>,
                        dim3(static_cast<unsigned>(nblocks * ((a.P + rows - 1) / rows))),
                        dim3(256), st, a);
    }
    return dispatch(state_update_kernel<T, N, false>, dim3(static_cast<unsigned>(nblocks)),
                    dim3(256), st, a);
}

// The compiled (io, P, N, Q) set of the chunked scan.
#define SSD_SCAN_VARIANT(IO, T, P, N, Q)                                    \
    {IO, P, N, Q, Q, &launch_chunk_prep_t<T, P, N, Q>,                      \
     &launch_chunk_scan_t<T, P, N, Q, false>, &launch_chunk_scan_t<T, P, N, Q, true>, false, false},
// the same kernels run at chunk QK < Q for a caller chunk of Q
#define SSD_SCAN_VARIANT_BLOCKED(IO, T, P, N, Q, QK)                        \
    {IO, P, N, Q, QK, &launch_chunk_prep_t<T, P, N, QK>,                    \
     &launch_chunk_scan_t<T, P, N, QK, false>, &launch_chunk_scan_t<T, P, N, QK, true>, false, false},

// bf16 shapes served by the transposing-read kernels of ssd_scan_tr.hip.
#define SSD_SCAN_VARIANT_TR(P, N, Q)                                        \
    {1, P, N, Q, Q, &launch_chunk_prep_t<uint16_t, P, N, Q>,                \
     &scan_tr_state_##P##_##N##_##Q, &scan_tr_output_##P##_##N##_##Q, true, true},
// ... at chunk QK < Q: their double-buffered tiles of a 256-token chunk
// (x 32 KiB and B 64 KiB per buffer at N = 128) do not fit the 160 KiB of LDS
#define SSD_SCAN_VARIANT_TR_BLOCKED(P, N, Q, QK)                            \
    {1, P, N, Q, QK, &launch_chunk_prep_t<uint16_t, P, N, QK>,              \
     &scan_tr_state_##P##_##N##_##QK, &scan_tr_output_##P##_##N##_##QK, true, true},

// Non-strict lookups take the first match, strict ones the first with
// kernel_Q == Q: blocked entries come before the native ones they stand in for.
static const ScanVariant kScanVariants[] = {
    SSD_SCAN_VARIANT(0, float, 16, 16, 32)
    SSD_SCAN_VARIANT(0, float, 16, 16, 64)
    SSD_SCAN_VARIANT(0, float, 16, 16, 128)
    SSD_SCAN_VARIANT(0, float, 64, 128, 64)
    SSD_SCAN_VARIANT(0, float, 64, 128, 128)
    SSD_SCAN_VARIANT_BLOCKED(0, float, 64, 128, 256, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 16, 16, 64)
    SSD_SCAN_VARIANT_TR(64, 64, 64)
    SSD_SCAN_VARIANT_TR(64, 64, 128)
    SSD_SCAN_VARIANT_TR_BLOCKED(64, 64, 256, 128)
    SSD_SCAN_VARIANT_TR(64, 128, 64)
    SSD_SCAN_VARIANT_TR(64, 128, 128)
    SSD_SCAN_VARIANT_TR_BLOCKED(64, 128, 256, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 128, 256)
    // further shapes of the generic kernel: state size 256, head dims 32 and
    // 128, chunk 32, state size 32 (bf16); state size 64, head dim 128 and
    // state size 256 at chunk 64 (fp32, whose wider tiles fit the LDS only so)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 256, 64)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 256, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 128, 128, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 32, 128, 128)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 128, 32)
    SSD_SCAN_VARIANT(1, uint16_t, 64, 32, 64)
    SSD_SCAN_VARIANT(0, float, 64, 64, 64)
    SSD_SCAN_VARIANT(0, float, 64, 64, 128)
    SSD_SCAN_VARIANT(0, float, 128, 128, 64)
    SSD_SCAN_VARIANT(0, float, 64, 256, 64)
};

const ScanVariant* find_scan_variant(int io, int64_t P, int64_t N, int64_t Q, bool strict) {
    for (const ScanVariant& v : kScanVariants)
        if (v.io == io && v.P == P && v.N == N && v.Q == Q && (!strict || v.kernel_Q == v.Q))
            return &v;
    return nullptr;
}

int scan_variant_count() {
    return static_cast<int>(sizeof(kScanVariants) / sizeof(kScanVariants[0]));
}

const ScanVariant* scan_variant_at(int i) { return &kScanVariants[i]; }

hipError_t launch_chunk_meta_bf16_64_128_128(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    return launch_chunk_prep_t<uint16_t, 64, 128, 128, false>(a, nblocks, st);
}

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
