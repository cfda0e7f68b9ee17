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
// Kernel pipeline of one ssd_chunk_scan_fwd call (one process, one GPU):
//   K1 dt_cumsum_kernel     dt = clamp(softplus(dt_raw + dt_bias)), segmented
//                           chunk cumsum of dt*A (wave-level segmented scan)
//   K2 chunk_state_kernel   per (row, head, segment of chunks): chunk states on
//                           bf16 MFMA from LDS-staged, transposed B and x tiles,
//                           chained inside the segment in registers; writes the
//                           segment's end state and its decay multiplier
//   K3 state_pass_kernel    fp32 pass over segments: each segment's incoming state
//   K4 chunk_output_kernel  per (row, head, segment): C.B^T masked-decay intra-chunk
//                           product, C.h_prev carried-state term and D skip on
//                           MFMA; the state is carried chunk to chunk in registers
//                           (recomputing the chunk state with K2's device code)
// and for decode:
//   K5 state_update_kernel  one token: coalesced in-place fp32 state update
//
// Segments exist only to give the GPU enough independent workgroups; with
// batch*heads large enough there is one segment per row and K2/K3 are skipped.
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

// ===========================================================================
// K1: dt transform + segmented chunk cumsum.
// grid (nc, ceil(H/16), batch), 256 threads.  Writes dtv and cs as (b, H, Lp)
// with Lp = nc*Q; padded tokens (t >= L) get dt = 0 (so they contribute nothing).
__global__ __launch_bounds__(256) void dt_cumsum_kernel(DtArgs a) {
    constexpr int kHB = 16;
    __shared__ float s_raw[256][kHB + 1];
    __shared__ int s_seq[256];
    const int c = blockIdx.x, h0 = blockIdx.y * kHB;
    const int64_t b = blockIdx.z;
    const int Q = a.Q;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < Q * kHB; idx += 256) {
        const int t = idx / kHB, hh = idx % kHB;
        float v = 0.0f;
        if (t0 + t < a.L && h0 + hh < a.H) v = a.dt_raw[(b * a.L + t0 + t) * a.H + h0 + hh];
        s_raw[t][hh] = v;
    }
    for (int t = tid; t < Q; t += 256) {
        int64_t tt = t0 + t < a.L ? t0 + t : a.L - 1;
        s_seq[t] = a.seq_idx ? a.seq_idx[b * a.L + tt] : 0;
    }
    __syncthreads();
    const int wave = tid / kWave, lane = tid % kWave;
    const int E = (Q + kWave - 1) / kWave;  // tokens per lane (<= 4)
    for (int hh = wave; hh < kHB; hh += 4) {
        const int h = h0 + hh;
        if (h >= a.H) break;
        const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
        const float Ah = a.A[h];
        float dtv[4], loc[4];
        int first_head = E;  // index of the first segment start inside this lane
        float run = 0.0f;
        for (int k = 0; k < E; ++k) {
            const int t = lane * E + k;
            float d = 0.0f;
            bool head = false;
            if (t < Q) {
                if (t0 + t < a.L)
                    d = dt_transform(s_raw[t][hh], bias, a.softplus, a.dt_min, a.dt_max);
                head = (t == 0) || (s_seq[t] != s_seq[t - 1]);
            }
            dtv[k] = d;
            const float av = d * Ah;
            run = (k == 0 || head) ? av : run + av;
            if (head && first_head == E) first_head = k;
            loc[k] = run;
        }
        // lane aggregate: sum since its last segment start (or the whole lane)
        const int lane_has_head = first_head < E;
        const float incl = wave_segmented_scan(loc[E - 1], lane_has_head);
        float excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0f;
        const int64_t base = (b * a.H + h) * a.Lp + t0;
        for (int k = 0; k < E; ++k) {
            const int t = lane * E + k;
            if (t < Q) {
                const float v = (k < first_head) ? excl + loc[k] : loc[k];
                a.dtv[base + t] = dtv[k];
                a.cs[base + t] = v;
            }
        }
    }
}

// ===========================================================================
// Shared tile configuration of K2 and K4.
template <typename T, int P, int N, int Q>
struct Cfg {
    static_assert(P % 16 == 0 && N % 16 == 0 && Q % 32 == 0, "tile shape");
    static constexpr int kVec = Io<T>::kVec;
    static constexpr int NP = (N + 31) / 32 * 32;  // n padded to the MFMA k step
    static constexpr int PAD = kVec;               // 16 bytes of row padding in LDS
    static constexpr int SB = NP + PAD;            // natural B rows   [Q][SB]
    static constexpr int SBW = Q + PAD;            // B^T*w rows       [N][SBW]
    static constexpr int SX = Q + PAD;             // x^T rows         [P][SX]
    static constexpr int SH = NP + PAD;            // h (operand) rows [P][SH]
    static constexpr int B_ELEMS = (Q * SB > N * SBW) ? Q * SB : N * SBW;
    static constexpr int NB = Q / 16;   // 16-row output blocks
    static constexpr int PB = P / 16;   // 16-column blocks of P
    static constexpr int NNB = N / 16;  // 16-row blocks of the state's n
    static constexpr int KN = NP / 32;  // k steps over n
    static constexpr int KQ = Q / 32;   // k steps over tokens
    static constexpr int MT = (NNB + 3) / 4;  // state n-blocks per wave
};

// The fp32 state tiles a wave keeps in registers: n-block nb = wave + 4m,
// p-block pb; lane (r16, q) holds h[16pb + r16][16nb + 4q + i], i = 0..3.
template <typename T, int P, int N, int Q>
struct StateRegs {
    f32x4_t v[Cfg<T, P, N, Q>::MT][Cfg<T, P, N, Q>::PB];
};

// Per-chunk token metadata staged in LDS.
template <int Q>
struct ChunkMeta {
    float cs[Q];
    float dt[Q];
    int seq[Q];
};

template <int Q>
__device__ __forceinline__ void load_chunk_meta(ChunkMeta<Q>& m, const ScanArgs& a, int64_t b,
                                                int h, int c) {
    const int64_t base = (b * a.H + h) * a.Lp + static_cast<int64_t>(c) * Q;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    for (int i = threadIdx.x; i < Q; i += 256) {
        m.cs[i] = a.cs[base + i];
        m.dt[i] = a.dtv[base + i];
        int64_t tt = t0 + i < a.L ? t0 + i : a.L - 1;
        m.seq[i] = a.seq_idx ? a.seq_idx[b * a.L + tt] : 0;
    }
}

// Sequence id of the token before chunk c (token 0 for the first chunk: the
// initial state belongs to the sequence holding token 0).
__device__ __forceinline__ int prev_last_seq(const ScanArgs& a, int64_t b, int c, int Q) {
    if (!a.seq_idx) return 0;
    const int64_t t = c == 0 ? 0 : static_cast<int64_t>(c) * Q - 1;
    return a.seq_idx[b * a.L + t];
}

// x tile (Q tokens x P) of head h -> LDS transposed: sX[p][j].  Each thread
// moves a block of 4 tokens x kVec columns and transposes it in registers.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void stage_x_transposed(T* sX, const T* __restrict__ x,
                                                   const ScanArgs& a, int64_t b, int h, int c) {
    using C_ = Cfg<T, P, N, Q>;
    constexpr int kV = C_::kVec;
    constexpr int CB = P / kV;            // column blocks per token
    constexpr int NBLK = (Q / 4) * CB;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    for (int blk = threadIdx.x; blk < NBLK; blk += 256) {
        const int j0 = (blk / CB) * 4, p0 = (blk % CB) * kV;
        Vec16<T> rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + j0 + r;
            rows[r] = (t < a.L) ? load16(x + ((b * a.L + t) * a.H + h) * P + p0) : zero16<T>();
        }
#pragma unroll
        for (int e = 0; e < kV; ++e) {
            Vec4<T> col;
#pragma unroll
            for (int r = 0; r < 4; ++r) col.v[r] = rows[r].v[e];
            store4(sX + (p0 + e) * C_::SX + j0, col);
        }
    }
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

// Writes one 4-token x kVec block of B, scaled by w_j, transposed into
// sBw[n][j].  `rows` holds B[j0 + r][n0 .. n0 + kVec).
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void store_bw_block(T* sBw, const Vec16<T> (&rows)[4],
                                               const ChunkMeta<Q>& m, int j0, int n0,
                                               float cs_last, int seq_last) {
    using C_ = Cfg<T, P, N, Q>;
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = state_weight<Q>(m, j0 + r, cs_last, seq_last);
#pragma unroll
    for (int e = 0; e < C_::kVec; ++e) {
        Vec4<T> col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = Io<T>::to_f32(rows[r].v[e]) * w[r];
            col.v[r] = Io<T>::from_f32(w[r] != 0.0f ? v : 0.0f);
        }
        store4(sBw + (n0 + e) * C_::SBW + j0, col);
    }
}

// Chunk-state MFMA shared by K2 and K4:
//   hreg.v[m][pb] (tile n-block nb = wave + 4m, p-block pb) += sum_j Bw^T[n][j] x[j][p]
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void chunk_state_mma(StateRegs<T, P, N, Q>& hreg,
                                                const T* sBw, const T* sX, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < C_::KQ; ++s) {
        Frag<T> xb[C_::PB];
#pragma unroll
        for (int pb = 0; pb < C_::PB; ++pb)
            xb[pb] = frag_load8(sX + (16 * pb + r16) * C_::SX + 32 * s + 8 * q);
#pragma unroll
        for (int m = 0; m < C_::MT; ++m) {
            const int nb = wave + 4 * m;
            if (nb < C_::NNB) {
                const Frag<T> af = frag_load8(sBw + (16 * nb + r16) * C_::SBW + 32 * s + 8 * q);
#pragma unroll
                for (int pb = 0; pb < C_::PB; ++pb) mma(hreg.v[m][pb], af, xb[pb]);
            }
        }
    }
}

// h_c = [no reset] exp(cs_last) h_{c-1} (+ S_c, accumulated afterwards); select, not multiply.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ void decay_state(StateRegs<T, P, N, Q>& hreg,
                                            bool keep, float e) {
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
        const int nb = wave + 4 * m;
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
        const int nb = wave + 4 * m;
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
__device__ __forceinline__ void state_to_lds(const StateRegs<T, P, N, Q>& hreg,
                                             T* sH, int wave, int lane) {
    using C_ = Cfg<T, P, N, Q>;
    const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < C_::MT; ++m) {
        const int nb = wave + 4 * m;
        if (nb < C_::NNB) {
#pragma unroll
            for (int pb = 0; pb < C_::PB; ++pb) {
                Vec4<T> v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v.v[i] = Io<T>::from_f32(hreg.v[m][pb][i]);
                store4(sH + (16 * pb + r16) * C_::SH + 16 * nb + 4 * q, v);
            }
        }
    }
}

// Decode the (row, segment, group, head-in-group) of this workgroup.
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

// ===========================================================================
// K2: chunk states of segments 0 .. nseg-2, chained inside the segment.
// grid = batch * (nseg-1) * H, 256 threads.
template <typename T, int P, int N, int Q>
__global__ __launch_bounds__(256) void chunk_state_kernel(ScanArgs a) {
    using C_ = Cfg<T, P, N, Q>;
    __shared__ __attribute__((aligned(16))) T sBw[N * C_::SBW];
    __shared__ __attribute__((aligned(16))) T sX[P * C_::SX];
    __shared__ __attribute__((aligned(16))) ChunkMeta<Q> meta;
    const WorkItem it = decode_work(a, a.nseg - 1);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const T* __restrict__ Bp = static_cast<const T*>(a.B);
    StateRegs<T, P, N, Q> hreg;
    state_load<T, P, N, Q>(hreg, nullptr, wave, lane);
    float mult = 1.0f;
    const int c_begin = it.seg * a.cps;
    const int c_end = min(c_begin + a.cps, a.nc);
    for (int c = c_begin; c < c_end; ++c) {
        load_chunk_meta<Q>(meta, a, it.b, it.h, c);
        const int seq_prev = prev_last_seq(a, it.b, c, Q);
        __syncthreads();
        const float cs_last = meta.cs[Q - 1];
        const int seq_last = meta.seq[Q - 1];
        stage_x_transposed<T, P, N, Q>(sX, x, a, it.b, it.h, c);
        {
            constexpr int kV = C_::kVec;
            constexpr int CB = N / kV;
            constexpr int NBLK = (Q / 4) * CB;
            const int64_t t0 = static_cast<int64_t>(c) * Q;
            for (int blk = threadIdx.x; blk < NBLK; blk += 256) {
                const int j0 = (blk / CB) * 4, n0 = (blk % CB) * kV;
                Vec16<T> rows[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t t = t0 + j0 + r;
                    rows[r] = (t < a.L) ? load16(Bp + ((it.b * a.L + t) * a.G + it.g) * N + n0)
                                        : zero16<T>();
                }
                store_bw_block<T, P, N, Q>(sBw, rows, meta, j0, n0, cs_last, seq_last);
            }
        }
        __syncthreads();
        const bool keep = seq_last == seq_prev;
        const float e = decay_exp(cs_last);
        decay_state<T, P, N, Q>(hreg, keep, e);
        mult = keep ? mult * e : 0.0f;
        chunk_state_mma<T, P, N, Q>(hreg, sBw, sX, wave, lane);
        __syncthreads();
    }
    const int64_t slot = (it.b * a.H + it.h) * a.nseg + it.seg;
    state_store<T, P, N, Q>(hreg, a.seg_state + slot * P * N, wave, lane);
    if (threadIdx.x == 0) a.seg_mult[slot] = mult;
}

// ===========================================================================
// K3: fp32 pass over segments.  grid (ceil(P*N/1024), batch*H), 256 threads,
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
// K4: chunk outputs with the state carried in registers.
// grid = batch * nseg * H, 256 threads.
template <typename T, int P, int N, int Q>
__global__ __launch_bounds__(256) void chunk_output_kernel(ScanArgs a) {
    using C_ = Cfg<T, P, N, Q>;
    __shared__ __attribute__((aligned(16))) T sB[C_::B_ELEMS];  // natural B, then B^T*w
    __shared__ __attribute__((aligned(16))) T sX[P * C_::SX];
    __shared__ __attribute__((aligned(16))) T sH[P * C_::SH];
    __shared__ __attribute__((aligned(16))) ChunkMeta<Q> meta;
    const WorkItem it = decode_work(a, a.nseg);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r16 = lane & 15, q = lane >> 4;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const T* __restrict__ Bp = static_cast<const T*>(a.B);
    const T* __restrict__ Cp = static_cast<const T*>(a.C);
    T* __restrict__ y = static_cast<T*>(a.y);
    const float Dh = a.D ? a.D[it.h] : 0.0f;
    const int64_t bh = it.b * a.H + it.h;

    StateRegs<T, P, N, Q> hreg;
    if (a.nseg == 1)
        state_load<T, P, N, Q>(hreg, a.init ? a.init + bh * P * N : nullptr, wave, lane);
    else
        state_load<T, P, N, Q>(hreg, a.seg_state + (bh * a.nseg + it.seg) * P * N, wave, lane);
    if (C_::NP > N) {  // zero the operand padding columns once
        for (int idx = threadIdx.x; idx < P * (C_::NP - N); idx += 256)
            sH[(idx / (C_::NP - N)) * C_::SH + N + idx % (C_::NP - N)] = Io<T>::from_f32(0.0f);
    }
    state_to_lds<T, P, N, Q>(hreg, sH, wave, lane);

    const int c_begin = it.seg * a.cps;
    const int c_end = min(c_begin + a.cps, a.nc);
    const bool last_seg = it.seg == a.nseg - 1;
    for (int c = c_begin; c < c_end; ++c) {
        const int64_t t0 = static_cast<int64_t>(c) * Q;
        load_chunk_meta<Q>(meta, a, it.b, it.h, c);
        const int seq_prev = prev_last_seq(a, it.b, c, Q);
        // natural B tile -> sB[j][n] (n >= N zero-filled)
        {
            constexpr int kV = C_::kVec;
            constexpr int CPR = C_::NP / kV;
            for (int li = threadIdx.x; li < Q * CPR; li += 256) {
                const int j = li / CPR, n0 = (li % CPR) * kV;
                const int64_t t = t0 + j;
                Vec16<T> v = zero16<T>();
                if (t < a.L && n0 < N) v = load16(Bp + ((it.b * a.L + t) * a.G + it.g) * N + n0);
                store16(sB + j * C_::SB + n0, v);
            }
        }
        stage_x_transposed<T, P, N, Q>(sX, x, a, it.b, it.h, c);
        __syncthreads();

        // ---- outputs: wave owns row-block pairs (k, NB-1-k), k = wave, wave+4, ...
        for (int pk = wave; pk < C_::NB / 2; pk += 4) {
#pragma unroll 1
            for (int half = 0; half < 2; ++half) {
                const int I = half == 0 ? pk : C_::NB - 1 - pk;
                const int i = 16 * I + r16;  // this lane's token inside the chunk
                const int64_t ti = t0 + i;
                // C_i fragments (operand for C.B^T and for C.h)
                Frag<T> cf[C_::KN];
#pragma unroll
                for (int s = 0; s < C_::KN; ++s) {
                    const int n0 = 32 * s + 8 * q;
                    if (ti < a.L && n0 < N)
                        cf[s] = frag_load8(Cp + ((it.b * a.L + ti) * a.G + it.g) * N + n0);
                    else
                        cf[s] = frag_zero<T>();
                }
                f32x4_t acc[C_::PB];
#pragma unroll
                for (int pb = 0; pb < C_::PB; ++pb) acc[pb] = acc_zero();
                // carried state: y^T[p][i] = sum_n h[p][n] C_i[n]
#pragma unroll
                for (int s = 0; s < C_::KN; ++s)
#pragma unroll
                    for (int pb = 0; pb < C_::PB; ++pb) {
                        const Frag<T> hf = frag_load8(sH + (16 * pb + r16) * C_::SH + 32 * s + 8 * q);
                        mma(acc[pb], hf, cf[s]);
                    }
                const float cs_i = meta.cs[i];
                const int seq_i = meta.seq[i];
                {
                    const bool keep = seq_i == seq_prev;
                    const float e = decay_exp(cs_i);
#pragma unroll
                    for (int pb = 0; pb < C_::PB; ++pb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float v = acc[pb][r] * e;
                            acc[pb][r] = keep ? v : 0.0f;
                        }
                }
                // intra-chunk: y^T[p][i] += sum_{j<=i} x^T[p][j] G[i][j],
                // G[i][j] = (C_i . B_j) exp(cs_i - cs_j) dt_j [same sequence]
                for (int u = 0; u <= I / 2; ++u) {
                    const int J0 = 2 * u, J1 = 2 * u + 1;
                    float g[8];
#pragma unroll
                    for (int hp = 0; hp < 2; ++hp) {
                        const int J = hp == 0 ? J0 : J1;
                        if (J <= I) {
                            f32x4_t t = acc_zero();  // t[r] = C_i . B_{16J+4q+r}
#pragma unroll
                            for (int s = 0; s < C_::KN; ++s) {
                                const Frag<T> bf = frag_load8(sB + (16 * J + r16) * C_::SB + 32 * s + 8 * q);
                                mma(t, bf, cf[s]);
                            }
                            const int jb = 16 * J + 4 * q;
                            const float4 csj = *reinterpret_cast<const float4*>(&meta.cs[jb]);
                            const float4 dtj = *reinterpret_cast<const float4*>(&meta.dt[jb]);
                            const int4 sqj = *reinterpret_cast<const int4*>(&meta.seq[jb]);
                            const float csv[4] = {csj.x, csj.y, csj.z, csj.w};
                            const float dtv[4] = {dtj.x, dtj.y, dtj.z, dtj.w};
                            const int sqv[4] = {sqj.x, sqj.y, sqj.z, sqj.w};
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const bool keep = (jb + r <= i) && (sqv[r] == seq_i);
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
                        const Frag<T> xf = frag_load4x2(row + 16 * J0 + 4 * q, row + 16 * J1 + 4 * q);
                        mma(acc[pb], xf, gf);
                    }
                }
                // D skip and store: lane holds y[i][16pb + 4q + r]
                if (ti < a.L) {
#pragma unroll
                    for (int pb = 0; pb < C_::PB; ++pb) {
                        Vec4<T> out;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float xv = Io<T>::to_f32(sX[(16 * pb + 4 * q + r) * C_::SX + i]);
                            out.v[r] = Io<T>::from_f32(acc[pb][r] + Dh * xv);
                        }
                        store4(y + ((it.b * a.L + ti) * a.H + it.h) * P + 16 * pb + 4 * q, out);
                    }
                }
            }
        }

        const bool need_state = (c + 1 < c_end) || (last_seg && a.final_states);
        __syncthreads();  // all reads of sB (natural) and sH are done
        if (need_state) {
            const float cs_last = meta.cs[Q - 1];
            const int seq_last = meta.seq[Q - 1];
            // natural B -> B^T * w, in place: read every block, then write
            constexpr int kV = C_::kVec;
            constexpr int CB = N / kV;
            constexpr int NBLK = (Q / 4) * CB;
            constexpr int PER = (NBLK + 255) / 256;
            Vec16<T> rows[PER][4];
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int blk = threadIdx.x + 256 * k;
                if (blk < NBLK) {
                    const int j0 = (blk / CB) * 4, n0 = (blk % CB) * kV;
#pragma unroll
                    for (int r = 0; r < 4; ++r) rows[k][r] = load16(sB + (j0 + r) * C_::SB + n0);
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int blk = threadIdx.x + 256 * k;
                if (blk < NBLK) {
                    const int j0 = (blk / CB) * 4, n0 = (blk % CB) * kV;
                    store_bw_block<T, P, N, Q>(sB, rows[k], meta, j0, n0, cs_last, seq_last);
                }
            }
            __syncthreads();
            const bool keep = seq_last == seq_prev;
            decay_state<T, P, N, Q>(hreg, keep, decay_exp(cs_last));
            chunk_state_mma<T, P, N, Q>(hreg, sB, sX, wave, lane);
            state_to_lds<T, P, N, Q>(hreg, sH, wave, lane);
        }
        __syncthreads();
    }
    if (last_seg && a.final_states)
        state_store<T, P, N, Q>(hreg, a.final_states + bh * P * N, wave, lane);
}

// ===========================================================================
// K5: one decode token.  grid = batch*H, 256 threads; N/4 lanes per state row
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

hipError_t launch_dt_cumsum(const DtArgs& a, int64_t batch, int nc, hipStream_t st) {
    dim3 grid(nc, (a.H + 15) / 16, static_cast<unsigned>(batch));
    hipLaunchKernelGGL(dt_cumsum_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

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

template <typename T, int P, int N, int Q>
static hipError_t launch_chunk_state_t(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    hipLaunchKernelGGL((chunk_state_kernel<T, P, N, Q>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, int P, int N, int Q>
static hipError_t launch_chunk_output_t(const ScanArgs& a, int64_t nblocks, hipStream_t st) {
    hipLaunchKernelGGL((chunk_output_kernel<T, P, N, Q>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, int N>
static hipError_t launch_state_update_t(const StepArgs& a, int64_t nblocks, hipStream_t st) {
    hipLaunchKernelGGL((state_update_kernel<T, N>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

// The compiled (io, P, N, Q) set of the chunked scan.
#define SSD_SCAN_VARIANT(IO, T, P, N, Q) \
    {IO, P, N, Q, &launch_chunk_state_t<T, P, N, Q>, &launch_chunk_output_t<T, P, N, Q>},

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

int scan_variant_count() { return static_cast<int>(sizeof(kScanVariants) / sizeof(kScanVariants[0])); }

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
