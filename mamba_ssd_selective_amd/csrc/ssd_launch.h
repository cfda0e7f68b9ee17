// ssd_launch.h -- argument blocks and launchers shared by the C-ABI layer
// (ssd_api.hip) and the kernels (ssd_kernels.hip).  Internal to libssd.so.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// K2 / K4 arguments (the dt transform and chunk cumsum run inside them).
struct ScanArgs {
    const void* x;          // (b, L, H, P)
    const void* B;          // (b, L, G, N)
    const void* C;          // (b, L, G, N)
    void* y;                // (b, L, H, P)
    const float* dt_raw;    // (b, L, H)
    const float* dt_bias;   // (H) or null
    const float* A;         // (H)
    int softplus;
    float dt_min, dt_max;
    const int32_t* seq_idx; // (b, L) or null
    // Where each row's tokens are (see row_span): by default row b is tokens
    // [b L, b L + L) of x, dt, B, C and y.  row_len (b) or null: row b ends
    // after row_len[b] tokens (clamped to [0, L]); its later tokens are
    // neither read nor written.  cu (b + 1) or null: packed rows, row b is
    // tokens [cu[b], cu[b+1]) of T (offsets clamped into [0, T], lengths to L).
    const int32_t* row_len;
    const int32_t* cu;
    int64_t T;
    // (b) or null: row b lives in slot slot[b] of buffers of `slots` rows of L
    // tokens each (its tokens at slot[b] L + t of x, dt, B and C), and its
    // initial and final states are those of the slot (init / final_states +
    // slot[b] H P N).  A slot outside [0, slots) marks a row that is not
    // computed: nothing of it is read or written.  Single-segment calls only.
    const int32_t* slot;
    int64_t slots;
    // emulated decode (slot rows only), or null.  pos (b): row b's length is
    // pos[b] + 1 (0 when pos[b] is outside [0, L)), in place of row_len.  Its
    // last token is the new one: chunk_prep reads it from tok_x (b, H, P),
    // tok_dt (b, H), tok_B and tok_C (b, G, N) (4-byte aligned) and writes
    // it into x, dt_raw, B and C (the slot's chunk buffers, writable here)
    // for the kernels after it.
    const int32_t* pos;
    const void* tok_x;
    const float* tok_dt;
    const void* tok_B;
    const void* tok_C;
    // (b, H, P) or null: decode output.  Only each row's last token (token
    // len - 1) is output, into y_last[b], and y is not written; a row writes
    // its final state only when it holds a whole chunk (len = L), so that its
    // slot's state moves on at chunk ends only.  Single-segment calls only.
    void* y_last;
    // decode output on the transposing-read kernels, in two launches: 1 = the
    // rows whose chunk does not complete; 2 = the others, on a grid of fewer
    // workgroups than work items (set by the launcher: dec_items work items,
    // workgroup k takes items k, k + gridDim.x, ...)
    int dec_pass;
    int64_t dec_items;
    // 1: every chunk takes the per-element exp(cs_i - cs_j) form of the
    // intra-chunk decay (no factoring), so that a token's output does not
    // depend on the tokens after it in its chunk (the strict mode)
    int exact_decay;
    const float* D;         // (H) or null
    const float* init;      // (b, H, P, N) or null
    float* final_states;    // (b, H, P, N) or null
    // (b, H, nseg, P*N) workspace: [P][N] for the generic kernels; for the
    // transposing-read kernels in register order, blocks [n-block][p-block]
    // of 64 lanes x 4 floats (the MFMA accumulator layout of both kernels)
    float* seg_state;
    float* seg_mult;        // (b, H, nseg) workspace
    // Per-token metadata workspace, one block [cs Q | dt Q | w Q] per (row, head,
    // chunk); cs, dtv and wgt point at the three arrays of block 0 (chunk
    // stride 3Q floats, see meta_offset).
    float* cs;              // segmented chunk cumsum of dt*A
    float* dtv;             // transformed dt (0 past L)
    float* wgt;             // chunk-state weights
    void* cbt;              // (b, nc, G, tiles, 64, 4) workspace: C.B^T tiles, io type
    // (b, nc, G, Q/16, N/32, 64, 8) workspace or null: the C rows of each chunk
    // in the output kernel's operand order (piece (I, s): lane (r16, q) holds
    // C[16I + r16][32s + 8q .. +7]), io type; written by chunk_prep when set.
    void* cmf;
    int64_t L;
    int H, G;
    int nc, nseg, cps;      // chunks, segments, chunks per segment
};

// K3 arguments.
struct PassArgs {
    float* seg_state;       // (b*H, nseg, P*N)
    const float* seg_mult;  // (b*H, nseg)
    const float* init;      // (b*H, P*N) or null
    int64_t PN;
    int nseg;
};

// K5 arguments.
struct StepArgs {
    float* state;           // (b, H, P, N)
    const void* x;          // (b, H, P)
    const float* dt;        // (b, H)
    const float* dt_bias;   // (H) or null
    int softplus;
    float dt_min, dt_max;
    const float* A;         // (H)
    const void* B;          // (b, G, N)
    const void* C;          // (b, G, N)
    const float* D;         // (H) or null
    void* y;                // (b, H, P)
    // state cache rows of the batch rows, or null (row b uses state row b);
    // an index outside [0, cache_rows) marks a padding row (skipped)
    const int32_t* state_idx;
    int64_t cache_rows;
    int H, P, G;
};

// Gradient kernels' arguments (ssd_bwd.hip; bf16 x, B, C, dy, dx, dB, dC).
struct BwdArgs {
    const void* x;          // (b, L, H, P)
    const void* B;          // (b, L, G, N)
    const void* C;          // (b, L, G, N)
    const void* dy;         // (b, L, H, P)
    const float* dt_raw;    // (b, L, H)
    const float* dt_bias;   // (H) or null
    const float* A;         // (H)
    const float* D;         // (H) or null
    int softplus;
    float dt_min, dt_max;
    const int32_t* seq_idx; // (b, L) or null
    const float* h_init;    // (b, H, P, N) or null
    const float* dh_final;  // (b, H, P, N) or null (zero)
    const float* cs;        // chunk_prep_kernel's metadata blocks (as ScanArgs::cs)
    // (b, H, nc, P, N) bf16 workspace: the state before each chunk and the
    // gradient after it, rounded once to the bf16 the gradient products take
    // them in (the walks themselves carry them in fp32)
    uint16_t* states;
    uint16_t* gstates;
    float* partials;        // (b, nc, H, 3) workspace: dA, dD, d(dt_bias) per chunk
    void* dx;               // (b, L, H, P)
    float* ddt;             // (b, L, H): gradient with respect to dt_raw
    float* dA;              // (H)
    void* dB;               // (b, L, G, N)
    void* dC;               // (b, L, G, N)
    float* dD;              // (H) or null
    float* ddt_bias;        // (H) or null
    float* dh_init;         // (b, H, P, N) or null
    // Segmented state walks (nseg > 1): the walk of every (direction, row,
    // head) is cut into nseg segments of cps chunks (in walk order).
    // seg_end (2, b*H, nseg, P*N) [p][n]: each segment's end state from a zero
    // start, then (after a pass over segments) its incoming state; seg_mult
    // (2, b*H, nseg): the product of the segment's chunk decays.
    float* seg_end;
    float* seg_mult;
    int nseg, cps;
    int64_t L;
    int batch, H, G, nc;
    int N;                  // state size: 128 or 64
};

// Mixer steps beside the scan (ssd_mixer.hip).
struct ConvArgs {
    const void* xbc;         // (b, L, dim) io; decode: (b, dim)
    const float* weight;     // (dim, 4)
    const float* bias;       // (dim) or null
    const void* state_in;    // (b, dim, 3) io or null (prefill)
    const int32_t* seq_idx;  // (b, L) or null (prefill)
    void* x_out;             // (b, L, nx): channels [0, nx)
    void* b_out;             // (b, L, nb): channels [nx, nx + nb)
    void* c_out;             // (b, L, nb): channels [nx + nb, dim)
    void* state_out;         // (b, dim, 3) io or null; decode: the state, updated in place
    // decode: conv-state cache rows of the batch rows, or null (as StepArgs)
    const int32_t* state_idx;
    int64_t cache_rows;
    int64_t L;
    int batch, dim, nx, nb;
};
struct NormArgs {
    const void* y;           // (rows, dim) io
    const void* z;           // (rows, dim) io
    const float* weight;     // (dim)
    void* out;               // (rows, dim) io
    int64_t rows;
    int dim, group;
    float eps;
};

typedef hipError_t (*ScanLaunchFn)(const ScanArgs&, int64_t nblocks, hipStream_t);

struct ScanVariant {
    int io;  // 0 = fp32, 1 = bf16
    int P, N, Q;
    // chunk size the kernels run with: Q itself, or a divisor of it whose
    // kernels serve the caller's chunk grid (the chunked form is the same
    // recurrence for any chunk size; only the rounding order differs).  Strict
    // calls, whose bits are defined on the caller's chunk grid, take only
    // variants with kernel_Q == Q.
    int kernel_Q;
    ScanLaunchFn chunk_prep;    // dt transform, chunk cumsum, weights, C.B^T tiles
    ScanLaunchFn chunk_state;   // segment states
    ScanLaunchFn chunk_output;  // outputs with the carried state
    // the output kernel forms each segment's incoming state from the earlier
    // segments' end states itself (no separate state pass)
    bool output_combines_segments;
    // the output kernel reads the C rows from chunk_prep's operand-order copy
    bool output_reads_c_copy;
};

// C.B^T tiles of one (row, chunk, group): for every 16-token row block I and
// u = 0 .. I/2 one tile pair (I, 2u), (I, 2u+1), stored lane by lane as
// [pair][lane][8 elements] (elements 0..3 from tile 2u, 4..7 from tile 2u+1,
// zeros where 2u+1 > I), so that one 16-byte (bf16) load per lane fetches a
// whole MFMA k step.  Pairs of row block I start at pair index cb_pair_base(I).
__host__ __device__ inline int cb_pair_base(int I) {
    const int h = I >> 1;
    return h * (h + 1) + ((I & 1) ? h + 1 : 0);
}

// Elements of io type in the C.B^T tile buffer of one (row, chunk, group).
__host__ __device__ inline int64_t cbt_elems_per_chunk_group(int64_t Q) {
    return static_cast<int64_t>(cb_pair_base(static_cast<int>(Q / 16))) * 64 * 8;
}

// bf16 scan kernels built on direct-to-LDS staging and transposing LDS reads
// (ssd_scan_tr.hip): segment states and outputs for P = 64.
hipError_t scan_tr_state_64_64_128(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_output_64_64_128(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_state_64_128_64(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_output_64_128_64(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_state_64_64_64(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_output_64_64_64(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_state_64_128_128(const ScanArgs& a, int64_t nblocks, hipStream_t st);
hipError_t scan_tr_output_64_128_128(const ScanArgs& a, int64_t nblocks, hipStream_t st);

// The variant serving (io, P, N, Q); strict: only one that runs the caller's
// chunk size itself.  Null when there is none.
const ScanVariant* find_scan_variant(int io, int64_t P, int64_t N, int64_t Q, bool strict = false);
int scan_variant_count();
const ScanVariant* scan_variant_at(int i);

// Events to bind to this host thread's next kernel dispatch (both null: none).
// Bound events take the dispatch's own start and end timestamps, so their
// elapsed time is the kernel's execution alone, without the launch gap and
// queue packets that separate event records on the stream would include.
struct DispatchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
DispatchEvents& dispatch_events();

// Every kernel of the library is launched through here.
template <typename... KArgs, typename... Args>
inline hipError_t dispatch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                           Args... args) {
    const DispatchEvents& ev = dispatch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
    return hipGetLastError();
}

// chunk_prep_kernel's per-token metadata alone (cs, dt, weights; no C.B^T
// tiles), bf16, P = 64, N = 128, Q = 128: one workgroup per (row, chunk, group).
hipError_t launch_chunk_meta_bf16_64_128_128(const ScanArgs& a, int64_t nblocks, hipStream_t st);

// Gradient kernels (bf16, P = 64, N = 128, Q = 128): the chains of states
// (forward: before each chunk; reverse: gradient after each chunk, then
// d(h_init); one launch), the per-(row, chunk, group) gradients, the per-head
// sums.
hipError_t launch_bwd_seg_ends(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_states(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_empty(const BwdArgs& a, int64_t nstate, hipStream_t st);

// Mixer steps (io 0 = fp32, 1 = bf16).
hipError_t launch_conv1d_fwd(int io, const ConvArgs& a, hipStream_t st);
hipError_t launch_conv1d_update(int io, const ConvArgs& a, hipStream_t st);
hipError_t launch_gated_rmsnorm(int io, const NormArgs& a, hipStream_t st);

hipError_t launch_state_pass(const PassArgs& a, int64_t bh, hipStream_t st);
hipError_t launch_copy_state(const float* src, float* dst, int64_t n, hipStream_t st);
// Chunk-emulating decode: the copies around the scan (widths in 4-byte words:
// wx = H*P*io/4, wd = H, wb = G*N*io/4; hpn = H*P*N).
// Cache slots <-> a (b, per_row) buffer: gather row r from slot idx[r] (zeros
// for an index outside [0, rows) or when cache is null); scatter row r to slot
// idx[r] (rows whose index is outside are skipped).  per_row % 4 == 0.
hipError_t launch_gather_slots(const float* cache, const int32_t* idx, int64_t rows, float* dst,
                               int64_t b, int64_t per_row, hipStream_t st);
hipError_t launch_scatter_slots(const float* src, const int32_t* idx, int64_t rows, float* cache,
                                int64_t b, int64_t per_row, hipStream_t st);
hipError_t launch_state_update(int io, int64_t N, const StepArgs& a, int64_t nblocks,
                               hipStream_t st);

}  // namespace ssd
