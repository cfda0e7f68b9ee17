/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD selective-scan library
 * (libssd.so, built from mamba_ssd_selective_amd/csrc).
 *
 * The operation (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1, operator
 * families 1 and 2, and section 3, Figure 2, box [F2]; "Nemotron 3 Nano - JAX
 * Implementation", Key Components, item 1), per batch row b and head h with
 * B/C group g = h / (H / G):
 *
 *   dt_t = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
 *   h_t  = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t      state P x N, fp32
 *   y_t  = h_t . C_t + D_h * x_t
 *
 * Prefill/training computes it as a chunked parallel scan (ssd_chunk_scan_fwd,
 * chunk size chosen by the caller; the pages use 128); decode computes it one
 * token at a time on a caller-held fp32 state (ssd_state_update).  Both use
 * the same device functions for the per-token arithmetic (RFC section 7:
 * train/prefill and decode share device functions).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous buffers.
 *    The caller owns all of them; the library allocates nothing and keeps no
 *    global buffers, so calls are re-entrant.  (One exception, on purpose:
 *    ssd_chunk_scan_fwd_noalloc takes its scratch from a static device array.)
 *    The other state the library keeps: the diagnostic timing hooks
 *    (ssd_set_timing_events), per host thread and off unless a caller sets
 *    them, and per-device launch sizes it queries once (compute units,
 *    workgroups per CU); no call's results depend on an earlier call.
 *  - Arguments are validated on the host before anything is launched.  Any
 *    failure returns a non-zero ssd_status and leaves every output untouched
 *    (fail closed, RFC section 4.1 and section 7 "Fail closed"); there is no
 *    fallback path.  Validation reads no device memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  A launch error is returned as SSD_ERR_HIP; device faults
 *    surface at the caller's next synchronisation.
 *  - Results are deterministic: fixed reduction order, no atomics
 *    (RFC section 4.1, WS1 rules).
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 1

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,      /* a required pointer is NULL                       */
    SSD_ERR_BAD_SHAPE = 2,     /* negative size, H % G != 0, batch*L too large ... */
    SSD_ERR_BAD_DTYPE = 3,     /* io dtype not one of ssd_dtype                    */
    SSD_ERR_UNSUPPORTED = 4,   /* (dtype, P, N, chunk) outside the compiled set    */
    SSD_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than required          */
    SSD_ERR_BAD_ARG = 6,       /* dt_min > dt_max, NaN clamp bound, ...            */
    SSD_ERR_ALIAS = 7,         /* an output overlaps an input it must not overlap  */
    SSD_ERR_HIP = 8,           /* a HIP launch returned an error                   */
    SSD_ERR_TOO_LARGE = 9,     /* needs more scratch than the library's static
                                  buffer holds (allocation-free entry point)       */
    SSD_ERR_BAD_SEQ_IDX = 10   /* seq_idx decreases along a row (opt-in check)     */
} ssd_status;

/* dtype of x, B, C and y.  A C caller may pass any int here (others are
 * rejected with SSD_ERR_BAD_DTYPE); in C++ the enum has int32_t as its fixed
 * underlying type so that every such value is a valid one, as in C. */
#ifdef __cplusplus
typedef enum : int32_t { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;
#else
typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;
#endif

typedef struct {
    int64_t batch;      /* b >= 0                                  */
    int64_t seqlen;     /* L >= 0 (any length; last chunk may be short) */
    int64_t nheads;     /* H >= 1                                  */
    int64_t headdim;    /* P                                       */
    int64_t dstate;     /* N                                       */
    int64_t ngroups;    /* G >= 1, H % G == 0                      */
    int64_t chunk_size; /* Q                                       */
} ssd_dims;

/* Bytes of device workspace ssd_chunk_scan_fwd needs for these dims (0 when
 * none).  Returns 0 as well for dims it would reject; call ssd_chunk_scan_fwd
 * to learn why. */
size_t ssd_chunk_scan_workspace_bytes(const ssd_dims* dims, ssd_dtype io);

/* Number of sequence segments a scan of these dims is split into (1 = each
 * row's state is carried through the whole row by one workgroup; more = the
 * rows are cut into segments whose states are chained by an extra pass).
 * Informational; 0 for dims the scan would reject. */
int64_t ssd_chunk_scan_segments(const ssd_dims* dims, ssd_dtype io);

/*
 * Opt-in checks of the seq_idx precondition of ssd_chunk_scan_fwd (every row
 * non-decreasing).  The scan itself never reads seq_idx on the host, so a
 * violation is not detected there; these calls are for debugging and for
 * callers that build seq_idx themselves.
 *   ssd_check_seq_idx_host: seq_idx is a HOST pointer (b, L) int32; pure host
 *     code.  Returns SSD_OK, SSD_ERR_BAD_SEQ_IDX at the first decrease,
 *     SSD_ERR_NULL_ARG (NULL with b * L > 0) or SSD_ERR_BAD_SHAPE (b or L < 0,
 *     or b * L values too many to address).
 *   ssd_check_seq_idx: seq_idx is a DEVICE pointer; the call copies it to the
 *     host on `stream`, waits for that copy (it synchronises the stream) and
 *     checks it as above.  SSD_ERR_BAD_SHAPE as well when b * L > 2^31 (the
 *     size of the host copy); SSD_ERR_HIP when the copy fails.
 */
ssd_status ssd_check_seq_idx_host(const int32_t* seq_idx, int64_t b, int64_t L);
ssd_status ssd_check_seq_idx(const int32_t* seq_idx, int64_t b, int64_t L, void* stream);

/* 1 when (io, headdim, dstate, chunk_size) is in the compiled set, else 0. */
int ssd_chunk_scan_supported(ssd_dtype io, int64_t headdim, int64_t dstate,
                             int64_t chunk_size);

/*
 * Chunked SSD scan over a batch of sequences (prefill / training forward).
 *
 *   x        (b, L, H, P)  io dtype
 *   dt       (b, L, H)     fp32, raw (before bias and softplus)
 *   dt_bias  (H)           fp32, or NULL = 0
 *   dt_softplus            non-zero: dt = softplus(dt + dt_bias); zero: dt = dt + dt_bias
 *   dt_min, dt_max         clamp applied after softplus; pass 0 and +INFINITY for none
 *   A        (H)           fp32, expected <= 0 (the caller forms -exp(A_log))
 *   B, C     (b, L, G, N)  io dtype
 *   D        (H)           fp32, or NULL = 0 (skip connection D * x)
 *   initial_states (b, H, P, N) fp32, or NULL = zero state; it belongs to the
 *                          sequence holding token 0 of each row
 *   seq_idx  (b, L)        int32, or NULL.  Packed sequences: non-decreasing
 *                          along each row; the state restarts from zero at every
 *                          token whose value differs from the previous token's.
 *                          (Non-monotone rows are a precondition violation: the
 *                          library does not read device memory to check them.)
 *   y        (b, L, H, P)  io dtype, output; must not overlap any input
 *   final_states (b, H, P, N) fp32 output or NULL: the state after token L-1 of
 *                          each row; may be the same pointer as initial_states
 *                          (exactly equal, not partially overlapping)
 *   workspace, workspace_bytes  device scratch of at least
 *                          ssd_chunk_scan_workspace_bytes(dims, io) bytes, 256-byte
 *                          aligned; contents on entry are ignored
 *   stream                 hipStream_t
 *
 * Supported set: see ssd_chunk_scan_supported.  L = 0 is allowed (final_states
 * then receives initial_states, or zeros).
 */
ssd_status ssd_chunk_scan_fwd(const ssd_dims* dims, ssd_dtype io, const void* x,
                              const float* dt, const float* dt_bias, int dt_softplus,
                              float dt_min, float dt_max, const float* A, const void* B,
                              const void* C, const float* D, const float* initial_states,
                              const int32_t* seq_idx, void* y, float* final_states,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssd_chunk_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it).  Same arguments, same
 * kernels and bitwise the same results as ssd_chunk_scan_fwd; the scratch
 * the scan needs comes from a static device array of the library
 * (SSD_NOALLOC_SCRATCH_BYTES per GPU, held by every GPU the library runs on
 * until the process ends).  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.
 *  - Dims whose workspace (ssd_chunk_scan_workspace_bytes) exceeds
 *    SSD_NOALLOC_SCRATCH_BYTES are rejected with SSD_ERR_TOO_LARGE before any
 *    launch.
 *  - The array's device address is looked up once per device, on the first
 *    call made with that device current; `stream` must belong to the current
 *    device.  A failed lookup returns SSD_ERR_HIP.
 *  - Every call on one GPU shares that GPU's array, and the scan writes each
 *    scratch word before reading it (nothing needs to start at zero).  Calls
 *    that overlap in time on one GPU (different streams, or host threads
 *    without ordering between them) race on the array and give wrong
 *    results: serialise them, for example on one stream.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_dims* dims, ssd_dtype io, const void* x,
                                      const float* dt, const float* dt_bias, int dt_softplus,
                                      float dt_min, float dt_max, const float* A,
                                      const void* B, const void* C, const float* D,
                                      const float* initial_states, const int32_t* seq_idx,
                                      void* y, float* final_states, void* stream);

/*
 * The forward scan of a batch of prompts whose states live in a state cache
 * (continuous batching: the per-sequence fp32 SSM state of RFC section 1,
 * operator family 2, kept in slots across prefill and decode).  Row r of the
 * batch is one sequence: its real tokens are [0, seq_lens[r]) of the row
 * (seq_lens NULL: all L; values are clamped to [0, L]); later tokens are
 * padding: they are not read, cost no work past the row's last chunk, and
 * leave the state as it is.  The
 * row starts from slot state_indices[r] of state_cache (cache_rows, H, P, N)
 * fp32 when init_from_cache != 0, else from zeros, and its state after its
 * last real token is written back to that slot.  An index outside
 * [0, cache_rows) marks a padding row: it is scanned from zeros and its state
 * is dropped.  The indices of the other rows must be distinct (two rows
 * naming one slot race); the library does not read device memory to check.
 * y (b, L, H, P): rows past a row's length are not written.  Other arguments as
 * ssd_chunk_scan_fwd (no seq_idx: a row is one sequence).  The workspace
 * (ssd_chunk_scan_cached_workspace_bytes, 256-byte aligned) holds the scan's
 * and the gathered states.  Dispatch order: slot gather, the scan's kernels,
 * slot scatter.  L = 0 reads no input (x, dt, A, B, C and y may be NULL): a
 * live row's slot is left as it is when init_from_cache != 0 and cleared to
 * zeros otherwise (one scatter launch).  strict != 0 runs every row as one segment of chunks whatever
 * the batch, and forms every intra-chunk decay exp(cs_i - cs_j) per element
 * (RFC section 4.1: batch-invariant arithmetic): a row's outputs and state
 * are then bitwise the same in any batch, and the chunk-emulating decode
 * (ssd_decode_emulated, always strict) continues them bit for bit.  strict = 0 lets the
 * library cut rows into segments to fill the GPU (faster for few rows; the
 * bits then depend on the number of rows x heads).
 */
size_t ssd_chunk_scan_cached_workspace_bytes(const ssd_dims* d, ssd_dtype io);
ssd_status ssd_chunk_scan_fwd_cached(const ssd_dims* d, ssd_dtype io, const void* x,
                                     const float* dt, const float* dt_bias, int dt_softplus,
                                     float dt_min, float dt_max, const float* A, const void* B,
                                     const void* C, const float* D, const int32_t* seq_lens,
                                     float* state_cache, int64_t cache_rows,
                                     const int32_t* state_indices, int init_from_cache, int strict,
                                     void* y, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Chunk-emulating decode (RFC section 1, operator family 1: "batch invariant"
 * covers how a sequence is split into prefill and decode steps; section 3,
 * Figure 2, box [F2]: the SSD scan's "chunk-emulating decode").  One token per
 * batch row; row r works on slot state_indices[r], whose new token sits at
 * offset positions[r] (0..Q-1) of its current chunk.  Per slot the caller
 * keeps:
 *   state_cache (slots, H, P, N) fp32: the state at the start of the slot's
 *                current chunk (for example from ssd_chunk_scan_fwd_cached
 *                over a prompt whose length is a multiple of Q);
 *   x_chunks (slots, Q, H, P) io, dt_chunks (slots, Q, H) fp32 (raw dt),
 *   b_chunks, c_chunks (slots, Q, G, N) io: the tokens of the current chunk so
 *                far (offsets below positions[r]; their contents past that
 *                are never read).
 * The call writes the new token into offset positions[r] of the slot's chunk
 * buffers, runs the chunked scan over offsets 0..positions[r] from the
 * chunk-start state, and writes y (b, H, P) io: the value the chunked prefill
 * gives that token.  When positions[r] = Q - 1 the chunk is complete and its
 * final state replaces the slot's chunk-start state.  An index outside
 * [0, cache_rows) or a position outside [0, Q) marks a padding row: its slot
 * and its y row are not touched.  Live rows must name distinct slots.
 * dims: batch b, seqlen = chunk_size = Q (one chunk), H, P, N, G as for the
 * scan and in its compiled set.  The scan reads each slot's chunk buffers and
 * chunk-start state in place (x_chunks, b_chunks, c_chunks, state_cache and y
 * 16-byte aligned) and computes only the 16-token row block that holds the
 * new token (the chunk's state only when it completes).  The workspace
 * (ssd_decode_emulated_workspace_bytes, 256-byte aligned) holds the chunk's
 * scan data.  This is the strict decode, not the fast one (ssd_state_update).
 * Dispatch order: chunk_prep (which also copies the new tokens into their
 * slots' chunk buffers), chunk_output for the rows whose chunk does not
 * complete, chunk_output for the others (a launch of at most as many
 * workgroups as the device runs at once, each taking several rows' heads).
 */
size_t ssd_decode_emulated_workspace_bytes(const ssd_dims* d, ssd_dtype io);
ssd_status ssd_decode_emulated(const ssd_dims* d, ssd_dtype io, const void* x, const float* dt,
                               const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                               const float* A, const void* B, const void* C, const float* D,
                               float* state_cache, void* x_chunks, float* dt_chunks,
                               void* b_chunks, void* c_chunks, int64_t cache_rows,
                               const int32_t* state_indices, const int32_t* positions, void* y,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length prefill (RFC section 8, open question 4: cu_seqlens-
 * aware chunking).  x (T, H, P), dt (T, H), B, C (T, G, N) hold nseq
 * sequences back to back, sequence r at tokens [cu_seqlens[r],
 * cu_seqlens[r+1]) (int32 on the device, nseq + 1 entries, non-decreasing
 * from 0 to T).  Each sequence is chunked from its own first token and runs
 * as one row of the cached prefill (ssd_chunk_scan_fwd_cached), read and
 * written in place in the packed layout (no copies, no padding work): it
 * starts from slot state_indices[r] of state_cache (or zeros) and its final
 * state is written back to that slot; strict as there.  y (T, H, P) receives
 * every sequence's outputs.  Its results are bitwise those of the cached
 * prefill over the same sequences as rows of one batch.  dims: batch = nseq,
 * seqlen = max_seqlen (no sequence longer: a longer one is cut to it, its
 * later tokens' y not written; offsets outside [0, T] are clamped, so that no
 * access leaves the buffers).  Workspace:
 * ssd_chunk_scan_varlen_workspace_bytes (the cached prefill's).  T = 0 reads
 * no token (x, dt, B, C, y may be NULL) and treats every sequence as empty.
 */
size_t ssd_chunk_scan_varlen_workspace_bytes(const ssd_dims* d, ssd_dtype io);
ssd_status ssd_chunk_scan_fwd_varlen(const ssd_dims* d, int64_t total_tokens, ssd_dtype io,
                                     const void* x, const float* dt, const float* dt_bias,
                                     int dt_softplus, float dt_min, float dt_max, const float* A,
                                     const void* B, const void* C, const float* D,
                                     const int32_t* cu_seqlens, float* state_cache,
                                     int64_t cache_rows, const int32_t* state_indices,
                                     int init_from_cache, int strict, void* y, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Bytes of device workspace ssd_chunk_scan_bwd needs for these dims (0 when
 * none, and for dims it would reject). */
size_t ssd_chunk_scan_bwd_workspace_bytes(const ssd_dims* dims, ssd_dtype io);

/*
 * Gradients of ssd_chunk_scan_fwd: the backward pass of the chunked scan that
 * training runs (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1, operator
 * family 1: the chunked parallel scan serves training).  Given the forward
 * inputs and the gradients of a loss with respect to y and to the final
 * states, writes the gradients with respect to every input.
 *
 *   x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D, initial_states,
 *   seq_idx          the forward call's inputs, same layouts and meaning
 *   dy       (b, L, H, P)  io dtype: gradient with respect to y
 *   d_final_states (b, H, P, N) fp32, or NULL = zero: gradient with respect
 *                          to final_states
 *   dx       (b, L, H, P)  io dtype output
 *   ddt      (b, L, H)     fp32 output: gradient with respect to the raw dt
 *                          (zero where the clamp binds)
 *   dA       (H)           fp32 output
 *   dB, dC   (b, L, G, N)  io dtype outputs (summed over each group's heads)
 *   dD, ddt_bias (H)       fp32 outputs, or NULL to skip
 *   d_initial_states (b, H, P, N) fp32 output, or NULL to skip
 *   workspace, workspace_bytes  device scratch of at least
 *                          ssd_chunk_scan_bwd_workspace_bytes(dims, io) bytes,
 *                          256-byte aligned; contents on entry are ignored
 *   stream                 hipStream_t
 *
 * No output may overlap an input, another output or the workspace
 * (SSD_ERR_ALIAS).  Supported set: io = SSD_BF16, headdim 64, dstate 128 or 64,
 * chunk_size 64, 128 or 256 (else SSD_ERR_UNSUPPORTED; the gradients are those
 * of the recurrence whatever the chunk size, and the kernels run 128-token
 * chunks); any b, L (L = 0 gives zero sums and d_initial_states =
 * d_final_states), H % G == 0.  Deterministic: every sum is taken in a fixed
 * order, without atomics.  A row's dx, ddt, dB, dC and d_initial_states are
 * bitwise the same in any batch (dA, dD and ddt_bias sum over the batch).
 */
ssd_status ssd_chunk_scan_bwd(const ssd_dims* dims, ssd_dtype io, const void* x,
                              const float* dt, const float* dt_bias, int dt_softplus,
                              float dt_min, float dt_max, const float* A, const void* B,
                              const void* C, const float* D, const float* initial_states,
                              const int32_t* seq_idx, const void* dy,
                              const float* d_final_states, void* dx, float* ddt, float* dA,
                              void* dB, void* dC, float* dD, float* ddt_bias,
                              float* d_initial_states, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The steps beside the scan in the Mamba-2 mixer (RL-Kernel RFC
 * "Nemotron-3-Nano-30B-A3B", section 3, Figure 2, box [F2]).
 *
 * ssd_conv1d_fwd: causal depthwise conv1d of width 4 + bias + SiLU over the
 * xBC channels (prefill), written straight into the scan's inputs:
 *   out_t[c] = silu(bias[c] + sum_{k<4} weight[c][k] * in_{t-3+k}[c]),
 * inputs before token 0 taken from conv_state_in (oldest first) or zero; with
 * seq_idx, an input of another sequence counts as zero (the state belongs to
 * the sequence of token 0).
 *   xbc      (b, L, dim)  io dtype, dim = nx + 2 * nb
 *   weight   (dim, 4) fp32;  width must be 4;  bias (dim) fp32 or NULL
 *   conv_state_in  (b, dim, 3) io dtype or NULL (zero)
 *   seq_idx  (b, L) int32 or NULL (as for ssd_chunk_scan_fwd)
 *   x_out    (b, L, nx) io: channels [0, nx)   (the scan's x as (b, L, H, P))
 *   b_out, c_out (b, L, nb) io: channels [nx, nx + nb) and [nx + nb, dim)
 *                          (the scan's B and C as (b, L, G, N))
 *   conv_state_out (b, dim, 3) io or NULL: the last three inputs (zero where
 *                          they belong to another sequence than the last
 *                          token's); may be exactly conv_state_in (in place)
 * Supported: io F32 or BF16; dim, nx, nb multiples of 8.
 */
ssd_status ssd_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t nx, int64_t nb,
                          ssd_dtype io, const void* xbc, const float* weight, int64_t width,
                          const float* bias, const void* conv_state_in, const int32_t* seq_idx,
                          void* x_out, void* b_out, void* c_out, void* conv_state_out,
                          void* stream);

/* One decode token of the conv: xbc (b, dim), conv_state (b, dim, 3) read and
 * updated in place (shifted by the new input); outputs x_out (b, nx), b_out,
 * c_out (b, nb).  Same supported set as ssd_conv1d_fwd. */
ssd_status ssd_conv1d_update(int64_t batch, int64_t dim, int64_t nx, int64_t nb, ssd_dtype io,
                             const void* xbc, const float* weight, int64_t width, const float* bias,
                             void* conv_state, void* x_out, void* b_out, void* c_out, void* stream);

/* ssd_conv1d_update on a conv-state cache (continuous batching; the
 * per-sequence conv state of RFC section 1, operator family 2): row r of
 * the batch reads and updates row state_indices[r] of conv_state_cache
 * (cache_rows, dim, 3) io dtype in place.  state_indices (batch) int32 on the
 * device.  An index outside [0, cache_rows) marks a padding row: its cache
 * row is not touched and its outputs are not written.  The indices of the
 * other rows must be distinct (two rows naming one cache row race); the
 * library does not read device memory to check.  Otherwise as
 * ssd_conv1d_update; cache_rows = batch with indices 0..batch-1 is the same
 * call. */
ssd_status ssd_conv1d_update_cached(int64_t batch, int64_t cache_rows, int64_t dim, int64_t nx,
                                    int64_t nb, ssd_dtype io, const void* xbc, const float* weight,
                                    int64_t width, const float* bias, void* conv_state_cache,
                                    const int32_t* state_indices, void* x_out, void* b_out,
                                    void* c_out, void* stream);

/* Gated group RMSNorm of the scan's output: per row and group of `group`
 * consecutive channels, v = y * silu(z) and out = v / sqrt(mean(v^2) + eps) *
 * weight.  y, z, out (rows, dim) io dtype; weight (dim) fp32; eps >= 0 (the
 * pages' RMSNorm epsilon is 1e-6).  Supported: group a multiple of 8, at most
 * 4096, dividing dim. */
ssd_status ssd_gated_rmsnorm(int64_t rows, int64_t dim, int64_t group, ssd_dtype io, const void* y,
                             const void* z, const float* weight, float eps, void* out, void* stream);

/*
 * One decode token per sequence: the per-token recurrent state update (RFC
 * section 1, operator family 1; the state is the fixed-size fp32 SSM state of
 * operator family 2).
 *
 *   state  (b, H, P, N) fp32, read and updated in place
 *   x      (b, H, P)    io dtype
 *   dt     (b, H)       fp32 raw;  dt_bias (H) or NULL; dt_softplus, dt_min, dt_max as above
 *   A      (H) fp32;  B, C (b, G, N) io dtype;  D (H) fp32 or NULL
 *   y      (b, H, P)    io dtype output, computed from the updated state
 *
 * Supported: io in {F32, BF16}; N in {16, 32, 64, 128, 256}; P >= 1; H % G == 0.
 */
ssd_status ssd_state_update(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                            int64_t ngroups, ssd_dtype io, float* state, const void* x,
                            const float* dt, const float* dt_bias, int dt_softplus,
                            float dt_min, float dt_max, const float* A, const void* B,
                            const void* C, const float* D, void* y, void* stream);

/* ssd_state_update on a state cache (continuous batching; the per-sequence
 * fp32 SSM state of RFC section 1, operator family 2, held in slots of one
 * buffer that outlives the batch): row
 * r of the batch reads and updates slot state_indices[r] of state_cache
 * (cache_rows, H, P, N) fp32 in place; x, dt, B, C, y keep the batch's rows.
 * state_indices (batch) int32 on the device.  An index outside
 * [0, cache_rows) marks a padding row: its slot is not touched and its y
 * rows are not written.  The indices of the other rows must be distinct (two
 * rows naming one slot race); the library does not read device memory to
 * check.  Otherwise as ssd_state_update; cache_rows = batch with indices
 * 0..batch-1 is the same call. */
ssd_status ssd_state_update_cached(int64_t batch, int64_t cache_rows, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype io,
                                   float* state_cache, const int32_t* state_indices,
                                   const void* x, const float* dt, const float* dt_bias,
                                   int dt_softplus, float dt_min, float dt_max, const float* A,
                                   const void* B, const void* C, const float* D, void* y,
                                   void* stream);

/* Per-kernel timing hooks (diagnostics).  After a call with events != NULL,
 * every ssd_chunk_scan_fwd / ssd_state_update call made on the same host
 * thread binds events[2k] and events[2k+1] to its k-th kernel dispatch, on
 * the call's stream, for k < count/2 (hipExtLaunchKernel's start and stop
 * events): they take that dispatch's own start and end timestamps, so
 * hipEventElapsedTime of the pair is the kernel's execution time.  The call
 * stores the number of kernels it launched in *launched (if not NULL).
 * `events` are hipEvent_t handles the caller created; the library only binds
 * them.  Kernel order of the scan: chunk_prep, [chunk_state, [state_pass,]]
 * chunk_output (chunk_state runs only when ssd_chunk_scan_segments(...) > 1,
 * state_pass only then and for kernels whose output pass does not combine the
 * segment states itself; L = 0 launches one state copy).  A NULL pair
 * events[2k], events[2k+1] skips kernel k.  Pass events = NULL to turn the
 * hooks off. */
void ssd_set_timing_events(void* const* events, int count, int* launched);

/* Static, human-readable text for a status code (never NULL). */
const char* ssd_status_string(int status);

/* SSD_ABI_VERSION of the built library. */
int ssd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
