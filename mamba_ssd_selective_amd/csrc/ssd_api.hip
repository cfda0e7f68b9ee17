// ssd_api.hip -- the C ABI of libssd.so (declared in include/ssd.h).
//
// Host side only: argument validation (fail closed before any launch, RL-Kernel
// RFC "Nemotron-3-Nano-30B-A3B" section 4.1 WS1 rules and section 7 "Fail
// closed"), workspace sizing, and the launch sequence of the chunked scan.
// Validation never touches the device, so it runs on machines without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/ssd.h"
#include "ssd_launch.h"

namespace {

// Rows x heads are cut into segments until there are about this many
// workgroups: one per CU of an MI355X (the scan kernels hold one workgroup per
// CU), so that every segment's workgroup runs in a single round.
constexpr int64_t kTargetWorkgroups = 256;
constexpr size_t kAlign = 256;

struct Plan {
    int64_t Qk = 0;  // chunk size the kernels run with
    int64_t nc = 0;
    int64_t nseg = 1, cps = 1;
    size_t off_cs = 0, off_dtv = 0, off_wgt = 0, off_cbt = 0, off_cmf = 0;
    bool has_cmf = false;
    size_t off_seg = 0, off_mult = 0, off_final = 0, total = 0;
};

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// one_segment: every row in one segment whatever the batch, so that a row's
// bits do not depend on the batch it is in (the strict mode's split; the scan
// then also takes the exact intra-chunk decay form in every chunk).
// The plan follows the variant that serves the call (strict calls: one that
// runs the caller's chunk size; others may run a divisor of it), and is laid
// out for the chunk size its kernels run with (Qk).
Plan make_plan(const ssd_dims& d, ssd_dtype io, bool one_segment = false) {
    Plan p;
    if (d.seqlen <= 0 || d.batch <= 0) return p;
    const ssd::ScanVariant* var =
        ssd::find_scan_variant(io, d.headdim, d.dstate, d.chunk_size, one_segment);
    const int64_t Qk = var ? var->kernel_Q : d.chunk_size;
    p.Qk = Qk;
    p.nc = (d.seqlen + Qk - 1) / Qk;
    const int64_t bh = d.batch * d.nheads;
    int64_t nseg = one_segment ? 1 : (kTargetWorkgroups + bh - 1) / bh;
    if (nseg < 1) nseg = 1;
    if (nseg > p.nc) nseg = p.nc;
    p.cps = (p.nc + nseg - 1) / nseg;
    p.nseg = (p.nc + p.cps - 1) / p.cps;
    const size_t f = sizeof(float);
    const size_t es = io == SSD_BF16 ? 2 : 4;
    // per-token metadata, one block [cs Q | dt Q | w Q] per (row, head, chunk)
    const size_t meta = static_cast<size_t>(bh * p.nc * Qk) * 3 * f;
    size_t off = 0;
    p.off_cs = off;
    p.off_dtv = off + static_cast<size_t>(Qk) * f;
    p.off_wgt = off + 2 * static_cast<size_t>(Qk) * f;
    off = align_up(off + meta);
    p.off_cbt = off;
    off = align_up(off + static_cast<size_t>(d.batch * p.nc * d.ngroups) *
                             static_cast<size_t>(ssd::cbt_elems_per_chunk_group(Qk)) * es);
    if (var != nullptr && var->output_reads_c_copy) {
        p.has_cmf = true;
        p.off_cmf = off;
        off = align_up(off + static_cast<size_t>(d.batch * p.nc * d.ngroups) *
                                 static_cast<size_t>(Qk * d.dstate) * es);
    }
    if (p.nseg > 1) {
        p.off_seg = off;
        off = align_up(off + static_cast<size_t>(bh * p.nseg * d.headdim * d.dstate) * f);
        p.off_mult = off;
        off = align_up(off + static_cast<size_t>(bh * p.nseg) * f);
        // where the final states go when the caller's final states are its
        // initial states: every segment's workgroup reads the initial state,
        // while the last segment's writes the final one, and with more
        // workgroups than fit at once the two can meet.  bh < 256 here, so
        // this area is below 256 states.
        p.off_final = off;
        off = align_up(off + static_cast<size_t>(bh * d.headdim * d.dstate) * f);
    }
    p.total = off;
    return p;
}

size_t io_size(ssd_dtype io) { return io == SSD_BF16 ? 2 : 4; }

// Workspace of a scan that may run in either mode (the strict flag is a
// call argument): the larger of the two plans.
size_t plan_bytes_any_mode(const ssd_dims& d, ssd_dtype io) {
    const size_t a = make_plan(d, io, false).total, b = make_plan(d, io, true).total;
    return a > b ? a : b;
}

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, size_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Span{a, a + bytes};
}
bool overlap(Span a, Span b) {
    if (a.lo == 0 || b.lo == 0 || a.hi == a.lo || b.hi == b.lo) return false;
    return a.lo < b.hi && b.lo < a.hi;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bad_clamp(float lo, float hi) { return isnan(lo) || isnan(hi) || lo > hi; }

// Optional per-kernel event recording (ssd_set_timing_events), per host thread.
struct TimingHooks {
    void* const* events = nullptr;
    int count = 0;
    int* launched = nullptr;
};
thread_local TimingHooks g_hooks;
thread_local ssd::DispatchEvents g_dispatch_events;

// Runs one launch (one kernel dispatch) with the k-th pair of timing events
// bound to it (when hooks are set).
template <typename F>
hipError_t timed_launch(int& k, hipStream_t, F&& launch) {
    const bool rec = g_hooks.events && 2 * k + 1 < g_hooks.count && g_hooks.events[2 * k] &&
                     g_hooks.events[2 * k + 1];
    ssd::DispatchEvents& ev = ssd::dispatch_events();
    if (rec) {
        ev.start = static_cast<hipEvent_t>(g_hooks.events[2 * k]);
        ev.stop = static_cast<hipEvent_t>(g_hooks.events[2 * k + 1]);
    }
    hipError_t e = launch();
    ev = ssd::DispatchEvents{};
    ++k;
    if (g_hooks.launched) *g_hooks.launched = k;
    return e;
}

// Shape checks shared by the workspace query and the scan entry point.
ssd_status check_scan_dims(const ssd_dims* d, ssd_dtype io) {
    if (!d) return SSD_ERR_NULL_ARG;
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_BAD_DTYPE;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1 || d->chunk_size < 1)
        return SSD_ERR_BAD_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    // index and grid limits: element offsets fit in int64, rows/heads in int
    if (d->batch > 65535 || d->nheads > 65535 || d->seqlen >= (int64_t(1) << 31))
        return SSD_ERR_BAD_SHAPE;
    if (!ssd::find_scan_variant(io, d->headdim, d->dstate, d->chunk_size))
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Chunk size the gradient kernels run with.
constexpr int64_t kBwdChunk = 128;

// The gradient path's compiled set: bf16, P = 64, N = 128 or 64, and chunk
// sizes 64, 128 and 256, all run as 128-token chunks.
ssd_status check_bwd_dims(const ssd_dims* d, ssd_dtype io) {
    if (!d) return SSD_ERR_NULL_ARG;
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_BAD_DTYPE;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1 || d->chunk_size < 1)
        return SSD_ERR_BAD_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (d->batch > 65535 || d->nheads > 65535 || d->seqlen >= (int64_t(1) << 31))
        return SSD_ERR_BAD_SHAPE;
    // the gradients of the scan are those of the recurrence whatever the
    // chunk size, so the caller's chunk grid (the forward's compiled chunks)
    // is served by the 128-token kernels
    if (io != SSD_BF16 || d->headdim != 64 || (d->dstate != 128 && d->dstate != 64) ||
        (d->chunk_size != 64 && d->chunk_size != 128 && d->chunk_size != 256))
        return SSD_ERR_UNSUPPORTED;
    // grids: (row, chunk, group) and (row, head) workgroups below 2^31
    const int64_t nc = (d->seqlen + kBwdChunk - 1) / kBwdChunk;
    if (d->batch * nc * d->ngroups >= (int64_t(1) << 31) || d->batch * d->nheads >= (int64_t(1) << 31))
        return SSD_ERR_BAD_SHAPE;
    return SSD_OK;
}

struct BwdPlan {
    int64_t nc = 0, nseg = 1, cps = 0;
    size_t off_meta = 0, off_states = 0, off_gstates = 0, off_partials = 0, off_seg = 0,
           off_mult = 0, total = 0;
};

// Chunks per segment of the gradient path's state walks.  Fixed in chunks
// (not chosen from rows x heads as the forward's segments are), so that a
// row's gradients are bitwise the same whatever batch it is in: at 8K, 4
// segments and 512 walk workgroups.
constexpr int64_t kBwdWalkChunks = 16;

// Workspace of the gradient path: the metadata blocks of chunk_prep_kernel,
// the bf16 state before and the gradient after every chunk, per-chunk sums,
// and (segmented walks) the segments' end states and decay products.
BwdPlan make_bwd_plan(const ssd_dims& d) {
    BwdPlan p;
    if (d.seqlen <= 0 || d.batch <= 0) return p;
    p.nc = (d.seqlen + kBwdChunk - 1) / kBwdChunk;
    p.cps = p.nc < kBwdWalkChunks ? p.nc : kBwdWalkChunks;
    p.nseg = (p.nc + p.cps - 1) / p.cps;
    const size_t bhc = static_cast<size_t>(d.batch * d.nheads * p.nc);
    size_t off = 0;
    p.off_meta = off;
    off = align_up(off + bhc * static_cast<size_t>(kBwdChunk) * 3 * sizeof(float));
    p.off_states = off;
    off = align_up(off + bhc * static_cast<size_t>(d.headdim * d.dstate) * sizeof(uint16_t));
    p.off_gstates = off;
    off = align_up(off + bhc * static_cast<size_t>(d.headdim * d.dstate) * sizeof(uint16_t));
    p.off_partials = off;
    off = align_up(off + bhc * 3 * sizeof(float));
    if (p.nseg > 1) {
        const size_t segs = static_cast<size_t>(2 * d.batch * d.nheads * p.nseg);
        p.off_seg = off;
        off = align_up(off + segs * static_cast<size_t>(d.headdim * d.dstate) * sizeof(float));
        p.off_mult = off;
        off = align_up(off + segs * sizeof(float));
    }
    p.total = off;
    return p;
}

}  // namespace

ssd::DispatchEvents& ssd::dispatch_events() { return g_dispatch_events; }

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

void ssd_set_timing_events(void* const* events, int count, int* launched) {
    g_hooks.events = events;
    g_hooks.count = events ? count : 0;
    g_hooks.launched = events ? launched : nullptr;
}

const char* ssd_status_string(int s) {
    switch (s) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL_ARG: return "a required pointer argument is NULL";
        case SSD_ERR_BAD_SHAPE: return "invalid shape (negative size, H % G != 0, or a size limit)";
        case SSD_ERR_BAD_DTYPE: return "io dtype is not SSD_F32 or SSD_BF16";
        case SSD_ERR_UNSUPPORTED: return "(dtype, headdim, dstate, chunk_size) is outside the compiled set";
        case SSD_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than required";
        case SSD_ERR_BAD_ARG: return "invalid argument (dt clamp bounds, or a buffer not 16-byte aligned)";
        case SSD_ERR_ALIAS: return "an output buffer overlaps an input it must not overlap";
        case SSD_ERR_HIP: return "a HIP kernel launch failed";
        case SSD_ERR_TOO_LARGE: return "needs more scratch than the allocation-free entry point's static buffer holds";
        case SSD_ERR_BAD_SEQ_IDX: return "seq_idx decreases along a row";
        default: return "unknown ssd_status";
    }
}

ssd_status ssd_check_seq_idx_host(const int32_t* seq_idx, int64_t b, int64_t L) {
    if (b < 0 || L < 0) return SSD_ERR_BAD_SHAPE;
    if (b == 0 || L == 0) return SSD_OK;
    if (!seq_idx) return SSD_ERR_NULL_ARG;
    // b * L int32 values must fit in the address space
    if (b > INT64_MAX / int64_t(sizeof(int32_t)) / L) return SSD_ERR_BAD_SHAPE;
    for (int64_t r = 0; r < b; ++r) {
        const int32_t* row = seq_idx + r * L;
        for (int64_t t = 1; t < L; ++t)
            if (row[t] < row[t - 1]) return SSD_ERR_BAD_SEQ_IDX;
    }
    return SSD_OK;
}

ssd_status ssd_check_seq_idx(const int32_t* seq_idx, int64_t b, int64_t L, void* stream) {
    if (b < 0 || L < 0) return SSD_ERR_BAD_SHAPE;
    if (b == 0 || L == 0) return SSD_OK;
    if (!seq_idx) return SSD_ERR_NULL_ARG;
    if (L > (int64_t(1) << 31) || b > (int64_t(1) << 31) / L) return SSD_ERR_BAD_SHAPE;
    std::vector<int32_t> host(static_cast<size_t>(b * L));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(host.data(), seq_idx, host.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                       hs) != hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess)
        return SSD_ERR_HIP;
    return ssd_check_seq_idx_host(host.data(), b, L);
}

int ssd_chunk_scan_supported(ssd_dtype io, int64_t headdim, int64_t dstate, int64_t chunk_size) {
    return ssd::find_scan_variant(io, headdim, dstate, chunk_size) != nullptr;
}

size_t ssd_chunk_scan_workspace_bytes(const ssd_dims* d, ssd_dtype io) {
    if (check_scan_dims(d, io) != SSD_OK) return 0;
    return make_plan(*d, io).total;
}

// Number of sequence segments the scan of these dims is split into (1 = the
// state is carried through each whole row inside one workgroup).  Informational.
int64_t ssd_chunk_scan_segments(const ssd_dims* d, ssd_dtype io) {
    if (check_scan_dims(d, io) != SSD_OK) return 0;
    return make_plan(*d, io).nseg;
}

}  // extern "C"

namespace {

// Where the scan's rows are (ScanArgs has the same fields):
//  row_len (b) or null: row r ends after row_len[r] tokens;
//  cu (b + 1) or null: packed rows, row r is tokens [cu[r], cu[r+1]) of the T
//    tokens of x, dt, B, C and y (no seq_idx then);
//  slot (b) or null: row r is slot slot[r] of buffers of `slots` rows of L
//    tokens, its initial and final states those of the slot;
//  y_last (b, H, P) or null: decode output (each row's last token only; a
//    row's final state is written only when it holds L tokens).
struct RowLayout {
    const int32_t* row_len = nullptr;
    const int32_t* cu = nullptr;
    int64_t T = 0;
    const int32_t* slot = nullptr;
    int64_t slots = 0;
    void* y_last = nullptr;
    // emulated decode: new-token offsets and arrays (ScanArgs::pos, tok_*)
    const int32_t* pos = nullptr;
    const void* tok_x = nullptr;
    const float* tok_dt = nullptr;
    const void* tok_B = nullptr;
    const void* tok_C = nullptr;
};

// The forward scan over rows laid out as `rl` says.  k counts the dispatches
// of the calling entry point; before() runs once the arguments are validated,
// ahead of the scan's first launch.
template <typename F>
ssd_status scan_fwd_impl(const ssd_dims* d, ssd_dtype io, const void* x, const float* dt,
                         const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                         const float* A, const void* B, const void* C, const float* D,
                         const float* initial_states, const int32_t* seq_idx,
                         const RowLayout& rl, void* y, float* final_states, void* workspace,
                         size_t workspace_bytes, hipStream_t hs, int& k, F&& before,
                         bool one_segment = false) {
    ssd_status st = check_scan_dims(d, io);
    if (st != SSD_OK) return st;
    if (one_segment && !ssd::find_scan_variant(io, d->headdim, d->dstate, d->chunk_size, true))
        return SSD_ERR_UNSUPPORTED;
    if (bad_clamp(dt_min, dt_max)) return SSD_ERR_BAD_ARG;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim,
                  N = d->dstate, G = d->ngroups;
    if (rl.cu && (seq_idx || rl.row_len || rl.slot || rl.T < 0)) return SSD_ERR_BAD_ARG;
    // slots and the decode output: single-segment scans of rows of one chunk
    if ((rl.slot || rl.y_last) && (!one_segment || seq_idx || rl.slots < 0 || L != d->chunk_size))
        return SSD_ERR_BAD_ARG;
    // tokens of x, dt, B, C (and y), and rows of states
    const int64_t toks = rl.cu ? rl.T : (rl.slot ? rl.slots * L : b * L);
    const int64_t srows = rl.slot ? rl.slots : b;
    const bool work = b > 0 && L > 0;
    if (work && (!x || !dt || !A || !B || !C || !(rl.y_last ? rl.y_last : y)))
        return SSD_ERR_NULL_ARG;
    const Plan plan = make_plan(*d, io, one_segment);
    if (plan.total > 0 &&
        (!workspace || workspace_bytes < plan.total ||
         (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0))
        return SSD_ERR_WORKSPACE;
    const void* vec_bufs[] = {x, B, C, y, rl.y_last, initial_states, final_states};
    for (const void* p : vec_bufs)
        if (p && !aligned16(p)) return SSD_ERR_BAD_ARG;
    const int64_t sbytes = srows * H * P * N * 4;
    if (initial_states && final_states && initial_states != final_states &&
        overlap(span(initial_states, sbytes), span(final_states, sbytes)))
        return SSD_ERR_ALIAS;
    const size_t es = io_size(io);
    const Span in_spans[] = {
        span(x, toks * H * P * es), span(dt, toks * H * 4), span(B, toks * G * N * es),
        span(C, toks * G * N * es), span(A, H * 4), span(dt_bias, dt_bias ? H * 4 : 0),
        span(D, D ? H * 4 : 0), span(seq_idx, seq_idx ? b * L * 4 : 0),
        span(rl.row_len, rl.row_len ? b * 4 : 0), span(rl.cu, rl.cu ? (b + 1) * 4 : 0),
        span(rl.slot, rl.slot ? b * 4 : 0),
    };
    const Span ys = rl.y_last ? span(rl.y_last, b * H * P * es) : span(y, toks * H * P * es);
    const Span fs = span(final_states, final_states ? sbytes : 0);
    const Span is = span(initial_states, initial_states ? sbytes : 0);
    const Span ws = span(workspace, plan.total);
    for (const Span& s : in_spans) {
        if (overlap(ys, s) || overlap(fs, s) || overlap(ws, s)) return SSD_ERR_ALIAS;
    }
    if (overlap(ys, fs) || overlap(ys, is) || overlap(ys, ws) || overlap(fs, ws) ||
        overlap(is, ws))
        return SSD_ERR_ALIAS;

    if (b == 0) return SSD_OK;
    if (before() != hipSuccess) return SSD_ERR_HIP;
    if (L == 0) {
        if (final_states) {
            if (timed_launch(k, hs, [&] {
                    return ssd::launch_copy_state(initial_states, final_states, b * H * P * N, hs);
                }) != hipSuccess)
                return SSD_ERR_HIP;
        }
        return SSD_OK;
    }
    const ssd::ScanVariant* var = ssd::find_scan_variant(io, P, N, d->chunk_size, one_segment);
    char* wsb = static_cast<char*>(workspace);

    ssd::ScanArgs sa{};
    sa.x = x;
    sa.B = B;
    sa.C = C;
    sa.y = y;
    sa.dt_raw = dt;
    sa.dt_bias = dt_bias;
    sa.A = A;
    sa.softplus = dt_softplus ? 1 : 0;
    sa.dt_min = dt_min;
    sa.dt_max = dt_max;
    sa.seq_idx = seq_idx;
    sa.row_len = rl.row_len;
    sa.cu = rl.cu;
    sa.T = rl.T;
    sa.slot = rl.slot;
    sa.slots = rl.slots;
    sa.y_last = rl.y_last;
    sa.pos = rl.pos;
    sa.tok_x = rl.tok_x;
    sa.tok_dt = rl.tok_dt;
    sa.tok_B = rl.tok_B;
    sa.tok_C = rl.tok_C;
    sa.exact_decay = one_segment ? 1 : 0;
    sa.D = D;
    sa.init = initial_states;
    sa.final_states = final_states;
    // final states written over the initial states they start from: to the
    // workspace first, copied over the initial states once the scan is done
    const bool final_in_ws = final_states && final_states == initial_states && plan.nseg > 1;
    if (final_in_ws) sa.final_states = reinterpret_cast<float*>(wsb + plan.off_final);
    sa.seg_state = plan.nseg > 1 ? reinterpret_cast<float*>(wsb + plan.off_seg) : nullptr;
    sa.seg_mult = plan.nseg > 1 ? reinterpret_cast<float*>(wsb + plan.off_mult) : nullptr;
    sa.cs = reinterpret_cast<float*>(wsb + plan.off_cs);
    sa.dtv = reinterpret_cast<float*>(wsb + plan.off_dtv);
    sa.wgt = reinterpret_cast<float*>(wsb + plan.off_wgt);
    sa.cbt = wsb + plan.off_cbt;
    sa.cmf = plan.has_cmf ? wsb + plan.off_cmf : nullptr;
    sa.L = L;
    sa.H = static_cast<int>(H);
    sa.G = static_cast<int>(G);
    sa.nc = static_cast<int>(plan.nc);
    sa.nseg = static_cast<int>(plan.nseg);
    sa.cps = static_cast<int>(plan.cps);

    if (timed_launch(k, hs, [&] { return var->chunk_prep(sa, b * plan.nc * G, hs); }) !=
        hipSuccess)
        return SSD_ERR_HIP;
    if (plan.nseg > 1) {
        if (timed_launch(k, hs, [&] {
                return var->chunk_state(sa, b * (plan.nseg - 1) * H, hs);
            }) != hipSuccess)
            return SSD_ERR_HIP;
        if (!var->output_combines_segments) {
            ssd::PassArgs pa;
            pa.seg_state = sa.seg_state;
            pa.seg_mult = sa.seg_mult;
            pa.init = initial_states;
            pa.PN = P * N;
            pa.nseg = static_cast<int>(plan.nseg);
            if (timed_launch(k, hs, [&] { return ssd::launch_state_pass(pa, b * H, hs); }) !=
                hipSuccess)
                return SSD_ERR_HIP;
        }
    }
    if (rl.y_last && var->output_combines_segments) {
        // decode output on the transposing-read kernels: the rows whose chunk
        // does not complete, then those whose chunk does
        for (int pass = 1; pass <= 2; ++pass) {
            sa.dec_pass = pass;
            if (timed_launch(k, hs, [&] { return var->chunk_output(sa, b * plan.nseg * H, hs); }) !=
                hipSuccess)
                return SSD_ERR_HIP;
        }
    } else if (timed_launch(k, hs, [&] { return var->chunk_output(sa, b * plan.nseg * H, hs); }) !=
               hipSuccess) {
        return SSD_ERR_HIP;
    }
    if (final_in_ws) {
        if (timed_launch(k, hs, [&] {
                return ssd::launch_copy_state(sa.final_states, final_states, b * H * P * N, hs);
            }) != hipSuccess)
            return SSD_ERR_HIP;
    }
    return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status ssd_chunk_scan_fwd(const ssd_dims* d, ssd_dtype io, const void* x, const float* dt,
                              const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                              const float* A, const void* B, const void* C, const float* D,
                              const float* initial_states, const int32_t* seq_idx, void* y,
                              float* final_states, void* workspace, size_t workspace_bytes,
                              void* stream) {
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    return scan_fwd_impl(d, io, x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D,
                         initial_states, seq_idx, RowLayout{}, y, final_states, workspace,
                         workspace_bytes, static_cast<hipStream_t>(stream), k,
                         [] { return hipSuccess; });
}

}  // extern "C"

namespace {

// Scratch of ssd_chunk_scan_fwd_noalloc: one copy per GPU, for the life of
// the process.  In host code `noalloc_scratch` names a host-side stand-in, not
// device memory: only the address that hipGetSymbolAddress returns for the
// current device is ever passed to a kernel.
__device__ __align__(256) char noalloc_scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of noalloc_scratch (looked up on its first
// use, with that device current), or null on failure.
void* noalloc_scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_dims* d, ssd_dtype io, const void* x,
                                      const float* dt, const float* dt_bias, int dt_softplus,
                                      float dt_min, float dt_max, const float* A, const void* B,
                                      const void* C, const float* D, const float* initial_states,
                                      const int32_t* seq_idx, void* y, float* final_states,
                                      void* stream) {
    ssd_status st = check_scan_dims(d, io);
    if (st != SSD_OK) return st;
    const size_t need = make_plan(*d, io).total;
    if (need > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (need > 0) {
        ws = noalloc_scratch_ptr();
        if (!ws) return SSD_ERR_HIP;
    }
    return ssd_chunk_scan_fwd(d, io, x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D,
                              initial_states, seq_idx, y, final_states, ws,
                              need > 0 ? SSD_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t ssd_chunk_scan_cached_workspace_bytes(const ssd_dims* d, ssd_dtype io) {
    if (check_scan_dims(d, io) != SSD_OK) return 0;
    if (d->batch == 0 || d->seqlen == 0) return 0;
    return align_up(plan_bytes_any_mode(*d, io)) +
           align_up(static_cast<size_t>(d->batch * d->nheads * d->headdim * d->dstate) * 4);
}

// The prefill of rows whose states live in cache slots: the rows are
// row_len-limited rows of L tokens (cu null) or packed rows at offsets cu
// into T tokens.
static ssd_status cached_prefill(const ssd_dims* d, ssd_dtype io, const void* x, const float* dt,
                                 const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                                 const float* A, const void* B, const void* C, const float* D,
                                 const int32_t* seq_lens, const int32_t* cu, int64_t T,
                                 float* state_cache, int64_t cache_rows,
                                 const int32_t* state_indices, int init_from_cache, int strict,
                                 void* y, void* workspace, size_t workspace_bytes, void* stream) {
    ssd_status st = check_scan_dims(d, io);
    if (st != SSD_OK) return st;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate;
    const int64_t k31 = int64_t(1) << 31;
    if (cache_rows < 0 || cache_rows >= k31) return SSD_ERR_BAD_SHAPE;
    if (cache_rows > 0 && H * P * N > (int64_t(1) << 60) / 4 / cache_rows) return SSD_ERR_BAD_SHAPE;
    if (bad_clamp(dt_min, dt_max)) return SSD_ERR_BAD_ARG;
    if (b > 0 && (!state_cache || !state_indices)) return SSD_ERR_NULL_ARG;
    if (state_cache && !aligned16(state_cache)) return SSD_ERR_BAD_ARG;
    const size_t need = ssd_chunk_scan_cached_workspace_bytes(d, io);
    if (need > 0 && (!workspace || workspace_bytes < need ||
                     (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0))
        return SSD_ERR_WORKSPACE;
    const size_t es = io_size(io);
    const int64_t G = d->ngroups;
    const int64_t toks = cu ? T : b * L;
    const Span cs = span(state_cache, cache_rows * H * P * N * 4);
    const Span others[] = {
        span(x, toks * H * P * es), span(dt, toks * H * 4), span(B, toks * G * N * es),
        span(C, toks * G * N * es), span(A, H * 4), span(dt_bias, dt_bias ? H * 4 : 0),
        span(D, D ? H * 4 : 0), span(seq_lens, seq_lens ? b * 4 : 0),
        span(cu, cu ? (b + 1) * 4 : 0), span(state_indices, state_indices ? b * 4 : 0),
        span(y, toks * H * P * es), span(workspace, need)};
    for (const Span& o : others)
        if (overlap(cs, o)) return SSD_ERR_ALIAS;
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    if (b == 0 || L == 0) {
        // nothing to scan (no input is read): a row that starts from its slot
        // keeps it as it is; one that starts from zeros ends in zeros, written
        // to its slot
        if (b > 0 && !init_from_cache) {
            hipStream_t hs0 = static_cast<hipStream_t>(stream);
            if (timed_launch(k, hs0, [&] {
                    return ssd::launch_scatter_slots(nullptr, state_indices, cache_rows, state_cache,
                                                     b, H * P * N, hs0);
                }) != hipSuccess)
                return SSD_ERR_HIP;
        }
        return SSD_OK;
    }
    const size_t scan_bytes = align_up(plan_bytes_any_mode(*d, io));
    float* states = reinterpret_cast<float*>(static_cast<char*>(workspace) + scan_bytes);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int64_t per_row = H * P * N;
    // the initial states gathered from their slots (zeros without them), the
    // scan's final states over them in place, then scattered back
    RowLayout rl;
    rl.row_len = seq_lens;
    rl.cu = cu;
    rl.T = T;
    st = scan_fwd_impl(d, io, x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D, states,
                       nullptr, rl, y, states, workspace, scan_bytes, hs, k, [&] {
                           return timed_launch(k, hs, [&] {
                               return ssd::launch_gather_slots(
                                   init_from_cache ? state_cache : nullptr, state_indices,
                                   cache_rows, states, b, per_row, hs);
                           });
                       }, strict != 0);
    if (st != SSD_OK) return st;
    if (timed_launch(k, hs, [&] {
            return ssd::launch_scatter_slots(states, state_indices, cache_rows, state_cache, b,
                                             per_row, hs);
        }) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd_cached(const ssd_dims* d, ssd_dtype io, const void* x,
                                     const float* dt, const float* dt_bias, int dt_softplus,
                                     float dt_min, float dt_max, const float* A, const void* B,
                                     const void* C, const float* D, const int32_t* seq_lens,
                                     float* state_cache, int64_t cache_rows,
                                     const int32_t* state_indices, int init_from_cache, int strict,
                                     void* y, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    return cached_prefill(d, io, x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D, seq_lens,
                          nullptr, 0, state_cache, cache_rows, state_indices, init_from_cache,
                          strict, y, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Chunk-emulating decode (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section
// 1, operator family 1, and section 3, Figure 2, box [F2]: the SSD scan runs
// train, prefill and decode with one arithmetic, so that how a sequence is
// split into prefill and decode steps does not change a bit of its outputs).
// A decode token at offset i of its chunk is not folded into a running state.
// Each slot keeps the state at its current chunk's start and that chunk's
// tokens so far.  A step runs the strict chunked scan on the slots in place,
// each row of length i + 1, in its decode-output form: chunk_prep takes the
// new token from the inputs and appends it to the slot's chunk buffers, and
// the output kernels compute only the row block of offset i and store only
// y at offset i, the value the chunked prefill computes for that token.  When
// the chunk is complete (i = Q - 1) the scan's state at its end replaces the
// slot's chunk-start state.
//
// Its workspace: the scan's (rows of one chunk, strict).
size_t emul_workspace(const ssd_dims& d, ssd_dtype io) {
    return align_up(make_plan(d, io, true).total);
}

ssd_status check_emul_dims(const ssd_dims* d, ssd_dtype io) {
    ssd_status st = check_scan_dims(d, io);
    if (st != SSD_OK) return st;
    if (d->seqlen != d->chunk_size) return SSD_ERR_BAD_SHAPE;  // the buffers hold one chunk
    const int64_t es = static_cast<int64_t>(io_size(io));
    if ((d->nheads * d->headdim * es) % 4 != 0 || (d->ngroups * d->dstate * es) % 4 != 0)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_decode_emulated_workspace_bytes(const ssd_dims* d, ssd_dtype io) {
    if (check_emul_dims(d, io) != SSD_OK || d->batch == 0) return 0;
    return emul_workspace(*d, io);
}

ssd_status ssd_decode_emulated(const ssd_dims* d, ssd_dtype io, const void* x, const float* dt,
                               const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                               const float* A, const void* B, const void* C, const float* D,
                               float* state_cache, void* x_chunks, float* dt_chunks,
                               void* b_chunks, void* c_chunks, int64_t cache_rows,
                               const int32_t* state_indices, const int32_t* positions, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
    ssd_status st = check_emul_dims(d, io);
    if (st != SSD_OK) return st;
    if (bad_clamp(dt_min, dt_max)) return SSD_ERR_BAD_ARG;
    const int64_t b = d->batch, Q = d->chunk_size, H = d->nheads, P = d->headdim, N = d->dstate,
                  G = d->ngroups;
    if (cache_rows < 0 || cache_rows >= (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
    if (cache_rows > 0 && Q * (H * P * N + H * P + 2 * G * N + H) > (int64_t(1) << 58) / cache_rows)
        return SSD_ERR_BAD_SHAPE;
    if (b == 0) return SSD_OK;
    if (!x || !dt || !A || !B || !C || !y || !state_cache || !x_chunks || !dt_chunks ||
        !b_chunks || !c_chunks || !state_indices || !positions)
        return SSD_ERR_NULL_ARG;
    if (!aligned16(state_cache)) return SSD_ERR_BAD_ARG;
    const void* word_bufs[] = {x, dt, B, C, y, x_chunks, dt_chunks, b_chunks, c_chunks};
    for (const void* p : word_bufs)
        if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return SSD_ERR_BAD_ARG;
    const size_t ws_need = emul_workspace(*d, io);
    if (!workspace || workspace_bytes < ws_need ||
        (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return SSD_ERR_WORKSPACE;
    const size_t es = io_size(io);
    // the caches (updated in place) against everything else and each other
    const Span caches[] = {span(state_cache, cache_rows * H * P * N * 4),
                           span(x_chunks, cache_rows * Q * H * P * es),
                           span(dt_chunks, cache_rows * Q * H * 4),
                           span(b_chunks, cache_rows * Q * G * N * es),
                           span(c_chunks, cache_rows * Q * G * N * es)};
    const Span others[] = {span(x, b * H * P * es), span(dt, b * H * 4), span(B, b * G * N * es),
                           span(C, b * G * N * es), span(A, H * 4),
                           span(dt_bias, dt_bias ? H * 4 : 0), span(D, D ? H * 4 : 0),
                           span(state_indices, b * 4), span(positions, b * 4),
                           span(y, b * H * P * es), span(workspace, ws_need)};
    for (size_t i = 0; i < 5; ++i) {
        for (const Span& o : others)
            if (overlap(caches[i], o)) return SSD_ERR_ALIAS;
        for (size_t j = i + 1; j < 5; ++j)
            if (overlap(caches[i], caches[j])) return SSD_ERR_ALIAS;
    }
    const Span ys = span(y, b * H * P * es);
    const Span ins[] = {span(x, b * H * P * es), span(dt, b * H * 4), span(B, b * G * N * es),
                        span(C, b * G * N * es), span(A, H * 4), span(dt_bias, dt_bias ? H * 4 : 0),
                        span(D, D ? H * 4 : 0), span(state_indices, b * 4), span(positions, b * 4),
                        span(workspace, ws_need)};
    for (const Span& o : ins)
        if (overlap(ys, o)) return SSD_ERR_ALIAS;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    // the scan of each slot's chunk in place: its chunk buffers and its
    // chunk-start state, decode output (y of the new token; the slot's state
    // replaced only when the chunk is complete).  chunk_prep reads the new
    // tokens from x, dt, B, C and appends them to the slots' chunk buffers.
    RowLayout rl;
    rl.slot = state_indices;
    rl.slots = cache_rows;
    rl.y_last = y;
    rl.pos = positions;
    rl.tok_x = x;
    rl.tok_dt = dt;
    rl.tok_B = B;
    rl.tok_C = C;
    return scan_fwd_impl(d, io, x_chunks, dt_chunks, dt_bias, dt_softplus, dt_min, dt_max, A,
                         b_chunks, c_chunks, D, state_cache, nullptr, rl, nullptr, state_cache,
                         workspace, ws_need, hs, k, [] { return hipSuccess; }, true);
}

size_t ssd_chunk_scan_varlen_workspace_bytes(const ssd_dims* d, ssd_dtype io) {
    return ssd_chunk_scan_cached_workspace_bytes(d, io);
}

ssd_status ssd_chunk_scan_fwd_varlen(const ssd_dims* d, int64_t total_tokens, ssd_dtype io,
                                     const void* x, const float* dt, const float* dt_bias,
                                     int dt_softplus, float dt_min, float dt_max, const float* A,
                                     const void* B, const void* C, const float* D,
                                     const int32_t* cu_seqlens, float* state_cache,
                                     int64_t cache_rows, const int32_t* state_indices,
                                     int init_from_cache, int strict, void* y, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    ssd_status st = check_scan_dims(d, io);
    if (st != SSD_OK) return st;
    const int64_t T = total_tokens;
    if (T < 0 || T > (int64_t(1) << 40)) return SSD_ERR_BAD_SHAPE;
    if (d->batch > 0 && !cu_seqlens) return SSD_ERR_NULL_ARG;
    // an empty packed batch reads no token
    if (d->batch > 0 && d->seqlen > 0 && T > 0 && (!x || !dt || !B || !C || !y))
        return SSD_ERR_NULL_ARG;
    // no tokens at all: as for rows of no tokens (nothing is read)
    ssd_dims dd = *d;
    if (T == 0) dd.seqlen = 0;
    return cached_prefill(&dd, io, x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D,
                          nullptr, cu_seqlens, T, state_cache, cache_rows, state_indices,
                          init_from_cache, strict, y, workspace, workspace_bytes, stream);
}

size_t ssd_chunk_scan_bwd_workspace_bytes(const ssd_dims* d, ssd_dtype io) {
    if (check_bwd_dims(d, io) != SSD_OK) return 0;
    return make_bwd_plan(*d).total;
}

ssd_status ssd_chunk_scan_bwd(const ssd_dims* d, ssd_dtype io, const void* x, const float* dt,
                              const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                              const float* A, const void* B, const void* C, const float* D,
                              const float* initial_states, const int32_t* seq_idx, const void* dy,
                              const float* d_final_states, void* dx, float* ddt, float* dA,
                              void* dB, void* dC, float* dD, float* ddt_bias,
                              float* d_initial_states, void* workspace, size_t workspace_bytes,
                              void* stream) {
    ssd_status st = check_bwd_dims(d, io);
    if (st != SSD_OK) return st;
    if (bad_clamp(dt_min, dt_max)) return SSD_ERR_BAD_ARG;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim,
                  N = d->dstate, G = d->ngroups;
    const bool work = b > 0 && L > 0;
    if (!A || !dA) return SSD_ERR_NULL_ARG;
    if (work && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return SSD_ERR_NULL_ARG;
    const BwdPlan plan = make_bwd_plan(*d);
    if (plan.total > 0 &&
        (!workspace || workspace_bytes < plan.total ||
         (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0))
        return SSD_ERR_WORKSPACE;
    const void* vec_bufs[] = {x, B, C, dy, dx, dB, dC, initial_states, d_final_states,
                              d_initial_states};
    for (const void* p : vec_bufs)
        if (p && !aligned16(p)) return SSD_ERR_BAD_ARG;
    const size_t es = io_size(io);
    const int64_t sbytes = b * H * P * N * 4;
    const Span ins[] = {
        span(x, b * L * H * P * es), span(dt, b * L * H * 4), span(B, b * L * G * N * es),
        span(C, b * L * G * N * es), span(A, H * 4), span(dt_bias, dt_bias ? H * 4 : 0),
        span(D, D ? H * 4 : 0), span(seq_idx, seq_idx ? b * L * 4 : 0),
        span(initial_states, initial_states ? sbytes : 0), span(dy, b * L * H * P * es),
        span(d_final_states, d_final_states ? sbytes : 0),
    };
    const Span outs[] = {
        span(dx, b * L * H * P * es), span(ddt, b * L * H * 4), span(dA, H * 4),
        span(dB, b * L * G * N * es), span(dC, b * L * G * N * es), span(dD, dD ? H * 4 : 0),
        span(ddt_bias, ddt_bias ? H * 4 : 0), span(d_initial_states, d_initial_states ? sbytes : 0),
        span(workspace, plan.total),
    };
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span& s : ins)
            if (overlap(outs[i], s)) return SSD_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j])) return SSD_ERR_ALIAS;
    }

    hipStream_t hs = static_cast<hipStream_t>(stream);
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    ssd::BwdArgs ba{};
    ba.x = x;
    ba.B = B;
    ba.C = C;
    ba.dy = dy;
    ba.dt_raw = dt;
    ba.dt_bias = dt_bias;
    ba.A = A;
    ba.D = D;
    ba.softplus = dt_softplus ? 1 : 0;
    ba.dt_min = dt_min;
    ba.dt_max = dt_max;
    ba.seq_idx = seq_idx;
    ba.h_init = initial_states;
    ba.dh_final = d_final_states;
    ba.dx = dx;
    ba.ddt = ddt;
    ba.dA = dA;
    ba.dB = dB;
    ba.dC = dC;
    ba.dD = dD;
    ba.ddt_bias = ddt_bias;
    ba.dh_init = d_initial_states;
    ba.L = L;
    ba.batch = static_cast<int>(b);
    ba.H = static_cast<int>(H);
    ba.G = static_cast<int>(G);
    ba.nc = static_cast<int>(plan.nc);
    ba.nseg = static_cast<int>(plan.nseg);
    ba.cps = static_cast<int>(plan.cps);
    ba.N = static_cast<int>(N);
    if (!work) {
        if (timed_launch(k, hs, [&] { return ssd::launch_bwd_empty(ba, b * H * P * N, hs); }) !=
            hipSuccess)
            return SSD_ERR_HIP;
        return SSD_OK;
    }
    char* wsb = static_cast<char*>(workspace);
    float* meta = reinterpret_cast<float*>(wsb + plan.off_meta);
    ba.cs = meta;
    ba.states = reinterpret_cast<uint16_t*>(wsb + plan.off_states);
    ba.gstates = reinterpret_cast<uint16_t*>(wsb + plan.off_gstates);
    ba.partials = reinterpret_cast<float*>(wsb + plan.off_partials);
    ba.seg_end = plan.nseg > 1 ? reinterpret_cast<float*>(wsb + plan.off_seg) : nullptr;
    ba.seg_mult = plan.nseg > 1 ? reinterpret_cast<float*>(wsb + plan.off_mult) : nullptr;

    // the per-token metadata of the forward pass (chunk_prep_kernel, no tiles)
    ssd::ScanArgs sa{};
    sa.B = B;
    sa.C = C;
    sa.dt_raw = dt;
    sa.dt_bias = dt_bias;
    sa.A = A;
    sa.softplus = ba.softplus;
    sa.dt_min = dt_min;
    sa.dt_max = dt_max;
    sa.seq_idx = seq_idx;
    sa.cs = meta;
    sa.dtv = meta + kBwdChunk;
    sa.wgt = meta + 2 * kBwdChunk;
    sa.L = L;
    sa.H = ba.H;
    sa.G = ba.G;
    sa.nc = ba.nc;
    sa.nseg = 1;
    sa.cps = ba.nc;
    if (timed_launch(k, hs, [&] { return ssd::launch_chunk_meta_bf16_64_128_128(sa, b * plan.nc * G, hs); }) !=
        hipSuccess)
        return SSD_ERR_HIP;
    if (plan.nseg > 1) {
        // segment ends from zero, then each segment's incoming state (one pass
        // per direction: from h_init forwards, from d(final states) backwards)
        if (timed_launch(k, hs, [&] { return ssd::launch_bwd_seg_ends(ba, hs); }) != hipSuccess)
            return SSD_ERR_HIP;
        for (int dir = 0; dir < 2; ++dir) {
            ssd::PassArgs pa;
            pa.seg_state = ba.seg_end + dir * b * H * plan.nseg * P * N;
            pa.seg_mult = ba.seg_mult + dir * b * H * plan.nseg;
            pa.init = dir == 0 ? initial_states : d_final_states;
            pa.PN = P * N;
            pa.nseg = static_cast<int>(plan.nseg);
            if (timed_launch(k, hs, [&] { return ssd::launch_state_pass(pa, b * H, hs); }) !=
                hipSuccess)
                return SSD_ERR_HIP;
        }
    }
    if (timed_launch(k, hs, [&] { return ssd::launch_bwd_states(ba, hs); }) != hipSuccess)
        return SSD_ERR_HIP;
    if (timed_launch(k, hs, [&] { return ssd::launch_bwd_chunk(ba, hs); }) != hipSuccess)
        return SSD_ERR_HIP;
    if (timed_launch(k, hs, [&] { return ssd::launch_bwd_reduce(ba, hs); }) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status ssd_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t nx, int64_t nb,
                          ssd_dtype io, const void* xbc, const float* weight, int64_t width,
                          const float* bias, const void* conv_state_in, const int32_t* seq_idx,
                          void* x_out, void* b_out, void* c_out, void* conv_state_out,
                          void* stream) {
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_BAD_DTYPE;
    if (batch < 0 || seqlen < 0 || nx < 0 || nb < 0 || dim != nx + 2 * nb || dim < 8)
        return SSD_ERR_BAD_SHAPE;
    if (width != 4 || dim % 8 != 0 || nx % 8 != 0 || nb % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (batch > 65535 || seqlen > int64_t(65535) * 32 || dim > (int64_t(1) << 30)) return SSD_ERR_BAD_SHAPE;
    const bool work = batch > 0 && seqlen > 0;
    if (!weight) return SSD_ERR_NULL_ARG;
    if (work && (!xbc || !x_out || (nb > 0 && (!b_out || !c_out)))) return SSD_ERR_NULL_ARG;
    const void* vec_bufs[] = {xbc, weight, x_out, b_out, c_out};
    for (const void* p : vec_bufs)
        if (p && !aligned16(p)) return SSD_ERR_BAD_ARG;
    const size_t es = io_size(io);
    const int64_t rows = batch * seqlen;
    const Span ins[] = {span(xbc, rows * dim * es), span(weight, dim * 16), span(bias, bias ? dim * 4 : 0),
                        span(seq_idx, seq_idx ? rows * 4 : 0)};
    const Span sin = span(conv_state_in, conv_state_in ? batch * dim * 3 * es : 0);
    const Span outs[] = {span(x_out, rows * nx * es), span(b_out, rows * nb * es), span(c_out, rows * nb * es),
                         span(conv_state_out, conv_state_out ? batch * dim * 3 * es : 0)};
    for (size_t i = 0; i < 4; ++i) {
        for (const Span& s : ins)
            if (overlap(outs[i], s)) return SSD_ERR_ALIAS;
        // the state may be updated in place (exactly the same buffer), the
        // outputs may not overlap the old state otherwise
        if (overlap(outs[i], sin) && !(i == 3 && conv_state_out == conv_state_in)) return SSD_ERR_ALIAS;
        for (size_t j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return SSD_ERR_ALIAS;
    }
    if (!work) return SSD_OK;
    ssd::ConvArgs ca{};
    ca.xbc = xbc;
    ca.weight = weight;
    ca.bias = bias;
    ca.state_in = conv_state_in;
    ca.seq_idx = seq_idx;
    ca.x_out = x_out;
    ca.b_out = b_out;
    ca.c_out = c_out;
    ca.state_out = conv_state_out;
    ca.L = seqlen;
    ca.batch = static_cast<int>(batch);
    ca.dim = static_cast<int>(dim);
    ca.nx = static_cast<int>(nx);
    ca.nb = static_cast<int>(nb);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    if (timed_launch(k, hs, [&] { return ssd::launch_conv1d_fwd(io, ca, hs); }) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

}  // extern "C"

namespace {

// One decode token of the conv with the conv states taken from a cache of
// cache_rows rows (state_idx[r] picks row r's; null: row r, cache_rows =
// batch).
ssd_status conv1d_update_impl(int64_t batch, int64_t cache_rows, int64_t dim, int64_t nx,
                              int64_t nb, ssd_dtype io, const void* xbc, const float* weight,
                              int64_t width, const float* bias, void* conv_state,
                              const int32_t* state_idx, void* x_out, void* b_out, void* c_out,
                              void* stream) {
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_BAD_DTYPE;
    if (batch < 0 || nx < 0 || nb < 0 || dim != nx + 2 * nb || dim < 8) return SSD_ERR_BAD_SHAPE;
    if (width != 4 || dim % 8 != 0 || nx % 8 != 0 || nb % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (batch > 65535 || dim > (int64_t(1) << 30)) return SSD_ERR_BAD_SHAPE;
    if (cache_rows < 0 || cache_rows > (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
    if (cache_rows > 0 && dim > (int64_t(1) << 52) / cache_rows) return SSD_ERR_BAD_SHAPE;
    if (!weight) return SSD_ERR_NULL_ARG;
    if (batch > 0 && (!xbc || !conv_state || !x_out || (nb > 0 && (!b_out || !c_out))))
        return SSD_ERR_NULL_ARG;
    const void* vec_bufs[] = {xbc, weight, x_out, b_out, c_out};
    for (const void* p : vec_bufs)
        if (p && !aligned16(p)) return SSD_ERR_BAD_ARG;
    const size_t es = io_size(io);
    const Span ins[] = {span(xbc, batch * dim * es), span(weight, dim * 16), span(bias, bias ? dim * 4 : 0),
                        span(state_idx, state_idx ? batch * 4 : 0)};
    const Span outs[] = {span(x_out, batch * nx * es), span(b_out, batch * nb * es), span(c_out, batch * nb * es),
                         span(conv_state, cache_rows * dim * 3 * es)};
    for (size_t i = 0; i < 4; ++i) {
        for (const Span& s : ins)
            if (overlap(outs[i], s)) return SSD_ERR_ALIAS;
        for (size_t j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return SSD_ERR_ALIAS;
    }
    if (batch == 0) return SSD_OK;
    ssd::ConvArgs ca{};
    ca.xbc = xbc;
    ca.weight = weight;
    ca.bias = bias;
    ca.x_out = x_out;
    ca.b_out = b_out;
    ca.c_out = c_out;
    ca.state_out = conv_state;
    ca.state_idx = state_idx;
    ca.cache_rows = cache_rows;
    ca.L = 1;
    ca.batch = static_cast<int>(batch);
    ca.dim = static_cast<int>(dim);
    ca.nx = static_cast<int>(nx);
    ca.nb = static_cast<int>(nb);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    if (timed_launch(k, hs, [&] { return ssd::launch_conv1d_update(io, ca, hs); }) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status ssd_conv1d_update(int64_t batch, int64_t dim, int64_t nx, int64_t nb, ssd_dtype io,
                             const void* xbc, const float* weight, int64_t width, const float* bias,
                             void* conv_state, void* x_out, void* b_out, void* c_out, void* stream) {
    return conv1d_update_impl(batch, batch, dim, nx, nb, io, xbc, weight, width, bias, conv_state,
                              nullptr, x_out, b_out, c_out, stream);
}

ssd_status ssd_conv1d_update_cached(int64_t batch, int64_t cache_rows, int64_t dim, int64_t nx,
                                    int64_t nb, ssd_dtype io, const void* xbc, const float* weight,
                                    int64_t width, const float* bias, void* conv_state_cache,
                                    const int32_t* state_indices, void* x_out, void* b_out,
                                    void* c_out, void* stream) {
    if (batch > 0 && !state_indices) return SSD_ERR_NULL_ARG;
    return conv1d_update_impl(batch, cache_rows, dim, nx, nb, io, xbc, weight, width, bias,
                              conv_state_cache, state_indices, x_out, b_out, c_out, stream);
}

ssd_status ssd_gated_rmsnorm(int64_t rows, int64_t dim, int64_t group, ssd_dtype io, const void* y,
                             const void* z, const float* weight, float eps, void* out, void* stream) {
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_BAD_DTYPE;
    if (rows < 0 || dim < 1 || group < 1 || dim % group != 0) return SSD_ERR_BAD_SHAPE;
    if (group % 8 != 0 || group > 4096) return SSD_ERR_UNSUPPORTED;
    if (rows > (int64_t(1) << 31) / (dim / group + 1) || dim > (int64_t(1) << 30)) return SSD_ERR_BAD_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return SSD_ERR_BAD_ARG;
    if (!weight) return SSD_ERR_NULL_ARG;
    if (rows > 0 && (!y || !z || !out)) return SSD_ERR_NULL_ARG;
    const void* vec_bufs[] = {y, z, weight, out};
    for (const void* p : vec_bufs)
        if (p && !aligned16(p)) return SSD_ERR_BAD_ARG;
    const size_t es = io_size(io);
    const Span os = span(out, rows * dim * es);
    if (overlap(os, span(y, rows * dim * es)) || overlap(os, span(z, rows * dim * es)) ||
        overlap(os, span(weight, dim * 4)))
        return SSD_ERR_ALIAS;
    if (rows == 0) return SSD_OK;
    ssd::NormArgs na{};
    na.y = y;
    na.z = z;
    na.weight = weight;
    na.out = out;
    na.rows = rows;
    na.dim = static_cast<int>(dim);
    na.group = static_cast<int>(group);
    na.eps = eps;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int k = 0;
    if (g_hooks.launched) *g_hooks.launched = 0;
    if (timed_launch(k, hs, [&] { return ssd::launch_gated_rmsnorm(io, na, hs); }) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

}  // extern "C"

namespace {

// The decode step with the state rows taken from a cache of cache_rows rows
// (state_idx[r] picks row r's; null: row r uses state row r, cache_rows =
// batch).
ssd_status state_update_impl(int64_t batch, int64_t cache_rows, int64_t nheads, int64_t headdim,
                             int64_t dstate, int64_t ngroups, ssd_dtype io, float* state,
                             const int32_t* state_idx, const void* x, const float* dt,
                             const float* dt_bias, int dt_softplus, float dt_min, float dt_max,
                             const float* A, const void* B, const void* C, const float* D, void* y,
                             void* stream) {
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_BAD_DTYPE;
    if (batch < 0 || cache_rows < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1)
        return SSD_ERR_BAD_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_BAD_SHAPE;
    // grid: one block per (row, head) (and, for few of them, per 8 or more of
    // its state rows), below 2^31; the cache's byte offsets below 2^62
    const int64_t k31 = int64_t(1) << 31;
    if (headdim > (int64_t(1) << 20) || nheads >= k31 || batch >= k31 || cache_rows >= k31)
        return SSD_ERR_BAD_SHAPE;
    if (batch * nheads >= k31 || batch * nheads * ((headdim + 7) / 8) >= k31)
        return SSD_ERR_BAD_SHAPE;
    if (cache_rows > 0 && nheads * headdim > (int64_t(1) << 52) / cache_rows)
        return SSD_ERR_BAD_SHAPE;
    if (dstate != 16 && dstate != 32 && dstate != 64 && dstate != 128 && dstate != 256)
        return SSD_ERR_UNSUPPORTED;
    if (bad_clamp(dt_min, dt_max)) return SSD_ERR_BAD_ARG;
    if (g_hooks.launched) *g_hooks.launched = 0;
    if (batch == 0) return SSD_OK;
    if (!state || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL_ARG;
    if (!aligned16(state)) return SSD_ERR_BAD_ARG;
    const size_t es = io_size(io);
    const int64_t b = batch, H = nheads, P = headdim, N = dstate, G = ngroups;
    const Span ss = span(state, cache_rows * H * P * N * 4);
    const Span ys = span(y, b * H * P * es);
    const Span ins[] = {span(x, b * H * P * es), span(dt, b * H * 4), span(B, b * G * N * es),
                        span(C, b * G * N * es), span(A, H * 4),
                        span(dt_bias, dt_bias ? H * 4 : 0), span(D, D ? H * 4 : 0),
                        span(state_idx, state_idx ? b * 4 : 0)};
    for (const Span& sp : ins)
        if (overlap(ss, sp) || overlap(ys, sp)) return SSD_ERR_ALIAS;
    if (overlap(ss, ys)) return SSD_ERR_ALIAS;

    ssd::StepArgs a;
    a.state = state;
    a.state_idx = state_idx;
    a.cache_rows = cache_rows;
    a.x = x;
    a.dt = dt;
    a.dt_bias = dt_bias;
    a.softplus = dt_softplus ? 1 : 0;
    a.dt_min = dt_min;
    a.dt_max = dt_max;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.y = y;
    a.H = static_cast<int>(H);
    a.P = static_cast<int>(P);
    a.G = static_cast<int>(G);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int k = 0;
    if (timed_launch(k, hs, [&] { return ssd::launch_state_update(io, N, a, b * H, hs); }) !=
        hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status ssd_state_update(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                            int64_t ngroups, ssd_dtype io, float* state, const void* x,
                            const float* dt, const float* dt_bias, int dt_softplus,
                            float dt_min, float dt_max, const float* A, const void* B,
                            const void* C, const float* D, void* y, void* stream) {
    return state_update_impl(batch, batch, nheads, headdim, dstate, ngroups, io, state, nullptr, x,
                             dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C, D, y, stream);
}

ssd_status ssd_state_update_cached(int64_t batch, int64_t cache_rows, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype io,
                                   float* state_cache, const int32_t* state_indices,
                                   const void* x, const float* dt, const float* dt_bias,
                                   int dt_softplus, float dt_min, float dt_max, const float* A,
                                   const void* B, const void* C, const float* D, void* y,
                                   void* stream) {
    if (batch > 0 && !state_indices) return SSD_ERR_NULL_ARG;
    return state_update_impl(batch, cache_rows, nheads, headdim, dstate, ngroups, io, state_cache,
                             state_indices, x, dt, dt_bias, dt_softplus, dt_min, dt_max, A, B, C,
                             D, y, stream);
}

}  // extern "C"
