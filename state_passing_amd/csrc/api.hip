// api.hip -- the C ABI declared in include/linrec.h: argument checking,
// the context (auxiliary stream + events), per-piece calls and the
// sequence-accumulation drivers that overlap the serial state transitions
// with the intra-chunk work of the neighbouring piece.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "launch.hpp"
#include "linrec.h"

using linrec::BwdIntraLaunch;
using linrec::DaFinishLaunch;
using linrec::FwdIntraLaunch;
using linrec::ScanLaunch;
using linrec::TensorArg;

struct TimedLaunch {
    int kind;
    hipEvent_t begin, end;
};

struct linrec_ctx {
    int device;
    void* scratch;          // this device's address of the no-allocation scratch
    hipError_t scratch_err; // result of looking that address up
    hipStream_t aux;        // state transitions
    hipEvent_t ev_start;    // inputs ready on the caller's stream
    hipEvent_t ev_scan;     // a piece's scan finished (aux)
    hipEvent_t ev_slot[2];  // a workspace slot's last reader finished (aux)
    // opt-in per-kernel timing (linrec_ctx_set_timing)
    int timing;
    std::vector<TimedLaunch> pending;
    std::vector<hipEvent_t> pool;
    double ms[LINREC_KERNEL_KINDS];
    int64_t count[LINREC_KERNEL_KINDS];
};

// Scratch of linrec_bwd_noalloc: the gradient records of one piece.  Each
// GPU the library runs on holds its own copy for the life of the process.
// In host code this name is only a stand-in for the symbol: kernels and
// runtime calls get the device address that linrec_ctx_create looks up with
// hipGetSymbolAddress (ctx->scratch).
static __device__ __align__(256) unsigned char scratch[LINREC_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kChunk = 64;
// Chunks per segment: the segment kernels rebuild every per-chunk state of a
// segment in registers; only the state at each segment boundary is stored.
constexpr int kSegChunks = 4;

int64_t chunks_of(int64_t tokens) { return (tokens + kChunk - 1) / kChunk; }
int64_t nseg_of(int64_t tokens) { return (chunks_of(tokens) + kSegChunks - 1) / kSegChunks; }

linrec_status hip_fail(hipError_t e, linrec_status code)
{
    g_last_hip_error = (int)e;
    return code;
}

int elem_size(int dtype) { return dtype == LINREC_BF16 ? 2 : 4; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

linrec_status check_desc(const linrec_desc* d)
{
    if (!d)
        return LINREC_E_NULL;
    if (d->dtype != LINREC_BF16 && d->dtype != LINREC_F32)
        return LINREC_E_DTYPE;
    // B: the sequence backward's launches carry another piece's segment sums
    // as a second set of grid rows z, so 2 B must fit the grid's 65535
    if (d->chunk != kChunk || d->B < 1 || d->H < 1 || d->B > 32767 || d->H > 65535 || d->T < 0 ||
        d->T > LINREC_MAX_T)
        return LINREC_E_SHAPE;
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128))
        return LINREC_E_SHAPE;
    if (d->out_dtype != LINREC_BF16 && d->out_dtype != LINREC_F32)
        return LINREC_E_DTYPE;
    if (d->dtype == LINREC_F32 && (d->dk != 64 || d->dv != 64 || d->out_dtype != LINREC_F32))
        return LINREC_E_DTYPE;
    if (d->decay != LINREC_DECAY_NONE && d->decay != LINREC_DECAY_HEAD &&
        d->decay != LINREC_DECAY_TOKEN)
        return LINREC_E_LAYOUT;
    return LINREC_OK;
}

// An activation view: 16-byte aligned rows, non-negative strides, rows at
// least `width` elements apart.
linrec_status check_act(const linrec_tensor& t, int width, int esz)
{
    if (!t.ptr)
        return LINREC_E_NULL;
    if (t.sb < 0 || t.sh < 0 || t.st < width)
        return LINREC_E_LAYOUT;
    if (!aligned(t.ptr, 16) || (t.st * esz) % 16 || (t.sh * esz) % 16 || (t.sb * esz) % 16)
        return LINREC_E_ALIGN;
    return LINREC_OK;
}

linrec_status check_decay(const linrec_desc* d, const linrec_tensor& a)
{
    if (d->decay == LINREC_DECAY_NONE)
        return LINREC_OK;
    if (!a.ptr)
        return LINREC_E_NULL;
    if (!aligned(a.ptr, 4))
        return LINREC_E_ALIGN;
    if (a.sh < 0 || (d->decay == LINREC_DECAY_TOKEN && (a.sb < 0 || a.st < 0)))
        return LINREC_E_LAYOUT;
    return LINREC_OK;
}

linrec_status check_state_ptr(const void* p, bool required)
{
    if (!p)
        return required ? LINREC_E_NULL : LINREC_OK;
    return aligned(p, 4) ? LINREC_OK : LINREC_E_ALIGN;
}

linrec_status check_buffer(const void* p)
{
    if (!p)
        return LINREC_E_WORKSPACE;
    return aligned(p, 16) ? LINREC_OK : LINREC_E_WORKSPACE;
}

linrec_status check_ctx(linrec_ctx* ctx)
{
    if (!ctx)
        return LINREC_E_NULL;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return hip_fail(e, LINREC_E_DEVICE);
    if (cur != ctx->device)
        return hip_fail(hipErrorInvalidDevice, LINREC_E_DEVICE);
    return LINREC_OK;
}

linrec_status check_pieces(const linrec_desc* d, int32_t npieces, const int32_t* lengths)
{
    if (npieces < 1)
        return LINREC_E_SHAPE;
    if (!lengths)
        return LINREC_E_NULL;
    int64_t sum = 0;
    for (int32_t i = 0; i < npieces; ++i) {
        if (lengths[i] < 1)
            return LINREC_E_SHAPE;
        sum += lengths[i];
    }
    return sum == d->T ? LINREC_OK : LINREC_E_SHAPE;
}

// Stored per-segment records (state or gradient, then the segment's
// log-decay) are fp32 whatever the activation dtype.
size_t per_seg_bytes(const linrec_desc* d)
{
    return (size_t)linrec::seg_record_floats(d->dk, d->dv) * sizeof(float);
}

int64_t total_nseg(int32_t npieces, const int32_t* lengths)
{
    int64_t n = 0;
    for (int32_t i = 0; i < npieces; ++i)
        n += nseg_of(lengths[i]);
    return n;
}

int64_t max_nseg(int32_t npieces, const int32_t* lengths)
{
    int64_t n = 0;
    for (int32_t i = 0; i < npieces; ++i)
        n = nseg_of(lengths[i]) > n ? nseg_of(lengths[i]) : n;
    return n;
}

TensorArg targ(const linrec_tensor& t) { return TensorArg{t.ptr, t.sb, t.sh, t.st}; }

// View of a tensor advanced by `tok` tokens.
TensorArg advance(const linrec_tensor& t, int64_t tok, int esz)
{
    return TensorArg{(const char*)t.ptr + tok * t.st * esz, t.sb, t.sh, t.st};
}

TensorArg advance_decay(const linrec_desc* d, const linrec_tensor& a, int64_t tok)
{
    if (d->decay != LINREC_DECAY_TOKEN)
        return targ(a);
    return TensorArg{(const float*)a.ptr + tok * a.st, a.sb, a.sh, a.st};
}

// All checks of a forward call except the piece list.
linrec_status check_fwd_args(const linrec_desc* d, const linrec_tensor& q,
                             const linrec_tensor& k, const linrec_tensor& v,
                             const linrec_tensor& decay, const float* S_in,
                             const linrec_tensor& o, const float* S_out, const void* states)
{
    linrec_status s;
    if ((s = check_desc(d)) != LINREC_OK)
        return s;
    if (d->T == 0)   // nothing is read or written but the carried state
        return (s = check_state_ptr(S_in, false)) != LINREC_OK ? s : check_state_ptr(S_out, true);
    const int esz = elem_size(d->dtype), osz = elem_size(d->out_dtype);
    if ((s = check_act(q, d->dk, esz)) != LINREC_OK || (s = check_act(k, d->dk, esz)) != LINREC_OK ||
        (s = check_act(v, d->dv, esz)) != LINREC_OK || (s = check_act(o, d->dv, osz)) != LINREC_OK)
        return s;
    if ((s = check_decay(d, decay)) != LINREC_OK)
        return s;
    if ((s = check_state_ptr(S_in, false)) != LINREC_OK ||
        (s = check_state_ptr(S_out, true)) != LINREC_OK)
        return s;
    return check_buffer(states);
}

linrec_status check_bwd_args(const linrec_desc* d, const linrec_tensor& q,
                             const linrec_tensor& k, const linrec_tensor& v,
                             const linrec_tensor& decay, const void* states,
                             const linrec_tensor& dO, const float* dS_out,
                             const linrec_tensor& dq, const linrec_tensor& dk,
                             const linrec_tensor& dv, const float* dS_in, const void* workspace)
{
    linrec_status s;
    if ((s = check_desc(d)) != LINREC_OK)
        return s;
    if (d->T == 0)   // nothing is read or written but the carried gradient
        return (s = check_state_ptr(dS_out, false)) != LINREC_OK ? s : check_state_ptr(dS_in, true);
    const int esz = elem_size(d->dtype), osz = elem_size(d->out_dtype);
    if ((s = check_act(q, d->dk, esz)) != LINREC_OK || (s = check_act(k, d->dk, esz)) != LINREC_OK ||
        (s = check_act(v, d->dv, esz)) != LINREC_OK || (s = check_act(dO, d->dv, esz)) != LINREC_OK ||
        (s = check_act(dq, d->dk, osz)) != LINREC_OK || (s = check_act(dk, d->dk, osz)) != LINREC_OK ||
        (s = check_act(dv, d->dv, osz)) != LINREC_OK)
        return s;
    if ((s = check_decay(d, decay)) != LINREC_OK)
        return s;
    if ((s = check_state_ptr(dS_out, false)) != LINREC_OK ||
        (s = check_state_ptr(dS_in, true)) != LINREC_OK)
        return s;
    if ((s = check_buffer(states)) != LINREC_OK)
        return s;
    return check_buffer(workspace);
}

// A piece of zero tokens: the carry passes through unchanged (zeros for a
// NULL input), one copy of B*H*n floats on `stream`.
linrec_status pass_carry(const linrec_desc* d, const float* in, float* out, int64_t n,
                         hipStream_t stream)
{
    if (in == out)
        return LINREC_OK;
    const hipError_t e = linrec::launch_carry_copy(in, out, (int64_t)d->B * d->H * n, stream);
    return e == hipSuccess ? LINREC_OK : hip_fail(e, LINREC_E_LAUNCH);
}

// Launch descriptions of one piece [tok0, tok0 + len) of the sequence.
ScanLaunch fwd_scan_of(const linrec_desc* d, const linrec_tensor& k, const linrec_tensor& v,
                       const linrec_tensor& decay, int64_t tok0, int32_t len,
                       const float* carry_in, float* carry_out, void* states,
                       int64_t seg0, int64_t nseg_total)
{
    const int esz = elem_size(d->dtype);
    ScanLaunch s{};
    s.dtype = d->dtype; s.dk = d->dk; s.dv = d->dv; s.B = d->B; s.H = d->H; s.N = (len + kChunk - 1) / kChunk; s.tail = len - (s.N - 1) * kChunk;
    s.m = kSegChunks;
    s.reverse = false;
    s.x = advance(k, tok0, esz);
    s.y = advance(v, tok0, esz);
    s.decay = advance_decay(d, decay, tok0);
    s.decay_kind = d->decay;
    s.carry_in = carry_in;
    s.carry_out = carry_out;
    s.store = (char*)states + seg0 * per_seg_bytes(d);
    s.store_nseg = nseg_total;
    return s;
}

FwdIntraLaunch fwd_intra_of(const linrec_desc* d, const linrec_tensor& q, const linrec_tensor& k,
                            const linrec_tensor& v, const linrec_tensor& decay,
                            const linrec_tensor& o, int64_t tok0, int32_t len,
                            const void* states, int64_t seg0, int64_t nseg_total)
{
    const int esz = elem_size(d->dtype), osz = elem_size(d->out_dtype);
    FwdIntraLaunch s{};
    s.dtype = d->dtype; s.out_dtype = d->out_dtype;
    s.dk = d->dk; s.dv = d->dv; s.B = d->B; s.H = d->H; s.N = (len + kChunk - 1) / kChunk; s.tail = len - (s.N - 1) * kChunk;
    s.m = kSegChunks;
    s.q = advance(q, tok0, esz);
    s.k = advance(k, tok0, esz);
    s.v = advance(v, tok0, esz);
    s.o = advance(o, tok0, osz);
    s.decay = advance_decay(d, decay, tok0);
    s.decay_kind = d->decay;
    s.states = (const char*)states + seg0 * per_seg_bytes(d);
    s.st_nseg = nseg_total;
    return s;
}

ScanLaunch bwd_scan_of(const linrec_desc* d, const linrec_tensor& q, const linrec_tensor& dO,
                       const linrec_tensor& decay, int64_t tok0, int32_t len,
                       const float* carry_in, float* carry_out, void* ghat)
{
    const int esz = elem_size(d->dtype);
    ScanLaunch s{};
    s.dtype = d->dtype; s.dk = d->dk; s.dv = d->dv; s.B = d->B; s.H = d->H; s.N = (len + kChunk - 1) / kChunk; s.tail = len - (s.N - 1) * kChunk;
    s.m = kSegChunks;
    s.reverse = true;
    s.x = advance(q, tok0, esz);
    s.y = advance(dO, tok0, esz);
    s.decay = advance_decay(d, decay, tok0);
    s.decay_kind = d->decay;
    s.carry_in = carry_in;
    s.carry_out = carry_out;
    s.store = ghat;
    s.store_nseg = nseg_of(len);
    return s;
}

BwdIntraLaunch bwd_intra_of(const linrec_desc* d, const linrec_tensor& q, const linrec_tensor& k,
                            const linrec_tensor& v, const linrec_tensor& decay,
                            const linrec_tensor& dO, const linrec_tensor& dq,
                            const linrec_tensor& dk, const linrec_tensor& dv, int64_t tok0,
                            int32_t len, const void* states, int64_t seg0,
                            int64_t nseg_total, const void* ghat)
{
    const int esz = elem_size(d->dtype), osz = elem_size(d->out_dtype);
    BwdIntraLaunch s{};
    s.dtype = d->dtype; s.out_dtype = d->out_dtype;
    s.dk = d->dk; s.dv = d->dv; s.B = d->B; s.H = d->H; s.N = (len + kChunk - 1) / kChunk; s.tail = len - (s.N - 1) * kChunk;
    s.m = kSegChunks;
    s.q = advance(q, tok0, esz);
    s.k = advance(k, tok0, esz);
    s.v = advance(v, tok0, esz);
    s.dO = advance(dO, tok0, esz);
    s.dq = advance(dq, tok0, osz);
    s.dk_ = advance(dk, tok0, osz);
    s.dv_ = advance(dv, tok0, osz);
    s.decay = advance_decay(d, decay, tok0);
    s.decay_kind = d->decay;
    s.states = (const char*)states + seg0 * per_seg_bytes(d);
    s.st_nseg = nseg_total;
    s.ghat = ghat;
    s.g_nseg = nseg_of(len);
    return s;
}

// The segment sums of a scan, as extra work of a segment-kernel launch.
linrec::SumArg sum_arg_of(const ScanLaunch& sc)
{
    linrec::SumArg a{};
    a.x = sc.x;
    a.y = sc.y;
    a.decay = sc.decay;
    a.decay_kind = sc.decay_kind;
    a.store = sc.store;
    a.store_nseg = sc.store_nseg;
    a.N = sc.N;
    a.m = sc.m;
    a.tail = sc.tail;
    a.nseg = (sc.N + sc.m - 1) / sc.m;
    return a;
}

hipError_t pool_event(linrec_ctx* ctx, hipEvent_t* ev)
{
    if (!ctx->pool.empty()) {
        *ev = ctx->pool.back();
        ctx->pool.pop_back();
        return hipSuccess;
    }
    // no system-scope release at the event: it would write back L2 after
    // the bracketed kernel and bill that to the kernel's duration
    return hipEventCreateWithFlags(ev, hipEventDisableSystemFence);
}

// Launch `fn` on `stream`; with timing on, the kernels it launches carry a pair
// of events as their own start and end stamps (launch_kernel).
template <typename F>
hipError_t timed_launch(linrec_ctx* ctx, int kind, hipStream_t stream, F fn)
{
    if (!ctx->timing)
        return fn();
    TimedLaunch t{kind, nullptr, nullptr};
    hipError_t e = pool_event(ctx, &t.begin);
    if (e == hipSuccess)
        e = pool_event(ctx, &t.end);
    if (e == hipSuccess) {
        // the events become the launched kernels' own start and end stamps
        linrec::launch_stamps() = linrec::LaunchStamps{t.begin, t.end};
        e = fn();
        linrec::launch_stamps() = linrec::LaunchStamps{};
    }
    if (e != hipSuccess) {
        if (t.begin)
            ctx->pool.push_back(t.begin);
        if (t.end)
            ctx->pool.push_back(t.end);
        return e;
    }
    ctx->pending.push_back(t);
    return hipSuccess;
}

#define LAUNCH(call)                                              \
    do {                                                          \
        hipError_t e_ = (call);                                   \
        if (e_ != hipSuccess)                                     \
            return hip_fail(e_, LINREC_E_LAUNCH);                 \
    } while (0)

// The state transition of a piece: segment sum, then fold.
#define LAUNCH_SCAN(ctx, desc, stream)                                                       \
    do {                                                                                    \
        LAUNCH(timed_launch((ctx), (desc).reverse ? LINREC_KERNEL_BWD_SUM : LINREC_KERNEL_FWD_SUM, \
                            (stream), [&] { return linrec::launch_seg_sum((desc), (stream)); })); \
        LAUNCH(timed_launch((ctx), (desc).reverse ? LINREC_KERNEL_BWD_FOLD : LINREC_KERNEL_FWD_FOLD, \
                            (stream), [&] { return linrec::launch_seg_fold((desc), (stream)); })); \
    } while (0)
#define LAUNCH_FWD_INTRA(ctx, desc, stream)                                                \
    LAUNCH(timed_launch((ctx), LINREC_KERNEL_FWD_SEG, (stream),                            \
                        [&] { return linrec::launch_fwd_intra((desc), (stream)); }))
#define LAUNCH_BWD_INTRA(ctx, desc, stream)                                                \
    LAUNCH(timed_launch((ctx), LINREC_KERNEL_BWD_SEG, (stream),                            \
                        [&] { return linrec::launch_bwd_intra((desc), (stream)); }))

#define HIPCHECK(call)                                            \
    do {                                                          \
        hipError_t e_ = (call);                                   \
        if (e_ != hipSuccess)                                     \
            return hip_fail(e_, LINREC_E_DEVICE);                 \
    } while (0)

}  // namespace

extern "C" {

linrec_status linrec_ctx_create(linrec_ctx** out, int device)
{
    if (!out)
        return LINREC_E_NULL;
    int prev = -1;
    HIPCHECK(hipGetDevice(&prev));
    HIPCHECK(hipSetDevice(device));
    linrec_ctx* c = new (std::nothrow) linrec_ctx();
    if (!c) {
        (void)hipSetDevice(prev);
        return LINREC_E_DEVICE;
    }
    c->device = device;
    hipError_t e = hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&c->ev_start, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&c->ev_scan, hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i)
        e = hipEventCreateWithFlags(&c->ev_slot[i], hipEventDisableTiming);
    // the no-allocation scratch's address on this device (the device is
    // current); a failure here only disables linrec_bwd_noalloc
    if (e == hipSuccess) {
        c->scratch_err = hipGetSymbolAddress(&c->scratch, HIP_SYMBOL(scratch));
        if (c->scratch_err != hipSuccess)
            c->scratch = nullptr;
    }
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        linrec_ctx_destroy(c);
        return hip_fail(e, LINREC_E_DEVICE);
    }
    *out = c;
    return LINREC_OK;
}

linrec_status linrec_ctx_destroy(linrec_ctx* ctx)
{
    if (!ctx)
        return LINREC_OK;
    if (ctx->aux)
        (void)hipStreamSynchronize(ctx->aux);
    if (ctx->ev_start)
        (void)hipEventDestroy(ctx->ev_start);
    if (ctx->ev_scan)
        (void)hipEventDestroy(ctx->ev_scan);
    for (hipEvent_t ev : ctx->ev_slot)
        if (ev)
            (void)hipEventDestroy(ev);
    for (const TimedLaunch& t : ctx->pending) {
        (void)hipEventDestroy(t.begin);
        (void)hipEventDestroy(t.end);
    }
    for (hipEvent_t e : ctx->pool)
        (void)hipEventDestroy(e);
    if (ctx->aux)
        (void)hipStreamDestroy(ctx->aux);
    delete ctx;
    return LINREC_OK;
}

linrec_status linrec_ctx_set_timing(linrec_ctx* ctx, int enable)
{
    if (!ctx)
        return LINREC_E_NULL;
    ctx->timing = enable ? 1 : 0;
    for (int k = 0; k < LINREC_KERNEL_KINDS; ++k) {
        ctx->ms[k] = 0.0;
        ctx->count[k] = 0;
    }
    for (const TimedLaunch& t : ctx->pending) {
        ctx->pool.push_back(t.begin);
        ctx->pool.push_back(t.end);
    }
    ctx->pending.clear();
    return LINREC_OK;
}

linrec_status linrec_ctx_kernel_times(linrec_ctx* ctx, int kind, int64_t* count, double* ms)
{
    if (!ctx || !count || !ms)
        return LINREC_E_NULL;
    if (kind < 0 || kind >= LINREC_KERNEL_KINDS)
        return LINREC_E_SHAPE;
    for (const TimedLaunch& t : ctx->pending) {
        float el = 0.f;
        hipError_t e = hipEventSynchronize(t.end);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&el, t.begin, t.end);
        if (e != hipSuccess)
            return hip_fail(e, LINREC_E_DEVICE);
        ctx->ms[t.kind] += el;
        ctx->count[t.kind] += 1;
        ctx->pool.push_back(t.begin);
        ctx->pool.push_back(t.end);
    }
    ctx->pending.clear();
    *count = ctx->count[kind];
    *ms = ctx->ms[kind];
    return LINREC_OK;
}

size_t linrec_states_bytes(const linrec_desc* d)
{
    if (check_desc(d) != LINREC_OK)
        return 0;
    return (size_t)d->B * (size_t)d->H * (size_t)nseg_of(d->T) * per_seg_bytes(d);
}

size_t linrec_bwd_workspace_bytes(const linrec_desc* d) { return linrec_states_bytes(d); }

size_t linrec_bwd_recompute_workspace_bytes(const linrec_desc* d)
{
    if (check_desc(d) != LINREC_OK || d->T == 0)
        return 0;
    return 2 * linrec_states_bytes(d) + (size_t)d->B * d->H * d->dk * d->dv * sizeof(float);
}

// Per-segment totals of the decay gradient, after the gradient records.
static size_t da_tot_bytes(const linrec_desc* d)
{
    const size_t raw = (size_t)d->B * d->H * (size_t)nseg_of(d->T) * sizeof(float);
    return (raw + 255) / 256 * 256;
}

size_t linrec_bwd_da_workspace_bytes(const linrec_desc* d)
{
    if (check_desc(d) != LINREC_OK || d->T == 0)
        return 0;
    return linrec_states_bytes(d) + da_tot_bytes(d);
}

size_t linrec_seq_states_bytes(const linrec_desc* d, int32_t npieces, const int32_t* lengths)
{
    if (check_desc(d) != LINREC_OK || check_pieces(d, npieces, lengths) != LINREC_OK)
        return 0;
    return (size_t)d->B * (size_t)d->H * (size_t)total_nseg(npieces, lengths) * per_seg_bytes(d);
}

// Two slots of gradient records, each sized for the longest piece: piece
// i - 1's are summed and folded while piece i's are read.
static size_t bwd_seq_slot_bytes(const linrec_desc* d, int32_t npieces, const int32_t* lengths)
{
    return (size_t)d->B * (size_t)d->H * (size_t)max_nseg(npieces, lengths) * per_seg_bytes(d);
}

size_t linrec_bwd_seq_workspace_bytes(const linrec_desc* d, int32_t npieces, const int32_t* lengths)
{
    if (check_desc(d) != LINREC_OK || check_pieces(d, npieces, lengths) != LINREC_OK)
        return 0;
    return 3 * bwd_seq_slot_bytes(d, npieces, lengths);
}

linrec_status linrec_fwd(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                         linrec_tensor k, linrec_tensor v, linrec_tensor decay,
                         const float* S_in, linrec_tensor o, float* S_out, void* states,
                         void* stream)
{
    linrec_status st = check_fwd_args(d, q, k, v, decay, S_in, o, S_out, states);
    if (st != LINREC_OK || (st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (d->T == 0)
        return pass_carry(d, S_in, S_out, (int64_t)d->dk * d->dv, s);
    const int64_t ns = nseg_of(d->T);
    const ScanLaunch sc = fwd_scan_of(d, k, v, decay, 0, d->T, S_in, S_out, states, 0, ns);
    const FwdIntraLaunch in = fwd_intra_of(d, q, k, v, decay, o, 0, d->T, states, 0, ns);
    LAUNCH_SCAN(ctx, sc, s);
    LAUNCH_FWD_INTRA(ctx, in, s);
    return LINREC_OK;
}

linrec_status linrec_bwd(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                         linrec_tensor k, linrec_tensor v, linrec_tensor decay,
                         const void* states, linrec_tensor dO, const float* dS_out,
                         linrec_tensor dq, linrec_tensor dk, linrec_tensor dv, float* dS_in,
                         void* workspace, void* stream)
{
    linrec_status st = check_bwd_args(d, q, k, v, decay, states, dO, dS_out, dq, dk, dv,
                                      dS_in, workspace);
    if (st != LINREC_OK || (st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (d->T == 0)
        return pass_carry(d, dS_out, dS_in, (int64_t)d->dk * d->dv, s);
    const int64_t ns = nseg_of(d->T);
    const ScanLaunch sc = bwd_scan_of(d, q, dO, decay, 0, d->T, dS_out, dS_in, workspace);
    const BwdIntraLaunch in =
        bwd_intra_of(d, q, k, v, decay, dO, dq, dk, dv, 0, d->T, states, 0, ns, workspace);
    LAUNCH_SCAN(ctx, sc, s);
    LAUNCH_BWD_INTRA(ctx, in, s);
    return LINREC_OK;
}

linrec_status linrec_bwd_noalloc(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                                 linrec_tensor k, linrec_tensor v, linrec_tensor decay,
                                 const void* states, linrec_tensor dO, const float* dS_out,
                                 linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                                 float* dS_in, void* stream)
{
    // the workspace check is done against the scratch below; any aligned
    // non-NULL pointer stands in for it in the common argument checks
    linrec_status st = check_bwd_args(d, q, k, v, decay, states, dO, dS_out, dq, dk, dv,
                                      dS_in, states);
    if (st != LINREC_OK)
        return st;
    if (linrec_bwd_workspace_bytes(d) > LINREC_NOALLOC_SCRATCH_BYTES)
        return LINREC_E_SCRATCH;
    if ((st = check_ctx(ctx)) != LINREC_OK)
        return st;
    if (d->T == 0)
        return pass_carry(d, dS_out, dS_in, (int64_t)d->dk * d->dv, (hipStream_t)stream);
    if (!ctx->scratch)
        return hip_fail(ctx->scratch_err != hipSuccess ? ctx->scratch_err : hipErrorInvalidSymbol,
                        LINREC_E_DEVICE);
    hipStream_t s = (hipStream_t)stream;
    const int64_t ns = nseg_of(d->T);
    const ScanLaunch sc = bwd_scan_of(d, q, dO, decay, 0, d->T, dS_out, dS_in, ctx->scratch);
    const BwdIntraLaunch in = bwd_intra_of(d, q, k, v, decay, dO, dq, dk, dv, 0, d->T, states, 0,
                                           ns, ctx->scratch);
    LAUNCH_SCAN(ctx, sc, s);
    LAUNCH_BWD_INTRA(ctx, in, s);
    return LINREC_OK;
}

linrec_status linrec_bwd_da(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                            linrec_tensor k, linrec_tensor v, linrec_tensor decay,
                            const void* states, linrec_tensor dO, const float* dS_out,
                            linrec_tensor dq, linrec_tensor dk, linrec_tensor dv, float* dS_in,
                            linrec_tensor da, const float* da_carry_in, float* da_carry_out,
                            void* workspace, void* stream)
{
    linrec_status st = check_bwd_args(d, q, k, v, decay, states, dO, dS_out, dq, dk, dv,
                                      dS_in, workspace);
    if (st != LINREC_OK)
        return st;
    if (d->decay == LINREC_DECAY_NONE)
        return LINREC_E_LAYOUT;
    if (d->T > 0) {
        if (!da.ptr)
            return LINREC_E_NULL;
        if (!aligned(da.ptr, 4))
            return LINREC_E_ALIGN;
        if (da.sb < 0 || da.sh < 0 || da.st < 1)
            return LINREC_E_LAYOUT;
    }
    if ((st = check_state_ptr(da_carry_in, false)) != LINREC_OK ||
        (st = check_state_ptr(da_carry_out, true)) != LINREC_OK || (st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (d->T == 0) {
        if ((st = pass_carry(d, dS_out, dS_in, (int64_t)d->dk * d->dv, s)) != LINREC_OK)
            return st;
        return pass_carry(d, da_carry_in, da_carry_out, 1, s);
    }
    const int64_t ns = nseg_of(d->T);
    float* tot = (float*)((char*)workspace + linrec_states_bytes(d));
    const ScanLaunch sc = bwd_scan_of(d, q, dO, decay, 0, d->T, dS_out, dS_in, workspace);
    BwdIntraLaunch in =
        bwd_intra_of(d, q, k, v, decay, dO, dq, dk, dv, 0, d->T, states, 0, ns, workspace);
    in.da = targ(da);
    in.da_tot = tot;
    DaFinishLaunch fin{};
    fin.B = d->B; fin.H = d->H; fin.N = (int)chunks_of(d->T); fin.m = kSegChunks;
    fin.tail = d->T - (fin.N - 1) * kChunk;
    fin.da = targ(da);
    fin.decay = targ(decay);
    fin.decay_kind = d->decay;
    fin.tot = tot;
    fin.carry_in = da_carry_in;
    fin.carry_out = da_carry_out;
    LAUNCH_SCAN(ctx, sc, s);
    LAUNCH_BWD_INTRA(ctx, in, s);
    LAUNCH(timed_launch(ctx, LINREC_KERNEL_DA_FINISH, s,
                        [&] { return linrec::launch_da_finish(fin, s); }));
    return LINREC_OK;
}

linrec_status linrec_bwd_recompute(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                                   linrec_tensor k, linrec_tensor v, linrec_tensor decay,
                                   const float* S_in, linrec_tensor dO, const float* dS_out,
                                   linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                                   float* dS_in, void* workspace, void* stream)
{
    // workspace: [state records | gradient records | one scratch state]
    linrec_status st = check_bwd_args(d, q, k, v, decay, workspace, dO, dS_out, dq, dk, dv,
                                      dS_in, workspace);
    if (st != LINREC_OK || (st = check_state_ptr(S_in, false)) != LINREC_OK ||
        (st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (d->T == 0)
        return pass_carry(d, dS_out, dS_in, (int64_t)d->dk * d->dv, s);
    const int64_t ns = nseg_of(d->T);
    char* ws = (char*)workspace;
    void* states = ws;
    void* grads = ws + linrec_states_bytes(d);
    float* scratch = (float*)(ws + 2 * linrec_states_bytes(d));
    const ScanLaunch fsc = fwd_scan_of(d, k, v, decay, 0, d->T, S_in, scratch, states, 0, ns);
    const ScanLaunch bsc = bwd_scan_of(d, q, dO, decay, 0, d->T, dS_out, dS_in, grads);
    const BwdIntraLaunch in =
        bwd_intra_of(d, q, k, v, decay, dO, dq, dk, dv, 0, d->T, states, 0, ns, grads);
    LAUNCH_SCAN(ctx, fsc, s);
    LAUNCH_SCAN(ctx, bsc, s);
    LAUNCH_BWD_INTRA(ctx, in, s);
    return LINREC_OK;
}

linrec_status linrec_fwd_seq(linrec_ctx* ctx, const linrec_desc* d, int32_t npieces,
                             const int32_t* lengths, linrec_tensor q, linrec_tensor k,
                             linrec_tensor v, linrec_tensor decay, const float* S_in,
                             linrec_tensor o, float* S_out, void* states, void* stream)
{
    linrec_status st = check_fwd_args(d, q, k, v, decay, S_in, o, S_out, states);
    if (st != LINREC_OK || (st = check_pieces(d, npieces, lengths)) != LINREC_OK ||
        (st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const int64_t nseg_total = total_nseg(npieces, lengths);
    HIPCHECK(hipEventRecord(ctx->ev_start, s));
    HIPCHECK(hipStreamWaitEvent(ctx->aux, ctx->ev_start, 0));
    int64_t tok0 = 0, seg0 = 0;
    for (int32_t i = 0; i < npieces; ++i) {
        // piece i's state transition: S carried in S_out from piece i-1
        const float* cin = i == 0 ? S_in : S_out;
        const ScanLaunch sc =
            fwd_scan_of(d, k, v, decay, tok0, lengths[i], cin, S_out, states, seg0, nseg_total);
        const FwdIntraLaunch in =
            fwd_intra_of(d, q, k, v, decay, o, tok0, lengths[i], states, seg0, nseg_total);
        LAUNCH_SCAN(ctx, sc, ctx->aux);
        HIPCHECK(hipEventRecord(ctx->ev_scan, ctx->aux));
        HIPCHECK(hipStreamWaitEvent(s, ctx->ev_scan, 0));
        LAUNCH_FWD_INTRA(ctx, in, s);
        tok0 += lengths[i];
        seg0 += nseg_of(lengths[i]);
    }
    return LINREC_OK;
}

linrec_status linrec_bwd_seq(linrec_ctx* ctx, const linrec_desc* d, int32_t npieces,
                             const int32_t* lengths, linrec_tensor q, linrec_tensor k,
                             linrec_tensor v, linrec_tensor decay, const void* states,
                             linrec_tensor dO, const float* dS_out, linrec_tensor dq,
                             linrec_tensor dk, linrec_tensor dv, float* dS_in, void* workspace,
                             void* stream)
{
    linrec_status st = check_bwd_args(d, q, k, v, decay, states, dO, dS_out, dq, dk, dv,
                                      dS_in, workspace);
    if (st != LINREC_OK || (st = check_pieces(d, npieces, lengths)) != LINREC_OK ||
        (st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const int64_t nseg_total = total_nseg(npieces, lengths);
    // Every launch goes to the caller's stream, one per piece: the segment
    // kernel of piece i carries, as extra work in the same launch, the fold
    // of piece i - 1 (which needs piece i's dS_in, left by the previous
    // launch) and the segment sums of piece i - 2 (which need nothing
    // carried).  The state transition thus runs beside the intra-chunk work
    // on the CUs the segment kernel leaves free, without a launch of its own.
    // A prologue does the last piece's sums and fold and the next piece's
    // sums.  The gradient records of piece j live in workspace slot j % 3:
    // one launch reads slot i % 3, folds slot (i - 1) % 3 and writes
    // slot (i - 2) % 3.
    const size_t slot_bytes = bwd_seq_slot_bytes(d, npieces, lengths);
    auto slot_ptr = [&](int32_t i) { return (void*)((char*)workspace + (i % 3) * slot_bytes); };
    std::vector<int64_t> tok0s(npieces), seg0s(npieces);
    for (int32_t i = 0, t0 = 0, g0 = 0; i < npieces; ++i) {
        tok0s[i] = t0;
        seg0s[i] = g0;
        t0 += lengths[i];
        g0 += (int32_t)nseg_of(lengths[i]);
    }
    auto scan_of = [&](int32_t i, const float* cin) {
        return bwd_scan_of(d, q, dO, decay, tok0s[i], lengths[i], cin, dS_in, slot_ptr(i));
    };
    const ScanLaunch last = scan_of(npieces - 1, dS_out);
    LAUNCH_SCAN(ctx, last, s);
    if (npieces > 1) {
        const ScanLaunch next = scan_of(npieces - 2, dS_in);
        LAUNCH(timed_launch(ctx, LINREC_KERNEL_BWD_SUM, s,
                            [&] { return linrec::launch_seg_sum(next, s); }));
    }
    for (int32_t i = npieces - 1; i >= 0; --i) {
        BwdIntraLaunch in = bwd_intra_of(d, q, k, v, decay, dO, dq, dk, dv, tok0s[i], lengths[i],
                                         states, seg0s[i], nseg_total, slot_ptr(i));
        if (i > 0) {
            const ScanLaunch prev = scan_of(i - 1, dS_in);
            in.fold = linrec::FoldArg{dS_in, dS_in, (float*)prev.store, prev.store_nseg,
                                      (int32_t)nseg_of(lengths[i - 1])};
        }
        if (i > 1) {
            const ScanLaunch sums = scan_of(i - 2, dS_in);
            in.sum = sum_arg_of(sums);
        }
        LAUNCH_BWD_INTRA(ctx, in, s);
    }
    return LINREC_OK;
}

namespace {

// Tokens of a delta-rule piece rounded up to whole chunks: the rows its
// workspace and saved buffers hold.
static size_t delta_tokens(const linrec_desc* d) { return (size_t)chunks_of(d->T) * kChunk; }

}  // namespace

size_t linrec_delta_workspace_bytes(const linrec_desc* d)
{
    if (check_desc(d) != LINREC_OK || d->dk != d->dv)
        return 0;
    // W_k, W_v, then P per chunk (64 x 64 per 64 tokens), then the decay
    // tables per chunk (256 per 64 tokens); a partial last chunk counts whole
    return (size_t)d->B * d->H * (size_t)delta_tokens(d) * (size_t)(d->dk + d->dv + kChunk + 4) * sizeof(float);
}

size_t linrec_delta_saved_bytes(const linrec_desc* d)
{
    if (check_desc(d) != LINREC_OK || d->dk != d->dv)
        return 0;
    const size_t bh = (size_t)d->B * d->H, Tp = delta_tokens(d);
    return bh * (Tp / kChunk * d->dk * d->dv + Tp * d->dv) * sizeof(float);
}

size_t linrec_delta_bwd_workspace_bytes(const linrec_desc* d)
{
    if (check_desc(d) != LINREC_OK || d->dk != d->dv)
        return 0;
    const size_t bh = (size_t)d->B * d->H, Tp = delta_tokens(d), N = Tp / kChunk;
    return bh * (Tp * (d->dk + 2 * d->dv + kChunk + 4) + N * kChunk * kChunk + N * d->dk * d->dv) *
           sizeof(float);
}

namespace {

static linrec_status check_beta(const linrec_tensor& beta)
{
    if (!beta.ptr)
        return LINREC_E_NULL;
    if (!aligned(beta.ptr, 4))
        return LINREC_E_ALIGN;
    if (beta.sb < 0 || beta.sh < 0 || beta.st < 0)
        return LINREC_E_LAYOUT;
    return LINREC_OK;
}

}  // namespace

namespace {

// Bytes of the delta rule's per-piece buffers for a piece of `len` tokens
// of the sequence d describes (rows rounded up to whole chunks).
static size_t delta_piece_saved_bytes(const linrec_desc* d, int32_t len)
{
    linrec_desc p = *d;
    p.T = len;
    return linrec_delta_saved_bytes(&p);
}

// Launch description of the delta-rule forward over tokens [tok0, tok0 + len)
// of the tensors, with that piece's workspace at `ws` and saved values at
// `saved` (may be NULL).
static linrec::DeltaFwdLaunch delta_fwd_of(const linrec_desc* d, int64_t tok0, int32_t len,
                                           const linrec_tensor& q, const linrec_tensor& k,
                                           const linrec_tensor& v, const linrec_tensor& beta,
                                           const linrec_tensor& decay, const float* S_in,
                                           const linrec_tensor& o, float* S_out, void* saved,
                                           void* ws)
{
    const int esz = elem_size(d->dtype), osz = elem_size(d->out_dtype);
    linrec_desc p = *d;
    p.T = len;
    linrec::DeltaFwdLaunch s{};
    s.dtype = d->dtype; s.out_dtype = d->out_dtype; s.dk = d->dk; s.dv = d->dv;
    s.B = d->B; s.H = d->H; s.T = len;
    s.q = advance(q, tok0, esz); s.k = advance(k, tok0, esz); s.v = advance(v, tok0, esz);
    s.beta = advance(beta, tok0, 4); s.o = advance(o, tok0, osz);
    s.decay = advance_decay(d, decay, tok0);
    s.decay_kind = d->decay;
    s.S_in = S_in;
    s.S_out = S_out;
    const size_t bh = (size_t)d->B * d->H, Tp = delta_tokens(&p);
    s.wk = (float*)ws;
    s.wv = s.wk + bh * Tp * d->dk;
    s.pm = s.wv + bh * Tp * d->dv;
    s.tabs = s.pm + bh * Tp * kChunk;
    if (saved) {
        s.s0 = (float*)saved;
        s.u = (float*)saved + bh * (Tp / kChunk) * d->dk * d->dv;
    }
    return s;
}

// Launch description of the delta-rule backward over tokens [tok0, tok0 + len).
static linrec::DeltaBwdLaunch delta_bwd_of(const linrec_desc* d, int64_t tok0, int32_t len,
                                           const linrec_tensor& q, const linrec_tensor& k,
                                           const linrec_tensor& v, const linrec_tensor& beta,
                                           const linrec_tensor& decay, const void* saved,
                                           const linrec_tensor& dO, const float* dS_out,
                                           const linrec_tensor& dq, const linrec_tensor& dk,
                                           const linrec_tensor& dv, const linrec_tensor& dbeta,
                                           float* dS_in, void* ws)
{
    const int esz = elem_size(d->dtype), osz = elem_size(d->out_dtype);
    linrec_desc p = *d;
    p.T = len;
    // workspace and saved rows cover whole chunks; the last may be partial
    const size_t bh = (size_t)d->B * d->H, T = delta_tokens(&p), N = T / kChunk;
    linrec::DeltaBwdLaunch s{};
    s.dtype = d->dtype; s.out_dtype = d->out_dtype; s.dk = d->dk; s.dv = d->dv;
    s.B = d->B; s.H = d->H; s.T = len;
    s.q = advance(q, tok0, esz); s.k = advance(k, tok0, esz); s.v = advance(v, tok0, esz);
    s.beta = advance(beta, tok0, 4); s.decay = advance_decay(d, decay, tok0);
    s.dO = advance(dO, tok0, esz);
    s.dq = advance(dq, tok0, osz); s.dk_ = advance(dk, tok0, osz); s.dv_ = advance(dv, tok0, osz);
    s.dbeta = advance(dbeta, tok0, 4);
    s.decay_kind = d->decay;
    s.s0 = (const float*)saved;
    s.u = (const float*)saved + bh * N * d->dk * d->dv;
    s.dS_out = dS_out;
    s.dS_in = dS_in;
    float* w = (float*)ws;
    s.wk = w;
    s.wv = s.wk + bh * T * d->dk;
    s.tm = s.wv + bh * T * d->dv;
    s.duy = s.tm + bh * N * kChunk * kChunk;
    s.dsc = s.duy + bh * T * d->dv;
    s.pm = s.dsc + bh * N * d->dk * d->dv;
    s.tabs = s.pm + bh * T * kChunk;
    return s;
}

// Largest piece of a sequence.
static int32_t longest_piece(int32_t npieces, const int32_t* lengths)
{
    int32_t m = 0;
    for (int32_t i = 0; i < npieces; ++i)
        m = std::max(m, lengths[i]);
    return m;
}

}  // namespace

linrec_status linrec_delta_fwd(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                               linrec_tensor k, linrec_tensor v, linrec_tensor beta,
                               linrec_tensor decay, const float* S_in, linrec_tensor o,
                               float* S_out, void* saved, void* workspace, void* stream)
{
    linrec_status st = check_fwd_args(d, q, k, v, decay, S_in, o, S_out, workspace);
    if (st != LINREC_OK)
        return st;
    if (d->dk != d->dv)
        return LINREC_E_SHAPE;
    if (d->T > 0 && (st = check_beta(beta)) != LINREC_OK)
        return st;
    if (saved && !aligned(saved, 16))
        return LINREC_E_WORKSPACE;
    if ((st = check_ctx(ctx)) != LINREC_OK)
        return st;
    if (d->T == 0)
        return pass_carry(d, S_in, S_out, (int64_t)d->dk * d->dv, (hipStream_t)stream);
    const linrec::DeltaFwdLaunch s =
        delta_fwd_of(d, 0, d->T, q, k, v, beta, decay, S_in, o, S_out, saved, workspace);
    LAUNCH(timed_launch(ctx, LINREC_KERNEL_DELTA_FWD, (hipStream_t)stream,
                        [&] { return linrec::launch_delta_fwd(s, (hipStream_t)stream); }));
    return LINREC_OK;
}

linrec_status linrec_delta_bwd(linrec_ctx* ctx, const linrec_desc* d, linrec_tensor q,
                               linrec_tensor k, linrec_tensor v, linrec_tensor beta,
                               linrec_tensor decay, const void* saved, linrec_tensor dO,
                               const float* dS_out, linrec_tensor dq, linrec_tensor dk,
                               linrec_tensor dv, linrec_tensor dbeta, float* dS_in,
                               void* workspace, void* stream)
{
    linrec_status st = check_bwd_args(d, q, k, v, decay, saved, dO, dS_out, dq, dk, dv, dS_in,
                                      workspace);
    if (st != LINREC_OK)
        return st;
    if (d->dk != d->dv)
        return LINREC_E_SHAPE;
    if (d->T > 0 && ((st = check_beta(beta)) != LINREC_OK || (st = check_beta(dbeta)) != LINREC_OK))
        return st;
    if ((st = check_ctx(ctx)) != LINREC_OK)
        return st;
    if (d->T == 0)
        return pass_carry(d, dS_out, dS_in, (int64_t)d->dk * d->dv, (hipStream_t)stream);
    const linrec::DeltaBwdLaunch s = delta_bwd_of(d, 0, d->T, q, k, v, beta, decay, saved, dO,
                                                  dS_out, dq, dk, dv, dbeta, dS_in, workspace);
    LAUNCH(timed_launch(ctx, LINREC_KERNEL_DELTA_BWD, (hipStream_t)stream,
                        [&] { return linrec::launch_delta_bwd(s, (hipStream_t)stream); }));
    return LINREC_OK;
}

size_t linrec_delta_seq_saved_bytes(const linrec_desc* d, int32_t npieces, const int32_t* lengths)
{
    if (check_desc(d) != LINREC_OK || d->dk != d->dv || check_pieces(d, npieces, lengths) != LINREC_OK)
        return 0;
    size_t n = 0;
    for (int32_t i = 0; i < npieces; ++i)
        n += delta_piece_saved_bytes(d, lengths[i]);
    return n;
}

size_t linrec_delta_fwd_seq_workspace_bytes(const linrec_desc* d, int32_t npieces,
                                            const int32_t* lengths)
{
    if (check_desc(d) != LINREC_OK || d->dk != d->dv || check_pieces(d, npieces, lengths) != LINREC_OK)
        return 0;
    linrec_desc p = *d;
    p.T = longest_piece(npieces, lengths);
    return linrec_delta_workspace_bytes(&p);
}

size_t linrec_delta_bwd_seq_workspace_bytes(const linrec_desc* d, int32_t npieces,
                                            const int32_t* lengths)
{
    if (check_desc(d) != LINREC_OK || d->dk != d->dv || check_pieces(d, npieces, lengths) != LINREC_OK)
        return 0;
    linrec_desc p = *d;
    p.T = longest_piece(npieces, lengths);
    return (size_t)std::min<int32_t>(npieces, 2) * linrec_delta_bwd_workspace_bytes(&p);
}

linrec_status linrec_delta_fwd_seq(linrec_ctx* ctx, const linrec_desc* d, int32_t npieces,
                                   const int32_t* lengths, linrec_tensor q, linrec_tensor k,
                                   linrec_tensor v, linrec_tensor beta, linrec_tensor decay,
                                   const float* S_in, linrec_tensor o, float* S_out, void* saved,
                                   void* workspace, void* stream)
{
    linrec_status st = check_fwd_args(d, q, k, v, decay, S_in, o, S_out, workspace);
    if (st != LINREC_OK || (st = check_pieces(d, npieces, lengths)) != LINREC_OK)
        return st;
    if (d->dk != d->dv)
        return LINREC_E_SHAPE;
    if ((st = check_beta(beta)) != LINREC_OK)
        return st;
    if (saved && !aligned(saved, 16))
        return LINREC_E_WORKSPACE;
    if ((st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    // Each piece's prep kernel, then its serial walk, on the caller's stream.
    // (The prep kernel of the next piece beside the walk, on a second stream,
    // slowed the walk, the critical path, by more than it saved.)
    int64_t tok0 = 0;
    size_t saved_off = 0;
    for (int32_t i = 0; i < npieces; ++i) {
        const linrec::DeltaFwdLaunch cur =
            delta_fwd_of(d, tok0, lengths[i], q, k, v, beta, decay, i == 0 ? S_in : S_out, o, S_out,
                         saved ? (char*)saved + saved_off : nullptr, workspace);
        LAUNCH(timed_launch(ctx, LINREC_KERNEL_DELTA_FWD, s,
                            [&] { return linrec::launch_delta_fwd(cur, s); }));
        tok0 += lengths[i];
        saved_off += delta_piece_saved_bytes(d, lengths[i]);
    }
    return LINREC_OK;
}

linrec_status linrec_delta_bwd_seq(linrec_ctx* ctx, const linrec_desc* d, int32_t npieces,
                                   const int32_t* lengths, linrec_tensor q, linrec_tensor k,
                                   linrec_tensor v, linrec_tensor beta, linrec_tensor decay,
                                   const void* saved, linrec_tensor dO, const float* dS_out,
                                   linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                                   linrec_tensor dbeta, float* dS_in, void* workspace,
                                   void* stream)
{
    linrec_status st = check_bwd_args(d, q, k, v, decay, saved, dO, dS_out, dq, dk, dv, dS_in,
                                      workspace);
    if (st != LINREC_OK || (st = check_pieces(d, npieces, lengths)) != LINREC_OK)
        return st;
    if (d->dk != d->dv)
        return LINREC_E_SHAPE;
    if ((st = check_beta(beta)) != LINREC_OK || (st = check_beta(dbeta)) != LINREC_OK)
        return st;
    if ((st = check_ctx(ctx)) != LINREC_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    // Pieces in reverse.  Each piece's prep kernel and serial walk run on the
    // caller's stream, the walks one after another (dS carried in dS_in).
    // The per-chunk gradient kernels of piece i, which need its walk but
    // nothing carried, run on the aux stream beside the prep and walk of
    // piece i - 1.  Piece i's buffers live in workspace slot i % 2; the prep
    // of piece i waits for the gradient kernels of piece i + 2, that slot's
    // last reader (one event per slot).
    linrec_desc p = *d;
    p.T = longest_piece(npieces, lengths);
    const size_t slot_bytes = linrec_delta_bwd_workspace_bytes(&p);
    int64_t tok0 = d->T;
    size_t off = linrec_delta_seq_saved_bytes(d, npieces, lengths);
    for (int32_t i = npieces - 1; i >= 0; --i) {
        tok0 -= lengths[i];
        off -= delta_piece_saved_bytes(d, lengths[i]);
        linrec::DeltaBwdLaunch cur = delta_bwd_of(
            d, tok0, lengths[i], q, k, v, beta, decay, (const char*)saved + off, dO,
            i == npieces - 1 ? dS_out : dS_in, dq, dk, dv, dbeta, dS_in,
            (char*)workspace + (i % 2) * slot_bytes);
        if (i + 2 < npieces)
            HIPCHECK(hipStreamWaitEvent(s, ctx->ev_slot[i % 2], 0));
        cur.parts = linrec::DELTA_PREP | linrec::DELTA_SERIAL;
        LAUNCH(timed_launch(ctx, LINREC_KERNEL_DELTA_BWD, s,
                            [&] { return linrec::launch_delta_bwd(cur, s); }));
        HIPCHECK(hipEventRecord(ctx->ev_start, s));
        HIPCHECK(hipStreamWaitEvent(ctx->aux, ctx->ev_start, 0));
        cur.parts = linrec::DELTA_GRAD;
        LAUNCH(timed_launch(ctx, LINREC_KERNEL_DELTA_BWD, ctx->aux,
                            [&] { return linrec::launch_delta_bwd(cur, ctx->aux); }));
        HIPCHECK(hipEventRecord(ctx->ev_slot[i % 2], ctx->aux));
    }
    // the caller's stream waits for the last gradient kernels
    HIPCHECK(hipEventRecord(ctx->ev_scan, ctx->aux));
    HIPCHECK(hipStreamWaitEvent(s, ctx->ev_scan, 0));
    return LINREC_OK;
}

const char* linrec_status_str(linrec_status s)
{
    // a C caller may pass any int; read it as one (an out-of-range value
    // loaded as the enum type is undefined in C++)
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case LINREC_OK: return "ok";
    case LINREC_E_NULL: return "required pointer is NULL";
    case LINREC_E_SHAPE: return "unsupported shape";
    case LINREC_E_DTYPE: return "unsupported dtype";
    case LINREC_E_LAYOUT: return "unsupported layout";
    case LINREC_E_ALIGN: return "misaligned pointer or stride";
    case LINREC_E_WORKSPACE: return "states/workspace missing or misaligned";
    case LINREC_E_DEVICE: return "HIP runtime error";
    case LINREC_E_LAUNCH: return "kernel launch failed";
    case LINREC_E_SCRATCH: return "the piece needs more than the fixed no-allocation scratch";
    }
    return "unknown status";
}

int linrec_last_hip_error(void) { return g_last_hip_error; }

int linrec_version(void) { return 100; }

}  // extern "C"
