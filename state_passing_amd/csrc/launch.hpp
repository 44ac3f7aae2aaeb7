// launch.hpp -- host-side launch descriptions shared by the C ABI and the
// kernel launchers (plain data; pointers are device addresses).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace linrec {

// Per-kernel timing.  When `stop` is set, the kernels launched on this thread
// carry the two events as their dispatch's own start and end stamps (so the
// measured time is the kernels' execution, as a kernel trace reports it, not
// queueing or the dispatch latency before them).  The first launch takes
// `start`; every launch takes `stop`, so a call that launches several kernels
// spans from the first one's start to the last one's end.
struct LaunchStamps {
    hipEvent_t start = nullptr, stop = nullptr;
};

inline LaunchStamps& launch_stamps()
{
    static thread_local LaunchStamps s;
    return s;
}

// Calls f with std::integral_constant<bool, ragged>: the kernels with the
// masking of a partial last chunk are instantiated apart, so pieces of whole
// chunks run code without it.
template <typename F>
inline hipError_t with_ragged(bool ragged, F&& f)
{
    return ragged ? f(std::integral_constant<bool, true>{}) : f(std::integral_constant<bool, false>{});
}

// Every kernel of the library is launched through here (no dynamic LDS).
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                          Args... args)
{
    LaunchStamps& st = launch_stamps();
    if (st.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, st.start, st.stop, 0, args...);
        st.start = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
    }
}

// Floats per stored segment record: a d_k x d_v state, then the segment's
// total log-decay, padded so records stay 256-byte aligned.
constexpr __host__ __device__ int64_t seg_record_floats(int dk, int dv) { return (int64_t)dk * dv + 64; }

struct TensorArg {
    const void* ptr;
    int64_t sb, sh, st;
};

// A piece has N chunks of 64 tokens, grouped into segments of m chunks (the
// last one may be shorter); its last chunk holds `tail` tokens (1..64), the
// tokens past them do not exist and are neither read nor written.  Per-segment records (seg_record_floats) live in
// a store laid out [B][H][nseg][record]; pointers are already offset to the
// piece's first segment and *_nseg is the store's segments per (b, h).

// Segment scan of one piece.  Forward: x = K, y = V, carry S_in -> S_out,
// store = state entering every segment.  Reverse: x = Q, y = dO, carry
// dS_out -> dS_in, store = gradient leaving every segment.
struct ScanLaunch {
    int dtype, dk, dv, B, H, N, m, tail;
    int out_dtype;           // unused by the scan; keeps one dispatch macro
    bool reverse;
    TensorArg x, y, decay;
    int decay_kind;
    const float* carry_in;   // may be NULL (zeros)
    float* carry_out;
    void* store;
    int64_t store_nseg;
};

// The previous piece's reverse fold carried along by a backward
// segment-kernel launch of the sequence driver (store == NULL: none).  Same meaning as the fold of a
// ScanLaunch: that piece's records (store, store_nseg per (b, h), nseg of
// them) and its carry.  Each workgroup of the launch folds an equal share of
// every head's state elements.
struct FoldArg {
    const float* carry_in;   // may be NULL (zeros); may alias carry_out
    float* carry_out;
    float* store;
    int64_t store_nseg;
    int nseg;
};

// Segment sums carried by a backward segment-kernel launch (the sequence
// backward): the reverse sums of another piece, whose q and dO views, decay
// view and records are given here, run as nseg extra workgroups of the
// launch, dispatched after the segment kernel's own.  nseg = 0: none.
struct SumArg {
    TensorArg x, y, decay;   // q, dO and decay of that piece
    int decay_kind;
    void* store;
    int64_t store_nseg;
    int N, m, nseg, tail;
};

struct FwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N, m, tail;
    TensorArg q, k, v, decay, o;
    int decay_kind;
    const void* states;
    int64_t st_nseg;
};

// da.ptr != NULL asks for the decay gradient: the kernel writes, per token,
// the reverse cumulative sum within its segment of q.dq - k.dk into da and
// each segment's total into da_tot ([B][H][nseg of the piece]).
struct BwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N, m, tail;
    TensorArg q, k, v, dO, decay, dq, dk_, dv_;
    int decay_kind;
    const void* states;
    int64_t st_nseg;
    const void* ghat;
    int64_t g_nseg;
    TensorArg da;
    float* da_tot;
    FoldArg fold;            // the previous piece's reverse fold, or none
    SumArg sum;              // the segment sums of the piece before that, or none
};

// Finishes the decay gradient of one piece: adds the totals of later
// segments and the carry from later pieces, divides by the decay, and
// writes the carry for the previous piece.
struct DaFinishLaunch {
    int B, H, N, m, tail;
    TensorArg da, decay;
    int decay_kind;
    const float* tot;
    const float* carry_in;   // may be NULL (zeros); may alias carry_out
    float* carry_out;
};

// Gated delta rule, forward over one piece: per-chunk W_k, W_v into the
// workspace (fp32 [B][H][T][d_k], then [B][H][T][d_v]), then the serial walk.
// The launches of a delta-rule piece, which a sequence driver may issue on
// different streams: the per-chunk prep kernel, the serial walk, and (in the
// backward) the per-chunk gradient kernels behind it.
enum : unsigned { DELTA_PREP = 1, DELTA_SERIAL = 2, DELTA_GRAD = 4 };
struct DeltaFwdLaunch {
    int dtype, out_dtype, dk, dv, B, H, T;
    TensorArg q, k, v, beta, decay, o;
    int decay_kind;
    const float* S_in;       // may be NULL (zeros)
    float* S_out;
    float* wk;
    float* wv;
    float* s0;               // optional: the state entering every chunk, [B][H][N][d_k][d_v]
    float* u;                // optional: U of every token, [B][H][T][d_v]
    float* pm;               // P = (Q K^T) .* D per chunk, [B][H][N][64][64] (workspace)
    float* tabs;             // the decay tables of every chunk, [B][H][N][256] (workspace)
    unsigned parts;          // DELTA_PREP | DELTA_SERIAL; 0: both
};

// Gated delta rule, backward over one piece, from the forward's saved s0 and
// u.  Workspace: W_k, W_v (as the forward), T then M per chunk
// ([B][H][N][64][64]), dU then Y ([B][H][T][d_v]), dS_C per chunk, P per
// chunk, the decay tables per chunk.
struct DeltaBwdLaunch {
    int dtype, out_dtype, dk, dv, B, H, T;
    TensorArg q, k, v, beta, decay, dO, dq, dk_, dv_, dbeta;
    int decay_kind;
    const float* s0;
    const float* u;
    const float* dS_out;     // may be NULL (zeros)
    float* dS_in;
    float* wk;
    float* wv;
    float* tm;
    float* duy;
    float* dsc;
    float* pm;
    float* tabs;
    unsigned parts;          // DELTA_PREP | DELTA_SERIAL | DELTA_GRAD; 0: all
};

// The state transition is two launches: the parallel segment sum, then the
// serial fold (both from the same description).
hipError_t launch_seg_sum(const ScanLaunch& s, hipStream_t stream);
hipError_t launch_seg_fold(const ScanLaunch& s, hipStream_t stream);
hipError_t launch_fwd_intra(const FwdIntraLaunch& s, hipStream_t stream);
hipError_t launch_bwd_intra(const BwdIntraLaunch& s, hipStream_t stream);
hipError_t launch_da_finish(const DaFinishLaunch& s, hipStream_t stream);
hipError_t launch_carry_copy(const float* src, float* dst, int64_t n, hipStream_t stream);
hipError_t launch_delta_fwd(const DeltaFwdLaunch& s, hipStream_t stream);
hipError_t launch_delta_bwd(const DeltaBwdLaunch& s, hipStream_t stream);

}  // namespace linrec
