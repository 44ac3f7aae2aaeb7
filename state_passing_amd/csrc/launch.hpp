// launch.hpp -- host-side launch descriptions shared by the C ABI and the
// kernel launchers (plain data; pointers are device addresses).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

// Floats per stored segment record: a d_k x d_v state, then the segment's
// total log-decay, padded so records stay 256-byte aligned.
constexpr __host__ __device__ int64_t seg_record_floats(int dk, int dv) { return (int64_t)dk * dv + 64; }

struct TensorArg {
    const void* ptr;
    int64_t sb, sh, st;
};

// A piece has N chunks of 64 tokens, grouped into segments of m chunks (the
// last one may be shorter).  Per-segment records (seg_record_floats) live in
// a store laid out [B][H][nseg][record]; pointers are already offset to the
// piece's first segment and *_nseg is the store's segments per (b, h).

// Segment scan of one piece.  Forward: x = K, y = V, carry S_in -> S_out,
// store = state entering every segment.  Reverse: x = Q, y = dO, carry
// dS_out -> dS_in, store = gradient leaving every segment.
struct ScanLaunch {
    int dtype, dk, dv, B, H, N, m;
    int out_dtype;           // unused by the scan; keeps one dispatch macro
    bool reverse;
    TensorArg x, y, decay;
    int decay_kind;
    const float* carry_in;   // may be NULL (zeros)
    float* carry_out;
    void* store;
    int64_t store_nseg;
};

struct FwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N, m;
    TensorArg q, k, v, decay, o;
    int decay_kind;
    const void* states;
    int64_t st_nseg;
};

// da.ptr != NULL asks for the decay gradient: the kernel writes, per token,
// the reverse cumulative sum within its segment of q.dq - k.dk into da and
// each segment's total into da_tot ([B][H][nseg of the piece]).
struct BwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N, m;
    TensorArg q, k, v, dO, decay, dq, dk_, dv_;
    int decay_kind;
    const void* states;
    int64_t st_nseg;
    const void* ghat;
    int64_t g_nseg;
    TensorArg da;
    float* da_tot;
};

// Finishes the decay gradient of one piece: adds the totals of later
// segments and the carry from later pieces, divides by the decay, and
// writes the carry for the previous piece.
struct DaFinishLaunch {
    int B, H, N, m;
    TensorArg da, decay;
    int decay_kind;
    const float* tot;
    const float* carry_in;   // may be NULL (zeros); may alias carry_out
    float* carry_out;
};

// The state transition is two launches: the parallel segment sum, then the
// serial fold (both from the same description).
hipError_t launch_seg_sum(const ScanLaunch& s, hipStream_t stream);
hipError_t launch_seg_fold(const ScanLaunch& s, hipStream_t stream);
hipError_t launch_fwd_intra(const FwdIntraLaunch& s, hipStream_t stream);
hipError_t launch_bwd_intra(const BwdIntraLaunch& s, hipStream_t stream);
hipError_t launch_da_finish(const DaFinishLaunch& s, hipStream_t stream);

}  // namespace linrec
