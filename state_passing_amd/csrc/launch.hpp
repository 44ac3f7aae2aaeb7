// launch.hpp -- host-side launch descriptions shared by the C ABI and the
// kernel launchers (plain data; pointers are device addresses).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

struct TensorArg {
    const void* ptr;
    int64_t sb, sh, st;
};

// A piece has N chunks of 64 tokens, grouped into segments of m chunks (the
// last one may be shorter).  Per-segment matrices are fp32 [d_v][d_k] in a
// store laid out [B][H][nseg][d_v][d_k]; pointers are already offset to the
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

struct BwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N, m;
    TensorArg q, k, v, dO, decay, dq, dk_, dv_;
    int decay_kind;
    const void* states;
    int64_t st_nseg;
    const void* ghat;
    int64_t g_nseg;
};

hipError_t launch_state_scan(const ScanLaunch& s, hipStream_t stream);
hipError_t launch_fwd_intra(const FwdIntraLaunch& s, hipStream_t stream);
hipError_t launch_bwd_intra(const BwdIntraLaunch& s, hipStream_t stream);

}  // namespace linrec
