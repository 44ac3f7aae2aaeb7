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

// One state-scan launch over N chunks of one piece.  Forward: x = K, y = V,
// carry S_in -> S_out, store = states.  Reverse: x = Q, y = dO, carry
// dS_out -> dS_in, store = per-chunk gradients.
struct ScanLaunch {
    int dtype, dk, dv, B, H, N;
    int out_dtype;           // unused by the scan; keeps one dispatch macro
    bool reverse;
    TensorArg x, y, decay;
    int decay_kind;
    const float* carry_in;   // may be NULL (zeros)
    float* carry_out;
    void* store;             // fp32, already offset to the piece's first chunk
    int64_t store_nchunks;   // chunks per (b,h) in the store
};

struct FwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N;
    TensorArg q, k, v, decay, o;
    int decay_kind;
    const void* states;
    int64_t st_nchunks;
};

struct BwdIntraLaunch {
    int dtype, out_dtype, dk, dv, B, H, N;
    TensorArg q, k, v, dO, decay, dq, dk_, dv_;
    int decay_kind;
    const void* states;
    int64_t st_nchunks;
    const void* ghat;
    int64_t g_nchunks;
};

hipError_t launch_state_scan(const ScanLaunch& s, hipStream_t stream);
hipError_t launch_fwd_intra(const FwdIntraLaunch& s, hipStream_t stream);
hipError_t launch_bwd_intra(const BwdIntraLaunch& s, hipStream_t stream);

}  // namespace linrec
