// kernels.hip -- gfx950 kernels of the chunkwise linear recurrence.
//
// Per (b,h) and chunk n of C = 64 tokens, with chunk-local cumulative
// log-decay lam_i (token i inclusive), gamma_i = exp(lam_i), gamma_C =
// exp(lam_63) and D_ij = exp(lam_i - lam_j) for j <= i (else 0):
//
//   state scan (forward):  store S_{n-1};  S_n = gamma_C S_{n-1} + (K .* gamma_C/gamma)^T V
//   intra (forward):       O = [(Q K^T) .* D] V + (Q .* gamma) S_{n-1}
//   state scan (reverse):  store G_n;  G_{n-1} = gamma_C G_n + (Q .* gamma)^T dO
//   intra (backward):      dQ = [(dO V^T) .* D] K + (dO S_{n-1}^T) .* gamma
//                          dK = [(V dO^T) .* D^T] Q + (V G_n^T) .* gamma_C/gamma
//                          dV = [(K Q^T) .* D^T] dO + (K .* gamma_C/gamma) G_n
//
// These are the chunk algebra of the token recurrence S_t = a_t S_{t-1} +
// k_t^T v_t, o_t = q_t S_t: the right-product form of linear attention
// (Linear Attention Sequence Parallelism, abstract) with a linear recurrence
// inside each chunk and chunks joined by boundary states (StateFlow, the
// gptget summary's method details).  G_n is the gradient of the loss with
// respect to the state leaving chunk n.
//
// Stored per-chunk matrices (S_{n-1} and G_n) are kept transposed, [d_v][d_k]
// with d_k contiguous, in the activation dtype: [B][H][nchunks][d_v][d_k].
#include "device.hpp"
#include "launch.hpp"

namespace linrec {

// ---------------------------------------------------------------------------
// State scan.  One wave per (b, h, 32x32 tile of the d_k x d_v state); the
// tile is carried in fp32 MFMA accumulators across the chunks of the piece
// (in order for the forward, reversed for the backward).  Per chunk: stage
// the X tile (K or Q, rows scaled by the decay factor, split hi + lo) and the
// Y tile (V or dO, exact) through LDS, store the carried tile (fp32), then
// carry = gamma_C carry + X^T Y.
//
// The carry is the only serial dependency, so the kernel is a software
// pipeline: the global loads of chunk it+2 are in flight while chunk it is
// staged and multiplied (two register buffers, 16-byte loads).
// ---------------------------------------------------------------------------
template <typename T>
struct ScanTile {
    static constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte vector
    static constexpr int NV = 32 / VEC;            // vectors per lane per 64x32 tile
    uint4 x[NV], y[NV];
};

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
    typedef bf16x8 type;
};
template <>
struct Vec16<float> {
    typedef floatx4 type;
};

template <typename T>
__device__ __forceinline__ void scan_load(ScanTile<T>& r, const T* xh, const T* yh, int64_t xst,
                                          int64_t yst, int64_t tok0)
{
    constexpr int VEC = ScanTile<T>::VEC, PR = 32 / VEC;
    const int l = lane_id();
#pragma unroll
    for (int p = 0; p < ScanTile<T>::NV; ++p) {
        const int idx = l + 64 * p, row = idx / PR, col = (idx % PR) * VEC;
        r.x[p] = *reinterpret_cast<const uint4*>(xh + (tok0 + row) * xst + col);
        r.y[p] = *reinterpret_cast<const uint4*>(yh + (tok0 + row) * yst + col);
    }
}

template <typename T, int DK, int DV, bool REVERSE>
__global__ __launch_bounds__(64) void state_scan_kernel(
    Act<const T> X, Act<const T> Y, DecayArg dec, const float* __restrict__ carry_in,
    float* __restrict__ carry_out, float* __restrict__ store, int64_t store_nchunks, int H, int N)
{
    constexpr int TF = 32, TC = 32;
    constexpr int PAD = Pad<T>::value;
    constexpr int XP = TF + PAD, YP = TC + PAD;
    constexpr int NTC = DV / TC;
    constexpr int VEC = ScanTile<T>::VEC, NV = ScanTile<T>::NV, PR = 32 / VEC;
    __shared__ __align__(16) T Xs[2][CHUNK * XP];
    __shared__ __align__(16) T Ys[CHUNK * YP];

    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int f0 = (tile / NTC) * TF, c0 = (tile % NTC) * TC;
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;

    // carry[fb][cb] holds S[f0 + 16fb + 4g + r][c0 + 16cb + t]
    floatx4 carry[2][2];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                carry[fb][cb][r] = carry_in
                    ? carry_in[(bh * DK + f0 + 16 * fb + 4 * g + r) * DV + c0 + 16 * cb + t]
                    : 0.f;

    const T* xh = X.head(b, h) + f0;
    const T* yh = Y.head(b, h) + c0;
    float* sh = store + bh * store_nchunks * (int64_t)(DV * DK);

    // row scale of the X vectors this lane stages, and the chunk decay; for a
    // per-head (or absent) decay they are the same for every chunk
    const bool const_decay = dec.kind != 2;
    float lm = chunk_log_cumsum(dec, b, h, 0);
    float lamC = __shfl(lm, 63, 64);
    float xs[NV];
#pragma unroll
    for (int p = 0; p < NV; ++p) {
        const float lr = __shfl(lm, (l + 64 * p) / PR, 64);
        xs[p] = REVERSE ? __expf(lr) : __expf(lamC - lr);
    }

    typedef typename Vec16<T>::type V;
    const auto chunk_of = [&](int it) { return REVERSE ? N - 1 - it : it; };

    // one pipeline stage: stage chunk `it` from `cur`, refill `cur` with chunk
    // it+2, store the carried tile and advance the carry
    const auto stage = [&](int it, ScanTile<T>& cur) {
        const int n = chunk_of(it);
        const int64_t tok0 = (int64_t)n * CHUNK;
        if (!const_decay) {
            lm = chunk_log_cumsum(dec, b, h, tok0);
            lamC = __shfl(lm, 63, 64);
#pragma unroll
            for (int p = 0; p < NV; ++p) {
                const float lr = __shfl(lm, (l + 64 * p) / PR, 64);
                xs[p] = REVERSE ? __expf(lr) : __expf(lamC - lr);
            }
        }
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = l + 64 * p, row = idx / PR, col = (idx % PR) * VEC;
            const V xv = __builtin_bit_cast(V, cur.x[p]);
            V hi, lo;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float v = (float)xv[e] * xs[p];
                hi[e] = (T)v;
                lo[e] = (T)(v - (float)hi[e]);
            }
            *reinterpret_cast<V*>(&Xs[0][row * XP + col]) = hi;
            if constexpr (sizeof(T) == 2)
                *reinterpret_cast<V*>(&Xs[1][row * XP + col]) = lo;
            *reinterpret_cast<uint4*>(&Ys[row * YP + col]) = cur.y[p];
        }
        if (it + 2 < N)
            scan_load(cur, xh, yh, X.st, Y.st, (int64_t)chunk_of(it + 2) * CHUNK);
        __syncthreads();

        // store the carried tile, transposed ([c][f], f contiguous), fp32
        float* sn = sh + (int64_t)n * (DV * DK);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                *reinterpret_cast<float4*>(sn + (int64_t)(c0 + 16 * cb + t) * DK + f0 + 16 * fb + 4 * g) =
                    float4{carry[fb][cb][0], carry[fb][cb][1], carry[fb][cb][2], carry[fb][cb][3]};

        // delta = X^T Y over the chunk's 64 tokens
        floatx4 dlt[2][2];
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                dlt[fb][cb] = zero4();
#pragma unroll
        for (int ks = 0; ks < CHUNK / 32; ++ks) {
            Split<T> a[2];
            Frag<T> bb[2];
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
                a[fb] = frag_cols_split(Xs[0], Xs[1], XP, 16 * fb, 32 * ks);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                bb[cb] = frag_cols(Ys, YP, 16 * cb, 32 * ks);
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    dlt[fb][cb] = mma(a[fb], bb[cb], dlt[fb][cb]);
        }
        const float gC = __expf(lamC);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                carry[fb][cb] = gC * carry[fb][cb] + dlt[fb][cb];
        __syncthreads();
    };

    ScanTile<T> buf0, buf1;
    scan_load(buf0, xh, yh, X.st, Y.st, (int64_t)chunk_of(0) * CHUNK);
    if (N > 1)
        scan_load(buf1, xh, yh, X.st, Y.st, (int64_t)chunk_of(1) * CHUNK);
    for (int it = 0; it < N; it += 2) {
        stage(it, buf0);
        if (it + 1 < N)
            stage(it + 1, buf1);
    }

#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                carry_out[(bh * DK + f0 + 16 * fb + 4 * g + r) * DV + c0 + 16 * cb + t] =
                    carry[fb][cb][r];
}

// ---------------------------------------------------------------------------
// Forward intra-chunk kernel.  One workgroup (4 waves) per (b, h, chunk).
// Wave w builds row block w of P = (Q K^T) .* D (split hi + lo) into LDS;
// then wave w owns output columns [w d_v/4, (w+1) d_v/4) of all 64 rows:
//   O = P V + gamma .* (Q S_{n-1})
// with the row scale gamma_i applied to the fp32 product.
// ---------------------------------------------------------------------------
template <typename T, typename OT, int DK, int DV>
__global__ __launch_bounds__(256) void fwd_intra_kernel(
    Act<const T> Q, Act<const T> K, Act<const T> V, DecayArg dec,
    const float* __restrict__ states, int64_t st_nchunks, Act<OT> O, int H)
{
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD, VP = DV + PAD, PP = CHUNK + PAD;
    __shared__ __align__(16) T Qs[CHUNK * QP];
    __shared__ __align__(16) T Ks[CHUNK * QP];
    __shared__ __align__(16) T Vs[CHUNK * VP];
    __shared__ __align__(16) T Ps[2][CHUNK * PP];
    __shared__ float lam[CHUNK];

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t tok0 = (int64_t)n * CHUNK;

    stage_rows<T, CHUNK, DK, 256>(Qs, QP, Q.head(b, h) + tok0 * Q.st, Q.st);
    stage_rows<T, CHUNK, DK, 256>(Ks, QP, K.head(b, h) + tok0 * K.st, K.st);
    stage_rows<T, CHUNK, DV, 256>(Vs, VP, V.head(b, h) + tok0 * V.st, V.st);
    if (w == 0)
        lam[l] = chunk_log_cumsum(dec, b, h, tok0);
    __syncthreads();

    // P row block w: P[i][j] = (q_i . k_j) exp(lam_i - lam_j) for j <= i
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        floatx4 acc = zero4();
        if (jb <= w) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mma(frag_rows(Qs, QP, 16 * w, 32 * ks), frag_rows(Ks, QP, 16 * jb, 32 * ks), acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * g + r, j = 16 * jb + t;
            const float val = (j <= i) ? acc[r] * __expf(lam[i] - lam[j]) : 0.f;
            put_split(Ps[0], Ps[1], i * PP + j, val);
        }
    }
    __syncthreads();

    constexpr int CPW = DV / 4;
    const float* St = states + ((int64_t)(b * H + h) * st_nchunks + n) * (int64_t)(DV * DK);
    OT* oh = O.head(b, h) + tok0 * O.st;
#pragma unroll
    for (int cbl = 0; cbl < CPW / 16; ++cbl) {
        const int cbase = w * CPW + 16 * cbl;
        Split<T> sf[DK / 32];      // B = S[f][c], k = f
#pragma unroll
        for (int fs = 0; fs < DK / 32; ++fs)
            sf[fs] = gfrag_rows_split<T>(St, DK, cbase, 32 * fs);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            floatx4 intra = zero4(), inter = zero4();
#pragma unroll
            for (int js = 0; js <= ib / 2; ++js)
                intra = mma(frag_rows_split(Ps[0], Ps[1], PP, 16 * ib, 32 * js),
                            frag_cols(Vs, VP, cbase, 32 * js), intra);
#pragma unroll
            for (int fs = 0; fs < DK / 32; ++fs)
                inter = mma(frag_rows(Qs, QP, 16 * ib, 32 * fs), sf[fs], inter);
            floatx4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[r] = intra[r] + __expf(lam[16 * ib + 4 * g + r]) * inter[r];
            store_tile<OT>(oh, O.st, 16 * ib, cbase, out);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward per-chunk kernel.  One workgroup (4 waves) per (b, h, chunk).
// Builds P = (Q K^T) .* D and A = (dO V^T) .* D in LDS (split hi + lo; wave
// w: row block w), then each wave owns a quarter of the columns of dQ, dK
// and dV.  The stored fp32 S_{n-1} and G_n are read as split fragments from
// global memory; decay factors scale the fp32 products' rows.
// ---------------------------------------------------------------------------
template <typename T, typename OT, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_intra_kernel(
    Act<const T> Q, Act<const T> K, Act<const T> V, Act<const T> dO, DecayArg dec,
    const float* __restrict__ states, int64_t st_nchunks, const float* __restrict__ ghat,
    int64_t g_nchunks, Act<OT> dQ, Act<OT> dK, Act<OT> dV, int H)
{
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD, VP = DV + PAD, PP = CHUNK + PAD;
    __shared__ __align__(16) T Qs[CHUNK * QP];
    __shared__ __align__(16) T Ks[CHUNK * QP];
    __shared__ __align__(16) T Vs[CHUNK * VP];
    __shared__ __align__(16) T dOs[CHUNK * VP];
    __shared__ __align__(16) T Ps[2][CHUNK * PP];
    __shared__ __align__(16) T As[2][CHUNK * PP];
    __shared__ float lam[CHUNK];

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t tok0 = (int64_t)n * CHUNK;
    const int64_t bh = (int64_t)b * H + h;

    stage_rows<T, CHUNK, DK, 256>(Qs, QP, Q.head(b, h) + tok0 * Q.st, Q.st);
    stage_rows<T, CHUNK, DK, 256>(Ks, QP, K.head(b, h) + tok0 * K.st, K.st);
    stage_rows<T, CHUNK, DV, 256>(Vs, VP, V.head(b, h) + tok0 * V.st, V.st);
    stage_rows<T, CHUNK, DV, 256>(dOs, VP, dO.head(b, h) + tok0 * dO.st, dO.st);
    if (w == 0)
        lam[l] = chunk_log_cumsum(dec, b, h, tok0);
    __syncthreads();
    const float lamC = lam[CHUNK - 1];
    const float* St = states + (bh * st_nchunks + n) * (int64_t)(DV * DK);   // S_{n-1}^T
    const float* Gt = ghat + (bh * g_nchunks + n) * (int64_t)(DV * DK);      // G_n^T

    // P and A, row block w
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        floatx4 accp = zero4(), acca = zero4();
        if (jb <= w) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                accp = mma(frag_rows(Qs, QP, 16 * w, 32 * ks), frag_rows(Ks, QP, 16 * jb, 32 * ks), accp);
#pragma unroll
            for (int ks = 0; ks < DV / 32; ++ks)
                acca = mma(frag_rows(dOs, VP, 16 * w, 32 * ks), frag_rows(Vs, VP, 16 * jb, 32 * ks), acca);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * g + r, j = 16 * jb + t;
            const float d = (j <= i) ? __expf(lam[i] - lam[j]) : 0.f;
            put_split(Ps[0], Ps[1], i * PP + j, accp[r] * d);
            put_split(As[0], As[1], i * PP + j, acca[r] * d);
        }
    }
    __syncthreads();

    // dQ = A K + gamma .* (dO S_{n-1}^T) ; wave w owns d_k columns [w DK/4, (w+1) DK/4)
    {
        OT* out = dQ.head(b, h) + tok0 * dQ.st;
#pragma unroll
        for (int fbl = 0; fbl < DK / 64; ++fbl) {
            const int fbase = w * (DK / 4) + 16 * fbl;
            Split<T> sf[DV / 32];  // B = S^T[c][f], k = c
#pragma unroll
            for (int cs = 0; cs < DV / 32; ++cs)
                sf[cs] = gfrag_cols_split<T>(St, DK, fbase, 32 * cs);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                floatx4 intra = zero4(), inter = zero4();
#pragma unroll
                for (int js = 0; js <= ib / 2; ++js)
                    intra = mma(frag_rows_split(As[0], As[1], PP, 16 * ib, 32 * js),
                                frag_cols(Ks, QP, fbase, 32 * js), intra);
#pragma unroll
                for (int cs = 0; cs < DV / 32; ++cs)
                    inter = mma(frag_rows(dOs, VP, 16 * ib, 32 * cs), sf[cs], inter);
                floatx4 res;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    res[r] = intra[r] + __expf(lam[16 * ib + 4 * g + r]) * inter[r];
                store_tile<OT>(out, dQ.st, 16 * ib, fbase, res);
            }
        }
    }

    // dK = A^T Q + (gamma_C / gamma) .* (V G_n^T) ; wave w owns d_k columns
    {
        OT* out = dK.head(b, h) + tok0 * dK.st;
#pragma unroll
        for (int fbl = 0; fbl < DK / 64; ++fbl) {
            const int fbase = w * (DK / 4) + 16 * fbl;
            Split<T> gf[DV / 32];  // B = G^T[c][f], k = c
#pragma unroll
            for (int cs = 0; cs < DV / 32; ++cs)
                gf[cs] = gfrag_cols_split<T>(Gt, DK, fbase, 32 * cs);
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                floatx4 intra = zero4(), inter = zero4();
#pragma unroll
                for (int is = jb / 2; is < 2; ++is)
                    intra = mma(frag_cols_split(As[0], As[1], PP, 16 * jb, 32 * is),
                                frag_cols(Qs, QP, fbase, 32 * is), intra);
#pragma unroll
                for (int cs = 0; cs < DV / 32; ++cs)
                    inter = mma(frag_rows(Vs, VP, 16 * jb, 32 * cs), gf[cs], inter);
                floatx4 res;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    res[r] = intra[r] + __expf(lamC - lam[16 * jb + 4 * g + r]) * inter[r];
                store_tile<OT>(out, dK.st, 16 * jb, fbase, res);
            }
        }
    }
    // dV = P^T dO + (gamma_C / gamma) .* (K G_n) ; wave w owns d_v columns
    {
        OT* out = dV.head(b, h) + tok0 * dV.st;
#pragma unroll
        for (int cbl = 0; cbl < DV / 64; ++cbl) {
            const int cbase = w * (DV / 4) + 16 * cbl;
            Split<T> gf[DK / 32];  // B = G[f][c], k = f
#pragma unroll
            for (int fs = 0; fs < DK / 32; ++fs)
                gf[fs] = gfrag_rows_split<T>(Gt, DK, cbase, 32 * fs);
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                floatx4 intra = zero4(), inter = zero4();
#pragma unroll
                for (int is = jb / 2; is < 2; ++is)
                    intra = mma(frag_cols_split(Ps[0], Ps[1], PP, 16 * jb, 32 * is),
                                frag_cols(dOs, VP, cbase, 32 * is), intra);
#pragma unroll
                for (int fs = 0; fs < DK / 32; ++fs)
                    inter = mma(frag_rows(Ks, QP, 16 * jb, 32 * fs), gf[fs], inter);
                floatx4 res;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    res[r] = intra[r] + __expf(lamC - lam[16 * jb + 4 * g + r]) * inter[r];
                store_tile<OT>(out, dV.st, 16 * jb, cbase, res);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers: dispatch (dtype, d_k, d_v) to a template instance.
// ---------------------------------------------------------------------------
namespace {

template <typename T>
Act<const T> cact(const TensorArg& a) { return Act<const T>{(const T*)a.ptr, a.sb, a.sh, a.st}; }
template <typename T>
Act<T> mact(const TensorArg& a) { return Act<T>{(T*)a.ptr, a.sb, a.sh, a.st}; }

DecayArg decay_arg(const TensorArg& d, int kind)
{
    return DecayArg{(const float*)d.ptr, d.sb, d.sh, d.st, kind};
}

template <typename T, typename OT, int DK, int DV>
hipError_t scan_impl(const ScanLaunch& s, hipStream_t stream)
{
    const dim3 grid((DK / 32) * (DV / 32), s.H, s.B), block(64);
    if (s.reverse)
        hipLaunchKernelGGL((state_scan_kernel<T, DK, DV, true>), grid, block, 0, stream,
                           cact<T>(s.x), cact<T>(s.y), decay_arg(s.decay, s.decay_kind),
                           s.carry_in, s.carry_out, (float*)s.store, s.store_nchunks, s.H, s.N);
    else
        hipLaunchKernelGGL((state_scan_kernel<T, DK, DV, false>), grid, block, 0, stream,
                           cact<T>(s.x), cact<T>(s.y), decay_arg(s.decay, s.decay_kind),
                           s.carry_in, s.carry_out, (float*)s.store, s.store_nchunks, s.H, s.N);
    return hipGetLastError();
}

template <typename T, typename OT, int DK, int DV>
hipError_t fwd_intra_impl(const FwdIntraLaunch& s, hipStream_t stream)
{
    const dim3 grid(s.N, s.H, s.B), block(256);
    hipLaunchKernelGGL((fwd_intra_kernel<T, OT, DK, DV>), grid, block, 0, stream,
                       cact<T>(s.q), cact<T>(s.k), cact<T>(s.v), decay_arg(s.decay, s.decay_kind),
                       (const float*)s.states, s.st_nchunks, mact<OT>(s.o), s.H);
    return hipGetLastError();
}

template <typename T, typename OT, int DK, int DV>
hipError_t bwd_intra_impl(const BwdIntraLaunch& s, hipStream_t stream)
{
    const dim3 grid(s.N, s.H, s.B), block(256);
    hipLaunchKernelGGL((bwd_intra_kernel<T, OT, DK, DV>), grid, block, 0, stream,
                       cact<T>(s.q), cact<T>(s.k), cact<T>(s.v), cact<T>(s.dO),
                       decay_arg(s.decay, s.decay_kind), (const float*)s.states, s.st_nchunks,
                       (const float*)s.ghat, s.g_nchunks, mact<OT>(s.dq), mact<OT>(s.dk_),
                       mact<OT>(s.dv_), s.H);
    return hipGetLastError();
}

}  // namespace

#define LINREC_DISPATCH_D(IMPL, T, OT, S, STREAM)                                       \
    do {                                                                               \
        if ((S).dk == 128 && (S).dv == 128) return IMPL<T, OT, 128, 128>(S, STREAM);   \
        if ((S).dk == 64 && (S).dv == 64) return IMPL<T, OT, 64, 64>(S, STREAM);       \
        if ((S).dk == 64 && (S).dv == 128) return IMPL<T, OT, 64, 128>(S, STREAM);     \
        if ((S).dk == 128 && (S).dv == 64) return IMPL<T, OT, 128, 64>(S, STREAM);     \
    } while (0)

// (activation dtype, output dtype, d_k, d_v) -> template instance.  fp32
// activations exist for d_k = d_v = 64 only.
#define LINREC_DISPATCH(IMPL, S, STREAM)                                               \
    do {                                                                               \
        if ((S).dtype == 0 && (S).out_dtype == 0) LINREC_DISPATCH_D(IMPL, bf16, bf16, S, STREAM); \
        if ((S).dtype == 0 && (S).out_dtype == 1) LINREC_DISPATCH_D(IMPL, bf16, float, S, STREAM); \
        if ((S).dtype == 1 && (S).out_dtype == 1 && (S).dk == 64 && (S).dv == 64)       \
            return IMPL<float, float, 64, 64>(S, STREAM);                              \
        return hipErrorInvalidValue;                                                   \
    } while (0)

hipError_t launch_state_scan(const ScanLaunch& s, hipStream_t stream)
{
    if (s.dtype == 0)
        LINREC_DISPATCH_D(scan_impl, bf16, float, s, stream);
    else if (s.dk == 64 && s.dv == 64)
        return scan_impl<float, float, 64, 64>(s, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_intra(const FwdIntraLaunch& s, hipStream_t stream)
{
    LINREC_DISPATCH(fwd_intra_impl, s, stream);
}

hipError_t launch_bwd_intra(const BwdIntraLaunch& s, hipStream_t stream)
{
    LINREC_DISPATCH(bwd_intra_impl, s, stream);
}

}  // namespace linrec
