// delta.hip -- gfx950 kernels of the gated delta-rule recurrence, forward.
//
// Per (b,h), row vectors q_t, k_t (d_k), v_t (d_v), gate a_t, write strength
// beta_t, and a d_k x d_v state:
//
//     S_t = a_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,   o_t = q_t S_t
//
// the recurrence of the Gated DeltaNet models StateFlow trains (the gptget
// summary, "Experimental design"; the pages name the model without writing
// it out), in the layer's d_k x d_v state orientation.
//
// Chunkwise form (C = 64 tokens, chunk-local cumulative log-decay lam_i,
// gamma_i = exp(lam_i), D_ij = gamma_i / gamma_j for j <= i, S_0 the state
// entering the chunk).  Reading the recurrence as S_t = a_t S_{t-1} + k_t^T
// u_t with u_t = beta_t (v_t - a_t k_t S_{t-1}), and unrolling a_t S_{t-1}
// inside the chunk, the new values U solve a unit lower-triangular system:
//
//     (I + A) U = diag(beta) (V - diag(gamma) K S_0),
//     A_ij = beta_i (gamma_i / gamma_j) k_i . k_j   for j < i, else 0,
//
// so with T = (I + A)^{-1}, W_v = T diag(beta) V and W_k = T diag(beta gamma) K:
//
//     U   = W_v - W_k S_0
//     O   = diag(gamma) Q S_0 + [(Q K^T) .* D] U
//     S_C = gamma_C S_0 + (K .* gamma_C / gamma)^T U.
//
// T, W_v and W_k depend on the chunk's own inputs only: delta_prep_kernel
// forms them for every chunk in parallel.  The state transition is affine
// with a d_k x d_k matrix, gamma_C I - K~^T W_k, so it is carried serially:
// delta_scan_kernel walks the piece's chunks for one (b, h) and one block of
// 16 state columns (the columns never mix).  Every product of two computed
// operands (W_k S, P U, K~^T U, S against Q) runs on bf16 MFMA with both
// operands as hi + lo pairs; the state is carried in fp32.
#include "device.hpp"
#include "launch.hpp"

namespace linrec {

// ---------------------------------------------------------------------------
// Per chunk: T = (I + A)^{-1}, then W_v, W_k (fp32, [B][H][T][d]).
// Workgroup = (chunk, h, b), 4 waves.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void delta_prep_kernel(Act<const T> K, Act<const T> V,
                                                         Act<const float> beta, DecayArg dec,
                                                         Act<float> Wk, Act<float> Wv, int H)
{
    constexpr int NT = 256, NW = 4;
    constexpr int PAD = Pad<T>::value;
    constexpr int KP = DK + PAD, VP = DV + PAD;
    constexpr int AP = CHUNK + 4;            // fp32 pitch of A and T
    __shared__ __align__(16) T Ks[CHUNK * KP];
    __shared__ __align__(16) T Vs[CHUNK * VP];
    __shared__ __align__(16) float As[CHUNK * AP];
    __shared__ __align__(16) float Ts[CHUNK * AP];
    __shared__ __align__(16) float tab[TAB_SIZE];
    __shared__ float bet[CHUNK];

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t tok0 = (int64_t)n * CHUNK;
    {
        ChunkRegs<T, DK, NT> rk;
        ChunkRegs<T, DV, NT> rv;
        chunk_load(rk, K.head(b, h) + tok0 * K.st, K.st);
        chunk_load(rv, V.head(b, h) + tok0 * V.st, V.st);
        chunk_store(rk, Ks, KP);
        chunk_store(rv, Vs, VP);
    }
    if (w == 0) {
        decay_tables(dec, decay_raw(dec, b, h, tok0), tab);
        bet[l] = beta.ptr[b * beta.sb + h * beta.sh + (tok0 + l) * beta.st];
    }
    __syncthreads();

    // A: strictly lower part of beta_i exp(lam_i - lam_j) (k_i . k_j)
    for (int tile = w; tile < 16; tile += NW) {
        const int ib = tile >> 2, jb = tile & 3;
        floatx4 acc = zero4();
        if (jb <= ib) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mma(frag_rows(Ks, KP, 16 * ib, 32 * ks), frag_rows(Ks, KP, 16 * jb, 32 * ks), acc);
        }
        const int j = 16 * jb + t;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * g + r;
            As[i * AP + j] = j < i ? bet[i] * __expf(tab[TAB_LAM + i] - tab[TAB_LAM + j]) * acc[r] : 0.f;
        }
    }
    __syncthreads();

    // T = (I + A)^{-1} by forward substitution, one column per lane of wave 0:
    // x_i = [i == j] - sum_{m < i} A_im x_m  (x_m = 0 for m < j)
    if (w == 0) {
        float x[CHUNK];
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) {
            float acc = i == l ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m)
                acc -= As[i * AP + m] * x[m];
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < CHUNK; ++i)
            Ts[i * AP + l] = x[i];
    }
    __syncthreads();

    // W^T[c][i] = sum_j X[j][c] (T[i][j] beta_j [gamma_j]) with X = V (W_v) or
    // K (W_k); transposed tiles so each lane stores four consecutive features
    constexpr int JV = 4 * (DV / 16), JOBS = JV + 4 * (DK / 16);
    for (int job = w; job < JOBS; job += NW) {
        const bool isk = job >= JV;
        const int jj = isk ? job - JV : job, ib = jj & 3, cb = jj >> 2;
        floatx4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < CHUNK / 32; ++ks) {
            float x[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int j = 32 * ks + 8 * g + r;
                x[r] = Ts[(16 * ib + t) * AP + j] * bet[j] * (isk ? tab[TAB_G + j] : 1.f);
            }
            const Split<T> top = split8<T>(x);
            acc = mma(isk ? frag_cols(Ks, KP, 16 * cb, 32 * ks) : frag_cols(Vs, VP, 16 * cb, 32 * ks), top,
                      acc);
        }
        Act<float>& W = isk ? Wk : Wv;
        store_tile_t<float>(W.head(b, h) + tok0 * W.st, W.st, 16 * ib, 16 * cb, acc);
    }
}

// ---------------------------------------------------------------------------
// Serial walk over a piece's chunks for one (b, h) and state columns
// [16 cb, 16 cb + 16).  4 waves; wave w carries state row blocks
// FPW w .. FPW w + FPW - 1 (fp32 result tiles) and computes the chunk's rows
// [16 w, 16 w + 16) of U and O.  Per chunk:
//   P = (Q K^T) .* D                      (fp32 tiles in LDS)
//   U = W_v - W_k S_0                      (rows of this wave)
//   O^T = gamma .* (S_0^T Q^T) + U^T P^T   (stored transposed: 4 features a lane)
//   S <- gamma_C S + (K .* gamma_C/gamma)^T U
// ---------------------------------------------------------------------------
template <typename T, typename OT, int DK, int DV>
__global__ __launch_bounds__(256) void delta_scan_kernel(Act<const T> Q, Act<const T> K,
                                                         Act<const float> Wk, Act<const float> Wv,
                                                         DecayArg dec, const float* S_in,
                                                         float* S_out, Act<OT> O, int H,
                                                         int N)
{
    constexpr int NT = 256, NW = 4, NFB = DK / 16, FPW = NFB / NW;
    static_assert(FPW >= 1 && FPW * NW == NFB, "d_k must be 64 or 128");
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD;
    constexpr int WP = DK + 4, CP = 16 + 4, PP = CHUNK + 4;   // fp32 pitches
    __shared__ __align__(16) T Qs[CHUNK * QP];
    __shared__ __align__(16) T Ks[CHUNK * QP];
    __shared__ __align__(16) float Wks[CHUNK * WP];
    __shared__ __align__(16) float Wvs[CHUNK * CP];
    __shared__ __align__(16) float Ps[CHUNK * PP];
    __shared__ __align__(16) float Ss[DK * CP];
    __shared__ __align__(16) float Us[CHUNK * CP];
    __shared__ __align__(16) float tab[TAB_SIZE];

    const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;
    const int cbase = 16 * cb;

    floatx4 S[FPW];   // S[16 fb + 4g + r][cbase + t], fb = FPW w + q
#pragma unroll
    for (int q = 0; q < FPW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[q][r] = S_in ? S_in[bh * DK * DV + (int64_t)(16 * (FPW * w + q) + 4 * g + r) * DV + cbase + t]
                           : 0.f;

    const T* qh = Q.head(b, h);
    const T* kh = K.head(b, h);
    const float* wkh = Wk.head(b, h);
    const float* wvh = Wv.head(b, h);
    for (int n = 0; n < N; ++n) {
        const int64_t tok0 = (int64_t)n * CHUNK;
        {
            ChunkRegs<T, DK, NT> rq, rk;
            chunk_load(rq, qh + tok0 * Q.st, Q.st);
            chunk_load(rk, kh + tok0 * K.st, K.st);
            chunk_store(rq, Qs, QP);
            chunk_store(rk, Ks, QP);
        }
        for (int idx = threadIdx.x; idx < CHUNK * DK / 4; idx += NT) {
            const int row = idx / (DK / 4), col = 4 * (idx % (DK / 4));
            *reinterpret_cast<floatx4*>(Wks + row * WP + col) =
                *reinterpret_cast<const floatx4*>(wkh + (tok0 + row) * Wk.st + col);
        }
        {
            const int row = threadIdx.x >> 2, col = 4 * (threadIdx.x & 3);
            *reinterpret_cast<floatx4*>(Wvs + row * CP + col) =
                *reinterpret_cast<const floatx4*>(wvh + (tok0 + row) * Wv.st + cbase + col);
        }
        if (w == 0)
            decay_tables(dec, decay_raw(dec, b, h, tok0), tab);
#pragma unroll
        for (int q = 0; q < FPW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Ss[(16 * (FPW * w + q) + 4 * g + r) * CP + t] = S[q][r];
        __syncthreads();

        // P = (Q K^T) .* D, causal, fp32
        const bool fac = decay_factored(tab);
        for (int tile = w; tile < 16; tile += NW) {
            const int ib = tile >> 2, jb = tile & 3;
            floatx4 acc = zero4();
            if (jb <= ib) {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks)
                    acc = mma(frag_rows(Qs, QP, 16 * ib, 32 * ks), frag_rows(Ks, QP, 16 * jb, 32 * ks), acc);
                acc = decay_mask<true>(acc, tab, 16 * ib, 16 * jb, fac);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Ps[(16 * ib + 4 * g + r) * PP + 16 * jb + t] = acc[r];
        }
        // U rows [16 w, 16 w + 16) = W_v - W_k S_0
        {
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mma(split_rows_f32<T>(Wks, WP, 16 * w, 32 * ks), split_cols_f32<T>(Ss, CP, 0, 32 * ks),
                          acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * g + r;
                Us[i * CP + t] = Wvs[i * CP + t] - acc[r];
            }
        }
        __syncthreads();

        // O^T[c][i] for tokens [16 w, 16 w + 16)
        {
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mma(split_cols_f32<T>(Ss, CP, 0, 32 * ks), frag_rows(Qs, QP, 16 * w, 32 * ks), acc);
            acc *= tab[TAB_G + 16 * w + t];
#pragma unroll
            for (int js = 0; js <= w / 2; ++js)
                acc = mma(split_cols_f32<T>(Us, CP, 0, 32 * js), split_rows_f32<T>(Ps, PP, 16 * w, 32 * js), acc);
            store_tile_t<OT>(O.head(b, h) + tok0 * O.st, O.st, 16 * w, cbase, acc);
        }
        // S <- gamma_C S + K~^T U for this wave's row blocks
        {
            const float gC = tab[TAB_G + CHUNK - 1];
            float kf[2][8];
            slot_factors(tab + TAB_F, kf);
#pragma unroll
            for (int q = 0; q < FPW; ++q) {
                const int fb = FPW * w + q;
                S[q] *= gC;
#pragma unroll
                for (int ks = 0; ks < CHUNK / 32; ++ks)
                    S[q] = mma(split_scaled<T>(frag_cols(Ks, QP, 16 * fb, 32 * ks), kf[ks]),
                               split_cols_f32<T>(Us, CP, 0, 32 * ks), S[q]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < FPW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S_out[bh * DK * DV + (int64_t)(16 * (FPW * w + q) + 4 * g + r) * DV + cbase + t] = S[q][r];
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
namespace {

template <typename T>
Act<const T> dact(const TensorArg& a) { return Act<const T>{(const T*)a.ptr, a.sb, a.sh, a.st}; }

template <typename T, typename OT, int DK, int DV>
hipError_t delta_fwd_impl(const DeltaFwdLaunch& s, hipStream_t stream)
{
    const DecayArg dec{(const float*)s.decay.ptr, s.decay.sb, s.decay.sh, s.decay.st, s.decay_kind};
    const Act<float> wk{s.wk, (int64_t)s.H * s.T * DK, (int64_t)s.T * DK, DK};
    const Act<float> wv{s.wv, (int64_t)s.H * s.T * DV, (int64_t)s.T * DV, DV};
    const int N = s.T / CHUNK;
    hipLaunchKernelGGL((delta_prep_kernel<T, DK, DV>), dim3(N, s.H, s.B), dim3(256), 0, stream,
                       dact<T>(s.k), dact<T>(s.v), dact<float>(s.beta), dec, wk, wv, s.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((delta_scan_kernel<T, OT, DK, DV>), dim3(DV / 16, s.H, s.B), dim3(256), 0,
                       stream, dact<T>(s.q), dact<T>(s.k), Act<const float>{wk.ptr, wk.sb, wk.sh, wk.st},
                       Act<const float>{wv.ptr, wv.sb, wv.sh, wv.st}, dec, s.S_in, s.S_out,
                       Act<OT>{(OT*)s.o.ptr, s.o.sb, s.o.sh, s.o.st}, s.H, N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_delta_fwd(const DeltaFwdLaunch& s, hipStream_t stream)
{
    if (s.dtype == 0 && s.dk == 128 && s.dv == 128)
        return s.out_dtype == 0 ? delta_fwd_impl<bf16, bf16, 128, 128>(s, stream)
                                : delta_fwd_impl<bf16, float, 128, 128>(s, stream);
    if (s.dtype == 0 && s.dk == 64 && s.dv == 64)
        return s.out_dtype == 0 ? delta_fwd_impl<bf16, bf16, 64, 64>(s, stream)
                                : delta_fwd_impl<bf16, float, 64, 64>(s, stream);
    if (s.dtype == 1 && s.dk == 64 && s.dv == 64 && s.out_dtype == 1)
        return delta_fwd_impl<float, float, 64, 64>(s, stream);
    return hipErrorInvalidValue;
}

}  // namespace linrec
