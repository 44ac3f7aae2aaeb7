// kernels.hip -- gfx950 kernels of the chunkwise linear recurrence.
//
// Per (b,h) and chunk n of C = 64 tokens, with chunk-local cumulative
// log-decay lam_i (token i inclusive), gamma_i = exp(lam_i), gamma_C =
// exp(lam_63) and D_ij = exp(lam_i - lam_j) for j <= i (else 0):
//
//   forward    O_n = gamma .* (Q_n S_{n-1}) + [(Q_n K_n^T) .* D] V_n
//              S_n = gamma_C S_{n-1} + (K_n .* gamma_C/gamma)^T V_n
//   backward   G_{n-1} = gamma_C G_n + (Q_n .* gamma)^T dO_n
//              dQ_n = gamma .* (dO_n S_{n-1}^T) + [(dO_n V_n^T) .* D] K_n
//              dK_n = gamma_C/gamma .* (V_n G_n^T) + [(V_n dO_n^T) .* D^T] Q_n
//              dV_n = gamma_C/gamma .* (K_n G_n)  + [(K_n Q_n^T) .* D^T] dO_n
//
// with G_n the gradient of the loss with respect to the state leaving chunk
// n.  This is the chunk algebra of the token recurrence S_t = a_t S_{t-1} +
// k_t^T v_t, o_t = q_t S_t: the right-product form of linear attention
// (Linear Attention Sequence Parallelism, abstract) with a linear recurrence
// inside each chunk and chunks joined by boundary states (StateFlow, the
// gptget summary's method details).
//
// Two levels.  Chunks are grouped into segments of m chunks.
//   * The state transition (a parallel segment-sum launch and a serial fold
//     launch per direction and piece) produces the state entering every
//     segment (the gradient leaving every segment in the reverse direction)
//     and the piece's boundary state.  Only those per-segment states reach
//     memory.
//   * The segment kernels (one workgroup per segment) walk the segment's
//     chunks with the state in fp32 registers, rebuilding every per-chunk
//     state on the fly; the backward walks forward for dQ (carrying S) and
//     then in reverse for dK and dV (carrying G).
// Per-segment records are fp32: the state [d_k][d_v] (the layout of S_in and
// S_out), then the segment's total log-decay, padded to 64 floats:
// [B][H][nseg][d_k * d_v + 64].
//
// Every operand these kernels compute (P, A, the decay-scaled K or Q, the
// carried states) enters the MFMA as a bf16 hi + lo pair against an exact
// bf16 activation; decay factors that depend only on an output row scale the
// fp32 product instead of an operand.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace linrec {

// Device side of SumArg.
template <typename T>
struct SumDev {
    Act<const T> X, Y;
    DecayArg dec;
    float* store;
    int64_t store_nseg;
    int N, m, nseg, tail;
};

// ---------------------------------------------------------------------------
// Shared pieces of the segment kernels.
// ---------------------------------------------------------------------------

// carry[fb][cbl] (rows f = 16fb + 4g + r, column cbase0 + 16cbl + t) <-
// gamma_C carry + X^T (Y .* yf) over the chunk: X (rows = tokens, d_k wide)
// exact, Y (rows = tokens) scaled per token by yf and split.  The per-token
// factor sits on the wave's own columns of Y, so each wave scales and splits
// only the quarter of the chunk it multiplies.
template <typename T, int DK, int NCB>
__device__ __forceinline__ void state_update(floatx4 (&carry)[DK / 16][NCB], const T* Xs, int xp,
                                             const T* Ys, int yp, int cbase0, float gC,
                                             const float (&yf)[2][8])
{
#pragma unroll
    for (int fb = 0; fb < DK / 16; ++fb)
#pragma unroll
        for (int cbl = 0; cbl < NCB; ++cbl)
            carry[fb][cbl] *= gC;
#pragma unroll
    for (int ks = 0; ks < CHUNK / 32; ++ks) {
        Split<T> y[NCB];
#pragma unroll
        for (int cbl = 0; cbl < NCB; ++cbl)
            y[cbl] = split_scaled<T>(frag_cols(Ys, yp, cbase0 + 16 * cbl, 32 * ks), yf[ks]);
#pragma unroll
        for (int fb = 0; fb < DK / 16; ++fb) {
            const Frag<T> a = frag_cols(Xs, xp, 16 * fb, 32 * ks);
#pragma unroll
            for (int cbl = 0; cbl < NCB; ++cbl)
                carry[fb][cbl] = mma(a, y[cbl], carry[fb][cbl]);
        }
    }
}

// Load a wave's columns of a stored [d_k][d_v] fp32 state into register tiles.
template <int DK, int DV, int NCB>
__device__ __forceinline__ void load_state(floatx4 (&st)[DK / 16][NCB], const float* src, int cbase0)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
#pragma unroll
    for (int fb = 0; fb < DK / 16; ++fb)
#pragma unroll
        for (int cbl = 0; cbl < NCB; ++cbl)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st[fb][cbl][r] = src[(int64_t)(16 * fb + 4 * g + r) * DV + cbase0 + 16 * cbl + t];
}

// Store a wave's register tiles of a state as [d_k][d_v] fp32.
template <int DK, int DV, int NCB>
__device__ __forceinline__ void store_state(float* dst, const floatx4 (&st)[DK / 16][NCB], int cbase0)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
#pragma unroll
    for (int fb = 0; fb < DK / 16; ++fb)
#pragma unroll
        for (int cbl = 0; cbl < NCB; ++cbl)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(int64_t)(16 * fb + 4 * g + r) * DV + cbase0 + 16 * cbl + t] = st[fb][cbl][r];
}

// Write a wave's register tiles of a state into an LDS plane pair laid out
// [c][f] (hi, lo).
template <typename T, int DK, int NCB>
__device__ __forceinline__ void put_state(T* hi, T* lo, int pitch, const floatx4 (&st)[DK / 16][NCB],
                                          int cbase0)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
#pragma unroll
    for (int fb = 0; fb < DK / 16; ++fb)
#pragma unroll
        for (int cbl = 0; cbl < NCB; ++cbl)
            put_split4(hi, lo, (cbase0 + 16 * cbl + t) * pitch + 16 * fb, st[fb][cbl]);
}

// ---------------------------------------------------------------------------
// State transition across a piece, in two launches.
//
// Segment sum (parallel over segments): workgroup = (b, h, segment), one
// wave per 16 state columns.  It folds the segment's chunks from a zero
// state with the same update the segment kernels use,
//   forward  U = gamma_C U + K^T (V .* gamma_C/gamma)      (chunks in order)
//   reverse  U = gamma_C U + Q^T (dO .* gamma)             (chunks reversed)
// and writes U and the segment's total log-decay into the segment's record.
//
// Fold (serial over segments, parallel over state elements): each thread
// walks the records in order, replacing U_s by the carried value and
// carrying  c <- exp(log Gamma_s) c + U_s;  it starts from S_in (dS_out) and
// ends with S_out (dS_in).  In the forward direction record s then holds the
// state entering segment s; in the reverse direction the gradient leaving it.
// ---------------------------------------------------------------------------
// The segment sum of segment s of head (b, h), in LDS the caller provides:
// two chunk buffers for X and for Y (pitches DK + PAD and DV + PAD) and two
// decay tables.  RAGGED: the piece's last chunk may be partial (`tail`
// tokens); otherwise every chunk is whole and the masking compiles away.
template <typename T, int DK, int DV, bool REVERSE, bool RAGGED>
__device__ __forceinline__ void seg_sum_body(Act<const T> X, Act<const T> Y, DecayArg dec,
                                             float* __restrict__ store, int64_t store_nseg, int H,
                                             int N, int tail, int m, int s, int h, int b, T* xs0,
                                             T* xs1, T* ys0, T* ys1, float* tb0, float* tb1)
{
    constexpr int NW = DV / 16, NT = NW * 64;
    constexpr int PAD = Pad<T>::value;
    constexpr int XP = DK + PAD, YP = DV + PAD;
    constexpr int64_t REC = seg_record_floats(DK, DV);

    const int w = wave_id();
    const int64_t bh = (int64_t)b * H + h;
    const int cbase = 16 * w;
    const int n0 = s * m, n1 = min(n0 + m, N), cnt = n1 - n0;
    const T* xh = X.head(b, h);
    const T* yh = Y.head(b, h);

    floatx4 U[DK / 16][1];
#pragma unroll
    for (int fb = 0; fb < DK / 16; ++fb)
        U[fb][0] = zero4();
    float seg_log = 0.f;

    ChunkRegs<T, DK, NT> rx;
    ChunkRegs<T, DV, NT> ry;
    // the piece's last chunk may be partial: `tail` tokens
    auto rows_of = [&](int c) { return RAGGED && c == N - 1 ? tail : CHUNK; };
    int n = REVERSE ? n1 - 1 : n0;
    int rw = rows_of(n);
    chunk_load(rx, xh + (int64_t)n * CHUNK * X.st, X.st, rw);
    chunk_load(ry, yh + (int64_t)n * CHUNK * Y.st, Y.st, rw);
    float ra = decay_raw(dec, b, h, (int64_t)n * CHUNK, rw);
    for (int it = 0; it < cnt; ++it) {
        // buffer it % 2 was last read in chunk it - 2, before every wave
        // passed the previous chunk's barrier
        T* xs = (it & 1) ? xs1 : xs0;
        T* ys = (it & 1) ? ys1 : ys0;
        float* tb = (it & 1) ? tb1 : tb0;
        chunk_store(rx, xs, XP, rw);
        chunk_store(ry, ys, YP, rw);
        if (w == 0)
            decay_tables(dec, ra, tb, rw);
        __syncthreads();
        if (it + 1 < cnt) {
            n = REVERSE ? n1 - 2 - it : n0 + 1 + it;
            rw = rows_of(n);
            const int64_t tn = (int64_t)n * CHUNK;
            chunk_load(rx, xh + tn * X.st, X.st, rw);
            chunk_load(ry, yh + tn * Y.st, Y.st, rw);
            ra = decay_raw(dec, b, h, tn, rw);
        }
        seg_log += tb[TAB_LAM + CHUNK - 1];
        float yf[2][8];
        slot_factors(tb + (REVERSE ? TAB_G : TAB_F), yf);
        state_update<T, DK, 1>(U, xs, XP, ys, YP, cbase, tb[TAB_G + CHUNK - 1], yf);
    }

    float* rec = store + (bh * store_nseg + s) * REC;
    store_state<DK, DV, 1>(rec, U, cbase);
    if (threadIdx.x == 0)
        rec[DK * DV] = seg_log;
}

template <typename T, int DK, int DV, bool REVERSE, bool RAGGED>
__global__ __launch_bounds__(DV / 16 * 64) void seg_sum_kernel(
    Act<const T> X, Act<const T> Y, DecayArg dec, float* __restrict__ store, int64_t store_nseg,
    int H, int N, int tail, int m)
{
    constexpr int PAD = Pad<T>::value;
    constexpr int XP = DK + PAD, YP = DV + PAD;
    // two buffers: chunk it + 1 is staged while chunk it may still be read,
    // so one barrier per chunk suffices
    __shared__ __align__(16) T Xs[2][CHUNK * XP];
    __shared__ __align__(16) T Ys[2][CHUNK * YP];
    __shared__ __align__(16) float tab[2][TAB_SIZE];
    seg_sum_body<T, DK, DV, REVERSE, RAGGED>(X, Y, dec, store, store_nseg, H, N, tail, m, blockIdx.x, blockIdx.y,
                                     blockIdx.z, Xs[0], Xs[1], Ys[0], Ys[1], tab[0], tab[1]);
}

// Fold of four consecutive state elements [e, e + 4) of head bh across the
// nseg records at base (in order, or from the last record back when
// REVERSE): each record's state is replaced by the carried value, then
// c <- exp(log Gamma_s) c + U_s.  Loads of a batch of records are issued
// before any of the batch's stores (each store goes to a slot just read).
template <int DK, int DV, bool REVERSE, int BATCH>
__device__ __forceinline__ void fold_elems(const float* carry_in, float* carry_out, float* base,
                                           int nseg, int64_t bh, int e)
{
    constexpr int64_t REC = seg_record_floats(DK, DV);
    const int64_t io = bh * (DK * DV) + e;                   // S_in / S_out: same layout
    floatx4 carry = carry_in ? *reinterpret_cast<const floatx4*>(carry_in + io) : floatx4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nseg; k0 += BATCH) {
        floatx4 u[BATCH];
        float lg[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int k = k0 + j;
            if (k < nseg) {
                const float* rec = base + (REVERSE ? nseg - 1 - k : k) * REC;
                u[j] = *reinterpret_cast<const floatx4*>(rec + e);
                lg[j] = rec[DK * DV];
            }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int k = k0 + j;
            if (k < nseg) {
                float* rec = base + (REVERSE ? nseg - 1 - k : k) * REC;
                *reinterpret_cast<floatx4*>(rec + e) = carry;
                const float f = __expf(lg[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    carry[i] = f * carry[i] + u[j][i];
            }
        }
    }
    *reinterpret_cast<floatx4*>(carry_out + io) = carry;
}

template <int DK, int DV, bool REVERSE>
__global__ __launch_bounds__(256) void seg_fold_kernel(
    const float* __restrict__ carry_in, float* __restrict__ carry_out, float* __restrict__ store,
    int64_t store_nseg, int H, int nseg)
{
    // four consecutive elements [f][c] of a record per thread
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * H + h;
    fold_elems<DK, DV, REVERSE, 16>(carry_in, carry_out, store + bh * store_nseg * seg_record_floats(DK, DV),
                                    nseg, bh, e);
}

// A fold carried by a segment-kernel launch (see FoldArg): workgroup
// (s, h, b) of the launch's nsegs_here takes a contiguous share of head
// (b, h)'s state elements, four per thread at a time.  Nothing in the launch
// reads or writes what the fold touches, so no workgroup waits on another.
template <int DK, int DV, bool REVERSE, int NT>
__device__ __forceinline__ void fold_share(const FoldArg& f, int b, int h, int H, int s, int nsegs_here)
{
    constexpr int UNITS = DK * DV / 4;
    const int per = (UNITS + nsegs_here - 1) / nsegs_here;
    const int u1 = min((s + 1) * per, UNITS);
    const int64_t bh = (int64_t)b * H + h;
    float* base = f.store + bh * f.store_nseg * seg_record_floats(DK, DV);
    for (int u = s * per + (int)threadIdx.x; u < u1; u += NT)
        fold_elems<DK, DV, REVERSE, 8>(f.carry_in, f.carry_out, base, f.nseg, bh, 4 * u);
}

// ---------------------------------------------------------------------------
// Forward segment kernel.  Workgroup = (b, h, segment), one wave per 16
// columns of d_v (8 waves at d_v = 128).  Wave w owns output and state
// columns [16w, 16w + 16) and carries its state columns across the
// segment's chunks in registers.  Per chunk the waves build P = (Q K^T) .* D
// (split) in LDS, then wave w computes
//   O[:, cols] = gamma .* (Q S_{n-1}[:, cols]) + P V[:, cols],
//   S_n[:, cols] = gamma_C S_{n-1}[:, cols] + K^T (V[:, cols] .* gamma_C/gamma).
// The state serves as the B operand straight from registers (k-slot order
// of the result tiles).  The next chunk's rows load while this one computes.
// ---------------------------------------------------------------------------
template <typename T, typename OT, int DK, int DV, bool RAGGED>
__global__ __launch_bounds__(DV / 16 * 64) void fwd_seg_kernel(
    Act<const T> Q, Act<const T> K, Act<const T> V, DecayArg dec,
    const float* __restrict__ bstates, int64_t bs_nseg, Act<OT> O, int H, int N, int tail, int m)
{
    constexpr int NW = DV / 16, NT = NW * 64;
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD, VP = DV + PAD, PP = CHUNK + PAD;
    // Q and a second copy of K are staged with their d_k index permuted
    // (chunk_store_perm), so that the Q S product reads Q in the state's
    // k-slot order with 16-byte reads; P = Q K^T contracts the two permuted
    // copies.  The plain K serves the state update.
    __shared__ __align__(16) T Qs[CHUNK * QP];
    __shared__ __align__(16) T Kp[CHUNK * QP];
    __shared__ __align__(16) T Ks[CHUNK * QP];
    __shared__ __align__(16) T Vs[CHUNK * VP];
    __shared__ __align__(16) T Ps[2][CHUNK * PP];
    __shared__ __align__(16) float tab[TAB_SIZE];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;
    const int cbase = 16 * w;
    const int n0 = s * m, n1 = min(n0 + m, N);

    const T* qh = Q.head(b, h);
    const T* kh = K.head(b, h);
    const T* vh = V.head(b, h);
    // the piece's last chunk may be partial: `tail` tokens
    auto rows_of = [&](int c) { return RAGGED && c == N - 1 ? tail : CHUNK; };
    ChunkRegs<T, DK, NT> rq, rk;
    ChunkRegs<T, DV, NT> rv;
    chunk_load(rq, qh + (int64_t)n0 * CHUNK * Q.st, Q.st, rows_of(n0));
    chunk_load(rk, kh + (int64_t)n0 * CHUNK * K.st, K.st, rows_of(n0));
    chunk_load(rv, vh + (int64_t)n0 * CHUNK * V.st, V.st, rows_of(n0));
    // the state load is in flight together with the first chunk's
    floatx4 S[DK / 16][1];
    load_state<DK, DV, 1>(S, bstates + (bh * bs_nseg + s) * seg_record_floats(DK, DV), cbase);
    float ra = decay_raw(dec, b, h, (int64_t)n0 * CHUNK, rows_of(n0));

    // P tiles of this wave: row block ib, column blocks jb0, jb0 + jstep, ...
    // (the second four waves take row blocks in reverse order, so the two
    // waves sharing a SIMD have 3 or 2 non-zero tiles between them)
    const int ib_p = (NW == 8 && w >= 4) ? 3 - (w & 3) : (w & 3);
    const int jb0 = NW == 8 ? w / 4 : 0, jstep = NW == 8 ? 2 : 1;

    for (int n = n0; n < n1; ++n) {
        const int64_t tok0 = (int64_t)n * CHUNK;
        const int rows_n = rows_of(n);
        chunk_store_perm(rq, Qs, QP, rows_n);
        chunk_store_perm(rk, Kp, QP, rows_n);
        chunk_store(rk, Ks, QP, rows_n);
        chunk_store(rv, Vs, VP, rows_n);
        if (w == 0)
            decay_tables(dec, ra, tab, rows_n);
        __syncthreads();
        if (n + 1 < n1) {
            const int64_t tn = (int64_t)(n + 1) * CHUNK;
            const int rw = rows_of(n + 1);
            chunk_load(rq, qh + tn * Q.st, Q.st, rw);
            chunk_load(rk, kh + tn * K.st, K.st, rw);
            chunk_load(rv, vh + tn * V.st, V.st, rw);
            ra = decay_raw(dec, b, h, tn, rw);
        }
        const bool fac = decay_factored(tab);

        // P^T tiles (rows = earlier tokens j, columns = later tokens i), so
        // each lane writes four consecutive j of one row i of P
#pragma unroll
        for (int jb = jb0; jb < 4; jb += jstep) {
            floatx4 acc = zero4();
            if (jb <= ib_p) {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks)
                    acc = mma(frag_rows(Kp, QP, 16 * jb, 32 * ks), frag_rows(Qs, QP, 16 * ib_p, 32 * ks), acc);
                acc = decay_mask<false>(acc, tab, 16 * jb, 16 * ib_p, fac);
            }
            put_split4(Ps[0], Ps[1], (16 * ib_p + t) * PP + 16 * jb, acc);
        }
        // S_{n-1} as split B fragments (k = f in result-tile k-slot order)
        Split<T> sf[DK / 32];
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            sf[ks] = split_tiles<T>(S[2 * ks][0], S[2 * ks + 1][0]);
        __syncthreads();

        // O^T tiles (rows = this wave's columns, columns = tokens), so each
        // lane ends up holding four consecutive outputs of one token
        OT* oh = O.head(b, h) + tok0 * O.st;
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mma(sf[ks], frag_rows(Qs, QP, 16 * ib, 32 * ks), acc);
            acc *= tab[TAB_G + 16 * ib + t];
#pragma unroll
            for (int js = 0; js <= ib / 2; ++js)
                acc = mma(frag_cols(Vs, VP, cbase, 32 * js),
                          frag_rows_split(Ps[0], Ps[1], PP, 16 * ib, 32 * js), acc);
            store_tile_t<OT>(oh, O.st, 16 * ib, cbase, acc, rows_n);
        }

        // S_n = gamma_C S_{n-1} + K^T (V .* gamma_C/gamma); the state after
        // the segment's last chunk is not needed here
        if (n + 1 < n1) {
            float vf[2][8];
            slot_factors(tab + TAB_F, vf);
            state_update<T, DK, 1>(S, Ks, QP, Vs, VP, cbase, tab[TAB_G + CHUNK - 1], vf);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Backward segment kernel.  Workgroup = (b, h, segment), one wave per 16
// columns of d_v (8 waves at d_v = 128).  Wave w carries state/gradient
// columns [16w, 16w + 16) and works on one row block rb of the outputs
// (w % 4 in the first half of the waves, 3 - w % 4 in the second); with 8
// waves, half w / 4 selects what else it does.
//   Walk 1 (chunks in order, S carried from the stored segment state):
//   S_{n-1} goes to LDS (split) and, for rows rb and the half's columns,
//       dQ = gamma .* (dO S_{n-1}^T) + A K,   A = (dO V^T) .* D,
//   then S_n = gamma_C S_{n-1} + K^T (V .* gamma_C/gamma).
//   Walk 2 (chunks in reverse, G carried from the stored segment gradient):
//   G_n goes to LDS (split); for rows rb, the first half computes
//       dV = gamma_C/gamma .* (K G_n) + P^T dO,   P = (Q K^T) .* D,
//   and the second half
//       dK = gamma_C/gamma .* (V G_n^T) + A^T Q
//   (with 4 waves, every wave does both); then
//   G_{n-1} = gamma_C G_n + Q^T (dO .* gamma).
// P and A are built per wave in registers in the orientation their product
// needs and used as split B operands directly (k-slot order of the
// frag_cols_perm reads of the other operand); outputs are computed
// transposed (one vector store per lane and tile).  The next chunk's rows
// load while this one computes; walk 2 starts on walk 1's last chunk, whose
// K, V, dO and decay tables are still in LDS, so only Q is loaded for it,
// and takes K, V and dO of the two chunks before it from registers that
// walk 1 filled: of the segment's K, V and dO only the first chunk's are
// read twice from memory.
// ---------------------------------------------------------------------------
template <typename T, typename OT, int DK, int DV, bool DA, bool RAGGED>
__global__ __launch_bounds__(DV / 16 * 64) void bwd_seg_kernel(
    Act<const T> Q, Act<const T> K, Act<const T> V, Act<const T> dO, DecayArg dec,
    const float* __restrict__ bstates, int64_t bs_nseg, const float* __restrict__ gstates,
    int64_t gs_nseg, Act<OT> dQ, Act<OT> dK, Act<OT> dV, Act<float> da, float* __restrict__ da_tot,
    int H, int N, int tail, int m, FoldArg fold, SumDev<T> sum)
{
    constexpr int NW = DV / 16, NT = NW * 64, NH = NW / 4;
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD, VP = DV + PAD;
    constexpr int FBW = (DK / 16) / NH;   // walk-1 dQ blocks per wave
    constexpr int MAXM = 4;               // chunks per segment (launcher: m <= MAXM)
    __shared__ __align__(16) T Qs[CHUNK * QP];
    __shared__ __align__(16) T Ks[CHUNK * QP];
    __shared__ __align__(16) T Vs[CHUNK * VP];
    __shared__ __align__(16) T dOs[CHUNK * VP];
    __shared__ __align__(16) T Ms[2][DV * QP];     // state / gradient, [c][f], split
    __shared__ __align__(16) float tab[TAB_SIZE];
    // decay gradient: q.dq per token (per half, per chunk of the segment), g per token
    __shared__ float qdq_s[DA ? NH * MAXM * CHUNK : 1];
    __shared__ float g_s[DA ? CHUNK : 1];

    const int s = blockIdx.x, h = blockIdx.y;
    const int nseg_here = (N + m - 1) / m;
    // With carried segment sums the grid has twice the batch rows: the
    // launch's own segments are z < B, the sums z >= B, so that every
    // segment workgroup is dispatched before any sum workgroup and the sums
    // fill CUs as segment workgroups finish.  The sums use this kernel's LDS.
    const int B = sum.nseg ? (int)gridDim.z / 2 : (int)gridDim.z;
    if ((int)blockIdx.z >= B) {
        if (s < sum.nseg)
            seg_sum_body<T, DK, DV, true, RAGGED>(sum.X, sum.Y, sum.dec, sum.store, sum.store_nseg, H, sum.N,
                                          sum.tail, sum.m, s, h, blockIdx.z - B, Qs, Ks, Vs, dOs, tab,
                                          reinterpret_cast<float*>(Ms[0]));
        return;
    }
    if (s >= nseg_here)
        return;
    const int b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;
    const int cbase = 16 * w;
    // waves w and w + 4 share a SIMD; giving them row blocks rb and 3 - rb
    // evens out the row-block-dependent tile work per SIMD
    const int half = w / 4, rb = half ? 3 - (w & 3) : (w & 3), fb0 = half * FBW;
    const int n0 = s * m, n1 = min(n0 + m, N);

    floatx4 C[DK / 16][1];   // carried state (walk 1) / gradient (walk 2)

    const T* qh = Q.head(b, h);
    const T* kh = K.head(b, h);
    const T* vh = V.head(b, h);
    const T* doh = dO.head(b, h);
    ChunkRegs<T, DK, NT> rq, rk;
    ChunkRegs<T, DV, NT> rv, rdo;
    // K, V and dO of the segment's chunks n1 - 3 (ka, va, da_) and n1 - 2
    // (kb, vb, db), kept from walk 1 for walk 2, which would otherwise read
    // them again.  They move through the pair as a queue (fixed registers,
    // no indexing).  The decay-gradient variant has no registers to spare.
    constexpr bool KEEP = !DA;
    ChunkRegs<T, DK, NT> ka, kb;
    ChunkRegs<T, DV, NT> va, vb, da_, db;

    // the piece's last chunk may be partial: `tail` tokens
    auto rows_of = [&](int c) { return RAGGED && c == N - 1 ? tail : CHUNK; };

    // ---------------- walk 1: dQ
    chunk_load(rk, kh + (int64_t)n0 * CHUNK * K.st, K.st, rows_of(n0));
    chunk_load(rv, vh + (int64_t)n0 * CHUNK * V.st, V.st, rows_of(n0));
    chunk_load(rdo, doh + (int64_t)n0 * CHUNK * dO.st, dO.st, rows_of(n0));
    load_state<DK, DV, 1>(C, bstates + (bh * bs_nseg + s) * seg_record_floats(DK, DV), cbase);
    float ra = decay_raw(dec, b, h, (int64_t)n0 * CHUNK, rows_of(n0));
    // the previous piece's fold, while the first chunk's loads are in flight
    if (fold.store)
        fold_share<DK, DV, true, NT>(fold, b, h, H, s, nseg_here);
    for (int n = n0; n < n1; ++n) {
        const int64_t tok0 = (int64_t)n * CHUNK;
        const int rows_n = rows_of(n);
        if (KEEP && n >= n1 - 3 && n < n1 - 1) {
            chunk_copy(ka, kb); chunk_copy(va, vb); chunk_copy(da_, db);
            chunk_copy(kb, rk); chunk_copy(vb, rv); chunk_copy(db, rdo);
        }
        chunk_store(rk, Ks, QP, rows_n);
        chunk_store(rv, Vs, VP, rows_n);
        chunk_store(rdo, dOs, VP, rows_n);
        if (w == 0)
            decay_tables(dec, ra, tab, rows_n);
        put_state<T, DK, 1>(Ms[0], Ms[1], QP, C, cbase);
        __syncthreads();
        if (n + 1 < n1) {
            const int64_t tn = (int64_t)(n + 1) * CHUNK;
            const int rw = rows_of(n + 1);
            chunk_load(rk, kh + tn * K.st, K.st, rw);
            chunk_load(rv, vh + tn * V.st, V.st, rw);
            chunk_load(rdo, doh + tn * dO.st, dO.st, rw);
            ra = decay_raw(dec, b, h, tn, rw);
        } else {
            chunk_load(rq, qh + tok0 * Q.st, Q.st, rows_n);
        }
        const bool fac = decay_factored(tab);

        // A^T tiles of row block rb: T[j][i] = (v_j . dO_i) D_ij, j-block jb
        floatx4 at[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            at[jb] = zero4();
            if (jb <= rb) {
#pragma unroll
                for (int cs = 0; cs < DV / 32; ++cs)
                    at[jb] = mma(frag_rows(Vs, VP, 16 * jb, 32 * cs), frag_rows(dOs, VP, 16 * rb, 32 * cs), at[jb]);
                at[jb] = decay_mask<false>(at[jb], tab, 16 * jb, 16 * rb, fac);
            }
        }
        const Split<T> a0 = split_tiles<T>(at[0], at[1]);
        const Split<T> a1 = split_tiles<T>(at[2], at[3]);
        // dQ^T tiles: lane (g,t) holds token 16rb + t
        const float rowg = tab[TAB_G + 16 * rb + t];

        OT* out = dQ.head(b, h) + tok0 * dQ.st;
        // decay gradient: this lane's q values for its dQ^T entries
        floatx4 qv[DA ? FBW : 1];
        if constexpr (DA) {
#pragma unroll
            for (int fbi = 0; fbi < FBW; ++fbi)
                qv[fbi] = 16 * rb + t < rows_n ? load4(qh + (tok0 + 16 * rb + t) * Q.st + 16 * (fb0 + fbi) + 4 * g)
                                               : zero4();
        }
        float qdq = 0.f;
#pragma unroll
        for (int fbi = 0; fbi < FBW; ++fbi) {
            const int fb = fb0 + fbi;
            floatx4 acc = zero4();
#pragma unroll
            for (int cs = 0; cs < DV / 32; ++cs)
                acc = mma(frag_cols_split(Ms[0], Ms[1], QP, 16 * fb, 32 * cs),
                          frag_rows(dOs, VP, 16 * rb, 32 * cs), acc);
            acc *= rowg;
            acc = mma(frag_cols_perm(Ks, QP, 16 * fb, 0), a0, acc);
            if (rb >= 2)
                acc = mma(frag_cols_perm(Ks, QP, 16 * fb, 32), a1, acc);
            if constexpr (DA)
                qdq += acc[0] * qv[fbi][0] + acc[1] * qv[fbi][1] + acc[2] * qv[fbi][2] +
                       acc[3] * qv[fbi][3];
            store_tile_t<OT>(out, dQ.st, 16 * rb, 16 * fb, acc, rows_n);
        }
        if constexpr (DA) {
            // sum over the four lane groups: this half's share of q.dq per token
            qdq += __shfl_xor(qdq, 16, 64);
            qdq += __shfl_xor(qdq, 32, 64);
            if (g == 0)
                qdq_s[(half * MAXM + (n - n0)) * CHUNK + 16 * rb + t] = qdq;
        }

        if (n + 1 < n1) {
            float vf[2][8];
            slot_factors(tab + TAB_F, vf);
            state_update<T, DK, 1>(C, Ks, QP, Vs, VP, cbase, tab[TAB_G + CHUNK - 1], vf);
        }
        __syncthreads();
    }

    // ---------------- walk 2: dK, dV
    load_state<DK, DV, 1>(C, gstates + (bh * gs_nseg + s) * seg_record_floats(DK, DV), cbase);
    float dcarry = 0.f;   // decay gradient: sum of g over the segment's later chunks (wave 0)
    for (int n = n1 - 1; n >= n0; --n) {
        const int64_t tok0 = (int64_t)n * CHUNK;
        const int rows_n = rows_of(n);
        chunk_store(rq, Qs, QP, rows_n);
        if (n < n1 - 1) {
            chunk_store(rk, Ks, QP, rows_n);
            chunk_store(rv, Vs, VP, rows_n);
            chunk_store(rdo, dOs, VP, rows_n);
            if (w == 0)
                decay_tables(dec, ra, tab, rows_n);
        }
        put_state<T, DK, 1>(Ms[0], Ms[1], QP, C, cbase);
        __syncthreads();
        if (n > n0) {
            const int64_t tn = (int64_t)(n - 1) * CHUNK;
            const int rw = rows_of(n - 1);
            chunk_load(rq, qh + tn * Q.st, Q.st, rw);
            if (KEEP && n >= n1 - 2) {
                chunk_copy(rk, kb); chunk_copy(rv, vb); chunk_copy(rdo, db);
                chunk_copy(kb, ka); chunk_copy(vb, va); chunk_copy(db, da_);
            } else {
                chunk_load(rk, kh + tn * K.st, K.st, rw);
                chunk_load(rv, vh + tn * V.st, V.st, rw);
                chunk_load(rdo, doh + tn * dO.st, dO.st, rw);
            }
            ra = decay_raw(dec, b, h, tn, rw);
        }
        const bool fac = decay_factored(tab);
        // dV^T and dK^T tiles: lane (g,t) holds token 16rb + t
        const float rowf = tab[TAB_F + 16 * rb + t];

        if (NH == 1 || half == 0) {
            // P tiles of column block rb: rows i (i-block ib), column j = 16rb + t
            floatx4 pt[4];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                pt[ib] = zero4();
                if (ib >= rb) {
#pragma unroll
                    for (int ks = 0; ks < DK / 32; ++ks)
                        pt[ib] = mma(frag_rows(Qs, QP, 16 * ib, 32 * ks), frag_rows(Ks, QP, 16 * rb, 32 * ks), pt[ib]);
                    pt[ib] = decay_mask<true>(pt[ib], tab, 16 * ib, 16 * rb, fac);
                }
            }
            const Split<T> p0 = split_tiles<T>(pt[0], pt[1]), p1 = split_tiles<T>(pt[2], pt[3]);
            OT* outv = dV.head(b, h) + tok0 * dV.st;
#pragma unroll
            for (int cb = 0; cb < DV / 16; ++cb) {
                floatx4 acc = zero4();
#pragma unroll
                for (int fs = 0; fs < DK / 32; ++fs)
                    acc = mma(frag_rows_split(Ms[0], Ms[1], QP, 16 * cb, 32 * fs),
                              frag_rows(Ks, QP, 16 * rb, 32 * fs), acc);
                acc *= rowf;
                if (rb < 2)
                    acc = mma(frag_cols_perm(dOs, VP, 16 * cb, 0), p0, acc);
                acc = mma(frag_cols_perm(dOs, VP, 16 * cb, 32), p1, acc);
                store_tile_t<OT>(outv, dV.st, 16 * rb, 16 * cb, acc, rows_n);
            }
        }
        if (NH == 1 || half == 1) {
            // A tiles of column block rb: rows i, column j = 16rb + t
            floatx4 atl[4];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                atl[ib] = zero4();
                if (ib >= rb) {
#pragma unroll
                    for (int cs = 0; cs < DV / 32; ++cs)
                        atl[ib] = mma(frag_rows(dOs, VP, 16 * ib, 32 * cs), frag_rows(Vs, VP, 16 * rb, 32 * cs), atl[ib]);
                    atl[ib] = decay_mask<true>(atl[ib], tab, 16 * ib, 16 * rb, fac);
                }
            }
            const Split<T> q0 = split_tiles<T>(atl[0], atl[1]), q1 = split_tiles<T>(atl[2], atl[3]);
            OT* outk = dK.head(b, h) + tok0 * dK.st;
            float kdk = 0.f;
#pragma unroll
            for (int fb = 0; fb < DK / 16; ++fb) {
                floatx4 acc = zero4();
#pragma unroll
                for (int cs = 0; cs < DV / 32; ++cs)
                    acc = mma(frag_cols_split(Ms[0], Ms[1], QP, 16 * fb, 32 * cs),
                              frag_rows(Vs, VP, 16 * rb, 32 * cs), acc);
                acc *= rowf;
                if (rb < 2)
                    acc = mma(frag_cols_perm(Qs, QP, 16 * fb, 0), q0, acc);
                acc = mma(frag_cols_perm(Qs, QP, 16 * fb, 32), q1, acc);
                if constexpr (DA) {
                    const floatx4 kk = load4(Ks + (16 * rb + t) * QP + 16 * fb + 4 * g);
                    kdk += acc[0] * kk[0] + acc[1] * kk[1] + acc[2] * kk[2] + acc[3] * kk[3];
                }
                store_tile_t<OT>(outk, dK.st, 16 * rb, 16 * fb, acc, rows_n);
            }
            if constexpr (DA) {
                // g = q.dq - k.dk for the tokens of row block rb
                kdk += __shfl_xor(kdk, 16, 64);
                kdk += __shfl_xor(kdk, 32, 64);
                if (g == 0) {
                    const int c = n - n0, tok = 16 * rb + t;
                    float qd = qdq_s[c * CHUNK + tok];
                    if constexpr (NH == 2)
                        qd += qdq_s[(MAXM + c) * CHUNK + tok];
                    g_s[tok] = qd - kdk;
                }
            }
        }

        // G_{n-1} = gamma_C G_n + Q^T (dO .* gamma); not needed after the
        // segment's first chunk
        if (n > n0) {
            float of[2][8];
            slot_factors(tab + TAB_G, of);
            state_update<T, DK, 1>(C, Qs, QP, dOs, VP, cbase, tab[TAB_G + CHUNK - 1], of);
        }
        __syncthreads();
        if constexpr (DA) {
            // reverse cumulative sum of g over the chunk (token = lane), plus
            // the segment's later chunks; g_s is next written after the next
            // iteration's first barrier
            if (w == 0) {
                float x = g_s[l];
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_down(x, off, 64);
                    if (l + off < 64)
                        x += y;
                }
                if (l < rows_n)
                    da.ptr[b * da.sb + h * da.sh + (tok0 + l) * da.st] = x + dcarry;
                dcarry += __shfl(x, 0, 64);
            }
        }
    }
    if constexpr (DA) {
        if (w == 0 && l == 0)
            da_tot[bh * nseg_here + s] = dcarry;
    }
}

// ---------------------------------------------------------------------------
// A piece of zero tokens passes its carry through: dst = src, or zeros when
// src is NULL (src may equal dst).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void carry_copy_kernel(const float* src, float* dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// Decay gradient of a piece, last step.  With g_t = q_t.dq_t - k_t.dk_t the
// gradient of the loss with respect to the log-decay of token r is the sum
// of g_t over t >= r (through the end of the sequence: the carry from later
// pieces), and da_r = that / a_r.  The segment kernel left the within-segment
// sums in da and the segment totals in tot.  One workgroup per (b, h): the
// totals of up to 1024 segments at a time are turned into suffix sums in LDS
// (an inclusive scan from the last segment), then every token of those
// segments is finished independently, four per thread with their loads
// issued together.  carry_out = carry_in + the piece's sum of g is the carry
// for the previous piece (it may alias carry_in: every thread reads carry_in
// before the first barrier, thread 0 writes carry_out after the last).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void da_finish_kernel(Act<float> da, DecayArg dec,
                                                         const float* __restrict__ tot,
                                                         const float* carry_in, float* carry_out,
                                                         int H, int T, int seg_len, int nseg)
{
    constexpr int NT = 1024;
    __shared__ float suf[NT + 1];   // suf[i]: sum of the block's totals from segment i on
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * H + h;
    float running = carry_in ? carry_in[bh] : 0.f;   // sum over every later segment
    float* dh = da.head(b, h);
    for (int end = nseg; end > 0; end -= NT) {
        const int start = max(0, end - NT), nb = end - start;
        // inclusive suffix scan of this block's totals
        float x = tid < nb ? tot[bh * nseg + start + tid] : 0.f;
        suf[tid] = x;
        if (tid == 0)
            suf[NT] = 0.f;
        __syncthreads();
        for (int off = 1; off < nb; off <<= 1) {
            const float y = tid + off < nb ? suf[tid + off] : 0.f;
            __syncthreads();
            x += y;
            suf[tid] = x;
            __syncthreads();
        }
        // tokens of segments start .. end - 1, four per thread
        const int t0 = start * seg_len, t1 = min(end * seg_len, T);
        for (int base = t0; base < t1; base += 4 * NT) {
            float v[4], a[4];
            int tok[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                tok[j] = base + j * NT + tid;
                if (tok[j] < t1) {
                    v[j] = dh[tok[j] * da.st];
                    a[j] = dec.kind == 1 ? dec.ptr[h * dec.sh]
                                         : dec.ptr[b * dec.sb + h * dec.sh + (int64_t)tok[j] * dec.st];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (tok[j] < t1) {
                    const int i = tok[j] / seg_len - start;
                    // totals of the later segments of this block, then of later blocks
                    dh[tok[j] * da.st] = (v[j] + suf[i + 1 < nb ? i + 1 : NT] + running) / a[j];
                }
            }
        }
        running += suf[0];
        __syncthreads();   // suf is rewritten by the next block
    }
    if (tid == 0)
        carry_out[bh] = running;
}

// ---------------------------------------------------------------------------
// Host-side launchers: dispatch (dtype, out dtype, d_k, d_v) to an instance.
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
hipError_t sum_impl(const ScanLaunch& s, hipStream_t stream)
{
    const dim3 grid((s.N + s.m - 1) / s.m, s.H, s.B), block(DV / 16 * 64);
    return with_ragged(s.tail < CHUNK, [&](auto rg) {
        constexpr bool RG = decltype(rg)::value;
        if (s.reverse)
            launch_kernel((seg_sum_kernel<T, DK, DV, true, RG>), grid, block, stream, cact<T>(s.x),
                          cact<T>(s.y), decay_arg(s.decay, s.decay_kind), (float*)s.store,
                          s.store_nseg, s.H, s.N, s.tail, s.m);
        else
            launch_kernel((seg_sum_kernel<T, DK, DV, false, RG>), grid, block, stream, cact<T>(s.x),
                          cact<T>(s.y), decay_arg(s.decay, s.decay_kind), (float*)s.store,
                          s.store_nseg, s.H, s.N, s.tail, s.m);
        return hipGetLastError();
    });
}

template <typename T, typename OT, int DK, int DV>
hipError_t fold_impl(const ScanLaunch& s, hipStream_t stream)
{
    const int nseg = (s.N + s.m - 1) / s.m;
    const dim3 grid(DK * DV / 1024, s.H, s.B), block(256);
    if (s.reverse)
        launch_kernel((seg_fold_kernel<DK, DV, true>), grid, block, stream, s.carry_in,
                      s.carry_out, (float*)s.store, s.store_nseg, s.H, nseg);
    else
        launch_kernel((seg_fold_kernel<DK, DV, false>), grid, block, stream, s.carry_in,
                      s.carry_out, (float*)s.store, s.store_nseg, s.H, nseg);
    return hipGetLastError();
}

template <typename T, typename OT, int DK, int DV>
hipError_t fwd_seg_impl(const FwdIntraLaunch& s, hipStream_t stream)
{
    const dim3 grid((s.N + s.m - 1) / s.m, s.H, s.B), block(DV / 16 * 64);
    return with_ragged(s.tail < CHUNK, [&](auto rg) {
        launch_kernel((fwd_seg_kernel<T, OT, DK, DV, decltype(rg)::value>), grid, block, stream,
                      cact<T>(s.q), cact<T>(s.k), cact<T>(s.v), decay_arg(s.decay, s.decay_kind),
                      (const float*)s.states, s.st_nseg, mact<OT>(s.o), s.H, s.N, s.tail, s.m);
        return hipGetLastError();
    });
}

template <typename T, typename OT, int DK, int DV>
hipError_t bwd_seg_impl(const BwdIntraLaunch& s, hipStream_t stream)
{
    if (s.m > 4 || s.sum.m > 4)
        return hipErrorInvalidValue;
    const SumDev<T> sum{cact<T>(s.sum.x), cact<T>(s.sum.y), decay_arg(s.sum.decay, s.sum.decay_kind),
                        (float*)s.sum.store, s.sum.store_nseg, s.sum.N, s.sum.m, s.sum.nseg, s.sum.tail};
    const int nseg = (s.N + s.m - 1) / s.m;
    const dim3 grid(s.sum.nseg ? max(nseg, s.sum.nseg) : nseg, s.H, s.sum.nseg ? 2 * s.B : s.B),
        block(DV / 16 * 64);
    const bool ragged = s.tail < CHUNK || (s.sum.nseg && s.sum.tail < CHUNK);
    return with_ragged(ragged, [&](auto rg) {
        constexpr bool RG = decltype(rg)::value;
        if (s.da.ptr)
            launch_kernel((bwd_seg_kernel<T, OT, DK, DV, true, RG>), grid, block, stream,
                          cact<T>(s.q), cact<T>(s.k), cact<T>(s.v), cact<T>(s.dO),
                          decay_arg(s.decay, s.decay_kind), (const float*)s.states, s.st_nseg,
                          (const float*)s.ghat, s.g_nseg, mact<OT>(s.dq), mact<OT>(s.dk_),
                          mact<OT>(s.dv_), mact<float>(s.da), s.da_tot, s.H, s.N, s.tail, s.m, s.fold,
                          sum);
        else
            launch_kernel((bwd_seg_kernel<T, OT, DK, DV, false, RG>), grid, block, stream,
                          cact<T>(s.q), cact<T>(s.k), cact<T>(s.v), cact<T>(s.dO),
                          decay_arg(s.decay, s.decay_kind), (const float*)s.states, s.st_nseg,
                          (const float*)s.ghat, s.g_nseg, mact<OT>(s.dq), mact<OT>(s.dk_),
                          mact<OT>(s.dv_), Act<float>{nullptr, 0, 0, 0}, nullptr, s.H, s.N,
                          s.tail, s.m, s.fold, sum);
        return hipGetLastError();
    });
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

hipError_t launch_seg_sum(const ScanLaunch& s, hipStream_t stream)
{
    if (s.dtype == 0)
        LINREC_DISPATCH_D(sum_impl, bf16, float, s, stream);
    else if (s.dk == 64 && s.dv == 64)
        return sum_impl<float, float, 64, 64>(s, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_seg_fold(const ScanLaunch& s, hipStream_t stream)
{
    if (s.dtype == 0)
        LINREC_DISPATCH_D(fold_impl, bf16, float, s, stream);
    else if (s.dk == 64 && s.dv == 64)
        return fold_impl<float, float, 64, 64>(s, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_intra(const FwdIntraLaunch& s, hipStream_t stream)
{
    LINREC_DISPATCH(fwd_seg_impl, s, stream);
}

hipError_t launch_bwd_intra(const BwdIntraLaunch& s, hipStream_t stream)
{
    LINREC_DISPATCH(bwd_seg_impl, s, stream);
}

hipError_t launch_carry_copy(const float* src, float* dst, int64_t n, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    launch_kernel(carry_copy_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), stream, src,
                  dst, n);
    return hipGetLastError();
}

hipError_t launch_da_finish(const DaFinishLaunch& s, hipStream_t stream)
{
    const int seg_len = s.m * CHUNK, nseg = (s.N + s.m - 1) / s.m;
    launch_kernel(da_finish_kernel, dim3(s.H, s.B), dim3(1024), stream, mact<float>(s.da),
                  decay_arg(s.decay, s.decay_kind), s.tot, s.carry_in, s.carry_out, s.H,
                  (s.N - 1) * CHUNK + s.tail, seg_len, nseg);
    return hipGetLastError();
}

}  // namespace linrec
