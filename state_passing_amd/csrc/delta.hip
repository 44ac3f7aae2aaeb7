// delta.hip -- gfx950 kernels of the gated delta-rule recurrence, forward and
// backward.
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

// 16 x 16 x 16 fp32 products on v_mfma_f32_16x16x4_f32: sub-step r contracts
// the k-slots {4g + r}.  X is read as rows of an fp32 LDS tile (lane (g,t)
// takes X[t][4g .. 4g + 3] in one read); Y either from LDS (Y[4g + r][t]) or
// as a result tile in registers (lane (g,t) holds Y[4g + r][t]), so results
// chain without moving between lanes.  Result: lane (g,t) gets D[4g + r][t].
__device__ __forceinline__ floatx4 mm16_f32(const float* X, int xp, const float* Y, int yp, floatx4 acc)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const floatx4 xa = *reinterpret_cast<const floatx4*>(X + t * xp + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[r], Y[(4 * g + r) * yp + t], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ floatx4 mm16_f32_reg(const float* X, int xp, floatx4 y, floatx4 acc)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const floatx4 xa = *reinterpret_cast<const floatx4*>(X + t * xp + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[r], y[r], acc, 0, 0, 0);
    return acc;
}

// ---------------------------------------------------------------------------
// Per chunk: T = (I + A)^{-1}, then W_v, W_k (fp32, [B][H][Tp][d], Tp the
// piece's tokens rounded up to whole chunks), P = (Q K^T) .* D and the decay
// tables for the serial kernels.  Workgroup = (chunk, h, b), 4 waves.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV, bool RAGGED>
__global__ __launch_bounds__(256) void delta_prep_kernel(Act<const T> Q, Act<const T> K, Act<const T> V,
                                                         Act<const float> beta, DecayArg dec,
                                                         Act<float> Wk, Act<float> Wv,
                                                         float* __restrict__ Pout,
                                                         float* __restrict__ Tout,
                                                         float* __restrict__ TabOut, int H, int tail)
{
    constexpr int NT = 256, NW = 4;
    constexpr int PAD = Pad<T>::value;
    constexpr int KP = DK + PAD, VP = DV + PAD;
    constexpr int AP = CHUNK + 4;            // fp32 pitch of A and T
    // Q is read only before T is formed: the two share one buffer, which
    // keeps the workgroup under half the CU's LDS (two per CU)
    constexpr int QT_BYTES = CHUNK * KP * (int)sizeof(T) > CHUNK * AP * 4 ? CHUNK * KP * (int)sizeof(T)
                                                                          : CHUNK * AP * 4;
    __shared__ __align__(16) unsigned char qt_buf[QT_BYTES];
    T* const Qs = reinterpret_cast<T*>(qt_buf);
    float* const Ts = reinterpret_cast<float*>(qt_buf);
    __shared__ __align__(16) T Ks[CHUNK * KP];
    __shared__ __align__(16) T Vs[CHUNK * VP];
    __shared__ __align__(16) float As[CHUNK * AP];
    __shared__ __align__(16) float tab[TAB_SIZE];
    __shared__ float bet[CHUNK];

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t tok0 = (int64_t)n * CHUNK;
    // the piece's last chunk may hold fewer tokens: the rows past them enter
    // as zeros (q, k, v) with beta = 0 and decay 1, so that they add nothing
    // to T, W, P or the state, and nothing is written for them but zeros
    const int rows = RAGGED && n == (int)gridDim.x - 1 ? tail : CHUNK;
    {
        // the gate and beta first: their use waits on nothing else
        float raw = 0.f, bt = 0.f;
        if (w == 0) {
            raw = decay_raw(dec, b, h, tok0, rows);
            bt = beta.ptr[b * beta.sb + h * beta.sh + (tok0 + (RAGGED ? min(l, rows - 1) : l)) * beta.st];
        }
        ChunkRegs<T, DK, NT> rq, rk;
        ChunkRegs<T, DV, NT> rv;
        chunk_load(rq, Q.head(b, h) + tok0 * Q.st, Q.st, rows);
        chunk_load(rk, K.head(b, h) + tok0 * K.st, K.st, rows);
        chunk_load(rv, V.head(b, h) + tok0 * V.st, V.st, rows);
        if (w == 0) {
            decay_tables(dec, raw, tab, rows);
            bet[l] = !RAGGED || l < rows ? bt : 0.f;
        }
        chunk_store(rq, Qs, KP, rows);
        chunk_store(rk, Ks, KP, rows);
        chunk_store(rv, Vs, VP, rows);
    }
    __syncthreads();
    // the chunk's decay tables for the serial kernels, [B][H][N][TAB_SIZE]
    if (threadIdx.x < TAB_SIZE / 4)
        *reinterpret_cast<floatx4*>(TabOut + (((int64_t)b * H + h) * gridDim.x + n) * TAB_SIZE +
                                    4 * threadIdx.x) = *reinterpret_cast<const floatx4*>(tab + 4 * threadIdx.x);

    // A: strictly lower part of beta_i exp(lam_i - lam_j) (k_i . k_j); and
    // P = (Q K^T) .* D (lower, diagonal included) for the serial kernels,
    // [B][H][N][64][64] fp32
    const bool fac = decay_factored(tab);
    float* pdst = Pout + (((int64_t)b * H + h) * gridDim.x + n) * CHUNK * CHUNK;
    for (int tile = w; tile < 16; tile += NW) {
        const int ib = tile >> 2, jb = tile & 3;
        floatx4 acc = zero4(), pacc = zero4();
        if (jb <= ib) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                acc = mma(frag_rows(Ks, KP, 16 * ib, 32 * ks), frag_rows(Ks, KP, 16 * jb, 32 * ks), acc);
                pacc = mma(frag_rows(Qs, KP, 16 * ib, 32 * ks), frag_rows(Ks, KP, 16 * jb, 32 * ks), pacc);
            }
            pacc = decay_mask<true>(pacc, tab, 16 * ib, 16 * jb, fac);
        }
        const int j = 16 * jb + t;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * g + r;
            As[i * AP + j] = j < i ? bet[i] * __expf(tab[TAB_LAM + i] - tab[TAB_LAM + j]) * acc[r] : 0.f;
            pdst[i * CHUNK + j] = pacc[r];
        }
    }
    __syncthreads();

    // T = (I + A)^{-1}, unit lower triangular, by 16 x 16 blocks (block
    // row i, column j).  Wave w inverts the diagonal block w by forward
    // substitution (lane c < 16 takes column c:
    // x_r = [r == c] - sum_{m < r} A_ww[r][m] x_m) and clears the blocks
    // right of it; then, one block diagonal at a time, wave i forms
    //     T_ij = -T_ii sum_{k = j .. i-1} A_ik T_kj
    // with fp32 MFMA (the blocks it needs are all on earlier diagonals).
    {
        if (l < 16) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == l ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m)
                    acc -= As[(16 * w + r) * AP + 16 * w + m] * x[m];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Ts[(16 * w + r) * AP + 16 * w + l] = x[r];
        }
        for (int e = l; e < 16 * 16 * (3 - w); e += 64)
            Ts[(16 * w + (e & 15)) * AP + 16 * (w + 1) + (e >> 4)] = 0.f;
        __syncthreads();
        for (int dg = 1; dg < 4; ++dg) {
            if (w >= dg) {
                const int i = w, j = w - dg;
                floatx4 m4 = zero4();
                for (int k = j; k < i; ++k)
                    m4 = mm16_f32(As + (16 * i) * AP + 16 * k, AP, Ts + (16 * k) * AP + 16 * j, AP, m4);
                floatx4 t4 = mm16_f32_reg(Ts + (16 * i) * AP + 16 * i, AP, m4, zero4());
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Ts[(16 * i + 4 * g + r) * AP + 16 * j + t] = -t4[r];
            }
            __syncthreads();
        }
        if (Tout) {   // the backward's copy: [B][H][N][64][64]
            float* dst = Tout + (((int64_t)b * H + h) * gridDim.x + n) * CHUNK * CHUNK;
            for (int e = 4 * (int)threadIdx.x; e < CHUNK * CHUNK; e += 4 * NT)
                *reinterpret_cast<floatx4*>(dst + e) =
                    *reinterpret_cast<const floatx4*>(Ts + (e / CHUNK) * AP + e % CHUNK);
        }
    }

    // W^T[c][i] = sum_j X[j][c] (T[i][j] beta_j [gamma_j]) with X = V (W_v) or
    // K (W_k); wave w takes the rows i of block w, so it forms its B operand
    // (T beta [gamma], split) once per k32 step and reuses it for every column
    // block; transposed tiles so each lane stores four consecutive features
#pragma unroll
    for (int isk = 0; isk < 2; ++isk) {
        Split<T> top[CHUNK / 32];
#pragma unroll
        for (int ks = 0; ks < CHUNK / 32; ++ks) {
            float x[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int j = 32 * ks + 8 * g + r;
                x[r] = Ts[(16 * w + t) * AP + j] * bet[j] * (isk ? tab[TAB_G + j] : 1.f);
            }
            top[ks] = split8<T>(x);
        }
        Act<float>& W = isk ? Wk : Wv;
        const T* X = isk ? Ks : Vs;
        const int XP = isk ? KP : VP;
        constexpr int NCB = (DK > DV ? DK : DV) / 16;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            if (cb < (isk ? DK : DV) / 16) {
                floatx4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < CHUNK / 32; ++ks)
                    acc = mma(frag_cols(X, XP, 16 * cb, 32 * ks), top[ks], acc);
                store_tile_t<float>(W.head(b, h) + tok0 * W.st, W.st, 16 * w, 16 * cb, acc);
            }
        }
    }
}

// Eight consecutive values of one row of an activation in global memory,
// as a fragment (frag_rows() layout: lane (g, t) holds row t, columns 8g ..).
template <typename T>
struct RowFrag;
template <>
struct RowFrag<bf16> {
    u32x4 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ Frag<bf16> frag() const
    {
        Frag<bf16> f;
        f.v = __builtin_bit_cast(bf16x8, v);
        return f;
    }
};
template <>
struct RowFrag<float> {
    floatx4 a, b;
    __device__ __forceinline__ void load(const float* p)
    {
        a = *reinterpret_cast<const floatx4*>(p);
        b = *reinterpret_cast<const floatx4*>(p + 4);
    }
    __device__ __forceinline__ Frag<float> frag() const
    {
        Frag<float> f;
        f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
        f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
        return f;
    }
};

// ---------------------------------------------------------------------------
// Workgroup -> (column block, head, batch) for the serial kernels, whose
// d_v / 16 column workgroups of one head all read that head's chunk operands
// (Q, K, W_k, P; dO in the backward).  Workgroups go to the eight XCDs in
// turn by flat index, and each XCD has its own L2; this mapping puts the
// column workgroups of one head on one XCD (flat index f: XCD f % 8, head
// group (f % 8) + 8 (f / 8 / ncb), column block (f / 8) % ncb), so that seven
// of every eight reads of those operands can hit the L2.  With B * H not a
// multiple of 8 the plain mapping is kept.
// ---------------------------------------------------------------------------
struct ColHead {
    int cb, h, b;
};

__device__ __forceinline__ ColHead xcd_col_head(int H, int B)
{
    const int ncb = gridDim.x;
    if ((B * H) % 8 != 0)
        return ColHead{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    const int f = blockIdx.x + ncb * (blockIdx.y + H * blockIdx.z);
    const int slot = f / 8;
    const int grp = f % 8 + 8 * (slot / ncb);
    return ColHead{slot % ncb, grp % H, grp / H};
}

// ---------------------------------------------------------------------------
// Serial walk over a piece's chunks for one (b, h) and state columns
// [16 cb, 16 cb + 16).  8 waves.  Per chunk n, with P = (Q K^T) .* D from the
// prep kernel:
//   U = W_v - W_k S_0                      (waves 0-3: rows [16 w, 16 w + 16))
//   S <- gamma_C S + (K .* gamma_C/gamma)^T U   (waves 0-3: state row blocks
//                                                FPW w .. FPW w + FPW - 1)
//   O^T = gamma .* (S_0^T Q^T) + U^T P^T   (waves 4-7, one chunk behind)
// The state's chain per chunk is U, then the update; the output is not on
// it, so waves 4-7 form chunk n - 1's output while waves 0-3 form chunk n's
// U, and waves 0-3 issue first on the SIMD each shares with one of waves
// 4-7.  K, the decay tables and the split S_0 and U planes are
// double-buffered in LDS (chunk n in buffer n % 2), which leaves two
// barriers per chunk: a buffer is written again two chunks later, after
// every wave has passed the barrier that follows its last reader.
// ---------------------------------------------------------------------------
template <typename T, typename OT, int DK, int DV, bool RAGGED>
__global__ __launch_bounds__(512) void delta_scan_kernel(Act<const T> Q, Act<const T> K,
                                                         Act<const float> Wk, Act<const float> Wv,
                                                         const float* __restrict__ Pm,
                                                         const float* __restrict__ tabs,
                                                         const float* S_in,
                                                         float* S_out, Act<OT> O,
                                                         float* __restrict__ s0_out,
                                                         float* __restrict__ u_out, int H, int N, int tail)
{
    constexpr int NT = 512, NFB = DK / 16;
    static_assert(NFB == 4 || NFB == 8, "d_k must be 64 or 128");
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD;
    __shared__ __align__(16) T Ks[2][CHUNK * QP];
    // the state and U as bf16 hi/lo planes, transposed ([column][f] and
    // [column][token]), so that every product reads them with 16-byte reads
    constexpr int SPP = DK + PAD, UPP = CHUNK + PAD;
    __shared__ __align__(16) T Ssp[2][2][16 * SPP];
    __shared__ __align__(16) T Usp[2][2][16 * UPP];
    __shared__ __align__(16) float tab[2][TAB_SIZE];

    const ColHead wg = xcd_col_head(H, gridDim.z);
    const int cb = wg.cb, h = wg.h, b = wg.b;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;
    const int cbase = 16 * cb;
    // roles: waves 0-3 form U (row block w) and carry the state; waves 4-7
    // form the output (row block w - 4)
    constexpr int FPW = NFB / 4;
    const bool urole = w < 4;
    const int rb = w & 3;
    if (urole)
        __builtin_amdgcn_s_setprio(1);

    floatx4 S[FPW];   // S[16 (FPW w + q) + 4g + r][cbase + t]
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
        S[q] = zero4();
        if (urole && S_in)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[q][r] = S_in[bh * DK * DV + (int64_t)(16 * (FPW * w + q) + 4 * g + r) * DV + cbase + t];
    }

    const T* kh = K.head(b, h);
    // Row operands of a wave's 16 tokens go from global memory straight into
    // the registers of the products that take them: W_k (rows of U's A
    // operand) and W_v (U's result-tile entries) in waves 0-3, Q and P (the
    // output's B operands) in waves 4-7, lane (g, t) holding row 16 rb + t,
    // columns 8g .. 8g + 7 of each k32 step.  Each is reloaded for the next
    // chunk as soon as the current chunk's products have taken it.  K, which
    // every wave reads transposed, and the decay tables are staged through
    // LDS, loaded a chunk ahead.
    // the last chunk may be partial (tail tokens): its row reads are clamped
    // to the last token; K's padded rows are zeroed in LDS, the prep
    // kernel's operands are zero there, and no output is stored for them
    auto rows_of = [&](int64_t tk) { return RAGGED && tk / CHUNK == N - 1 ? tail : CHUNK; };
    const T* qh = Q.head(b, h);
    const float* wkrow = Wk.head(b, h) + (int64_t)(16 * rb + t) * Wk.st + 8 * g;
    const float* prow = Pm + bh * (int64_t)N * CHUNK * CHUNK + (16 * rb + t) * CHUNK + 8 * g;
    const float* wvh = Wv.head(b, h) + cbase + t;
    const float* th = tabs + bh * (int64_t)N * TAB_SIZE;
    constexpr int NKS = DK / 32;
    typedef RowFrag<T> QF;
    floatx4 wk[NKS][2], pv[2][2];
    float wv[4];
    QF qv[NKS];
    auto load_wk_wv = [&](int64_t tk) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            wk[ks][0] = *reinterpret_cast<const floatx4*>(wkrow + tk * Wk.st + 32 * ks);
            wk[ks][1] = *reinterpret_cast<const floatx4*>(wkrow + tk * Wk.st + 32 * ks + 4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wv[r] = wvh[(tk + 16 * rb + 4 * g + r) * Wv.st];
    };
    auto load_q_p = [&](int64_t tk) {
        const T* qrow = qh + (tk + (RAGGED ? min(16 * rb + t, rows_of(tk) - 1) : 16 * rb + t)) * Q.st + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qv[ks].load(qrow + 32 * ks);
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            pv[js][0] = *reinterpret_cast<const floatx4*>(prow + tk * CHUNK + 32 * js);
            pv[js][1] = *reinterpret_cast<const floatx4*>(prow + tk * CHUNK + 32 * js + 4);
        }
    };
    ChunkRegs<T, DK, NT> rk;
    floatx4 rtab = zero4();
    auto load_k_tab = [&](int64_t tk) {
        if (threadIdx.x < TAB_SIZE / 4)
            rtab = *reinterpret_cast<const floatx4*>(th + tk / CHUNK * TAB_SIZE + 4 * threadIdx.x);
        chunk_load(rk, kh + tk * K.st, K.st, rows_of(tk));
    };
    load_k_tab(0);
    if (urole)
        load_wk_wv(0);
    else
        load_q_p(0);
    // O^T[c][i] of chunk nn, tokens [16 rb, 16 rb + 16) (waves 4-7), from
    // its buffers (nn % 2) and the registers holding its Q and P rows
    auto out_tile = [&](int nn) {
        const int bf = nn & 1;
        floatx4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            acc = mma(frag_rows_split(Ssp[bf][0], Ssp[bf][1], SPP, 0, 32 * ks), qv[ks].frag(), acc);
        acc *= tab[bf][TAB_G + 16 * rb + t];
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            if (js <= rb / 2) {
                const float x[8] = {pv[js][0][0], pv[js][0][1], pv[js][0][2], pv[js][0][3],
                                    pv[js][1][0], pv[js][1][1], pv[js][1][2], pv[js][1][3]};
                acc = mma(frag_rows_split(Usp[bf][0], Usp[bf][1], UPP, 0, 32 * js), split8<T>(x), acc);
            }
        }
        return acc;
    };
    // The top of chunk n: its K and decay tables into LDS, the state entering
    // it as split planes (waves 0-3), and that state for the backward.
    auto chunk_top = [&](int n) {
        const int cur = n & 1;
        chunk_store(rk, Ks[cur], QP, rows_of((int64_t)n * CHUNK));
        if (threadIdx.x < TAB_SIZE / 4)
            *reinterpret_cast<floatx4*>(tab[cur] + 4 * threadIdx.x) = rtab;
        if (urole)
#pragma unroll
            for (int q = 0; q < FPW; ++q) {
                const int fb = FPW * w + q;
                put_split4(Ssp[cur][0], Ssp[cur][1], t * SPP + 16 * fb, S[q]);
                if (s0_out)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s0_out[((bh * N + n) * DK + 16 * fb + 4 * g + r) * DV + cbase + t] = S[q][r];
            }
    };
    // S <- gamma_C S + K~^T U of chunk n for this wave's row blocks
    auto update = [&](int n) {
        const int cur = n & 1;
        if (urole) {
            const float gC = tab[cur][TAB_G + CHUNK - 1];
            float kf[2][8];
            slot_factors(tab[cur] + TAB_F, kf);
#pragma unroll
            for (int q = 0; q < FPW; ++q) {
                const int fb = FPW * w + q;
                S[q] *= gC;
#pragma unroll
                for (int ks = 0; ks < CHUNK / 32; ++ks)
                    S[q] = mma(split_scaled<T>(frag_cols(Ks[cur], QP, 16 * fb, 32 * ks), kf[ks]),
                               frag_rows_split(Usp[cur][0], Usp[cur][1], UPP, 0, 32 * ks), S[q]);
            }
        }
    };
    // Chunk n: U and the update (waves 0-3), the output of chunk n - 1
    // (waves 4-7); the last chunk's output follows the loop.  The
    // two roles run separate loops with the same two barriers per chunk, so
    // that each loop carries only its own operands from one chunk to the
    // next and waits for them only where they are used.
    if (urole) {
        for (int n = 0; n < N; ++n) {
            const int cur = n & 1;
            const int64_t tok0 = (int64_t)n * CHUNK;
            chunk_top(n);
            __syncthreads();
            if (n + 1 < N)
                load_k_tab(tok0 + CHUNK);
            // U rows [16 w, 16 w + 16) = W_v - W_k S_0
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const float x[8] = {wk[ks][0][0], wk[ks][0][1], wk[ks][0][2], wk[ks][0][3],
                                    wk[ks][1][0], wk[ks][1][1], wk[ks][1][2], wk[ks][1][3]};
                acc = mma(split8<T>(x), frag_rows_split(Ssp[cur][0], Ssp[cur][1], SPP, 0, 32 * ks), acc);
            }
            floatx4 u4;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                u4[r] = wv[r] - acc[r];
            if (n + 1 < N)
                load_wk_wv(tok0 + CHUNK);
            if (u_out)    // U for the backward, [B][H][T][DV]
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    u_out[(bh * (int64_t)N * CHUNK + tok0 + 16 * rb + 4 * g + r) * DV + cbase + t] = u4[r];
            put_split4(Usp[cur][0], Usp[cur][1], t * UPP + 16 * rb, u4);
            __syncthreads();
            update(n);
        }
    } else {
        for (int n = 0; n < N; ++n) {
            const int64_t tok0 = (int64_t)n * CHUNK;
            chunk_top(n);
            __syncthreads();
            if (n + 1 < N)
                load_k_tab(tok0 + CHUNK);
            if (n >= 1) {
                const floatx4 acc = out_tile(n - 1);
                load_q_p(tok0);
                const int64_t tp = tok0 - CHUNK;
                store_tile_t<OT>(O.head(b, h) + tp * O.st, O.st, 16 * rb, cbase, acc, rows_of(tp));
            }
            __syncthreads();
            update(n);
        }
        // the last chunk's output: its U was written before the loop's last
        // barrier, and no buffer is written after it
        const int64_t tp = (int64_t)(N - 1) * CHUNK;
        store_tile_t<OT>(O.head(b, h) + tp * O.st, O.st, 16 * rb, cbase, out_tile(N - 1), rows_of(tp));
    }
    if (urole)
#pragma unroll
        for (int q = 0; q < FPW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S_out[bh * DK * DV + (int64_t)(16 * (FPW * w + q) + 4 * g + r) * DV + cbase + t] = S[q][r];
}

// ---------------------------------------------------------------------------
// Backward.  With dO the chunk's output gradient and dS_C the gradient of
// the state leaving it (G, carried from later chunks):
//
//   dU   = P^T dO + K~ dS_C                         (K~ = K .* gamma_C/gamma)
//   dS_0 = (Q .* gamma)^T dO + gamma_C dS_C - W_k^T dU          (serial)
//   Y    = T^T dU,   dV = beta .* Y
//   dA   = -Y U^T,   M = dA .* (gamma_i / gamma_j) for j < i, else 0
//   dbeta_i = < V_i - gamma_i (K S_0)_i, Y_i > + sum_j M_ij k_i . k_j
//   dQ   = gamma .* (dO S_0^T) + [(dO U^T) .* D] K
//   dK   = [(dO U^T) .* D]^T Q + gamma_C/gamma .* (U dS_C^T)
//          - beta gamma .* (Y S_0^T) + beta .* (M K) + M^T (beta .* K)
//
// (through W = T R with T = (I + A)^{-1}: dT = dU ((I + A) U)^T, so
// dA = -T^T dT T^T = -Y U^T.)  The gate is not differentiated.
// ---------------------------------------------------------------------------

// Serial reverse walk over a piece's chunks for one (b, h) and gradient
// columns [16 cb, 16 cb + 16), 8 waves.  Writes dU ([B][H][T][DV] fp32), the
// gradient leaving every chunk (dS_C, per chunk [B][H][N][DK][DV]) and dS_in.
// Per chunk the gradient's chain is
//   dU   = P^T dO + (K .* gamma_C/gamma) dS_C        (waves 0-3: rows 16 w ..)
//   dS_0 = gamma_C dS_C + (Q .* gamma)^T dO - W_k^T dU  (waves 0-3: row blocks
//                                                   FPW w .. FPW w + FPW - 1)
// whose terms P^T dO and (Q .* gamma)^T dO do not depend on dS: waves 4-7
// form them for the next (earlier) chunk while waves 0-3 walk the current
// one, and pass them through LDS in the result-tile layout of the waves that
// add them.  Q, dO, the decay tables and those terms are double-buffered
// (chunk n in buffer n % 2); two barriers per chunk.
template <typename T, int DK, int DV, bool RAGGED>
__global__ __launch_bounds__(512) void delta_bscan_kernel(Act<const T> Q, Act<const T> K,
                                                          Act<const T> dO, Act<const float> Wk,
                                                          const float* __restrict__ Pm,
                                                          const float* __restrict__ tabs,
                                                          const float* dS_out,
                                                          float* dS_in, float* __restrict__ dU_out,
                                                          float* __restrict__ dsc_out, int H, int N, int tail)
{
    constexpr int NT = 512, NFB = DK / 16, FPW = NFB / 4;
    static_assert(NFB == 4 || NFB == 8, "d_k must be 64 or 128");
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD, OP = 16 + PAD;
    __shared__ __align__(16) T Qs[2][CHUNK * QP];
    __shared__ __align__(16) T dOs[2][CHUNK * OP];
    // the carried gradient and dU as bf16 hi/lo planes, transposed
    constexpr int SPP = DK + PAD, UPP = CHUNK + PAD;
    __shared__ __align__(16) T Gsp[2][16 * SPP];
    __shared__ __align__(16) T dUsp[2][16 * UPP];
    __shared__ __align__(16) float tab[2][TAB_SIZE];
    // the terms that do not depend on dS, per chunk: (Q .* gamma)^T dO as
    // NFB result tiles, then P^T dO as 4 (64 lanes x 4 values each)
    __shared__ __align__(16) float XY[2][(NFB + 4) * 256];

    const ColHead wg = xcd_col_head(H, gridDim.z);
    const int cb = wg.cb, h = wg.h, b = wg.b;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;
    const int cbase = 16 * cb;
    // roles: waves 0-3 walk the gradient (row block w of dU, feature blocks
    // FPW w .. of dS); waves 4-7 form the next chunk's dS-free terms (row
    // block w - 4 of P^T dO, feature blocks FPW (w - 4) .. of (Q .* gamma)^T dO)
    const bool chain = w < 4;
    const int rb = w & 3;
    if (chain)
        __builtin_amdgcn_s_setprio(1);

    floatx4 G[FPW];   // dS[16 fb + 4g + r][cbase + t], fb = FPW w + q
#pragma unroll
    for (int q = 0; q < FPW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            G[q][r] = chain && dS_out
                          ? dS_out[bh * DK * DV + (int64_t)(16 * (FPW * w + q) + 4 * g + r) * DV + cbase + t]
                          : 0.f;

    const T* qh = Q.head(b, h);
    const T* doh = dO.head(b, h);
    const float* th = tabs + bh * (int64_t)N * TAB_SIZE;
    // Operands only one wave reads go from global memory straight into the
    // registers of its products, in fragment layout, a chunk ahead: K rows
    // 16 w .. (dU's A operand) and the W_k columns of the wave's feature
    // blocks (the gradient update's W_k^T) in waves 0-3, P columns
    // 16 (w - 4) .. (P^T dO) in waves 4-7.  Q and dO, which waves 4-7 read
    // transposed, and the decay tables are staged through LDS by every wave.
    constexpr int NKS = DK / 32;
    // the last chunk may be partial (tail tokens): row reads are clamped to
    // its last token, Q and dO are zeroed past it in LDS, and dU is zero
    // there (the prep kernel's W_k and P are zero for those tokens)
    auto rows_of = [&](int64_t tk) { return RAGGED && tk / CHUNK == N - 1 ? tail : CHUNK; };
    const T* kh = K.head(b, h);
    const float* pcol = Pm + bh * (int64_t)N * CHUNK * CHUNK + 8 * g * CHUNK + 16 * rb + t;
    const float* wkcol = Wk.head(b, h) + (int64_t)(8 * g) * Wk.st + 16 * FPW * rb + t;
    RowFrag<T> kv[NKS];
    float pc[2][8], wkc[FPW][2][8];
    auto load_k = [&](int64_t tk) {
        const T* krow = kh + (tk + (RAGGED ? min(16 * rb + t, rows_of(tk) - 1) : 16 * rb + t)) * K.st + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            kv[ks].load(krow + 32 * ks);
    };
    auto load_p = [&](int64_t tk) {
#pragma unroll
        for (int js = 0; js < 2; ++js)
#pragma unroll
            for (int r = 0; r < 8; ++r)
                pc[js][r] = pcol[tk * CHUNK + (32 * js + r) * CHUNK];
    };
    auto load_wk = [&](int64_t tk) {
#pragma unroll
        for (int q = 0; q < FPW; ++q)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    wkc[q][ks][r] = wkcol[(tk + 32 * ks + r) * Wk.st + 16 * q];
    };
    constexpr int VEC = 16 / sizeof(T), PER = 16 / VEC;   // 16-byte vectors per dO slice row
    static_assert(CHUNK * PER <= NT, "chunk split");
    ChunkRegs<T, DK, NT> rq;
    floatx4 rtab = zero4();
    u32x4 rdo = {0u, 0u, 0u, 0u};
    auto load_q_do_tab = [&](int64_t tk) {
        if (threadIdx.x < TAB_SIZE / 4)
            rtab = *reinterpret_cast<const floatx4*>(th + tk / CHUNK * TAB_SIZE + 4 * threadIdx.x);
        chunk_load(rq, qh + tk * Q.st, Q.st, rows_of(tk));
        if (threadIdx.x < CHUNK * PER) {
            const int row = RAGGED ? min((int)threadIdx.x / PER, rows_of(tk) - 1) : (int)threadIdx.x / PER;
            const int col = VEC * (threadIdx.x % PER);
            rdo = *reinterpret_cast<const u32x4*>(doh + (tk + row) * dO.st + cbase + col);
        }
    };
    auto store_q_do_tab = [&](int m) {
        const int bf = m & 1, rows_m = rows_of((int64_t)m * CHUNK);
        chunk_store(rq, Qs[bf], QP, rows_m);
        if (threadIdx.x < CHUNK * PER) {
            const int row = threadIdx.x / PER, col = VEC * (threadIdx.x % PER);
            *reinterpret_cast<u32x4*>(dOs[bf] + row * OP + col) =
                !RAGGED || row < rows_m ? rdo : u32x4{0u, 0u, 0u, 0u};
        }
        if (threadIdx.x < TAB_SIZE / 4)
            *reinterpret_cast<floatx4*>(tab[bf] + 4 * threadIdx.x) = rtab;
    };
    // waves 4-7: chunk m's (Q .* gamma)^T dO tiles of feature blocks
    // FPW rb .. and P^T dO tile of row block rb, into XY[m % 2]
    auto free_terms = [&](int m) {
        const int bf = m & 1;
        float qf[2][8];
        slot_factors(tab[bf] + TAB_G, qf);
#pragma unroll
        for (int q = 0; q < FPW; ++q) {
            const int fb = FPW * rb + q;
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < CHUNK / 32; ++ks)
                acc = mma(split_scaled<T>(frag_cols(Qs[bf], QP, 16 * fb, 32 * ks), qf[ks]),
                          frag_cols(dOs[bf], OP, 0, 32 * ks), acc);
            *reinterpret_cast<floatx4*>(XY[bf] + (fb * 64 + l) * 4) = acc;
        }
        floatx4 acc = zero4();
#pragma unroll
        for (int js = 0; js < 2; ++js)
            if (js >= rb / 2)
                acc = mma(split8<T>(pc[js]), frag_cols(dOs[bf], OP, 0, 32 * js), acc);
        *reinterpret_cast<floatx4*>(XY[bf] + ((NFB + rb) * 64 + l) * 4) = acc;
    };

    // prologue: the last chunk's staged operands and dS-free terms
    const int64_t last = (int64_t)(N - 1) * CHUNK;
    load_q_do_tab(last);
    if (chain) {
        load_k(last);
        load_wk(last);
    } else {
        load_p(last);
    }
    store_q_do_tab(N - 1);
    if (N > 1)
        load_q_do_tab(last - CHUNK);
    __syncthreads();
    if (!chain) {
        free_terms(N - 1);
        if (N > 1)
            load_p(last - CHUNK);
    }

    // Chunk n (in reverse): the gradient's chain in waves 0-3, chunk n - 1's
    // dS-free terms in waves 4-7.  The two roles run separate loops with the
    // same two barriers per chunk, so that each loop carries only its own
    // operands from one chunk to the next.
    if (chain) {
        for (int n = N - 1; n >= 0; --n) {
            const int cur = n & 1;
            const int64_t tok0 = (int64_t)n * CHUNK;
            const int rows_n = rows_of(tok0);
#pragma unroll
            for (int q = 0; q < FPW; ++q) {
                put_split4(Gsp[0], Gsp[1], t * SPP + 16 * (FPW * w + q), G[q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int f = 16 * (FPW * w + q) + 4 * g + r;
                    dsc_out[((bh * N + n) * DK + f) * DV + cbase + t] = G[q][r];
                }
            }
            if (n > 0)
                store_q_do_tab(n - 1);
            __syncthreads();
            if (n > 1)
                load_q_do_tab(tok0 - 2 * CHUNK);
            const float gC = tab[cur][TAB_G + CHUNK - 1];

            // dU rows [16 w, 16 w + 16): P^T dO (j >= i) + (gamma_C/gamma_i) K dS_C
            {
                const floatx4 acc = *reinterpret_cast<const floatx4*>(XY[cur] + ((NFB + w) * 64 + l) * 4);
                floatx4 acc2 = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc2 = mma(kv[ks].frag(), frag_rows_split(Gsp[0], Gsp[1], SPP, 0, 32 * ks), acc2);
                if (n > 0)
                    load_k(tok0 - CHUNK);
                floatx4 u4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * w + 4 * g + r;
                    u4[r] = !RAGGED || i < rows_n ? acc[r] + tab[cur][TAB_F + i] * acc2[r] : 0.f;
                    dU_out[(bh * (int64_t)N * CHUNK + tok0 + i) * DV + cbase + t] = u4[r];
                }
                put_split4(dUsp[0], dUsp[1], t * UPP + 16 * w, u4);
            }
            __syncthreads();

            // dS <- gamma_C dS + (Q .* gamma)^T dO - W_k^T dU, this wave's row blocks
#pragma unroll
            for (int q = 0; q < FPW; ++q) {
                const int fb = FPW * w + q;
                const floatx4 acc = *reinterpret_cast<const floatx4*>(XY[cur] + (fb * 64 + l) * 4);
                floatx4 acc2 = zero4();
#pragma unroll
                for (int ks = 0; ks < CHUNK / 32; ++ks)
                    acc2 = mma(split8<T>(wkc[q][ks]), frag_rows_split(dUsp[0], dUsp[1], UPP, 0, 32 * ks), acc2);
                G[q] = gC * G[q] + acc - acc2;
            }
            if (n > 0)
                load_wk(tok0 - CHUNK);
        }
#pragma unroll
        for (int q = 0; q < FPW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dS_in[bh * DK * DV + (int64_t)(16 * (FPW * w + q) + 4 * g + r) * DV + cbase + t] = G[q][r];
    } else {
        for (int n = N - 1; n >= 0; --n) {
            const int64_t tok0 = (int64_t)n * CHUNK;
            if (n > 0)
                store_q_do_tab(n - 1);
            __syncthreads();
            if (n > 1)
                load_q_do_tab(tok0 - 2 * CHUNK);
            if (n > 0) {
                free_terms(n - 1);
                if (n > 1)
                    load_p(tok0 - 2 * CHUNK);
            }
            __syncthreads();
        }
    }
}

// Per chunk, first part: Y = T^T dU (written over dU), dV, M (written over
// T) and dbeta.  Workgroup = (chunk, h, b), 8 waves (its LDS holds one
// workgroup per CU); wave w owns token rows [16 rb, 16 rb + 16), rb = w % 4,
// and half of the column blocks of Y and dV (ch = w / 4) and of the row
// block's M tiles; the two waves of a row block add their shares of dbeta
// through LDS.
template <typename T, typename OT, int DK, int DV, bool RAGGED>
__global__ __launch_bounds__(512) void delta_bgrad1_kernel(Act<const T> K, Act<const T> V,
                                                           Act<const float> beta,
                                                           const float* __restrict__ tabs,
                                                           const float* __restrict__ s0,
                                                           const float* __restrict__ u,
                                                           float* __restrict__ Tm, float* __restrict__ dUY,
                                                           Act<OT> dVo, Act<float> dbeta, int H, int tail)
{
    constexpr int NT = 512;
    constexpr int PAD = Pad<T>::value;
    constexpr int KP = DK + PAD, SPP = DK + PAD;
    constexpr int UP = DV + 4, AP = CHUNK + 4;
    // One LDS region serves three phases in turn: T and dU (Y from them);
    // S_0 as bf16 hi/lo planes, transposed ([c][f]), for K S_0; then Y and U
    // for the gradient of A.
    constexpr int PH1 = (CHUNK * AP + CHUNK * UP) * 4;
    constexpr int PH2 = 2 * DV * SPP * (int)sizeof(T);
    constexpr int PH3 = 2 * CHUNK * UP * 4;
    constexpr int RBYTES = PH1 > PH2 ? (PH1 > PH3 ? PH1 : PH3) : (PH2 > PH3 ? PH2 : PH3);
    __shared__ __align__(16) T Ks[CHUNK * KP];
    __shared__ __align__(16) unsigned char region[RBYTES];
    __shared__ __align__(16) float tab[TAB_SIZE];
    __shared__ float bet[CHUNK];
    __shared__ float dbp[2][CHUNK];   // each column half's share of dbeta
    float* const Ts = reinterpret_cast<float*>(region);
    float* const dUs = Ts + CHUNK * AP;
    T* const S0h = reinterpret_cast<T*>(region);
    T* const S0l = S0h + DV * SPP;
    float* const Ys = reinterpret_cast<float*>(region);
    float* const Us = Ys + CHUNK * UP;

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z, N = gridDim.x;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    constexpr int NCB = DV / 16, CPW = NCB / 2;   // column blocks, per wave
    const int rb = w & 3, ch = w >> 2, cb0 = ch * CPW;
    const int64_t bh = (int64_t)b * H + h;
    const int64_t tok0 = (int64_t)n * CHUNK;
    float* Tc = Tm + (bh * N + n) * CHUNK * CHUNK;
    const float* S0 = s0 + (bh * N + n) * DK * DV;
    const float* uc = u + (bh * (int64_t)N * CHUNK + tok0) * DV;
    float* yc = dUY + (bh * (int64_t)N * CHUNK + tok0) * DV;
    const T* vh = V.head(b, h) + tok0 * V.st;
    // the last chunk may be partial: reads stay on its tokens, K and beta
    // are zero past them, and nothing is stored for them but workspace rows
    const int rows = RAGGED && n == N - 1 ? tail : CHUNK;

    // every global read of the kernel but S_0 is issued here, together:
    // beta, the decay tables, K, T, dU, U, and this lane's V values
    constexpr int NTV = CHUNK * CHUNK / 4 / NT, NUV = CHUNK * DV / 4 / NT;
    static_assert(NTV * NT * 4 == CHUNK * CHUNK && NUV * NT * 4 == CHUNK * DV, "chunk split");
    float bt = 0.f;
    floatx4 rtab = zero4(), rt[NTV], rdu[NUV], ru[NUV];
    if (threadIdx.x < CHUNK)
        bt = beta.ptr[b * beta.sb + h * beta.sh + (tok0 + (RAGGED ? min((int)threadIdx.x, rows - 1) : (int)threadIdx.x)) * beta.st];
    if (threadIdx.x < TAB_SIZE / 4)
        rtab = *reinterpret_cast<const floatx4*>(tabs + (bh * N + n) * TAB_SIZE + 4 * threadIdx.x);
    ChunkRegs<T, DK, NT> rk;
    chunk_load(rk, K.head(b, h) + tok0 * K.st, K.st, rows);
#pragma unroll
    for (int i = 0; i < NTV; ++i)
        rt[i] = *reinterpret_cast<const floatx4*>(Tc + 4 * (threadIdx.x + NT * i));
#pragma unroll
    for (int i = 0; i < NUV; ++i) {
        rdu[i] = *reinterpret_cast<const floatx4*>(yc + 4 * (threadIdx.x + NT * i));
        ru[i] = *reinterpret_cast<const floatx4*>(uc + 4 * (threadIdx.x + NT * i));
    }
    float vv[CPW][4];   // V[16 rb + 4 g + r][16 (cb0 + c) + t]
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            vv[c][r] = (float)vh[(RAGGED ? min(16 * rb + 4 * g + r, rows - 1) : 16 * rb + 4 * g + r) * V.st +
                                 16 * (cb0 + c) + t];

    if (threadIdx.x < CHUNK)
        bet[threadIdx.x] = !RAGGED || (int)threadIdx.x < rows ? bt : 0.f;
    if (threadIdx.x < TAB_SIZE / 4)
        *reinterpret_cast<floatx4*>(tab + 4 * threadIdx.x) = rtab;
    chunk_store(rk, Ks, KP, rows);
#pragma unroll
    for (int i = 0; i < NTV; ++i) {
        const int e = 4 * (threadIdx.x + NT * i);
        *reinterpret_cast<floatx4*>(Ts + (e / CHUNK) * AP + e % CHUNK) = rt[i];
    }
#pragma unroll
    for (int i = 0; i < NUV; ++i) {
        const int e = 4 * (threadIdx.x + NT * i);
        *reinterpret_cast<floatx4*>(dUs + (e / DV) * UP + e % DV) = rdu[i];
    }
    __syncthreads();

    // Y rows [16 rb, 16 rb + 16), this wave's column blocks:
    // Y[i][c] = sum_{m >= i} T[m][i] dU[m][c]
    floatx4 Y[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        Y[c] = zero4();
        for (int ms = rb / 2; ms < 2; ++ms)
            Y[c] = mma(split_cols_f32<T>(Ts, AP, 16 * rb, 32 * ms),
                       split_cols_f32<T>(dUs, UP, 16 * (cb0 + c), 32 * ms), Y[c]);
    }
    {
        // Y to the workspace (over dU, which every thread read before the
        // barrier above) and dV
        OT* dvh = dVo.head(b, h) + tok0 * dVo.st;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rb + 4 * g + r, col = 16 * (cb0 + c) + t;
                yc[i * DV + col] = Y[c][r];
                if (!RAGGED || i < rows)
                    dvh[i * dVo.st + col] = (OT)(bet[i] * Y[c][r]);
            }
    }
    // S_0 (fp32 [f][c]) in result-tile order: lane (g, t) of wave w takes
    // the tiles w, w + 8, ... of the NFB x NCB tiles (tile = fb NCB + cb)
    constexpr int NFB = DK / 16, SPW = NFB * NCB / 8;
    float sv[SPW][4];
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
        const int fb = (w + 8 * k) / NCB, cb = (w + 8 * k) % NCB;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sv[k][r] = S0[(16 * fb + 4 * g + r) * DV + 16 * cb + t];
    }
    __syncthreads();   // every wave has read T and dU
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
        const int fb = (w + 8 * k) / NCB, cb = (w + 8 * k) % NCB;
        put_split4(S0h, S0l, (16 * cb + t) * SPP + 16 * fb, floatx4{sv[k][0], sv[k][1], sv[k][2], sv[k][3]});
    }
    __syncthreads();

    // (K S_0) of rows 16 rb; z = V - gamma (K S_0); dbeta gets < z_i, Y_i >
    float db[4] = {0.f, 0.f, 0.f, 0.f};   // dbeta of rows 16 rb + 4g + r, this lane's columns
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        floatx4 ks0 = zero4();
#pragma unroll
        for (int fs = 0; fs < DK / 32; ++fs)
            ks0 = mma(frag_rows(Ks, KP, 16 * rb, 32 * fs),
                      frag_rows_split(S0h, S0l, SPP, 16 * (cb0 + c), 32 * fs), ks0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * rb + 4 * g + r;
            db[r] += (vv[c][r] - tab[TAB_G + i] * ks0[r]) * Y[c][r];
        }
    }
    __syncthreads();   // every wave has read S_0
    // Y and U to LDS (over S_0)
    {
        auto* ysv = (volatile __attribute__((address_space(3))) float*)Ys;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ysv[(16 * rb + 4 * g + r) * UP + 16 * (cb0 + c) + t] = Y[c][r];
    }
#pragma unroll
    for (int i = 0; i < NUV; ++i) {
        const int e = 4 * (threadIdx.x + NT * i);
        *reinterpret_cast<floatx4*>(Us + (e / DV) * UP + e % DV) = ru[i];
    }
    __syncthreads();
    // dA = -Y U^T (j < i), M = dA .* gamma_i / gamma_j, this wave's column
    // blocks jb = ch, ch + 2, ... of the row block; sum_j M_ij k_i . k_j
    // into dbeta
    for (int jb = ch; jb <= rb; jb += 2) {
        floatx4 dA = zero4(), gk = zero4();
#pragma unroll
        for (int cs = 0; cs < DV / 32; ++cs)
            dA = mma(split_rows_f32<T>(Ys, UP, 16 * rb, 32 * cs), split_rows_f32<T>(Us, UP, 16 * jb, 32 * cs), dA);
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            gk = mma(frag_rows(Ks, KP, 16 * rb, 32 * ks), frag_rows(Ks, KP, 16 * jb, 32 * ks), gk);
        const int j = 16 * jb + t;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * rb + 4 * g + r;
            const float m = j < i ? -dA[r] * __expf(tab[TAB_LAM + i] - tab[TAB_LAM + j]) : 0.f;
            Tc[i * CHUNK + j] = m;
            db[r] += m * gk[r];
        }
    }
    for (int jb = rb + 1 + ch; jb < 4; jb += 2)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Tc[(16 * rb + 4 * g + r) * CHUNK + 16 * jb + t] = 0.f;
    // row sums over the 16 lanes of a group, then over the row block's two
    // waves
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x = db[r];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        if (t == 0)
            dbp[ch][16 * rb + 4 * g + r] = x;
    }
    __syncthreads();
    if (threadIdx.x < CHUNK && (!RAGGED || (int)threadIdx.x < rows))
        dbeta.ptr[b * dbeta.sb + h * dbeta.sh + (tok0 + threadIdx.x) * dbeta.st] =
            dbp[0][threadIdx.x] + dbp[1][threadIdx.x];
}

// Per chunk, second part: dQ and dK.  Workgroup = (chunk, h, b), one wave
// per feature block (d_k / 16, at least 4); wave w owns feature blocks
// w, w + NW, ... of both, every row block.  The LDS holds one workgroup per
// CU, so the waves of that one workgroup are all the CU's latency hiding.
template <int DK>
constexpr int bgrad2_waves() { return DK / 16 >= 8 ? 8 : 4; }

template <typename T, typename OT, int DK, int DV, bool RAGGED>
__global__ __launch_bounds__(64 * bgrad2_waves<DK>()) void delta_bgrad2_kernel(Act<const T> Q, Act<const T> K, Act<const T> dO,
                                                           Act<const float> beta,
                                                           const float* __restrict__ tabs,
                                                           const float* __restrict__ s0,
                                                           const float* __restrict__ dsc,
                                                           const float* __restrict__ u,
                                                           const float* __restrict__ Y,
                                                           const float* __restrict__ Mg, Act<OT> dQo,
                                                           Act<OT> dKo, int H, int tail)
{
    constexpr int NW = bgrad2_waves<DK>(), NT = 64 * NW;
    constexpr int PAD = Pad<T>::value;
    constexpr int QP = DK + PAD, OP = DV + PAD;
    constexpr int UP = DV + 4, AP = CHUNK + 4;
    __shared__ __align__(16) T Qs[CHUNK * QP];
    __shared__ __align__(16) T Ks[CHUNK * QP];
    __shared__ __align__(16) T dOs[CHUNK * OP];
    __shared__ __align__(16) float Us[CHUNK * UP];
    __shared__ __align__(16) float Ys[CHUNK * UP];
    __shared__ __align__(16) float Ms[CHUNK * AP];
    __shared__ __align__(16) float dPs[CHUNK * AP];
    __shared__ __align__(16) float tab[TAB_SIZE];
    __shared__ float bet[CHUNK];

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z, N = gridDim.x;
    const int w = wave_id(), l = lane_id(), t = l & 15, g = l >> 4;
    const int64_t bh = (int64_t)b * H + h;
    const int64_t tok0 = (int64_t)n * CHUNK;
    const float* S0 = s0 + (bh * N + n) * DK * DV;
    const float* dSC = dsc + (bh * N + n) * DK * DV;
    const float* uc = u + (bh * (int64_t)N * CHUNK + tok0) * DV;
    const float* yc = Y + (bh * (int64_t)N * CHUNK + tok0) * DV;
    const float* Mc = Mg + (bh * N + n) * CHUNK * CHUNK;
    // the last chunk may be partial: reads stay on its tokens, Q, K, dO and
    // beta are zero past them, and no gradient is stored for them
    const int rows = RAGGED && n == N - 1 ? tail : CHUNK;

    // Wave w takes the feature blocks fb = w, w + 4, ... of dQ and dK, every
    // row block of each; the rows of S_0 and dS_C it needs (as B operands,
    // row 16 fb + t, columns 32 cs + 8 g ..) are read once, up front,
    // together with everything else the kernel reads.
    constexpr int NFB = DK / 16, FBW = NFB / NW, NCS = DV / 32;
    static_assert(FBW * NW == NFB, "d_k must be 64 or 128");
    constexpr int NUV = CHUNK * DV / 4 / NT, NMV = CHUNK * CHUNK / 4 / NT;
    static_assert(NUV * NT * 4 == CHUNK * DV && NMV * NT * 4 == CHUNK * CHUNK, "chunk split");
    float bt = 0.f;
    floatx4 rtab = zero4(), ru[NUV], ry[NUV], rm[NMV];
    floatx4 s0r[FBW][NCS][2], dsr[FBW][NCS][2];
    if (threadIdx.x < CHUNK)
        bt = beta.ptr[b * beta.sb + h * beta.sh + (tok0 + (RAGGED ? min((int)threadIdx.x, rows - 1) : (int)threadIdx.x)) * beta.st];
    if (threadIdx.x < TAB_SIZE / 4)
        rtab = *reinterpret_cast<const floatx4*>(tabs + (bh * N + n) * TAB_SIZE + 4 * threadIdx.x);
    ChunkRegs<T, DK, NT> rq, rk;
    ChunkRegs<T, DV, NT> ro;
    chunk_load(rq, Q.head(b, h) + tok0 * Q.st, Q.st, rows);
    chunk_load(rk, K.head(b, h) + tok0 * K.st, K.st, rows);
    chunk_load(ro, dO.head(b, h) + tok0 * dO.st, dO.st, rows);
#pragma unroll
    for (int i = 0; i < NUV; ++i) {
        ru[i] = *reinterpret_cast<const floatx4*>(uc + 4 * (threadIdx.x + NT * i));
        ry[i] = *reinterpret_cast<const floatx4*>(yc + 4 * (threadIdx.x + NT * i));
    }
#pragma unroll
    for (int i = 0; i < NMV; ++i)
        rm[i] = *reinterpret_cast<const floatx4*>(Mc + 4 * (threadIdx.x + NT * i));
#pragma unroll
    for (int q = 0; q < FBW; ++q)
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            const int off = (16 * (w + NW * q) + t) * DV + 32 * cs + 8 * g;
            s0r[q][cs][0] = *reinterpret_cast<const floatx4*>(S0 + off);
            s0r[q][cs][1] = *reinterpret_cast<const floatx4*>(S0 + off + 4);
            dsr[q][cs][0] = *reinterpret_cast<const floatx4*>(dSC + off);
            dsr[q][cs][1] = *reinterpret_cast<const floatx4*>(dSC + off + 4);
        }

    if (threadIdx.x < CHUNK)
        bet[threadIdx.x] = !RAGGED || (int)threadIdx.x < rows ? bt : 0.f;
    if (threadIdx.x < TAB_SIZE / 4)
        *reinterpret_cast<floatx4*>(tab + 4 * threadIdx.x) = rtab;
    chunk_store(rq, Qs, QP, rows);
    chunk_store(rk, Ks, QP, rows);
    chunk_store(ro, dOs, OP, rows);
#pragma unroll
    for (int i = 0; i < NUV; ++i) {
        const int e = 4 * (threadIdx.x + NT * i);
        *reinterpret_cast<floatx4*>(Us + (e / DV) * UP + e % DV) = ru[i];
        *reinterpret_cast<floatx4*>(Ys + (e / DV) * UP + e % DV) = ry[i];
    }
#pragma unroll
    for (int i = 0; i < NMV; ++i) {
        const int e = 4 * (threadIdx.x + NT * i);
        *reinterpret_cast<floatx4*>(Ms + (e / CHUNK) * AP + e % CHUNK) = rm[i];
    }
    __syncthreads();

    // dP .* D = (dO U^T) .* D, causal (incl. the diagonal)
    const bool fac = decay_factored(tab);
    for (int tile = w; tile < 16; tile += NW) {
        const int ib = tile >> 2, jb = tile & 3;
        floatx4 acc = zero4();
        if (jb <= ib) {
#pragma unroll
            for (int cs = 0; cs < DV / 32; ++cs)
                acc = mma(frag_rows(dOs, OP, 16 * ib, 32 * cs), split_rows_f32<T>(Us, UP, 16 * jb, 32 * cs), acc);
            acc = decay_mask<true>(acc, tab, 16 * ib, 16 * jb, fac);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dPs[(16 * ib + 4 * g + r) * AP + 16 * jb + t] = acc[r];
    }
    __syncthreads();

    OT* outq = dQo.head(b, h) + tok0 * dQo.st;
    OT* outk = dKo.head(b, h) + tok0 * dKo.st;
#pragma unroll
    for (int q = 0; q < FBW; ++q) {
        const int fb = w + NW * q;
        Split<T> s0f[NCS], dsf[NCS];
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            const float xs[8] = {s0r[q][cs][0][0], s0r[q][cs][0][1], s0r[q][cs][0][2], s0r[q][cs][0][3],
                                 s0r[q][cs][1][0], s0r[q][cs][1][1], s0r[q][cs][1][2], s0r[q][cs][1][3]};
            const float xd[8] = {dsr[q][cs][0][0], dsr[q][cs][0][1], dsr[q][cs][0][2], dsr[q][cs][0][3],
                                 dsr[q][cs][1][0], dsr[q][cs][1][1], dsr[q][cs][1][2], dsr[q][cs][1][3]};
            s0f[cs] = split8<T>(xs);
            dsf[cs] = split8<T>(xd);
        }
        for (int rb = 0; rb < 4; ++rb) {
            // dQ[i][f] = gamma_i (dO S_0^T)[i][f] + (dP .* D) K
            {
                floatx4 acc = zero4();
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs)
                    acc = mma(frag_rows(dOs, OP, 16 * rb, 32 * cs), s0f[cs], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] *= tab[TAB_G + 16 * rb + 4 * g + r];
                for (int js = 0; js <= rb / 2; ++js)
                    acc = mma(split_rows_f32<T>(dPs, AP, 16 * rb, 32 * js), frag_cols(Ks, QP, 16 * fb, 32 * js), acc);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!RAGGED || 16 * rb + 4 * g + r < rows)
                        outq[(16 * rb + 4 * g + r) * dQo.st + 16 * fb + t] = (OT)acc[r];
            }
            // dK[j][f]: five terms with different row factors
            {
                floatx4 acc = zero4(), a1 = zero4(), a2 = zero4(), a3 = zero4();
                for (int is = rb / 2; is < 2; ++is) {
                    // (dP .* D)^T Q  and  M^T (beta .* K)    (i >= j)
                    acc = mma(split_cols_f32<T>(dPs, AP, 16 * rb, 32 * is), frag_cols(Qs, QP, 16 * fb, 32 * is), acc);
                    float bf[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        bf[r] = bet[32 * is + 8 * g + r];
                    acc = mma(split_cols_f32<T>(Ms, AP, 16 * rb, 32 * is),
                              split_scaled<T>(frag_cols(Ks, QP, 16 * fb, 32 * is), bf), acc);
                }
                for (int is = 0; is <= rb / 2; ++is)   // M K  (i < j)
                    a3 = mma(split_rows_f32<T>(Ms, AP, 16 * rb, 32 * is), frag_cols(Ks, QP, 16 * fb, 32 * is), a3);
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs) {
                    a1 = mma(split_rows_f32<T>(Us, UP, 16 * rb, 32 * cs), dsf[cs], a1);
                    a2 = mma(split_rows_f32<T>(Ys, UP, 16 * rb, 32 * cs), s0f[cs], a2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * rb + 4 * g + r;
                    acc[r] += tab[TAB_F + j] * a1[r] - bet[j] * tab[TAB_G + j] * a2[r] + bet[j] * a3[r];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!RAGGED || 16 * rb + 4 * g + r < rows)
                        outk[(16 * rb + 4 * g + r) * dKo.st + 16 * fb + t] = (OT)acc[r];
            }
        }
    }
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
    // workspace rows cover whole chunks (Tp tokens); the last may be partial
    const int N = (s.T + CHUNK - 1) / CHUNK, tail = s.T - (N - 1) * CHUNK;
    const int64_t Tp = (int64_t)N * CHUNK;
    const Act<float> wk{s.wk, (int64_t)s.H * Tp * DK, Tp * DK, DK};
    const Act<float> wv{s.wv, (int64_t)s.H * Tp * DV, Tp * DV, DV};
    const unsigned parts = s.parts ? s.parts : DELTA_PREP | DELTA_SERIAL;
    return with_ragged(tail < CHUNK, [&](auto rg) {
        constexpr bool RG = decltype(rg)::value;
        if (parts & DELTA_PREP) {
            launch_kernel((delta_prep_kernel<T, DK, DV, RG>), dim3(N, s.H, s.B), dim3(256), stream,
                          dact<T>(s.q), dact<T>(s.k), dact<T>(s.v), dact<float>(s.beta), dec, wk, wv, s.pm,
                          nullptr, s.tabs, s.H, tail);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || !(parts & DELTA_SERIAL))
                return e;
        }
        launch_kernel((delta_scan_kernel<T, OT, DK, DV, RG>), dim3(DV / 16, s.H, s.B), dim3(512),
                      stream, dact<T>(s.q), dact<T>(s.k), Act<const float>{wk.ptr, wk.sb, wk.sh, wk.st},
                      Act<const float>{wv.ptr, wv.sb, wv.sh, wv.st}, (const float*)s.pm, (const float*)s.tabs,
                      s.S_in, s.S_out, Act<OT>{(OT*)s.o.ptr, s.o.sb, s.o.sh, s.o.st}, s.s0, s.u, s.H, N, tail);
        return hipGetLastError();
    });
}

template <typename T, typename OT, int DK, int DV>
hipError_t delta_bwd_impl(const DeltaBwdLaunch& s, hipStream_t stream)
{
    const DecayArg dec{(const float*)s.decay.ptr, s.decay.sb, s.decay.sh, s.decay.st, s.decay_kind};
    const int N = (s.T + CHUNK - 1) / CHUNK, tail = s.T - (N - 1) * CHUNK;
    const int64_t Tp = (int64_t)N * CHUNK;
    const Act<float> wk{s.wk, (int64_t)s.H * Tp * DK, Tp * DK, DK};
    const Act<float> wv{s.wv, (int64_t)s.H * Tp * DV, Tp * DV, DV};
    const unsigned parts = s.parts ? s.parts : DELTA_PREP | DELTA_SERIAL | DELTA_GRAD;
    return with_ragged(tail < CHUNK, [&](auto rg) {
        constexpr bool RG = decltype(rg)::value;
        hipError_t e = hipSuccess;
        if (parts & DELTA_PREP) {
            launch_kernel((delta_prep_kernel<T, DK, DV, RG>), dim3(N, s.H, s.B), dim3(256), stream,
                          dact<T>(s.q), dact<T>(s.k), dact<T>(s.v), dact<float>(s.beta), dec, wk, wv, s.pm,
                          s.tm, s.tabs, s.H, tail);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
        if (parts & DELTA_SERIAL) {
            launch_kernel((delta_bscan_kernel<T, DK, DV, RG>), dim3(DV / 16, s.H, s.B), dim3(512), stream,
                          dact<T>(s.q), dact<T>(s.k), dact<T>(s.dO),
                          Act<const float>{wk.ptr, wk.sb, wk.sh, wk.st}, (const float*)s.pm,
                          (const float*)s.tabs, s.dS_out, s.dS_in, s.duy, s.dsc, s.H, N, tail);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
        if (!(parts & DELTA_GRAD))
            return e;
        launch_kernel((delta_bgrad1_kernel<T, OT, DK, DV, RG>), dim3(N, s.H, s.B), dim3(512), stream,
                      dact<T>(s.k), dact<T>(s.v), dact<float>(s.beta), (const float*)s.tabs, (const float*)s.s0,
                      (const float*)s.u, s.tm, s.duy, Act<OT>{(OT*)s.dv_.ptr, s.dv_.sb, s.dv_.sh, s.dv_.st},
                      Act<float>{(float*)s.dbeta.ptr, s.dbeta.sb, s.dbeta.sh, s.dbeta.st}, s.H, tail);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        launch_kernel((delta_bgrad2_kernel<T, OT, DK, DV, RG>), dim3(N, s.H, s.B), dim3(64 * bgrad2_waves<DK>()), stream,
                      dact<T>(s.q), dact<T>(s.k), dact<T>(s.dO), dact<float>(s.beta), (const float*)s.tabs,
                      (const float*)s.s0, (const float*)s.dsc, (const float*)s.u, (const float*)s.duy,
                      (const float*)s.tm, Act<OT>{(OT*)s.dq.ptr, s.dq.sb, s.dq.sh, s.dq.st},
                      Act<OT>{(OT*)s.dk_.ptr, s.dk_.sb, s.dk_.sh, s.dk_.st}, s.H, tail);
        return hipGetLastError();
    });
}

}  // namespace

hipError_t launch_delta_bwd(const DeltaBwdLaunch& s, hipStream_t stream)
{
    if (s.dtype == 0 && s.dk == 128 && s.dv == 128)
        return s.out_dtype == 0 ? delta_bwd_impl<bf16, bf16, 128, 128>(s, stream)
                                : delta_bwd_impl<bf16, float, 128, 128>(s, stream);
    if (s.dtype == 0 && s.dk == 64 && s.dv == 64)
        return s.out_dtype == 0 ? delta_bwd_impl<bf16, bf16, 64, 64>(s, stream)
                                : delta_bwd_impl<bf16, float, 64, 64>(s, stream);
    if (s.dtype == 1 && s.dk == 64 && s.dv == 64 && s.out_dtype == 1)
        return delta_bwd_impl<float, float, 64, 64>(s, stream);
    return hipErrorInvalidValue;
}

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
