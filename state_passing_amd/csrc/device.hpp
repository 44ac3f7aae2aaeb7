// device.hpp -- gfx950 building blocks shared by the linear-recurrence kernels.
//
// Conventions (one wave = 64 lanes; lane l = 16*g + t, g = l/16, t = l%16):
//
//   MFMA 16x16, k = 32 per step ("k32 step").  An operand fragment holds 8
//   values per lane.  For A (M x K) lane (g,t) holds A[t][8g + r], r = 0..7;
//   for B (K x N) it holds B[8g + r][t].  The result tile D (16 x 16 fp32)
//   gives lane (g,t) the values D[4g + r][t], r = 0..3.
//     bf16: one v_mfma_f32_16x16x32_bf16 per k32 step.
//     fp32: eight v_mfma_f32_16x16x4_f32; sub-step r contracts the four
//           k-slots {8g + r : g = 0..3}, so both dtypes share one fragment
//           layout and any k-slot order shared by A and B is exact.
//
//   LDS tiles are row-major with a pitch in elements.  frag_rows() reads an
//   operand whose M/N index runs down LDS rows (k contiguous in a row: one
//   16-byte read for bf16); frag_cols() reads one whose k index runs down
//   LDS rows (gfx950 ds_read_b64_tr_b16 transposing reads for bf16, scalar
//   reads for fp32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

constexpr int CHUNK = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;
// 16 raw bytes as a native vector (HIP's uint4 is a struct: copies of it
// become memcpy calls that keep staging registers in private memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Decay description as the kernels see it (kind: 0 none, 1 per head, 2 per token).
struct DecayArg {
    const float* ptr;
    int64_t sb, sh, st;
    int kind;
};

// Strided activation view (element strides; the feature index is contiguous).
template <typename T>
struct Act {
    T* ptr;
    int64_t sb, sh, st;
    __device__ __forceinline__ T* head(int b, int h) const { return ptr + b * sb + h * sh; }
};

// LDS row padding.  32 bytes per row keep 16-byte row reads (frag_rows) and
// the transposing reads (frag_cols, frag_cols_perm) near the LDS peak.
template <typename T>
struct Pad { static constexpr int value = 32 / sizeof(T); };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
    bf16x8 v;
};
template <>
struct Frag<float> {
    float v[8];
};

__device__ __forceinline__ floatx4 mma(const Frag<bf16>& a, const Frag<bf16>& b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma(const Frag<float>& a, const Frag<float>& b, floatx4 c)
{
#pragma unroll
    for (int r = 0; r < 8; ++r)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[r], b.v[r], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// ---- fragment reads from LDS -------------------------------------------

// lane (g,t) <- tile[rbase + t][kbase + 8g + r]
__device__ __forceinline__ Frag<bf16> frag_rows(const bf16* tile, int pitch, int rbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(tile + (rbase + t) * pitch + kbase + 8 * g);
    return f;
}

__device__ __forceinline__ Frag<float> frag_rows(const float* tile, int pitch, int rbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const float4* p = reinterpret_cast<const float4*>(tile + (rbase + t) * pitch + kbase + 8 * g);
    const float4 a = p[0], b = p[1];
    Frag<float> f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}

// lane (g,t) <- tile[kbase + 8g + r][cbase + t]
// ds_read_b64_tr_b16: within each 16-lane group, lane t addresses row
// R + t/4, columns c0 + 4(t%4) .. +3, and receives column c0 + t of rows
// R .. R+3.  Two reads cover the 8 k-slots.
__device__ __forceinline__ Frag<bf16> frag_cols(const bf16* tile, int pitch, int cbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const bf16* p = tile + (kbase + 8 * g + (t >> 2)) * pitch + cbase + 4 * (t & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * pitch));
    Frag<bf16> f;
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return f;
}

__device__ __forceinline__ Frag<float> frag_cols(const float* tile, int pitch, int cbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    Frag<float> f;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        f.v[r] = tile[(kbase + 8 * g + r) * pitch + cbase + t];
    return f;
}

// Fragments in the k-slot order of a pair of 16x16 result tiles: slot r < 4
// is k = kbase + 4g + r (first tile's rows), slot r >= 4 is k = kbase + 16 +
// 4g + (r - 4) (second tile's rows).  A result tile held in registers can
// then serve as the other operand without moving between lanes.
//   frag_cols_perm: lane (g,t) <- tile[k(slot)][cbase + t]
// (a row read in that order is frag_rows() of a tile staged with
// chunk_store_perm()).
__device__ __forceinline__ Frag<bf16> frag_cols_perm(const bf16* tile, int pitch, int cbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const bf16* p = tile + (kbase + 4 * g + (t >> 2)) * pitch + cbase + 4 * (t & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * pitch));
    Frag<bf16> f;
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return f;
}

__device__ __forceinline__ Frag<float> frag_cols_perm(const float* tile, int pitch, int cbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    Frag<float> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f.v[r] = tile[(kbase + 4 * g + r) * pitch + cbase + t];
        f.v[4 + r] = tile[(kbase + 16 + 4 * g + r) * pitch + cbase + t];
    }
    return f;
}

// A chunk's rows of one activation (64 x D elements) spread over the NT
// threads of a workgroup as 16-byte vectors: chunk_load() issues the global
// loads into registers, chunk_store() later writes them to LDS, so the loads
// of the next chunk can be in flight while the current one is processed.
template <typename T, int D, int NT>
struct ChunkRegs {
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int PER_ROW = D / VEC;
    static constexpr int NV = CHUNK * PER_ROW / NT;
    static_assert(NV * NT == CHUNK * PER_ROW && NV >= 1 && NV <= 4,
                  "chunk must split evenly over the threads, 1 to 4 vectors each");
    u32x4 v0, v1, v2, v3;
};

template <int P, typename R>
__device__ __forceinline__ u32x4& chunk_vec(R& r)
{
    if constexpr (P == 0)
        return r.v0;
    else if constexpr (P == 1)
        return r.v1;
    else if constexpr (P == 2)
        return r.v2;
    else
        return r.v3;
}

// d = s, vector by vector (only the NV vectors in use).
template <typename T, int D, int NT>
__device__ __forceinline__ void chunk_copy(ChunkRegs<T, D, NT>& d, const ChunkRegs<T, D, NT>& s)
{
    constexpr int NV = ChunkRegs<T, D, NT>::NV;
    d.v0 = s.v0;
    if constexpr (NV > 1)
        d.v1 = s.v1;
    if constexpr (NV > 2)
        d.v2 = s.v2;
    if constexpr (NV > 3)
        d.v3 = s.v3;
}

template <int P, typename T, int D, int NT>
__device__ __forceinline__ void chunk_load_one(ChunkRegs<T, D, NT>& r, const T* src, int64_t ld, int rows)
{
    typedef ChunkRegs<T, D, NT> R;
    if constexpr (P < R::NV) {
        const int idx = threadIdx.x + NT * P, row = idx / R::PER_ROW, col = (idx % R::PER_ROW) * R::VEC;
        // no branch: a row past the end reads the last row that exists;
        // chunk_store() writes zeros in its place
        chunk_vec<P>(r) = *reinterpret_cast<const u32x4*>(src + min(row, rows - 1) * ld + col);
    }
}

template <int P, typename T, int D, int NT>
__device__ __forceinline__ void chunk_store_one(ChunkRegs<T, D, NT>& r, T* lds, int pitch)
{
    typedef ChunkRegs<T, D, NT> R;
    if constexpr (P < R::NV) {
        const int idx = threadIdx.x + NT * P, row = idx / R::PER_ROW, col = (idx % R::PER_ROW) * R::VEC;
        *reinterpret_cast<u32x4*>(lds + row * pitch + col) = chunk_vec<P>(r);
    }
}

// Zeros over the rows >= rows of what chunk_store_one<P> wrote, by the same
// thread (so it lands after that thread's own store).
template <int P, typename T, int D, int NT>
__device__ __forceinline__ void chunk_zero_one(T* lds, int pitch, int rows)
{
    typedef ChunkRegs<T, D, NT> R;
    if constexpr (P < R::NV) {
        const int idx = threadIdx.x + NT * P, row = idx / R::PER_ROW, col = (idx % R::PER_ROW) * R::VEC;
        if (row >= rows)
            *reinterpret_cast<u32x4*>(lds + row * pitch + col) = u32x4{0u, 0u, 0u, 0u};
    }
}

// rows: the chunk's tokens that exist (1..64; the last chunk of a piece may
// be partial); nothing past them is read (chunk_store() with the same rows
// writes zeros for them).
template <typename T, int D, int NT>
__device__ __forceinline__ void chunk_load(ChunkRegs<T, D, NT>& r, const T* src, int64_t ld,
                                           int rows = CHUNK)
{
    chunk_load_one<0>(r, src, ld, rows);
    chunk_load_one<1>(r, src, ld, rows);
    chunk_load_one<2>(r, src, ld, rows);
    chunk_load_one<3>(r, src, ld, rows);
}

// rows: as given to the chunk_load() that filled r; rows past them are
// written as zeros (only a piece's last chunk can be partial, and whole
// chunks take no extra instruction but one uniform branch).
template <typename T, int D, int NT>
__device__ __forceinline__ void chunk_store(ChunkRegs<T, D, NT>& r, T* lds, int pitch, int rows = CHUNK)
{
    chunk_store_one<0>(r, lds, pitch);
    chunk_store_one<1>(r, lds, pitch);
    chunk_store_one<2>(r, lds, pitch);
    chunk_store_one<3>(r, lds, pitch);
    if (rows < CHUNK) {
        chunk_zero_one<0, T, D, NT>(lds, pitch, rows);
        chunk_zero_one<1, T, D, NT>(lds, pitch, rows);
        chunk_zero_one<2, T, D, NT>(lds, pitch, rows);
        chunk_zero_one<3, T, D, NT>(lds, pitch, rows);
    }
}

// chunk_store() into a tile whose rows hold the k index permuted so that
// the k-slot order of the result tiles becomes contiguous: within every 32
// elements, the 4-element unit u (k = 4u .. 4u + 3) sits at unit position
// 2 (u % 4) + u / 4.  frag_rows() of such a tile then returns exactly what
// two 8-byte reads at k and k + 16 would return from the plain tile, with one 16-byte read; two
// such tiles contract correctly with each other as well.
__device__ __forceinline__ int perm_unit(int u) { return 8 * (u >> 3) + 2 * (u & 3) + ((u >> 2) & 1); }

template <int P, typename T, int D, int NT>
__device__ __forceinline__ void chunk_store_perm_one(ChunkRegs<T, D, NT>& r, T* lds, int pitch)
{
    typedef ChunkRegs<T, D, NT> R;
    if constexpr (P < R::NV) {
        const int idx = threadIdx.x + NT * P, row = idx / R::PER_ROW, col = (idx % R::PER_ROW) * R::VEC;
        const u32x4 v = chunk_vec<P>(r);
        T* base = lds + row * pitch;
        if constexpr (sizeof(T) == 2) {   // two 4-element units per vector
            const int u = col / 4;
            *reinterpret_cast<u32x2*>(base + 4 * perm_unit(u)) = u32x2{v.x, v.y};
            *reinterpret_cast<u32x2*>(base + 4 * perm_unit(u + 1)) = u32x2{v.z, v.w};
        } else {                           // one unit per vector
            *reinterpret_cast<u32x4*>(base + 4 * perm_unit(col / 4)) = v;
        }
    }
}

// Zeros at the permuted positions chunk_store_perm_one<P> wrote, for rows >=
// rows, by the same thread.
template <int P, typename T, int D, int NT>
__device__ __forceinline__ void chunk_zero_perm_one(T* lds, int pitch, int rows)
{
    typedef ChunkRegs<T, D, NT> R;
    if constexpr (P < R::NV) {
        const int idx = threadIdx.x + NT * P, row = idx / R::PER_ROW, col = (idx % R::PER_ROW) * R::VEC;
        if (row >= rows) {
            T* base = lds + row * pitch;
            if constexpr (sizeof(T) == 2) {
                const int u = col / 4;
                *reinterpret_cast<u32x2*>(base + 4 * perm_unit(u)) = u32x2{0u, 0u};
                *reinterpret_cast<u32x2*>(base + 4 * perm_unit(u + 1)) = u32x2{0u, 0u};
            } else {
                *reinterpret_cast<u32x4*>(base + 4 * perm_unit(col / 4)) = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
}

template <typename T, int D, int NT>
__device__ __forceinline__ void chunk_store_perm(ChunkRegs<T, D, NT>& r, T* lds, int pitch,
                                                 int rows = CHUNK)
{
    chunk_store_perm_one<0>(r, lds, pitch);
    chunk_store_perm_one<1>(r, lds, pitch);
    chunk_store_perm_one<2>(r, lds, pitch);
    chunk_store_perm_one<3>(r, lds, pitch);
    if (rows < CHUNK) {
        chunk_zero_perm_one<0, T, D, NT>(lds, pitch, rows);
        chunk_zero_perm_one<1, T, D, NT>(lds, pitch, rows);
        chunk_zero_perm_one<2, T, D, NT>(lds, pitch, rows);
        chunk_zero_perm_one<3, T, D, NT>(lds, pitch, rows);
    }
}

// ---- decay ----------------------------------------------------------------

// The raw decay this lane needs for the chunk starting at tok0 (token = lane
// for per-token decay), so that it can be loaded a chunk ahead.
// rows: the chunk's tokens that exist; a lane past them reads the last
// one (no branch) and decay_tables() with the same rows gives it decay 1.
__device__ __forceinline__ float decay_raw(const DecayArg& d, int b, int h, int64_t tok0,
                                          int rows = CHUNK)
{
    if (d.kind == 0)
        return 1.f;
    if (d.kind == 1)
        return d.ptr[h * d.sh];
    return d.ptr[b * d.sb + h * d.sh + (tok0 + min(lane_id(), rows - 1)) * d.st];
}

// Inclusive cumulative log of the chunk's decays from decay_raw() values
// (token = lane); called by a full wave.
__device__ __forceinline__ float decay_log_cumsum(const DecayArg& d, float raw, int rows = CHUNK)
{
    const int lane = lane_id();
    if (d.kind == 0)
        return 0.f;
    // tokens past `rows` decay by 1
    if (d.kind == 1)
        return (float)(min(lane, rows - 1) + 1) * logf(raw);
    float x = lane < rows ? logf(raw) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off)
            x += y;
    }
    return x;
}

// Per-chunk decay tables in LDS, indexed by token within the chunk:
//   lam  chunk-local inclusive cumulative log-decay,
//   G    gamma   = exp(lam),
//   F    gamma_C / gamma = exp(lam_C - lam)   (in (0, 1]),
//   E    gamma / gamma_C = exp(lam - lam_C)   (>= 1; clamped),
// so that D_ij = exp(lam_i - lam_j) = E_i F_j.  The product form is used
// only when the chunk's total log-decay lam_C is at least FACTOR_MIN_LOG,
// which keeps E far from overflow; otherwise masks take one exp per entry.
enum { TAB_LAM = 0, TAB_G = CHUNK, TAB_F = 2 * CHUNK, TAB_E = 3 * CHUNK, TAB_SIZE = 4 * CHUNK };
constexpr float FACTOR_MIN_LOG = -40.f;

// Fill the tables from decay_raw() values (token = lane); one full wave.
__device__ __forceinline__ void decay_tables(const DecayArg& d, float raw, float* tab, int rows = CHUNK)
{
    const int l = lane_id();
    const float lam = decay_log_cumsum(d, raw, rows);
    const float lamC = __shfl(lam, CHUNK - 1, 64);
    tab[TAB_LAM + l] = lam;
    tab[TAB_G + l] = __expf(lam);
    tab[TAB_F + l] = __expf(lamC - lam);
    tab[TAB_E + l] = __expf(fminf(lam - lamC, 80.f));
}

// Whether the chunk's masks may use the E F product (wave-uniform).
__device__ __forceinline__ bool decay_factored(const float* tab)
{
    return __builtin_amdgcn_readfirstlane((int)(tab[TAB_LAM + CHUNK - 1] >= FACTOR_MIN_LOG)) != 0;
}

// Causal decay mask of a 16x16 score tile in result layout (lane (g,t)
// holds rows rbase + 4g + r, column cbase + t).  LATER_ROWS: the rows are
// the later token i and the column the earlier token j, else the reverse.
// Entries with j > i become 0, the others are multiplied by D_ij.
template <bool LATER_ROWS>
__device__ __forceinline__ floatx4 decay_mask(floatx4 x, const float* tab, int rbase, int cbase,
                                              bool factored)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const int c = cbase + t;
    floatx4 y;
    if (factored) {
        const floatx4 rv =
            *reinterpret_cast<const floatx4*>(tab + (LATER_ROWS ? TAB_E : TAB_F) + rbase + 4 * g);
        const float cv = tab[(LATER_ROWS ? TAB_F : TAB_E) + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = rbase + 4 * g + r;
            const bool keep = LATER_ROWS ? rr >= c : rr <= c;
            y[r] = keep ? x[r] * (rv[r] * cv) : 0.f;
        }
    } else {
        const floatx4 rl = *reinterpret_cast<const floatx4*>(tab + TAB_LAM + rbase + 4 * g);
        const float cl = tab[TAB_LAM + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = rbase + 4 * g + r;
            const bool keep = LATER_ROWS ? rr >= c : rr <= c;
            y[r] = keep ? x[r] * __expf(LATER_ROWS ? rl[r] - cl : cl - rl[r]) : 0.f;
        }
    }
    return y;
}

// Per-lane factors for the k-slots of a frag_cols() read over tokens (slot
// r of k32 step ks is token 32ks + 8g + r), from one decay table.
__device__ __forceinline__ void slot_factors(const float* table, float (&f)[2][8])
{
    const int g = lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(table + 32 * ks + 8 * g);
        const floatx4 b = *reinterpret_cast<const floatx4*>(table + 32 * ks + 8 * g + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f[ks][r] = a[r];
            f[ks][4 + r] = b[r];
        }
    }
}

// ---- split operands ---------------------------------------------------------
//
// A computed MFMA operand (P, the decay-scaled K or Q, a carried state) is
// not a bf16 input, and rounding it to bf16 once would cost about 2^-9 of
// relative accuracy per element.  It is therefore carried as hi + lo, two
// bf16 values whose sum holds ~16 significant bits, and multiplied against
// the exact bf16 activation with two MFMAs.  For fp32 activations the fp32
// MFMA is used directly and there is no remainder.
template <typename T>
struct Split;
template <>
struct Split<bf16> {
    Frag<bf16> hi, lo;
};
template <>
struct Split<float> {
    Frag<float> hi;
};

// hi = x with its low 16 mantissa bits cleared (exactly the upper half of
// the fp32 pattern, so a bf16 by truncation), lo = bf16(x - hi) rounded to
// nearest even; x - hi is exact, and hi + lo carries ~16 significant bits.
// Two values at a time: hi and lo each come back as one packed bf16 pair.
// Returns {hi pair, lo pair}.
__device__ __forceinline__ u32x2 split2(float x0, float x1)
{
    const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
    const float r0 = x0 - __uint_as_float(b0 & 0xffff0000u);
    const float r1 = x1 - __uint_as_float(b1 & 0xffff0000u);
    const bf16x2 l = {(bf16)r0, (bf16)r1};
    return u32x2{(b1 & 0xffff0000u) | (b0 >> 16), __builtin_bit_cast(uint32_t, l)};
}

template <typename T>
__device__ __forceinline__ Split<T> split8(const float (&x)[8]);

template <>
__device__ __forceinline__ Split<bf16> split8<bf16>(const float (&x)[8])
{
    const u32x2 p0 = split2(x[0], x[1]), p1 = split2(x[2], x[3]);
    const u32x2 p2 = split2(x[4], x[5]), p3 = split2(x[6], x[7]);
    const u32x4 h = {p0.x, p1.x, p2.x, p3.x}, l = {p0.y, p1.y, p2.y, p3.y};
    Split<bf16> s;
    s.hi.v = __builtin_bit_cast(bf16x8, h);
    s.lo.v = __builtin_bit_cast(bf16x8, l);
    return s;
}

template <>
__device__ __forceinline__ Split<float> split8<float>(const float (&x)[8])
{
    Split<float> s;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        s.hi.v[r] = x[r];
    return s;
}

__device__ __forceinline__ floatx4 mma(const Frag<bf16>& a, const Split<bf16>& b, floatx4 c)
{
    return mma(a, b.lo, mma(a, b.hi, c));
}
__device__ __forceinline__ floatx4 mma(const Split<bf16>& a, const Frag<bf16>& b, floatx4 c)
{
    return mma(a.lo, b, mma(a.hi, b, c));
}
__device__ __forceinline__ floatx4 mma(const Frag<float>& a, const Split<float>& b, floatx4 c)
{
    return mma(a, b.hi, c);
}
__device__ __forceinline__ floatx4 mma(const Split<float>& a, const Frag<float>& b, floatx4 c)
{
    return mma(a.hi, b, c);
}

// Split operand from two 16x16 result tiles in registers (k-slot order of
// the result tiles).
template <typename T>
__device__ __forceinline__ Split<T> split_tiles(const floatx4& a, const floatx4& b)
{
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return split8<T>(x);
}

// Split operand from a fragment of exact inputs times a per-slot factor.
template <typename T>
__device__ __forceinline__ Split<T> split_scaled(const Frag<T>& f, const float (&s)[8])
{
    float x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        x[r] = (float)f.v[r] * s[r];
    return split8<T>(x);
}


// Product of two computed operands, each a hi + lo pair: hi.hi + hi.lo +
// lo.hi (the lo.lo term lies below fp32 rounding).
__device__ __forceinline__ floatx4 mma(const Split<bf16>& a, const Split<bf16>& b, floatx4 c)
{
    return mma(a.lo, b.hi, mma(a.hi, b.lo, mma(a.hi, b.hi, c)));
}
__device__ __forceinline__ floatx4 mma(const Split<float>& a, const Split<float>& b, floatx4 c)
{
    return mma(a.hi, b.hi, c);
}

// Split operands read from an fp32 LDS tile: frag_rows() / frag_cols()
// patterns (k contiguous in a row, or k running down the rows).
template <typename T>
__device__ __forceinline__ Split<T> split_rows_f32(const float* tile, int pitch, int rbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const float* p = tile + (rbase + t) * pitch + kbase + 8 * g;
    const floatx4 a = *reinterpret_cast<const floatx4*>(p);
    const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return split8<T>(x);
}

template <typename T>
__device__ __forceinline__ Split<T> split_cols_f32(const float* tile, int pitch, int cbase, int kbase)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    float x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        x[r] = tile[(kbase + 8 * g + r) * pitch + cbase + t];
    return split8<T>(x);
}

// Split fragments read from LDS plane pairs.
template <typename T>
__device__ __forceinline__ Split<T> frag_rows_split(const T* hi, const T* lo, int pitch, int rbase, int kbase)
{
    Split<T> s;
    s.hi = frag_rows(hi, pitch, rbase, kbase);
    if constexpr (sizeof(T) == 2)
        s.lo = frag_rows(lo, pitch, rbase, kbase);
    return s;
}

template <typename T>
__device__ __forceinline__ Split<T> frag_cols_split(const T* hi, const T* lo, int pitch, int cbase, int kbase)
{
    Split<T> s;
    s.hi = frag_cols(hi, pitch, cbase, kbase);
    if constexpr (sizeof(T) == 2)
        s.lo = frag_cols(lo, pitch, cbase, kbase);
    return s;
}

// Write the 4 values of a result tile a lane holds (rows 4g + r, column t) as
// four consecutive elements of an LDS row of a plane pair (the tile lands
// transposed: LDS row = tile column).
template <typename T>
__device__ __forceinline__ void put_split4(T* hi, T* lo, int idx, const floatx4& x)
{
    // idx: the lane's row and the tile's first column; lane (g, t) holds
    // columns 4g .. 4g + 3 of that row.  bf16: lanes g and g ^ 1 trade
    // halves (v_permlane16_swap swaps odd 16-lane rows of one register with
    // even rows of the other), so that even g writes the hi plane and odd g
    // the lo plane, each 8 consecutive columns in one 16-byte store: 16
    // lanes at 16 rows with 8-byte stores conflict in the LDS banks.
    const int g = lane_id() >> 4;
    if constexpr (sizeof(T) == 2) {
        const u32x2 p0 = split2(x[0], x[1]), p1 = split2(x[2], x[3]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(p0.x, p0.y, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(p1.x, p1.y, false, false);
        T* plane = (g & 1) ? lo : hi;
        *reinterpret_cast<u32x4*>(plane + idx + 8 * (g >> 1)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    } else {
        *reinterpret_cast<floatx4*>(hi + idx + 4 * g) = x;
    }
}

// Four consecutive values of an activation row as fp32.
__device__ __forceinline__ floatx4 load4(const bf16* p)
{
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ floatx4 load4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

// Store a 16x16 fp32 result tile computed transposed (lane (g,t) holds
// rows 4g + r of the transpose, i.e. row rbase + t, columns cbase + 4g + r of
// the output) to row-major global memory as OT: one 8-byte (bf16) or 16-byte
// (fp32) store per lane.
template <typename OT>
__device__ __forceinline__ void store_tile_t(OT* base, int64_t ld, int rbase, int cbase, floatx4 acc,
                                             int rows = CHUNK);

template <>
__device__ __forceinline__ void store_tile_t<bf16>(bf16* base, int64_t ld, int rbase, int cbase, floatx4 acc,
                                                   int rows)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    const bf16x4 v = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
    bf16x4* p = reinterpret_cast<bf16x4*>(base + (rbase + t) * ld + cbase + 4 * g);
    if (rows >= CHUNK)           // wave-uniform: whole chunks store without lane masks
        *p = v;
    else if (rbase + t < rows)
        *p = v;
}

template <>
__device__ __forceinline__ void store_tile_t<float>(float* base, int64_t ld, int rbase, int cbase, floatx4 acc,
                                                    int rows)
{
    const int l = lane_id(), t = l & 15, g = l >> 4;
    floatx4* p = reinterpret_cast<floatx4*>(base + (rbase + t) * ld + cbase + 4 * g);
    if (rows >= CHUNK)
        *p = acc;
    else if (rbase + t < rows)
        *p = acc;
}

}  // namespace linrec
