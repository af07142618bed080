// clr_device.h -- device-side building blocks for the gfx950 (CDNA4) kernels.
//
// Matrix products use the wave64 matrix cores through one abstraction: a
// "k32 step" multiplies a 16 x 32 A tile by a 32 x 16 B tile into a 16 x 16
// fp32 accumulator tile.
//
//   lane l, r = l & 15, g = l >> 4 (0..3)
//   accumulator (D) tile:  lane holds D[4g + i][r],            i = 0..3
//   A fragment:            lane holds A[r][kmap(g, i)],        i = 0..7
//   B fragment:            lane holds B[kmap(g, i)][r],        i = 0..7
//   kmap(g, i) = 4g + i for i < 4,  16 + 4g + (i - 4) for i >= 4.
//
// The k ordering inside an MFMA is immaterial as long as A and B agree, and
// this kmap makes two vertically adjacent accumulator tiles (rows 0..15 and
// 16..31 of a 32-row block) *exactly* a B fragment, and the transpose of an
// A fragment.  Chained products therefore stay in registers.
//
// bf16 elements use v_mfma_f32_16x16x32_bf16 (one instruction per k32 step);
// fp32 elements use eight v_mfma_f32_16x16x4_f32 (lane group g supplies k
// slot g of each).  Accumulation is fp32 in both cases.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace clr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BLK = 64;  // tokens per kernel-level block (chunk)

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// XCD-aware placement of the sequential scans.  Work-groups are dispatched to
// the 8 XCDs round-robin (group i -> XCD i % 8) and each XCD has its own L2.
// All value slices of one (batch, head) read the same per-block operands, so
// they are put on one XCD: group w -> (batch * H + head) index
// p = (w % 8) + 8 * (w / (8 NV)), value slice vb = (w / 8) % NV.
// Returns false for the padding groups of the last round (p >= BH).
constexpr int NXCD = 8;
__device__ __forceinline__ bool scan_coords(int w, int NV, int BH, int H, int& b, int& h, int& vb) {
    const int p = (w % NXCD) + NXCD * (w / (NXCD * NV));
    vb = (w / NXCD) % NV;
    if (p >= BH) return false;
    b = p / H;
    h = p % H;
    return true;
}
__device__ __forceinline__ bool scan_coords(int NV, int BH, int H, int& b, int& h, int& vb) {
    return scan_coords((int)blockIdx.x, NV, BH, H, b, h, vb);
}
inline unsigned scan_grid(int NV, int BH) { return (unsigned)(((BH + NXCD - 1) / NXCD) * NXCD * NV); }

// ---------------------------------------------------------------------------
// Fragments
// ---------------------------------------------------------------------------
template <typename E> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };
// A fragment's eight elements as fp32 (lo: elements 0..3, hi: 4..7).
__device__ __forceinline__ Frag<float> widen(const Frag<float>& x) { return x; }
__device__ __forceinline__ Frag<float> widen(const Frag<bf16>& x) {
    Frag<float> y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        y.lo[i] = (float)x.v[i];
        y.hi[i] = (float)x.v[4 + i];
    }
    return y;
}

// Four contiguous elements <-> f32x4.
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const bf16* p) {
    bf16x4 t = *(const bf16x4*)p;
    return f32x4{(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void st4(bf16* p, f32x4 v) {
    bf16x4 t;
    t[0] = (bf16)v[0]; t[1] = (bf16)v[1]; t[2] = (bf16)v[2]; t[3] = (bf16)v[3];
    *(bf16x4*)p = t;
}

// A fragment from a row-major tile whose k index is contiguous:
// p points at X[m0 + r][k0 + 4g]; the second half is 16 elements further.
__device__ __forceinline__ Frag<bf16> ldfrag(const bf16* p) {
    Frag<bf16> f;
    bf16x4 a = *(const bf16x4*)p;
    bf16x4 b = *(const bf16x4*)(p + 16);
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}
__device__ __forceinline__ Frag<float> ldfrag(const float* p) {
    Frag<float> f;
    f.lo = *(const f32x4*)p;
    f.hi = *(const f32x4*)(p + 16);
    return f;
}
// ldfrag of row `row` of a token-major tile (row stride ld), zero if the
// row lies past the end of the sequence (row >= nvalid).
template <typename E>
__device__ __forceinline__ Frag<E> ldfrag_row(const E* base, int row, int nvalid, size_t ld, int col) {
    if (row < nvalid) return ldfrag(base + (size_t)row * ld + col);
    Frag<E> f;
    if constexpr (sizeof(E) == 2) {
        f.v = bf16x8{};
    } else {
        f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
        f.hi = f.lo;
    }
    return f;
}

// A fragment whose elements are scaled by s[i] (per k index) before rounding.
__device__ __forceinline__ Frag<bf16> ldfrag_scaled(const bf16* p, f32x4 slo, f32x4 shi) {
    f32x4 a = ld4(p), b = ld4(p + 16);
    Frag<bf16> f;
    f.v = bf16x8{(bf16)(a[0] * slo[0]), (bf16)(a[1] * slo[1]), (bf16)(a[2] * slo[2]), (bf16)(a[3] * slo[3]),
                 (bf16)(b[0] * shi[0]), (bf16)(b[1] * shi[1]), (bf16)(b[2] * shi[2]), (bf16)(b[3] * shi[3])};
    return f;
}
__device__ __forceinline__ Frag<float> ldfrag_scaled(const float* p, f32x4 slo, f32x4 shi) {
    Frag<float> f;
    f.lo = ld4(p) * slo;
    f.hi = ld4(p + 16) * shi;
    return f;
}

// B fragment (or transposed A fragment) from two vertically adjacent
// accumulator tiles: rows 0..15 in lo, rows 16..31 in hi.
template <typename E> __device__ __forceinline__ Frag<E> frag_from_acc(f32x4 lo, f32x4 hi);
template <> __device__ __forceinline__ Frag<bf16> frag_from_acc<bf16>(f32x4 lo, f32x4 hi) {
    Frag<bf16> f;
    f.v = bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                 (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
    return f;
}
template <> __device__ __forceinline__ Frag<float> frag_from_acc<float>(f32x4 lo, f32x4 hi) {
    Frag<float> f;
    f.lo = lo;
    f.hi = hi;
    return f;
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Split operands.  An fp32 value x is carried into a bf16 product as the pair
// hi = bf16(x), lo = bf16(x - hi): hi + lo holds about 16 significant bits,
// and a product with a bf16 operand b is hi*b + lo*b (two matrix-core
// instructions, fp32 accumulation).  With two split operands the lo*lo term,
// below 2^-16 relative, is left out.  Used where the block form of the delta
// rule cancels: with repeated keys and beta near 1, the new values U of one
// key telescope within a block, so a rounding of U (or of T, or of the
// adjoints that T multiplies) of one bf16 ulp is amplified in the sums over
// tokens.  fp32 elements are not split (Frag2<float> is one fragment).
// ---------------------------------------------------------------------------
template <typename E> struct Frag2;
template <> struct Frag2<bf16> { Frag<bf16> hi, lo; };
template <> struct Frag2<float> { Frag<float> hi; };

// From eight fp32 elements in fragment order (i = 0..3 in a, 4..7 in b).
template <typename E> __device__ __forceinline__ Frag2<E> split8(f32x4 a, f32x4 b);
template <> __device__ __forceinline__ Frag2<bf16> split8<bf16>(f32x4 a, f32x4 b) {
    Frag2<bf16> x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16 ha = (bf16)a[i], hb = (bf16)b[i];
        x.hi.v[i] = ha;
        x.hi.v[4 + i] = hb;
        x.lo.v[i] = (bf16)(a[i] - (float)ha);
        x.lo.v[4 + i] = (bf16)(b[i] - (float)hb);
    }
    return x;
}
// A split pair from its two stored halves (fp32: the value itself).
__device__ __forceinline__ Frag2<bf16> pair_of(const Frag<bf16>& hi, const Frag<bf16>& lo) { return Frag2<bf16>{hi, lo}; }
__device__ __forceinline__ Frag2<float> pair_of(const Frag<float>& hi, const Frag<float>&) { return Frag2<float>{hi}; }
template <> __device__ __forceinline__ Frag2<float> split8<float>(f32x4 a, f32x4 b) {
    Frag2<float> x;
    x.hi.lo = a;
    x.hi.hi = b;
    return x;
}
// Split B fragment (or transposed A fragment) from two vertically adjacent
// fp32 accumulator tiles, as frag_from_acc.
template <typename E> __device__ __forceinline__ Frag2<E> split_acc(f32x4 lo, f32x4 hi) { return split8<E>(lo, hi); }

__device__ __forceinline__ void mma2(f32x4& acc, const Frag2<bf16>& a, const Frag<bf16>& b) {
    mma(acc, a.hi, b);
    mma(acc, a.lo, b);
}
__device__ __forceinline__ void mma2(f32x4& acc, const Frag<bf16>& a, const Frag2<bf16>& b) {
    mma(acc, a, b.hi);
    mma(acc, a, b.lo);
}
__device__ __forceinline__ void mma2(f32x4& acc, const Frag2<bf16>& a, const Frag2<bf16>& b) {
    mma(acc, a.hi, b.hi);
    mma(acc, a.hi, b.lo);
    mma(acc, a.lo, b.hi);
}
__device__ __forceinline__ void mma2(f32x4& acc, const Frag2<float>& a, const Frag<float>& b) { mma(acc, a.hi, b); }
__device__ __forceinline__ void mma2(f32x4& acc, const Frag<float>& a, const Frag2<float>& b) { mma(acc, a, b.hi); }
__device__ __forceinline__ void mma2(f32x4& acc, const Frag2<float>& a, const Frag2<float>& b) { mma(acc, a.hi, b.hi); }

// ---------------------------------------------------------------------------
// Fragment-packed ("kmap-32") order.  Within every aligned group of 32
// indices, index kmap(g, i) is stored at position 8g + i, so the eight
// elements of one lane's fragment are contiguous (one 16-byte load for bf16).
// Four consecutive indices starting at a multiple of 4 stay consecutive.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kperm(int idx) {  // index -> stored position
    const int c = idx & 31;
    const int p = c < 16 ? ((c >> 2) << 3) + (c & 3) : (((c - 16) >> 2) << 3) + 4 + (c & 3);
    return (idx & ~31) + p;
}
__device__ __forceinline__ int kunperm(int pos) {  // stored position -> index
    const int p = pos & 31, g = p >> 3, i = p & 7;
    return (pos & ~31) + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
}
// Fragment from packed storage: p points at X[row][k0 + 8g].
__device__ __forceinline__ Frag<bf16> ldfragP(const bf16* p) {
    Frag<bf16> f;
    f.v = *(const bf16x8*)p;
    return f;
}
__device__ __forceinline__ Frag<float> ldfragP(const float* p) {
    Frag<float> f;
    f.lo = *(const f32x4*)p;
    f.hi = *(const f32x4*)(p + 4);
    return f;
}
// Store two vertically adjacent accumulator tiles (rows 0..15 in lo, 16..31
// in hi) of one lane into packed storage at p = &X[col][k0 + 8g].
__device__ __forceinline__ void st8P(bf16* p, f32x4 lo, f32x4 hi) {
    *(bf16x8*)p = bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                         (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
}
__device__ __forceinline__ void st8P(float* p, f32x4 lo, f32x4 hi) {
    *(f32x4*)p = lo;
    *(f32x4*)(p + 4) = hi;
}

// ---------------------------------------------------------------------------
// Row-major LDS tiles and transposing fragment reads.
//
// A 16-bit ds_read_b64_tr_b16 works on groups of 16 lanes: lane L' of a group
// points at four consecutive elements M[L'][0..3], and lane i of the group
// receives M[4j + (i >> 2)][i & 3], j = 0..3.  With lane L' = 16g + 4j + q
// pointing at X[k0 + 4g + j][n0 + 4q], lane (r, g) receives
// X[k0 + 4g + j][n0 + r], j = 0..3: the k-half of a B fragment of a
// row-major X[k][n] (equivalently an A fragment of X^T).  Every matrix a
// block kernel needs in both orientations is therefore staged once, row-major
// (whole 16-byte LDS writes), and read transposed where needed.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// B fragment (k = k0 .. k0 + 31, n = n0 .. n0 + 15) of a row-major matrix
// X[k][n] in LDS with row pitch P elements (P a multiple of 4).
__device__ __forceinline__ Frag<bf16> ldfrag_tr(const bf16* X, int P, int k0, int n0, int l) {
    const int g = l >> 4, j = (l >> 2) & 3, q = l & 3;
    const bf16* p = X + (k0 + 4 * g + j) * P + n0 + 4 * q;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * P));
    Frag<bf16> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}
__device__ __forceinline__ Frag<float> ldfrag_tr(const float* X, int P, int k0, int n0, int l) {
    const int r = l & 15, g = l >> 4;
    Frag<float> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.lo[i] = X[(k0 + 4 * g + i) * P + n0 + r];
        f.hi[i] = X[(k0 + 16 + 4 * g + i) * P + n0 + r];
    }
    return f;
}

// Coalesced staging of an R x CC token-major tile (global row stride ld) by a
// 256-thread work-group, in two steps so that a kernel can put the loads of
// several tiles in flight together: load_rows() issues every 16-byte load at
// once (rows >= nvalid read as zeros), store_rows() writes the registers
// row-major into LDS with row pitch P (whole 16-byte writes).
template <typename E, int R, int CC, int NT = 256> struct RowsRegs {
    static constexpr int VEC = 16 / (int)sizeof(E), PER_ROW = CC / VEC, UNITS = R * PER_ROW;
    static constexpr int N = (UNITS + NT - 1) / NT;
    uint4 u[N];
};
template <typename E, int R, int CC, int NT = 256>
__device__ __forceinline__ RowsRegs<E, R, CC, NT> load_rows(const E* __restrict__ src, size_t ld, int nvalid) {
    using X = RowsRegs<E, R, CC, NT>;
    X x;
#pragma unroll
    for (int j = 0; j < X::N; ++j) {
        const int idx = threadIdx.x + NT * j, t = idx / X::PER_ROW, cb = idx % X::PER_ROW;
        x.u[j] = (idx < X::UNITS && t < nvalid) ? *(const uint4*)(src + (size_t)t * ld + cb * X::VEC)
                                                : uint4{0u, 0u, 0u, 0u};
    }
    return x;
}
template <typename E, int R, int CC, int P, int NT = 256>
__device__ __forceinline__ void store_rows(const RowsRegs<E, R, CC, NT>& x, E* dst) {
    using X = RowsRegs<E, R, CC, NT>;
    static_assert(P % X::VEC == 0, "row pitch must keep 16-byte alignment");
#pragma unroll
    for (int j = 0; j < X::N; ++j) {
        const int idx = threadIdx.x + NT * j, t = idx / X::PER_ROW, cb = idx % X::PER_ROW;
        if (idx < X::UNITS) *(uint4*)(dst + t * P + cb * X::VEC) = x.u[j];
    }
}

// ---------------------------------------------------------------------------
// Tiled ("fragment-major") storage of a block-local matrix X[R][C], C a
// multiple of 32.  The 16 x 32 fragment f = (row / 16) * (C / 32) + col / 32
// is one contiguous run in lane order: lane l = 16g + r holds the A-fragment
// elements X[16 (f / (C/32)) + r][32 (f % (C/32)) + kmap(g, i)], i = 0..7.
//   bf16: 64 lanes x 16 bytes = 1 KB per fragment;
//   fp32: 2 KB per fragment, i = 0..3 in the first KB, i = 4..7 in the second.
// One wave therefore reads or writes a fragment as whole 1-KB runs (eight
// full 128-byte lines per instruction) instead of sixteen partial rows, which
// is what bounds a scan's operand stream on this chip.  Four consecutive
// columns starting at a multiple of 4 stay contiguous.
// ---------------------------------------------------------------------------
template <typename E>
__device__ __forceinline__ size_t toff(int row, int col, int C) {
    const int f = (row >> 4) * (C >> 5) + (col >> 5);
    const int p = kperm(col & 31);
    const int lane = ((p >> 3) << 4) + (row & 15), i = p & 7;
    if constexpr (sizeof(E) == 2) return ((size_t)f * 64 + lane) * 8 + i;
    else return (((size_t)f * 2 + (i >> 2)) * 64 + lane) * 4 + (i & 3);
}
// Elements per 1-KB unit, and this lane's offset inside a unit.
template <typename E> constexpr int UNIT_ELEMS = 1024 / (int)sizeof(E);
template <typename E> constexpr int LANE_ELEMS = 16 / (int)sizeof(E);
// Fragment f of a tiled matrix.
__device__ __forceinline__ Frag<bf16> ldfragT(const bf16* base, int f, int l) {
    Frag<bf16> x;
    x.v = *(const bf16x8*)(base + ((size_t)f * 64 + l) * 8);
    return x;
}
__device__ __forceinline__ Frag<float> ldfragT(const float* base, int f, int l) {
    Frag<float> x;
    x.lo = *(const f32x4*)(base + ((size_t)(2 * f) * 64 + l) * 4);
    x.hi = *(const f32x4*)(base + ((size_t)(2 * f + 1) * 64 + l) * 4);
    return x;
}
// Store two vertically adjacent accumulator tiles (rows 0..15 in lo, 16..31
// in hi), which are exactly an A fragment of the transposed 32 x 16 block, as
// fragment f of a tiled matrix.
__device__ __forceinline__ void st8T(bf16* base, int f, int l, f32x4 lo, f32x4 hi) {
    *(bf16x8*)(base + ((size_t)f * 64 + l) * 8) = bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                                                         (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
}
__device__ __forceinline__ void st8T(float* base, int f, int l, f32x4 lo, f32x4 hi) {
    *(f32x4*)(base + ((size_t)(2 * f) * 64 + l) * 4) = lo;
    *(f32x4*)(base + ((size_t)(2 * f + 1) * 64 + l) * 4) = hi;
}
__device__ __forceinline__ void st8T(bf16* base, int f, int l, const Frag<bf16>& x) {
    *(bf16x8*)(base + ((size_t)f * 64 + l) * 8) = x.v;
}

// Tiled global storage of X[R][C], one 16-byte unit per thread and iteration
// (coalesced 1-KB runs).  get4(row, col) returns X[row][col .. col + 3]
// (col a multiple of 4) as fp32; the values are rounded to E on the store.
template <typename E, int R, int C, typename F>
__device__ __forceinline__ void store_tiled(E* __restrict__ dst, F get4) {
    constexpr int UNITS = R * C * (int)sizeof(E) / 16;
    for (int u = threadIdx.x; u < UNITS; u += blockDim.x) {
        int f, lane, half;
        if constexpr (sizeof(E) == 2) { f = u >> 6; lane = u & 63; half = 0; }
        else { f = u >> 7; half = (u >> 6) & 1; lane = u & 63; }
        const int row = 16 * (f / (C / 32)) + (lane & 15), g = lane >> 4, c0 = 32 * (f % (C / 32));
        if constexpr (sizeof(E) == 2) {
            const f32x4 lo = get4(row, c0 + 4 * g), hi = get4(row, c0 + 16 + 4 * g);
            *(bf16x8*)(dst + (size_t)u * 8) = bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                                                     (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
        } else {
            *(f32x4*)(dst + (size_t)u * 4) = get4(row, c0 + (half ? 16 : 0) + 4 * g);
        }
    }
}

// Tiled global X[R][C] -> transposed LDS dst[c * DP + r] = X[r][c]
// (coalesced 16-byte reads).
template <typename E, int R, int C, int DP>
__device__ __forceinline__ void stage_T_tiled(const E* __restrict__ src, E* dst) {
    constexpr int UNITS = R * C * (int)sizeof(E) / 16;
    for (int u = threadIdx.x; u < UNITS; u += blockDim.x) {
        int f, lane, half;
        if constexpr (sizeof(E) == 2) { f = u >> 6; lane = u & 63; half = 0; }
        else { f = u >> 7; half = (u >> 6) & 1; lane = u & 63; }
        const int row = 16 * (f / (C / 32)) + (lane & 15), g = lane >> 4, c0 = 32 * (f % (C / 32));
        if constexpr (sizeof(E) == 2) {
            const bf16x8 v = *(const bf16x8*)(src + (size_t)u * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[(c0 + 4 * g + i) * DP + row] = v[i];
                dst[(c0 + 16 + 4 * g + i) * DP + row] = v[4 + i];
            }
        } else {
            const f32x4 v = *(const f32x4*)(src + (size_t)u * 4);
            const int c = c0 + (half ? 16 : 0) + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(c + i) * DP + row] = v[i];
        }
    }
}

// Tiled global X[R][C] -> row-major LDS (row pitch P), in two steps like
// load_rows / store_rows: every 16-byte unit is loaded at once, then each
// unit's two 4-element halves are written to their rows.
template <typename E, int R, int C, int NT = 256> struct TiledRegs {
    static constexpr int UNITS = R * C * (int)sizeof(E) / 16, N = (UNITS + NT - 1) / NT;
    uint4 u[N];
};
template <typename E, int R, int C, int NT = 256>
__device__ __forceinline__ TiledRegs<E, R, C, NT> load_tiled(const E* __restrict__ src) {
    TiledRegs<E, R, C, NT> x;
#pragma unroll
    for (int j = 0; j < x.N; ++j) {
        const int u = threadIdx.x + NT * j;
        x.u[j] = u < x.UNITS ? *(const uint4*)(src + (size_t)u * (16 / sizeof(E))) : uint4{0u, 0u, 0u, 0u};
    }
    return x;
}
template <typename E, int R, int C, int P, int NT = 256>
__device__ __forceinline__ void store_untiled(const TiledRegs<E, R, C, NT>& x, E* dst) {
#pragma unroll
    for (int j = 0; j < x.N; ++j) {
        const int u = threadIdx.x + NT * j;
        if (u >= x.UNITS) continue;
        if constexpr (sizeof(E) == 2) {
            const int f = u >> 6, lane = u & 63;
            const int row = 16 * (f / (C / 32)) + (lane & 15), c = 32 * (f % (C / 32)) + 4 * (lane >> 4);
            *(uint2*)(dst + row * P + c) = uint2{x.u[j].x, x.u[j].y};
            *(uint2*)(dst + row * P + c + 16) = uint2{x.u[j].z, x.u[j].w};
        } else {
            const int f = u >> 7, half = (u >> 6) & 1, lane = u & 63;
            const int row = 16 * (f / (C / 32)) + (lane & 15), c = 32 * (f % (C / 32)) + 16 * half + 4 * (lane >> 4);
            *(uint4*)(dst + row * P + c) = x.u[j];
        }
    }
}

// Tiled fp32 global X[R][C] (loaded with load_tiled<float, ...>) -> row-major
// LDS in the element type E, split: hi[r * P + c] = E(X[r][c]) and, for bf16,
// lo[r * P + c] = bf16(X[r][c] - hi).  For E = float only hi is written.
template <typename E, int R, int C, int P, int NT = 256>
__device__ __forceinline__ void store_untiled_split(const TiledRegs<float, R, C, NT>& x, E* hi, E* lo) {
#pragma unroll
    for (int j = 0; j < x.N; ++j) {
        const int u = threadIdx.x + NT * j;
        if (u >= x.UNITS) continue;
        const int f = u >> 7, half = (u >> 6) & 1, lane = u & 63;
        const int row = 16 * (f / (C / 32)) + (lane & 15), c = 32 * (f % (C / 32)) + 16 * half + 4 * (lane >> 4);
        const f32x4 v = *(const f32x4*)&x.u[j];
        if constexpr (sizeof(E) == 2) {
            bf16x4 h, o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = (bf16)v[i];
                o[i] = (bf16)(v[i] - (float)h[i]);
            }
            *(bf16x4*)(hi + row * P + c) = h;
            *(bf16x4*)(lo + row * P + c) = o;
        } else {
            *(f32x4*)(hi + row * P + c) = v;
        }
    }
}

// Tiled fp32 global X[R][C] -> row-major LDS in the element type (rounded).
template <typename E, int R, int C, int P, int NT = 256>
__device__ __forceinline__ void store_untiled_round(const TiledRegs<float, R, C, NT>& x, E* dst) {
#pragma unroll
    for (int j = 0; j < x.N; ++j) {
        const int u = threadIdx.x + NT * j;
        if (u >= x.UNITS) continue;
        const int f = u >> 7, half = (u >> 6) & 1, lane = u & 63;
        const int row = 16 * (f / (C / 32)) + (lane & 15), c = 32 * (f % (C / 32)) + 16 * half + 4 * (lane >> 4);
        st4(dst + row * P + c, *(const f32x4*)&x.u[j]);
    }
}

// Split fragments of a matrix staged as a (hi, lo) pair of LDS tiles: the
// row-major read of ldfrag and the transposing read of ldfrag_tr.
__device__ __forceinline__ Frag2<bf16> ldfrag2(const bf16* hi, const bf16* lo) { return Frag2<bf16>{ldfrag(hi), ldfrag(lo)}; }
__device__ __forceinline__ Frag2<float> ldfrag2(const float* hi, const float*) { return Frag2<float>{ldfrag(hi)}; }
__device__ __forceinline__ Frag2<bf16> ldfrag_tr2(const bf16* hi, const bf16* lo, int P, int k0, int n0, int l) {
    return Frag2<bf16>{ldfrag_tr(hi, P, k0, n0, l), ldfrag_tr(lo, P, k0, n0, l)};
}
__device__ __forceinline__ Frag2<float> ldfrag_tr2(const float* hi, const float*, int P, int k0, int n0, int l) {
    return Frag2<float>{ldfrag_tr(hi, P, k0, n0, l)};
}
// Split fragment f of a matrix stored tiled as a (hi, lo) pair (lo unused for fp32).
__device__ __forceinline__ Frag2<bf16> ldfragT2(const bf16* hi, const bf16* lo, int f, int l) {
    return Frag2<bf16>{ldfragT(hi, f, l), ldfragT(lo, f, l)};
}
__device__ __forceinline__ Frag2<float> ldfragT2(const float* hi, const float*, int f, int l) { return Frag2<float>{ldfragT(hi, f, l)}; }

// Accumulator-tiled fp32 storage of an [M][N] matrix: the 16 x 16 tile
// (mb, nb) is 1 KB in lane order, lane l = 16g + r holding rows 16 mb + 4g + i
// (i = 0..3) of column 16 nb + r.  Tiles are ordered nb-major: tile index
// nb * (M / 16) + mb, so one 16-column slice is contiguous.
__device__ __forceinline__ size_t atoff(int mb, int nb, int M, int l) {
    return ((size_t)nb * (M / 16) + mb) * 256 + (size_t)l * 4;
}

// Four contiguous elements kept in their storage type (fewer registers than
// f32x4 for bf16), converted on use.
template <typename E> struct Raw4;
template <> struct Raw4<bf16> { bf16x4 v; };
template <> struct Raw4<float> { f32x4 v; };
__device__ __forceinline__ Raw4<bf16> ldraw4(const bf16* p) { return Raw4<bf16>{*(const bf16x4*)p}; }
__device__ __forceinline__ Raw4<float> ldraw4(const float* p) { return Raw4<float>{*(const f32x4*)p}; }
__device__ __forceinline__ f32x4 cvt4(Raw4<bf16> x) {
    return f32x4{(float)x.v[0], (float)x.v[1], (float)x.v[2], (float)x.v[3]};
}
__device__ __forceinline__ f32x4 cvt4(Raw4<float> x) { return x.v; }
// Four fp32 values rounded to E (as a product operand would take them).
template <typename E> __device__ __forceinline__ Raw4<E> to_raw4(f32x4 v);
template <> __device__ __forceinline__ Raw4<bf16> to_raw4<bf16>(f32x4 v) {
    return Raw4<bf16>{bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]}};
}
template <> __device__ __forceinline__ Raw4<float> to_raw4<float>(f32x4 v) { return Raw4<float>{v}; }

// Inclusive prefix sum over the 64 lanes of a wave (lane order).
// Four consecutive floats (16-byte aligned, LDS or global) read together and
// kept ahead of any per-element condition: the empty asm stops the compiler
// from sinking each read under its own branch and waiting on it separately.
__device__ __forceinline__ f32x4 ld4_now(const float* p) {
    f32x4 v = *(const f32x4*)p;
    asm volatile("" : "+v"(v));
    return v;
}

// The value of lane src(l) by a DPP move (CTRL), for the rows in ROW_MASK;
// 0 where the source lane lies outside the row or the row is masked off.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes: within each 16-lane row by
// row_shr 1, 2, 4, 8, then the row totals by row_bcast 15 (into rows 1 and 3)
// and row_bcast 31 (into rows 2 and 3).
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_move<0x111>(x);
    x += dpp_move<0x112>(x);
    x += dpp_move<0x114>(x);
    x += dpp_move<0x118>(x);
    x += dpp_move<0x142, 0xA>(x);
    x += dpp_move<0x143, 0xC>(x);
    return x;
}

// Sum over the 16 lanes of each row (lanes 16 k .. 16 k + 15); every lane of
// the row gets it.  DPP lane moves (quad_perm [1,0,3,2], [2,3,0,1], then
// row_half_mirror and row_mirror) instead of LDS permutes; each step adds a
// partner that holds an equal partial, the same sums as xor 1, 2, 4, 8.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_move<0xB1>(x);
    x += dpp_move<0x4E>(x);
    x += dpp_move<0x141>(x);
    x += dpp_move<0x140>(x);
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace clr
