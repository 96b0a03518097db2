// Device helpers for the gfx950 attention kernels: MFMA operand traits,
// swizzled LDS tile addressing, the Philox4x32-10 generator and small
// wave-level utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;


// ---------------------------------------------------------------------------
// MFMA 32x32 traits.  For every 32x32xK instruction used here a lane l holds
//   A[m = l % 32][k = (l / 32) * E + e]      e = 0..E-1
//   B[k = (l / 32) * E + e][n = l % 32]
//   C[m = 8 * (r / 4) + 4 * (l / 32) + r % 4][n = l % 32]   r = 0..15
// with K = 2E.  16-bit inputs use the gfx950 32x32x16 shapes (E = 8), fp32
// inputs the 32x32x2 fp32 shape (E = 1).
template <class T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int E = 8;
    typedef bf16x8 frag;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<f16> {
    static constexpr int E = 8;
    typedef f16x8 frag;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int E = 1;
    typedef float frag;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// Type used for the probability operand of the forward's P*V product (and
// for V in LDS there).  For bf16 inputs P is rounded to fp16 (11-bit
// significand) instead of bf16 (8 bits) and the product reads an fp16 copy
// of V scaled by a power of two per (b, h) (see fa_fwd.hip).
template <class T> struct PvType { typedef T type; };
template <> struct PvType<bf16> { typedef f16 type; };

template <class T> __device__ inline float to_f32(T x) { return (float)x; }
template <class T> __device__ inline T from_f32(float x) { return (T)x; }

// fragment <-> 16-byte (or 4-byte) memory
template <class T> __device__ inline typename Mma<T>::frag load_frag(const T* p) {
    if constexpr (Mma<T>::E == 8) {
        return *reinterpret_cast<const typename Mma<T>::frag*>(p);
    } else {
        return *p;
    }
}

template <class T> __device__ inline typename Mma<T>::frag zero_frag() {
    typename Mma<T>::frag z;
    if constexpr (Mma<T>::E == 8) {
        for (int e = 0; e < 8; ++e) z[e] = (T)0.0f;
    } else {
        z = 0.0f;
    }
    return z;
}

__device__ inline f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// ---------------------------------------------------------------------------
// Row-major LDS tile of ROWS x COLS elements of T, addressed in 16-byte units
// with an XOR swizzle of the unit index by the row so that lanes reading the
// same column of consecutive rows fall in different banks.  Each swizzle is a
// bijection on the units of 8 consecutive rows (a 128-byte bank window) and,
// for rows of up to 256 bytes, also on the (window offset, unit) pairs of 16
// consecutive rows (a 256-byte window).
template <class T, int COLS>
struct Swz {
    static constexpr int EPU = 16 / (int)sizeof(T);   // elements per 16-byte unit
    static constexpr int U = COLS / EPU;              // units per row
    static_assert(COLS % EPU == 0, "row must be a whole number of 16-byte units");
    __device__ static inline int f(int row) {
        if constexpr (U >= 16) return (row ^ (row >> 4)) & 15;
        else if constexpr (U == 8) return (row ^ (row >> 3)) & 7;
        else if constexpr (U == 4) return ((row >> 1) ^ (row >> 3)) & 3;
        else if constexpr (U == 2) return ((row >> 2) ^ (row >> 3)) & 1;
        else return 0;
    }
    // element offset of (row, col); a run of up to EPU elements starting at a
    // col that is a multiple of the run length stays contiguous.
    __device__ static inline int off(int row, int col) {
        const int u = col / EPU;
        return row * COLS + ((u ^ f(row)) * EPU) + (col % EPU);
    }
};

// Row-major tile read both row-wise (16 consecutive rows, one 16-byte unit
// each) and with the LDS transpose read (4 consecutive rows x 4 consecutive
// units per 32 lanes).  With 64 banks of 4 bytes, a 256-byte row puts every
// row at the same bank offset, so the swizzle must make (row mod 16) -> unit
// a bijection and also spread 4 consecutive rows over 4 different unit
// quartets: unit bits 2-3 take the row's low two bits, unit bits 0-1 the next
// two.  For 128-byte rows the row's low bit picks the half of the 256-byte
// window, the next bit goes to unit bit 2, the two above to unit bits 0-1.
template <class T, int COLS>
struct SwzTr {
    static constexpr int EPU = 16 / (int)sizeof(T);
    static constexpr int U = COLS / EPU;
    static_assert(COLS % EPU == 0 && U >= 8, "rows of at least 128 bytes");
    __device__ static inline int f(int row) {
        if constexpr (U >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
        else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    }
    __device__ static inline int off(int row, int col) {
        const int u = col / EPU;
        return row * COLS + ((u ^ f(row)) * EPU) + (col % EPU);
    }
};

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit products on counter words 0 and 2, the key added into the
// high halves, and the key advanced by the two Weyl increments per round.
struct u32q { uint32_t x, y, z, w; };

__device__ inline u32q philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                     uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // full 64-bit products: one v_mad_u64_u32 each instead of a lo/hi pair
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// One generator call decides the block of keys 4g .. 4g+3 x query rows 2m,
// 2m+1: counter (g, m, bh, off); output word e belongs to key 4g+e, its low
// 16 bits to row 2m and its high 16 bits to row 2m+1; an element is kept iff
// its 16-bit value is >= thr.  Eight keep bits, in one of two orders:
//   ROWS:  bit 4s + e = (key 4g+e, row 2m+s)   (a row's 4 keys contiguous)
//   PAIRS: bit 2e + s = (key 4g+e, row 2m+s)   (a key's 2 rows contiguous)
template <bool ROWS>
__device__ inline uint32_t keep8(uint32_t g, uint32_t m, uint32_t bh, uint32_t off, uint32_t k0, uint32_t k1,
                                 uint32_t thr) {
    const u32q r = philox4x32_10(g, m, bh, off, k0, k1);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t out = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (uint32_t)((w[e] & 0xFFFFu) >= thr), hi = (uint32_t)((w[e] >> 16) >= thr);
        out |= ROWS ? ((lo << e) | (hi << (4 + e))) : ((lo | (hi << 1)) << (2 * e));
    }
    return out;
}

// DPP moves within a quad of lanes: every lane reads lane TP of its quad, or
// the lanes of each pair swap (quad_perm [1, 0, 3, 2]).
template <int TP> __device__ inline uint32_t quad_bcast(uint32_t w) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, TP * 0x55, 0xF, 0xF, false);   // quad_perm [TP,TP,TP,TP]
}
__device__ inline uint32_t pair_swap(uint32_t w) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xB1, 0xF, 0xF, false);
}

// Keep bits of this lane's query row i for the 16 keys 4*g0 .. 4*g0+15 (bit r
// = key 4*g0 + r), where lanes l and l ^ 1 hold rows i and i ^ 1 of one pair
// with the same keys.  The pair needs four calls (one per key group); the lane
// with row parity s runs those of groups g0 + 2s and g0 + 2s + 1, and the two
// lanes swap results with one DPP move.  Both lanes of every pair must be
// active.
__device__ inline uint32_t keep16_row(uint32_t g0, uint32_t i, uint32_t bh, uint32_t off, uint32_t k0,
                                      uint32_t k1, uint32_t thr) {
    const uint32_t s = i & 1u;
    const uint32_t w = keep8<true>(g0 + 2 * s, i >> 1, bh, off, k0, k1, thr) |
                       (keep8<true>(g0 + 2 * s + 1, i >> 1, bh, off, k0, k1, thr) << 8);
    const uint32_t o = pair_swap(w);
    const uint32_t a = s ? o : w;        // groups g0, g0 + 1 (bytes 0, 1)
    const uint32_t b = s ? w : o;        // groups g0 + 2, g0 + 3
    const uint32_t sh = 4 * s;           // this row's nibble of each byte
    return ((a >> sh) & 0xFu) | (((a >> (8 + sh)) & 0xFu) << 4) | (((b >> sh) & 0xFu) << 8) |
           (((b >> (8 + sh)) & 0xFu) << 12);
}

// Keep bits of this lane's key for 16 consecutive queries i0 .. i0+15 (i0
// even; bit r = query i0 + r), where the 4 lanes of each quad hold the 4 keys
// of one group (lane % 4 == key % 4).  The 8 row pairs take 8 calls: lane t of
// the quad runs pairs t and t + 4, and the quad shares the results with DPP
// quad broadcasts.  All 4 lanes of every quad must be active.
__device__ inline uint32_t keep16_quad(uint32_t key, uint32_t i0, uint32_t bh, uint32_t off, uint32_t k0,
                                       uint32_t k1, uint32_t thr, int lane) {
    const uint32_t t = (uint32_t)lane & 3u;
    const uint32_t m0 = (i0 >> 1) + t;
    const uint32_t w = keep8<false>(key >> 2, m0, bh, off, k0, k1, thr) |
                       (keep8<false>(key >> 2, m0 + 4, bh, off, k0, k1, thr) << 8);
    const uint32_t W[4] = {quad_bcast<0>(w), quad_bcast<1>(w), quad_bcast<2>(w), quad_bcast<3>(w)};
    const uint32_t ks = key & 3u;
    uint32_t out = 0;
    // byte c of W[tp] is pair tp + 4c: its bits 2ks, 2ks + 1 are queries i0 + 2(tp + 4c) + {0, 1}
#pragma unroll
    for (int tp = 0; tp < 4; ++tp)
#pragma unroll
        for (int c = 0; c < 2; ++c) out |= ((W[tp] >> (8 * c + 2 * ks)) & 3u) << (2 * tp + 8 * c);
    return out;
}

// ---------------------------------------------------------------------------
// Reductions over the lane pair (l, l ^ 32) with the gfx950 half-swap: the
// two results of v_permlane32_swap hold, between them, v of lane l and of
// lane l ^ 32 in every lane (which one is where depends on the half, but
// max and sum do not care).
__device__ inline float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA row order within a 32-row block: slot m holds row 16*((m/4)%2) +
// 4*(m/8) + m%4, so accumulator register r of lane half h is row 16*h + r.
__device__ inline int row_slot(int r) {
    return (r & ~31) | (((r >> 2) & 3) * 8 + ((r >> 4) & 1) * 4 + (r & 3));
}
__device__ inline int slot_row(int m) {
    return (m & ~31) | (((m >> 2) & 1) * 16 + ((m >> 3) & 3) * 4 + (m & 3));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Stage ROWS x D elements (rows row0.. of a row-major [N][D] head slab) into
// a swizzled LDS tile whose rows are in MFMA row order, with 16-byte
// buffer-to-LDS loads.  One such load writes the 64 lanes' 16 bytes to 64
// consecutive LDS units, so each lane fetches the global chunk that belongs
// at its unit.  The buffer descriptor covers only the rows that exist, so
// rows past N read as zeros (the hardware range check).  Issued by all NW
// waves of the workgroup (`wave` must be wave-uniform); completion is awaited
// with s_waitcnt before the barrier that publishes the tile.  (The buffer
// form rather than the global one: with a global load to LDS in flight the
// compiler turns every wait on an LDS read into a full drain.)
template <class T, int ROWS, int D, int NW = 4>
__device__ inline void dma_rows(T* tile, const T* head, int row0, int N, int wave, int lane) {
    typedef SwzTr<T, D> L;
    constexpr int EPU = 16 / (int)sizeof(T);
    constexpr int UPR = D / EPU;
    constexpr int UNITS = ROWS * UPR;
    static_assert(UNITS % (64 * NW) == 0, "tile must be a whole number of workgroup-wide loads");
    const int rows = N - row0 < ROWS ? N - row0 : ROWS;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(head + (size_t)row0 * D), (short)0, rows * D * (int)sizeof(T), 0x00020000);
#pragma unroll
    for (int n = 0; n < UNITS / (64 * NW); ++n) {
        const int blk = n * NW + wave;                // this wave's 64-unit block
        const int P = blk * 64 + lane;                // LDS unit written by this lane
        const int slot = P / UPR, pu = P % UPR;
        const int u = pu ^ L::f(slot);
        const uint32_t off = (uint32_t)((slot_row(slot) * D + u * EPU) * (int)sizeof(T));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + blk * 64 * EPU), 16, off, 0, 0, 0);
    }
}

// Transposed MFMA operand from a natural (row-major, swizzled, MFMA row
// order) 16-bit LDS tile, with the gfx950 LDS transpose read: the result is
// the 8 values X[k][c] for k = k-slots 8*(lane/32) .. +7 and c = col0 +
// lane%32, where k-slot q maps to tile row rowof(q).  Within each 16-lane
// group the transpose read hands destination lane j, element e, element j%4
// of the 8 bytes addressed by source lane j/4 + 4e; so source lane s of group
// G addresses row k = 8*(G/2) + 4*h + s/4 (h = 0, 1: the two halves of the
// fragment), columns col0 + 16*(G%2) + 4*(s%4) .. +3.  frag_tr_off gives
// the element offset of half h for this lane.
template <class T, int D, class RowOf>
__device__ inline int frag_tr_off(int col0, RowOf rowof, int lane, int h) {
    typedef SwzTr<T, D> L;
    const int G = lane >> 4, s = lane & 15;
    const int col = col0 + 16 * (G & 1) + 4 * (s & 3);
    const int k = 8 * (G >> 1) + 4 * h + (s >> 2);
    return L::off(rowof(k), col);
}

// The two transpose reads of a 16-bit fragment at given addresses (halves
// h = 0, 1 as frag_tr_off computes them).
template <class T>
__device__ inline typename Mma<T>::frag frag_tr_at(const T* p0, const T* p1) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    union { v4s h[2]; typename Mma<T>::frag f; } u;
    u.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
    u.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p1);
    return u.f;
}

template <class T, int D, class RowOf>
__device__ inline typename Mma<T>::frag load_frag_tr(const T* tile, int col0, RowOf rowof, int lane) {
    typedef SwzTr<T, D> L;
    if constexpr (Mma<T>::E == 8) {
        return frag_tr_at<T>(tile + frag_tr_off<T, D>(col0, rowof, lane, 0),
                             tile + frag_tr_off<T, D>(col0, rowof, lane, 1));
    } else {
        // one element per lane (k-slot lane/32): a plain read
        return tile[L::off(rowof(lane >> 5), col0 + (lane & 31))];
    }
}

// NC independent chains acc[c] += A(c, ks) x B(c, ks) over KS steps, with
// the A operands read from LDS by afrag(c, ks) PF steps ahead of their MFMA
// (LDS latency under load is several MFMA issue times) and the B operands
// in registers.  The fences keep the compiler from sinking the reads.
template <class T, int NC, int KS, int PF, class AFrag, class BFrag>
__device__ inline void lds_chain(f32x16 (&acc)[NC], AFrag afrag, BFrag bfrag) {
    typedef Mma<T> MM;
    constexpr int P = PF < KS ? PF : KS - 1;
    typename MM::frag af[P + 1][NC];
#pragma unroll
    for (int st = 0; st < P; ++st)
#pragma unroll
        for (int c = 0; c < NC; ++c) af[st][c] = afrag(c, st);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + P < KS) {
#pragma unroll
            for (int c = 0; c < NC; ++c) af[(ks + P) % (P + 1)][c] = afrag(c, ks + P);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = MM::mma(af[ks % (P + 1)][c], bfrag(c, ks), acc[c]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Chains of MFMAs acc[db] += R(s) x X(s, db) (or X x R) whose one operand
// is read from a natural 16-row-group tile with the transpose read and whose
// other operand R(s) is in registers.  Step s = (blk, u) covers 16 k-slots:
// k-slot kk is tile row 32*blk + row_slot(16*(kk/E) + u*E + kk%E), i.e. 16
// consecutive keys (or queries) of the register operand's lane half.  For
// 16-bit tiles row_slot(16a + 8u + b) = 16u + row_slot(16a + b) (b < 8) and
// the swizzle depends on a row's low 4 bits only, so the lane's read
// addresses are per-lane offsets fixed for the kernel plus a constant per
// step: TrOffsets holds the former.
template <class T, int D>
struct TrOffsets {
    int v[D / 32][2];
    __device__ explicit TrOffsets(int lane) {
        if constexpr (Mma<T>::E == 8) {
            auto rowof = [](int kk) { return row_slot(16 * (kk / 8) + kk % 8); };
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h) v[db][h] = frag_tr_off<T, D>(db * 32, rowof, lane, h);
        }
    }
};

// Steps run over (blk < NBLK, u < 16/E, db < D/32) with db fastest; the
// transposed operands are read PF steps ahead of their MFMA.  reg(blk, u)
// gives the register operand; TR_A puts the transposed operand first.
template <class T, int D, int NBLK, bool TR_A, int PF, class Reg>
__device__ inline void tr_chain(f32x16 (&acc)[D / 32], const T* tile, const TrOffsets<T, D>& to, Reg reg,
                                int lane) {
    typedef Mma<T> MM;
    constexpr int E = MM::E, QU = 16 / E, DB = D / 32, NS = NBLK * QU * DB;
    auto xfrag = [&](int st) {
        const int db = st % DB, u = (st / DB) % QU, blk = st / (DB * QU);
        if constexpr (E == 8) {
            const T* p = tile + (blk * 32 + u * 16) * D;
            return frag_tr_at<T>(p + to.v[db][0], p + to.v[db][1]);
        } else {
            auto rowof = [=](int kk) { return blk * 32 + row_slot(16 * kk + u); };
            return load_frag_tr<T, D>(tile, db * 32, rowof, lane);
        }
    };
    typename MM::frag xf[PF + 1];
#pragma unroll
    for (int st = 0; st < PF; ++st) xf[st] = xfrag(st);
    typename MM::frag r;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        if (st + PF < NS) xf[(st + PF) % (PF + 1)] = xfrag(st + PF);
        const int db = st % DB, u = (st / DB) % QU, blk = st / (DB * QU);
        if (db == 0) r = reg(blk, u);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (TR_A) acc[db] = MM::mma(xf[st % (PF + 1)], r, acc[db]);
        else acc[db] = MM::mma(r, xf[st % (PF + 1)], acc[db]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Map a linear workgroup id to a work item (head * per_head + rank, rank 0 the
// heaviest item of its head) so that each of the 8 XCDs -- which receive
// workgroups round-robin and have their own L2 -- works on one contiguous range
// of heads.  The grid has 8 * ceil(heads * per_head / 8) workgroups; ids with
// no item get -1.  Inside an XCD's range the items are dispatched head by head,
// or, with `by_rank` and a head count that splits evenly over the XCDs, rank by
// rank (the heaviest item of every head in the range first), so that when the
// range holds many short heads no heavy item is left to start last.
__device__ inline int xcd_item(int wg, int heads, int per_head, bool by_rank) {
    const int x = wg & 7, k = wg >> 3;
    if (by_rank && heads % 8 == 0) {
        const int nh = heads / 8;                      // heads per XCD; k < nh * per_head
        return (x * nh + k % nh) * per_head + k / nh;
    }
    const int total = heads * per_head;
    const int item = x * ((total + 7) / 8) + k;
    return item < total ? item : -1;
}

// Four floats stored as one 8- or 16-byte vector of T.
template <class T> __device__ inline void store4(T* p, float a, float b, float c, float d);
template <> __device__ inline void store4<f16>(f16* p, float a, float b, float c, float d) {
    f16x4 w = {(f16)a, (f16)b, (f16)c, (f16)d};
    *reinterpret_cast<f16x4*>(p) = w;
}
template <> __device__ inline void store4<bf16>(bf16* p, float a, float b, float c, float d) {
    bf16x4 w = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4*>(p) = w;
}
template <> __device__ inline void store4<float>(float* p, float a, float b, float c, float d) {
    f32x4 w = {a, b, c, d};
    *reinterpret_cast<f32x4*>(p) = w;
}

// A 16-bit MFMA operand (8 consecutive values) or an fp32 one (1 value) from
// floats, rounded to the operand type.
template <class TV> __device__ inline typename Mma<TV>::frag pack_p(const float* p) {
    if constexpr (Mma<TV>::E == 8) {
        typename Mma<TV>::frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (TV)p[e];
        return f;
    } else {
        return p[0];
    }
}

}  // namespace fa
