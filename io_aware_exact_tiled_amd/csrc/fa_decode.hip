// Decode attention (split key/value cache) for gfx950.
//
// A few new query rows per (b, h) against a long key/value cache: the regime
// the Self-Attention tutorial (infra-guide, section 11.2, decode phase)
// describes as memory-bound -- each step reads the whole cache for a handful
// of queries.  So the cache is cut into chunks that many workgroups read in
// parallel, each chunk exactly once, and the per-chunk softmax partials are
// merged with the two-block rule of the FlashAttention summary ("Method",
// incremental softmax: m = max(m1, m2), l = e^{m1-m} l1 + e^{m2-m} l2).
//
// decode_split_kernel: one workgroup per (sequence b, K/V head g, block of 32
//   query rows, chunk s of the sequence's valid rows).  The S chunks split the
//   len_b valid rows evenly (32-row multiples), so the workgroups of a
//   sequence read equal amounts; rows at or past len_b are never read, so the
//   cache past them may hold anything.  The 32 rows are those of the G = H/Hkv
//   query heads that read head g, times the Nq decode rows (row r = hh*Nq + i,
//   query head g*G + hh, decode row i; rows past G*Nq are padding), so every
//   byte of K and V is read once for the whole group.  Four waves take the
//   chunk's 32-key tiles round-robin:
//     S^T = K_t Q^T           MFMA, K rows loaded from global straight into the
//                             A operand, Q^T in registers (one query per lane)
//     masks                   keys >= len_b; causal: key > len_b - Nq + i
//     online softmax          as in the forward kernel (lazy rescale, base 2)
//     O^T += V_t^T P^T        V_t staged per wave in LDS (buffer-to-LDS loads,
//                             double-buffered), read with the transpose read.
//                             bf16: P is split into bf16 high and low parts and
//                             both products accumulate (the extra MFMAs are free
//                             in this memory-bound kernel; P keeps ~16 bits)
//   then the four waves' partials merge in LDS and the workgroup writes, per
//   query row, O_s (normalised by its own l) and lse2_s = m + log2 l.
// decode_merge_kernel: per query row, the splits' (O_s, lse2_s) with the same
//   rule: O = sum_s w_s O_s / sum_s w_s, w_s = 2^(lse2_s - max), LSE = (max +
//   log2 sum w) ln 2; splits holding no valid key (lse2 = -inf) are skipped.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <class T, int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
    typedef Mma<T> MM;
    constexpr int E = MM::E;            // 8 (16-bit inputs only)
    constexpr int KS = D / (2 * E);
    constexpr int DB = D / 32;
    constexpr int PU = 16 / E;          // P*V MFMA steps per 32-key tile
    constexpr int TT = 32 * D;          // elements of one wave's V tile
    constexpr float RESCALE = 8.0f;
    constexpr bool SPLIT_P = std::is_same<T, bf16>::value;   // bf16: P as hi + lo
    static_assert(E == 8, "16-bit inputs");

    // per wave: two V tiles; after the loop the same memory holds the four
    // waves' partial O^T (4 x 32 x D floats = 4 x 2 x TT x 2 bytes)
    __shared__ __attribute__((aligned(16))) T sV[4 * 2 * TT];
    __shared__ float sM[4 * 32], sL[4 * 32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ln = lane & 31;
    const int G = a.H / a.Hkv, R = G * a.Nq;
    // work item: (b, g, query block, split), split fastest
    int item = (int)blockIdx.x;
    const int s = item % a.S; item /= a.S;
    const int qb = item % a.QBn; item /= a.QBn;
    const int g = item % a.Hkv;
    const int b = item / a.Hkv;
    const int Nk = a.Nk, Nq = a.Nq;
    int L = Nk;
    if (a.kv_lens) {
        const int x = a.kv_lens[b];
        L = x < 0 ? 0 : (x > Nk ? Nk : x);
    }
    const int Cb = ((L + a.S - 1) / a.S + 31) & ~31;  // rows per chunk of this sequence
    const int c0 = min(s * Cb, L);
    const int c1 = min(c0 + Cb, L);
    const size_t koff = ((size_t)b * a.Hkv + g) * (size_t)Nk * D;
    const T* __restrict__ Kg = (const T*)a.k + koff;
    const T* __restrict__ Vg = (const T*)a.v + koff;

    // this lane's query row (MFMA column): r = qb*32 + ln
    const int r = qb * 32 + ln;
    const bool rok = r < R;
    const int hh = rok ? r / Nq : 0, qi = rok ? r % Nq : 0;
    const int h = g * G + hh;
    const size_t qrow = (((size_t)b * a.H + h) * Nq + qi);     // row of Q / O / LSE
    const int qpos = L - Nq + qi;                              // its position in the sequence
    typename MM::frag qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = rok ? load_frag<T>((const T*)a.q + qrow * D + ks * 2 * E + hl * E) : zero_frag<T>();

    const TrOffsets<T, D> tro(lane);
    const float c = a.scale_log2;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = zero16();

    // tiles of this wave: kt = c0 + 32 * (wave + 4 n), n = 0, 1, ...
    const int ntile = c1 > c0 ? (c1 - c0 + 31) / 32 : 0;
    const int nmine = ntile > wave ? (ntile - wave + 3) / 4 : 0;
    T* vbuf = sV + wave * 2 * TT;
    auto kt_of = [&](int n) { return c0 + 32 * (wave + 4 * n); };
    typename MM::frag kf[2][KS];
    auto load_k = [&](int n, int slot) {
        int row = kt_of(n) + ln;
        row = row < c1 ? row : c1 - 1;                 // masked below as a key >= c1
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[slot][ks] = load_frag<T>(Kg + (size_t)row * D + ks * 2 * E + hl * E);
    };
    // rows at or past c1 arrive as zeros (the descriptor ends there)
    auto load_v = [&](int n, int slot) { dma_rows<T, 32, D, 1>(vbuf + slot * TT, Vg, kt_of(n), c1, 0, lane); };

    if (nmine > 0) {
        load_k(0, 0);
        load_v(0, 0);
    }
    // one tile; the buffer slot is a compile-time constant so that the K
    // fragments stay in registers
    auto step = [&](int n, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        __builtin_amdgcn_s_waitcnt(0);                 // tile n's K and V have landed
        if (n + 1 < nmine) {
            load_k(n + 1, slot ^ 1);
            load_v(n + 1, slot ^ 1);
        }
        const int kt = kt_of(n);
        // ---- S^T = K_t Q^T: accumulator lane column = query row, register = key
        f32x16 sacc = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = MM::mma(kf[slot][ks], qf[ks], sacc);
        // keys in MFMA row order: register r of lane half h is key 8(r/4) + 4h + r%4
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int key = kt + 8 * (q / 4) + 4 * hl + (q % 4);
            if (!rok || key >= c1 || (a.causal && key > qpos)) sacc[q] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < 16; ++q) mx = fmaxf(mx, sacc[q]);
        mx = pair_max(mx) * c;
        if (__builtin_expect(__any(mx > m_run + RESCALE), 0)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int q = 0; q < 16; ++q) oacc[db][q] *= alpha;
        }
        const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
        float p[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            p[q] = fast_exp2(fmaf(sacc[q], c, -m_ref));
            l_run += p[q];
        }
        // ---- O^T += V_t^T P^T.  k-slot kk of step u is the key of register
        // 8u + kk%8 of lane half kk/8: key 8(kk%8 / 4 + 2u) + 4(kk/8) + kk%4 of
        // the tile, which the staging put in LDS row row_slot(key)
        typename MM::frag phi[PU], plo[PU];
#pragma unroll
        for (int u = 0; u < PU; ++u) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = p[u * E + e];
                const T hi = (T)x;
                phi[u][e] = hi;
                if constexpr (SPLIT_P) plo[u][e] = (T)(x - (float)hi);
            }
        }
        const T* vt = vbuf + slot * TT;
#pragma unroll
        for (int u = 0; u < PU; ++u) {
            auto rowof = [=](int kk) { return row_slot(8 * ((kk % 8) / 4 + 2 * u) + 4 * (kk / 8) + kk % 4); };
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const typename MM::frag vf = load_frag_tr<T, D>(vt, db * 32, rowof, lane);
                oacc[db] = MM::mma(vf, phi[u], oacc[db]);
                if constexpr (SPLIT_P) oacc[db] = MM::mma(vf, plo[u], oacc[db]);
            }
        }
    };
    for (int n = 0; n < nmine; n += 2) {
        step(n, std::integral_constant<int, 0>{});
        if (n + 1 < nmine) step(n + 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(0);

    // ---- merge the four waves' partials in LDS
    __syncthreads();                                   // every wave is done with its V tiles
    // [wave][32 rows][D] floats; row r's columns are rotated by 4 (r % 32)
    // floats so that the 32 rows a store or a load touches at once fall in
    // different banks (unrotated, rows D floats apart share one bank)
    float* sO = reinterpret_cast<float*>(sV);
    auto so_at = [&](int row, int col) { return sO + row * D + ((col + 4 * (row & 31)) & (D - 1)); };
    const float l_tot = pair_sum(l_run);
    if (hl == 0) {
        sM[wave * 32 + ln] = m_run;
        sL[wave * 32 + ln] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 v4 = {oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
            *reinterpret_cast<f32x4*>(so_at(wave * 32 + ln, db * 32 + 8 * g4 + 4 * hl)) = v4;
        }
    __syncthreads();
    {
        constexpr int TPR = 8;                         // threads per row
        constexpr int CPT = D / TPR;                   // columns per thread
        const int n = tid / TPR, col0 = (tid % TPR) * CPT;
        const int rr = qb * 32 + n;
        if (rr < R) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, sM[w * 32 + n]);
            float cw[4], lsum = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                cw[w] = (M == -INFINITY) ? 0.0f : fast_exp2(sM[w * 32 + n] - M);
                lsum += cw[w] * sL[w * 32 + n];
            }
            const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
            const int hh2 = rr / Nq, qi2 = rr % Nq;
            const size_t row = ((size_t)b * a.H + g * G + hh2) * Nq + qi2;     // (b, h, i)
            float* op = a.opart + (row * a.S + s) * D + col0;
#pragma unroll
            for (int j = 0; j < CPT; j += 4) {
                f32x4 v4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(so_at(w * 32 + n, col0 + j));
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] += cw[w] * x[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] *= inv;
                *reinterpret_cast<f32x4*>(op + j) = v4;
            }
            if (col0 == 0) a.lpart[row * a.S + s] = lsum > 0.0f ? M + log2f(lsum) : -INFINITY;
        }
    }
}

template <class T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    // one wave per query row; each lane owns D/64 columns.  The splits' lse2
    // values are read 64 at a time (one per lane) and their weights handed to
    // every lane with readlane, so that the partial-O loads of a batch of
    // splits are independent and in flight together.
    constexpr int CPL = D / 64;
    constexpr int U = 8;                               // partial rows per batch
    const int lane = threadIdx.x & 63;
    const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const size_t rows = (size_t)a.B * a.H * a.Nq;
    if (row >= rows) return;
    const int S = a.S;
    const float* lp = a.lpart + row * S;
    const float* op = a.opart + row * S * D + lane * CPL;
    float M = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += 64)
        if (s0 + lane < S) M = fmaxf(M, lp[s0 + lane]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    float acc[CPL], wsum = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < S; s0 += 64) {
            const float ls = s0 + lane < S ? lp[s0 + lane] : -INFINITY;
            const float wl = fast_exp2(ls - M);        // 0 for a split without valid keys
            wsum += wl;
            const int n = min(64, S - s0);
            for (int j = 0; j < n; j += U) {
                float w[U], v[U][CPL];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = j + u < n ? j + u : n - 1;
                    const float wk = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k));
                    w[u] = j + u < n ? wk : 0.0f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) v[u][c] = op[(size_t)(s0 + k) * D + c];
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w[u], v[u][c], acc[c]);
            }
        }
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) wsum += __shfl_xor(wsum, x);
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    T* o = (T*)a.o + row * D + lane * CPL;
    if constexpr (CPL == 2) {
        typedef T t2 __attribute__((ext_vector_type(2)));
        t2 w2 = {(T)(acc[0] * inv), (T)(acc[1] * inv)};
        *reinterpret_cast<t2*>(o) = w2;
    } else {
        o[0] = (T)(acc[0] * inv);
    }
    if (lane == 0) a.lse[row] = wsum > 0.0f ? (M + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
}

namespace {
template <class T, int D>
hipError_t launch_t(const DecodeArgs& a, const hipEvent_t* ev, hipStream_t st) {
    DecodeArgs copy = a;
    void* args[] = {(void*)&copy};
    const size_t nsplit = (size_t)a.B * a.Hkv * a.QBn * a.S;
    hipError_t e = ev ? hipEventRecord(ev[0], st) : hipSuccess;
    if (e != hipSuccess) return e;
    e = hipLaunchKernel((const void*)&decode_split_kernel<T, D>, dim3((unsigned)nsplit), dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
    const size_t rows = (size_t)a.B * a.H * a.Nq;
    e = hipLaunchKernel((const void*)&decode_merge_kernel<T, D>, dim3((unsigned)((rows + 3) / 4)), dim3(256),
                        args, 0, st);
    if (e != hipSuccess) return e;
    return ev ? hipEventRecord(ev[2], st) : hipSuccess;
}
}  // namespace

hipError_t launch_decode(const DecodeArgs& a, fa_dtype dt, int d, const hipEvent_t* ev, hipStream_t s) {
    if (dt == FA_BF16) return d == 64 ? launch_t<bf16, 64>(a, ev, s) : launch_t<bf16, 128>(a, ev, s);
    return d == 64 ? launch_t<f16, 64>(a, ev, s) : launch_t<f16, 128>(a, ev, s);
}

}  // namespace fa
