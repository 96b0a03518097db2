// Forward pass of tiled exact attention for gfx950.
//
// One workgroup (4 waves) owns BR = 128 query rows of one (b, h); each wave
// owns 32 of them.  The workgroup walks the key/value tiles of BC = 64 keys
// that hold at least one valid pair (FlashAttention summary, xyznot.com,
// "Method"; the query-outer / key-inner loop order of the tutorial's section
// 12.2 pseudocode), staging K_j and V_j^T in LDS, and per tile:
//   S^T = K_j Q_i^T          MFMA, fp32 accumulation, one query per lane column
//   masks on edge tiles      causal j > i, key padding j >= len_b, N tail
//   m_new = max(m, rowmax)   lane-local max over 16 keys + one cross-half swap
//   P = exp2(S*scale*log2e - m_new),  l = e^{m - m_new} l + rowsum(P)
//   dropout keep bits        Philox4x32-10, one call per 4 keys
//   O^T = e^{m - m_new} O^T + V_j^T P^T     MFMA
// and finally writes O = O^T / l and LSE = m + ln l (incremental softmax of
// the summary's "Method" steps 2-4 with the normalisation deferred to the end,
// as in the explainer's simplified forward, azimuth.plus).
//
// Layout choices (MI355X-specific, not from the pages):
//  * S is computed transposed (keys on MFMA rows, queries on columns) so that
//    every lane holds one query row: the row max needs one cross-half swap,
//    the row sum none until the epilogue, and the per-row rescale of O is a
//    lane-local multiply.
//  * K rows are stored in LDS in MFMA row order: MFMA row m takes key
//    16*((m/4)%2) + 4*(m/8) + m%4, so that lane (l/32) of the accumulator
//    holds 16 *consecutive* keys in registers r = 0..15.  Those 16 values are
//    then exactly the B operand of the P*V product (8 consecutive keys per
//    MFMA per lane half), with no register shuffles.
//  * V is stored transposed (d rows, key columns) so the A operand of V^T P^T
//    is one 16-byte LDS read per MFMA.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

template <class TV> __device__ inline void store4(TV* p, float a, float b, float c, float d);
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

// MFMA row slot of key r within a 32-key block (see the file comment).
__device__ inline int key_slot(int r) { return row_slot(r); }

}  // namespace

template <class T, int D, bool DROP>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
    typedef typename PvType<T>::type TV;
    typedef Mma<T> MS;
    typedef Mma<TV> MV;
    constexpr int E = MS::E;
    constexpr int EV = MV::E;
    constexpr int BR = FWD_BR, BC = FWD_BC;
    constexpr int KS = D / (2 * E);     // MFMA steps over d in S^T
    constexpr int KB = BC / 32;         // 32-key blocks per tile
    constexpr int DB = D / 32;          // 32-wide column blocks of O
    constexpr int PU = 16 / EV;         // P*V MFMAs per 32-key block
    constexpr int EPU = 16 / (int)sizeof(T);
    constexpr int DC = D / EPU;         // 16-byte chunks per row of K / V
    constexpr int KT = BC * DC;         // K staging: one 16-byte chunk per task
    constexpr int KN = (KT + 255) / 256;
    constexpr int VT = (BC / 4) * DC;   // V staging: 4 rows x one chunk per task
    constexpr int VN = (VT + 255) / 256;
    constexpr int TILE_K = BC * D;      // elements of one K (or V^T) buffer
    constexpr float RESCALE = 8.0f;     // log2 headroom before the running max moves
    typedef Swz<T, D> LK;
    typedef Swz<TV, BC> LV;

    __shared__ __attribute__((aligned(16))) T sK[2 * TILE_K];
    __shared__ __attribute__((aligned(16))) TV sV[2 * TILE_K];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane >> 5, ln = lane & 31;
    const int N = a.N, H = a.H;
    const int Tr = (N + BR - 1) / BR, Tc = (N + BC - 1) / BC;
    // work item: contiguous ranges per XCD; inside a head, heaviest tiles first
    const int total = Tr * H * a.B;
    const int item = xcd_item((int)blockIdx.x, (total + 7) / 8);
    if (item >= total) return;
    const int bhi = item / Tr, r_ = item % Tr;
    const int it = a.mask.causal ? (Tr - 1 - r_) : r_;
    const int b = bhi / H, h = bhi % H;
    const int q0 = it * BR, qw0 = q0 + wave * 32;
    const size_t bh = (size_t)bhi;
    const size_t hoff = bh * (size_t)N * D;
    const T* __restrict__ Qg = (const T*)a.q + hoff;
    const T* __restrict__ Kg = (const T*)a.k + hoff;
    const T* __restrict__ Vg = (const T*)a.v + hoff;
    (void)b; (void)h;

    int kend = N;
    if (a.mask.key_lens) {
        const int L = a.mask.key_lens[bhi / H];
        kend = L < 0 ? 0 : (L > N ? N : L);
    }
    int j_end = min(Tc, (kend + BC - 1) / BC);
    if (a.mask.causal) j_end = min(j_end, (min(q0 + BR, N) - 1) / BC + 1);
    const uint8_t* bmask = a.mask.block_mask ? a.mask.block_mask + (size_t)(q0 / MASK_TILE) * a.mask.mask_T
                                             : nullptr;
    const int rev = a.reverse_kv;
    // next visited key tile after position jj of the walk (or -1)
    auto tile_at = [&](int jj) -> int {
        for (; jj < j_end; ++jj) {
            const int j = rev ? (j_end - 1 - jj) : jj;
            if (!bmask || bmask[(j * BC) / MASK_TILE]) return jj;
        }
        return -1;
    };

    uint8_t* vis = a.tile_visits ? a.tile_visits + (bh * Tr + it) * (size_t)Tc : nullptr;
    if (vis)
        for (int j = tid; j < Tc; j += 256) vis[j] = 0;

    // Q_i^T as the B operand: lane column = query qw0 + ln, rows = d
    const int qrow = qw0 + ln;
    typename MS::frag qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = (qrow < N) ? load_frag<T>(Qg + (size_t)qrow * D + ks * 2 * E + hl * E)
                            : zero_frag<T>();

    // ---- staging: global -> registers (prefetch) -> LDS
    u32x4 kreg[KN];
    u32x4 vreg[VN][4];
    auto load_tile = [&](int j) {
        const int kv0 = j * BC;
#pragma unroll
        for (int n = 0; n < KN; ++n) {
            const int t = tid + n * 256;
            const int key = kv0 + t / DC;
            u32x4 z = {0u, 0u, 0u, 0u};
            kreg[n] = (t < KT && key < N) ? *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + (t % DC) * EPU)
                                          : z;
        }
#pragma unroll
        for (int n = 0; n < VN; ++n) {
            const int t = tid + n * 256;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int key = kv0 + (t / DC) * 4 + kk;
                u32x4 z = {0u, 0u, 0u, 0u};
                vreg[n][kk] = (t < VT && key < N)
                                  ? *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + (t % DC) * EPU)
                                  : z;
            }
        }
    };
    auto store_tile = [&](int buf) {
        T* k = sK + buf * TILE_K;
        TV* v = sV + buf * TILE_K;
#pragma unroll
        for (int n = 0; n < KN; ++n) {
            const int t = tid + n * 256;
            if (t < KT) *reinterpret_cast<u32x4*>(k + LK::off(key_slot(t / DC), (t % DC) * EPU)) = kreg[n];
        }
#pragma unroll
        for (int n = 0; n < VN; ++n) {
            const int t = tid + n * 256;
            if (t < VT) {
                const int dc = t % DC, kg = t / DC;
                const T* x0 = reinterpret_cast<const T*>(&vreg[n][0]);
                const T* x1 = reinterpret_cast<const T*>(&vreg[n][1]);
                const T* x2 = reinterpret_cast<const T*>(&vreg[n][2]);
                const T* x3 = reinterpret_cast<const T*>(&vreg[n][3]);
#pragma unroll
                for (int dd = 0; dd < EPU; ++dd)
                    store4<TV>(v + LV::off(dc * EPU + dd, kg * 4), to_f32(x0[dd]), to_f32(x1[dd]),
                               to_f32(x2[dd]), to_f32(x3[dd]));
            }
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = zero16();

    const float c = a.scale_log2;
    const int causal = a.mask.causal;

    int jj = tile_at(0);
    if (jj >= 0) {
        load_tile(rev ? (j_end - 1 - jj) : jj);
        store_tile(0);
    }
    __syncthreads();
    int buf = 0;
    while (jj >= 0) {
        const int j = rev ? (j_end - 1 - jj) : jj;
        const int kv0 = j * BC;
        if (vis && tid == 0) vis[j] = 1;
        const int jn = tile_at(jj + 1);
        if (jn >= 0) load_tile(rev ? (j_end - 1 - jn) : jn);   // in flight during this tile's math

        // one tile of math; element masks only on tiles that straddle the
        // diagonal, the padding boundary or the N tail
        auto tile_math = [&](bool edge) {
            const T* k = sK + buf * TILE_K;
            const TV* v = sV + buf * TILE_K;
            // ---- S^T = K_j Q^T (operands of one 32-key block loaded together)
            // (software-pipelined: the K operands of step ks+1 are read
            // before the MFMAs of step ks are issued; not with dropout at
            // d=128, where the registers are short)
            constexpr bool PIPE = !(DROP && D == 128);
            auto fence = [] { if constexpr (PIPE) __builtin_amdgcn_sched_barrier(0); };
            f32x16 s[KB];
            __builtin_amdgcn_s_setprio(1);
            {
                typename MS::frag kf[2][KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    s[kb] = zero16();
                    kf[0][kb] = load_frag<T>(k + LK::off(kb * 32 + ln, hl * E));
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (!PIPE && ks > 0) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
                            kf[ks & 1][kb] = load_frag<T>(k + LK::off(kb * 32 + ln, ks * 2 * E + hl * E));
                    }
                    if (PIPE && ks + 1 < KS) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
                            kf[(ks + 1) & 1][kb] = load_frag<T>(k + LK::off(kb * 32 + ln, (ks + 1) * 2 * E + hl * E));
                    }
                    fence();
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) s[kb] = MS::mma(kf[ks & 1][kb], qf[ks], s[kb]);
                    fence();
                }
            }
            __builtin_amdgcn_s_setprio(0);
            if (__builtin_expect(edge, 0)) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb * 32 + hl * 16 + r;
                        if (key >= kend || (causal && key > qrow)) s[kb][r] = -INFINITY;
                    }
            }
            // ---- online softmax; the reference max only moves when some row's
            // max exceeds it by more than 2^RESCALE, so P <= 2^RESCALE
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, wave_xor32(mx)) * c;
            if (__builtin_expect(__any(mx > m_run + RESCALE), 0)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;

            float p[KB][16];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[kb][r] = fast_exp2(fmaf(s[kb][r], c, -m_ref));
                    l_run += p[kb][r];
                }
            if constexpr (DROP) {
                const uint32_t g0 = (uint32_t)(kv0 + hl * 16) >> 2;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint32_t bits = keep4(g0 + kb * 8 + g, (uint32_t)qrow, (uint32_t)bh, a.drop.off,
                                                    a.drop.k0, a.drop.k1, a.drop.thr);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (!((bits >> e) & 1u)) p[kb][g * 4 + e] = 0.0f;
                    }
            }
            // ---- O^T += V_j^T P^T
            // (software-pipelined over the flattened (kb, u, db) steps, two
            // V^T operands ahead)
            __builtin_amdgcn_s_setprio(1);
            {
                constexpr int NS = KB * PU * DB, PF = PIPE ? 2 : 1;
                auto vfrag = [&](int st) {
                    const int db = st % DB, u = (st / DB) % PU, kb = st / (DB * PU);
                    return load_frag<TV>(v + LV::off(db * 32 + ln, kb * 32 + hl * 16 + u * EV));
                };
                typename MV::frag vf[PF + 1];
#pragma unroll
                for (int st = 0; st < PF; ++st) vf[st] = vfrag(st);
                typename MV::frag bp;
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    if (st + PF < NS) vf[(st + PF) % (PF + 1)] = vfrag(st + PF);
                    const int db = st % DB, u = (st / DB) % PU, kb = st / (DB * PU);
                    if (db == 0) bp = pack_p<TV>(&p[kb][u * EV]);
                    fence();
                    oacc[db] = MV::mma(vf[st % (PF + 1)], bp, oacc[db]);
                    fence();
                }
            }
            __builtin_amdgcn_s_setprio(0);
        };
        if (!(causal && kv0 > qw0 + 31))   // else: no valid key for this wave's rows
            tile_math((kv0 + BC > kend) || (causal && kv0 + BC - 1 > qw0));
        if (jn >= 0) store_tile(buf ^ 1);   // that buffer was last read before the previous barrier
        __syncthreads();
        buf ^= 1;
        jj = jn;
    }

    // ---- epilogue: O = O^T / l, LSE = m + ln l
    const float l_tot = l_run + wave_xor32(l_run);
    float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if constexpr (DROP) inv *= a.drop.keep_scale;
    if (qrow < N) {
        const size_t orow = hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = db * 32 + 8 * g + 4 * hl;
                const float v0 = oacc[db][4 * g] * inv, v1 = oacc[db][4 * g + 1] * inv;
                const float v2 = oacc[db][4 * g + 2] * inv, v3 = oacc[db][4 * g + 3] * inv;
                if (a.o_f32) store4<float>((float*)a.o + orow + dcol, v0, v1, v2, v3);
                else store4<T>((T*)a.o + orow + dcol, v0, v1, v2, v3);
            }
        if (hl == 0)
            a.lse[bh * N + qrow] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f
                                                : -INFINITY;
    }
}

namespace {
template <class T, int D, bool DROP>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    const int total = ((a.N + FWD_BR - 1) / FWD_BR) * a.H * a.B;
    dim3 grid((unsigned)(8 * ((total + 7) / 8)));
    FwdArgs copy = a;
    void* args[] = {(void*)&copy};
    if (a.ev_begin) {
        const hipError_t e = hipEventRecord(a.ev_begin, s);
        if (e != hipSuccess) return e;
    }
    const hipError_t e = hipLaunchKernel((const void*)&fwd_kernel<T, D, DROP>, grid, dim3(256), args, 0, s);
    if (e != hipSuccess || !a.ev_end) return e;
    return hipEventRecord(a.ev_end, s);
}

template <class T>
hipError_t launch_d(const FwdArgs& a, int d, hipStream_t s) {
    const bool drop = a.drop.thr != 0;
    if (d == 64) return drop ? launch_t<T, 64, true>(a, s) : launch_t<T, 64, false>(a, s);
    return drop ? launch_t<T, 128, true>(a, s) : launch_t<T, 128, false>(a, s);
}
}  // namespace

hipError_t launch_fwd(const FwdArgs& a, fa_dtype dt, int d, hipStream_t s) {
    switch (dt) {
        case FA_BF16: return launch_d<bf16>(a, d, s);
        case FA_F16: return launch_d<f16>(a, d, s);
        default: return launch_d<float>(a, d, s);
    }
}

}  // namespace fa
