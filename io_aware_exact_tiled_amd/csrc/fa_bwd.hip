// Backward pass of tiled exact attention for gfx950.
//
// The pages state only that the backward pass recomputes S and P on chip from
// Q, K, V and the saved softmax statistics instead of reading a stored N x N
// matrix (FlashAttention summary, xyznot.com, core ideas, recomputation;
// azimuth.plus explainer, "three ideas in one kernel", recomputation).  The
// gradients follow from the definition with the softmax Jacobian:
//     D_i = sum_k dO_ik O_ik                (pre-pass)
//     P   = exp(S - LSE_i)                  recomputed per tile
//     dV_j += (P o Z / (1-p))^T dO_i
//     dP   = (dO_i V_j^T) o Z / (1-p)
//     dS   = P o (dP - D_i)
//     dK_j += scale dS^T Q_i,   dQ_i += scale dS K_j
//
// Kernels, in launch order on the caller's stream:
//   1. bwd_pre:   D = rowsum(dO o O) (fp32) and the fp32 dQ accumulator set to 0.
//   2. bwd_main:  one workgroup (4 waves) per 128 keys of one (b, h); each wave
//                 owns 32 keys and keeps K_j, V_j in registers and dK_j, dV_j
//                 in fp32 accumulators.  It walks the query tiles of 32 rows
//                 that hold a valid pair.  dQ contributions go through LDS
//                 (dS) and fp32 atomic adds into the workspace.
//   3. bwd_dq:    dQ = scale * accumulator, rounded to the input dtype.
//
// Layout choices (MI355X-specific): S and dP are computed with queries on the
// MFMA rows and keys on the columns, so each lane holds one key and 16
// consecutive queries (query rows are staged in LDS in MFMA row order, as in
// the forward kernel).  Those registers are directly the A operand of
// dV += P^T dO and dK += dS^T Q; the B operands dO and Q are staged a second
// time transposed (d rows, query columns).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

template <class T> __device__ inline void store4g(T* p, float a, float b, float c, float d);
template <> __device__ inline void store4g<f16>(f16* p, float a, float b, float c, float d) {
    f16x4 w = {(f16)a, (f16)b, (f16)c, (f16)d};
    *reinterpret_cast<f16x4*>(p) = w;
}
template <> __device__ inline void store4g<bf16>(bf16* p, float a, float b, float c, float d) {
    bf16x4 w = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4*>(p) = w;
}
template <> __device__ inline void store4g<float>(float* p, float a, float b, float c, float d) {
    f32x4 w = {a, b, c, d};
    *reinterpret_cast<f32x4*>(p) = w;
}

template <class T> __device__ inline typename Mma<T>::frag pack_f(const float* p) {
    if constexpr (Mma<T>::E == 8) {
        typename Mma<T>::frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (T)p[e];
        return f;
    } else {
        return p[0];
    }
}

__device__ inline int row_slot(int r) {
    return (r & ~31) | (((r >> 2) & 3) * 8 + ((r >> 4) & 1) * 4 + (r & 3));
}

}  // namespace

// ---------------------------------------------------------------------------
// D = rowsum(dO o O); dQ accumulator = 0.  8 consecutive elements per lane.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPB = 256 / LPR;             // rows per block
    const size_t rows = (size_t)a.B * a.H * a.N;
    const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c0 = (threadIdx.x % LPR) * 8;
    float acc = 0.0f;
    if (row < rows) {
        const T* dO = (const T*)a.dout + row * D + c0;
        float g[8], o[8];
        if constexpr (sizeof(T) == 2) {
            typedef T t8 __attribute__((ext_vector_type(8)));
            const t8 x = *reinterpret_cast<const t8*>(dO);
#pragma unroll
            for (int e = 0; e < 8; ++e) g[e] = (float)x[e];
        } else {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(dO);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(dO + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { g[e] = x0[e]; g[e + 4] = x1[e]; }
        }
        if (a.o_f32 || sizeof(T) == 4) {
            const float* O = (const float*)a.o + row * D + c0;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(O);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(O + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { o[e] = x0[e]; o[e + 4] = x1[e]; }
        } else {
            typedef T t8 __attribute__((ext_vector_type(8)));
            const t8 x = *reinterpret_cast<const t8*>((const T*)a.o + row * D + c0);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (float)x[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(g[e], o[e], acc);
        float* dq = a.dq_acc + row * D + c0;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(dq) = z;
        *reinterpret_cast<f32x4*>(dq + 4) = z;
    }
#pragma unroll
    for (int s = LPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, WAVE);
    if (row < rows && (threadIdx.x % LPR) == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
template <class T, int D, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdArgs a) {
    typedef Mma<T> MM;
    constexpr int E = MM::E;
    constexpr int BR = BWD_BR, BC = BWD_BC;       // 32 queries per step, 128 keys per workgroup
    constexpr int KS = D / (2 * E);               // MFMA steps over d
    constexpr int DB = D / 32;
    constexpr int QU = 16 / E;                    // MFMA steps over the 32 queries
    constexpr int EPU = 16 / (int)sizeof(T);
    typedef Swz<T, D> LQ;      // Q, dO natural: BR rows (MFMA row order) x D
    typedef Swz<T, BR> LT;     // Q^T, dO^T: D rows x BR queries
    typedef Swz<T, BC> LS;     // dS: BR rows x BC keys;  K^T: D rows x BC keys

    __shared__ __attribute__((aligned(16))) T sQ[BR * D];
    __shared__ __attribute__((aligned(16))) T sdO[BR * D];
    __shared__ __attribute__((aligned(16))) T sQt[D * BR];
    __shared__ __attribute__((aligned(16))) T sdOt[D * BR];
    __shared__ __attribute__((aligned(16))) T sdS[BR * BC];
    __shared__ __attribute__((aligned(16))) T sKt[D * BC];
    __shared__ float sLse[BR];
    __shared__ float sDel[BR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane >> 5, ln = lane & 31;
    const int N = a.N, H = a.H;
    const int Tr = (N + BR - 1) / BR, Tc = (N + BC - 1) / BC;
    const int jt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int kbase = jt * BC, kw0 = kbase + wave * 32;
    const size_t bh = (size_t)b * H + h;
    const size_t hoff = bh * (size_t)N * D;
    const T* __restrict__ Qg = (const T*)a.q + hoff;
    const T* __restrict__ Kg = (const T*)a.k + hoff;
    const T* __restrict__ Vg = (const T*)a.v + hoff;
    const T* __restrict__ dOg = (const T*)a.dout + hoff;
    const float* __restrict__ lseg = a.lse + bh * N;
    const float* __restrict__ delg = a.delta + bh * N;
    float* __restrict__ dqacc = a.dq_acc + hoff;

    int kend = N;
    if (a.mask.key_lens) {
        const int L = a.mask.key_lens[b];
        kend = L < 0 ? 0 : (L > N ? N : L);
    }
    const int causal = a.mask.causal;
    const int i_begin = (causal && kbase < kend) ? kbase / BR : 0;
    const int i_end = (kbase < kend) ? Tr : 0;          // all keys padded: nothing to do

    // tile-visit map: this workgroup owns column jt of the [Tr][Tc] map
    uint8_t* vis = a.tile_visits ? a.tile_visits + bh * Tr * (size_t)Tc + jt : nullptr;
    if (vis) {
        for (int i = tid; i < Tr; i += 256)
            if (i < i_begin || i >= i_end) vis[(size_t)i * Tc] = 0;
    }

    const int krow = kw0 + ln;           // this lane's key
    typename MM::frag kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bool ok = krow < N;
        kf[ks] = ok ? load_frag<T>(Kg + (size_t)krow * D + ks * 2 * E + hl * E) : zero_frag<T>();
        vf[ks] = ok ? load_frag<T>(Vg + (size_t)krow * D + ks * 2 * E + hl * E) : zero_frag<T>();
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dk[db] = zero16(); dv[db] = zero16(); }

    // K^T for the dQ product: D rows x 128 keys
    if (i_begin < i_end) {
        constexpr int DC = D / EPU;
        for (int t = tid; t < (BC / 4) * DC; t += 256) {
            const int dc = t % DC, kg = t / DC;
            T x[4][EPU];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int key = kbase + kg * 4 + kk;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (key < N) val = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + dc * EPU);
                *reinterpret_cast<u32x4*>(&x[kk][0]) = val;
            }
#pragma unroll
            for (int dd = 0; dd < EPU; ++dd)
                store4g<T>(sKt + LS::off(dc * EPU + dd, kg * 4), to_f32(x[0][dd]), to_f32(x[1][dd]),
                           to_f32(x[2][dd]), to_f32(x[3][dd]));
        }
    }

    const float c = a.scale_log2;
    const float LOG2E = 1.4426950408889634f;
    const uint8_t* bmcol = a.mask.block_mask ? a.mask.block_mask + (kbase / MASK_TILE) : nullptr;

    for (int i = i_begin; i < i_end; ++i) {
        const int q0 = i * BR;
        if (bmcol && bmcol[(size_t)(q0 / MASK_TILE) * a.mask.mask_T] == 0) {
            if (vis && tid == 0) vis[(size_t)i * Tc] = 0;
            continue;
        }
        if (vis && tid == 0) vis[(size_t)i * Tc] = 1;

        __syncthreads();   // previous step's LDS readers are done
        // ---- stage Q_i, dO_i (natural, MFMA row order) and transposed, plus LSE, D
        {
            constexpr int DC = D / EPU;
            for (int t = tid; t < 2 * (BR / 4) * DC; t += 256) {
                const int which = t / ((BR / 4) * DC);          // 0: Q, 1: dO
                const int tt = t % ((BR / 4) * DC);
                const int dc = tt % DC, qg = tt / DC;
                const T* src = which ? dOg : Qg;
                T* nat = which ? sdO : sQ;
                T* tr = which ? sdOt : sQt;
                T x[4][EPU];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int r = qg * 4 + kk;
                    const int q = q0 + r;
                    u32x4 val = {0u, 0u, 0u, 0u};
                    if (q < N) val = *reinterpret_cast<const u32x4*>(src + (size_t)q * D + dc * EPU);
                    *reinterpret_cast<u32x4*>(&x[kk][0]) = val;
                    *reinterpret_cast<u32x4*>(nat + LQ::off(row_slot(r), dc * EPU)) = val;
                }
#pragma unroll
                for (int dd = 0; dd < EPU; ++dd)
                    store4g<T>(tr + LT::off(dc * EPU + dd, qg * 4), to_f32(x[0][dd]), to_f32(x[1][dd]),
                               to_f32(x[2][dd]), to_f32(x[3][dd]));
            }
            if (tid < BR) {
                const int q = q0 + tid;
                sLse[tid] = q < N ? lseg[q] * LOG2E : INFINITY;
                sDel[tid] = q < N ? delg[q] : 0.0f;
            }
        }
        __syncthreads();

        const bool wave_live = !(causal && kw0 > q0 + BR - 1) && kw0 < kend;
        if (wave_live) {
            // ---- S = Q_i K_j^T and dP_hat = dO_i V_j^T (queries on rows, keys on columns)
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const typename MM::frag aq = load_frag<T>(sQ + LQ::off(ln, ks * 2 * E + hl * E));
                s = MM::mma(aq, kf[ks], s);
                const typename MM::frag ao = load_frag<T>(sdO + LQ::off(ln, ks * 2 * E + hl * E));
                dp = MM::mma(ao, vf[ks], dp);
            }
            // lane holds key krow and queries q0 + hl*16 + r
            float lse2[16], del[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) { lse2[r] = sLse[hl * 16 + r]; del[r] = sDel[hl * 16 + r]; }
            float p[16], pd[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = q0 + hl * 16 + r;
                const bool valid = (q < N) && (krow < kend) && !(causal && krow > q);
                p[r] = valid ? fast_exp2(fmaf(s[r], c, -lse2[r])) : 0.0f;
            }
            if constexpr (DROP) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t q = (uint32_t)(q0 + hl * 16 + r);
                    const uint32_t bits = keep4((uint32_t)krow >> 2, q, (uint32_t)bh, a.drop.off, a.drop.k0,
                                                a.drop.k1, a.drop.thr);
                    const float z = ((bits >> (krow & 3)) & 1u) ? a.drop.keep_scale : 0.0f;
                    pd[r] = p[r] * z;
                    ds[r] = p[r] * (dp[r] * z - del[r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pd[r] = p[r];
                    ds[r] = p[r] * (dp[r] - del[r]);
                }
            }
            // ---- dV_j += Pd^T dO_i ;  dK_j += dS^T Q_i
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const typename MM::frag ap = pack_f<T>(&pd[u * E]);
                const typename MM::frag as = pack_f<T>(&ds[u * E]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const typename MM::frag bo = load_frag<T>(sdOt + LT::off(db * 32 + ln, hl * 16 + u * E));
                    dv[db] = MM::mma(ap, bo, dv[db]);
                    const typename MM::frag bq = load_frag<T>(sQt + LT::off(db * 32 + ln, hl * 16 + u * E));
                    dk[db] = MM::mma(as, bq, dk[db]);
                }
            }
            // ---- dS to LDS for the dQ product (rows = queries, cols = keys)
#pragma unroll
            for (int r = 0; r < 16; ++r) sdS[LS::off(hl * 16 + r, wave * 32 + ln)] = (T)ds[r];
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) sdS[LS::off(hl * 16 + r, wave * 32 + ln)] = (T)0.0f;
        }
        __syncthreads();

        // ---- dQ_i += dS K_j : output 32 x D split over the waves
        {
            constexpr int SPLIT = (DB >= 4) ? 1 : 4 / DB;      // waves sharing one column block
            constexpr int KEYS = BC / SPLIT;
            const int db = wave % DB;
            const int kpart = (wave / DB) % SPLIT;
            if (wave < DB * SPLIT) {
                f32x16 acc = zero16();
#pragma unroll
                for (int ks = 0; ks < KEYS / (2 * E); ++ks) {
                    const int kc = kpart * KEYS + ks * 2 * E + hl * E;
                    const typename MM::frag as = load_frag<T>(sdS + LS::off(ln, kc));
                    const typename MM::frag bk = load_frag<T>(sKt + LS::off(db * 32 + ln, kc));
                    acc = MM::mma(as, bk, acc);
                }
                const int dcol = db * 32 + ln;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = q0 + 8 * (r / 4) + 4 * hl + (r % 4);
                    if (q < N) unsafeAtomicAdd(dqacc + (size_t)q * D + dcol, acc[r]);
                }
            }
        }
    }

    // ---- dK_j = scale * acc, dV_j = acc (lane holds column db*32+ln, rows = keys)
    T* dKg = (T*)a.dk + hoff;
    T* dVg = (T*)a.dv + hoff;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kw0 + 8 * (r / 4) + 4 * hl + (r % 4);
            if (key < N) {
                dKg[(size_t)key * D + db * 32 + ln] = (T)(dk[db][r] * a.scale);
                dVg[(size_t)key * D + db * 32 + ln] = (T)dv[db][r];
            }
        }
}

// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ acc, T* __restrict__ dq,
                                                     size_t n, float scale) {
    for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (size_t)gridDim.x * 256 * 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(acc + i);
        store4g<T>(dq + i, x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale);
    }
}

namespace {
template <class T, int D, bool DROP>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
    BwdArgs copy = a;
    void* args[] = {(void*)&copy};
    const size_t rows = (size_t)a.B * a.H * a.N;
    constexpr int RPB = 256 / (D / 8);
    hipError_t e = hipLaunchKernel((const void*)&bwd_pre_kernel<T, D>, dim3((unsigned)((rows + RPB - 1) / RPB)),
                                   dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
    dim3 grid((a.N + BWD_BC - 1) / BWD_BC, a.H, a.B);
    if (a.ev_begin && (e = hipEventRecord(a.ev_begin, s)) != hipSuccess) return e;
    e = hipLaunchKernel((const void*)&bwd_main_kernel<T, D, DROP>, grid, dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
    if (a.ev_end && (e = hipEventRecord(a.ev_end, s)) != hipSuccess) return e;
    const float* acc = a.dq_acc;
    T* dq = (T*)a.dq;
    size_t n = rows * D;
    float scale = a.scale;
    size_t blocks = (n / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    void* args2[] = {(void*)&acc, (void*)&dq, (void*)&n, (void*)&scale};
    return hipLaunchKernel((const void*)&bwd_dq_kernel<T>, dim3((unsigned)blocks), dim3(256), args2, 0, s);
}

template <class T>
hipError_t launch_d(const BwdArgs& a, int d, hipStream_t s) {
    const bool drop = a.drop.thr != 0;
    if (d == 64) return drop ? launch_t<T, 64, true>(a, s) : launch_t<T, 64, false>(a, s);
    return drop ? launch_t<T, 128, true>(a, s) : launch_t<T, 128, false>(a, s);
}
}  // namespace

hipError_t launch_bwd(const BwdArgs& a, fa_dtype dt, int d, hipStream_t s) {
    switch (dt) {
        case FA_BF16: return launch_d<bf16>(a, d, s);
        case FA_F16: return launch_d<f16>(a, d, s);
        default: return launch_d<float>(a, d, s);
    }
}

}  // namespace fa
