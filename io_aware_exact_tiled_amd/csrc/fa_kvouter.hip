// Forward pass in the key/value-outer loop order, kept as an IO ablation.
//
// The FlashAttention explainer's step-by-step algorithm (and the summary's
// "Method") walks key/value blocks in the outer loop and query blocks in the
// inner one: K_j and V_j stay on chip while every query block that sees them
// loads its running O_i, l_i, m_i from HBM, updates them and stores them
// back.  That order moves T_c * N * d elements of Q and of O per head (the
// summary's Theta(N^2 d^2 / M) with B_c ~ M / 4d), against about N * d for
// the query-outer fwd_kernel, whose running statistics never leave
// registers.  This kernel computes the same O and LSE in that order so the
// IO model can be checked against measured HBM bytes.
//
// fwd_kvo_kernel<T, D, BC>: one workgroup per (b, h, group g of G).  Group g
// takes the 128-row query blocks it = g, g + G, ... (32 rows per wave), so K
// and V are read G times per head.  For each key tile j (BC keys; K_j and V_j
// double-buffered in LDS with the buffer-to-LDS loads, the next tile landing
// during this one's work) each wave walks its rows of those blocks:
//   load Q rows (registers), the running O (fp32 workspace, accumulator
//   layout), m and l -- or start from O = 0, m = -inf, l = 0 on tile 0;
//   S^T = K_j Q^T, masks, the online-softmax step of fwd_kernel (base 2,
//   lazy rescale), O^T += V_j^T P^T (bf16: P as a high and a low bf16 part,
//   both multiplied, since there is no fp16 V copy here);
//   store O, m, l back -- or, on the last key tile the rows see, write
//   O / l in the output dtype and LSE = m + ln l.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <class T, int D, int BC>
__global__ __launch_bounds__(256, 1) void fwd_kvo_kernel(KvoArgs a) {
    typedef Mma<T> MM;
    constexpr int E = MM::E;            // 8: 16-bit inputs only
    constexpr int BR = 128;             // query block (4 waves x 32 rows)
    constexpr int KS = D / (2 * E);
    constexpr int KB = BC / 32;
    constexpr int DB = D / 32;
    constexpr int TILE = BC * D;
    constexpr float RESCALE = 8.0f;
    constexpr bool SPLIT_P = std::is_same<T, bf16>::value;
    static_assert(E == 8, "16-bit inputs");
    typedef SwzTr<T, D> LK;

    __shared__ __attribute__((aligned(16))) T sK[2 * TILE];
    __shared__ __attribute__((aligned(16))) T sV[2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ln = lane & 31;
    const int N = a.N, G = a.G;
    const int Tr = (N + BR - 1) / BR, Tc = (N + BC - 1) / BC;
    const int bh = (int)blockIdx.x / G, g = (int)blockIdx.x % G;
    if (g >= Tr) return;                               // host keeps G <= Tr; defensive
    const size_t hoff = (size_t)bh * N * D;
    const T* __restrict__ Qg = (const T*)a.q + hoff;
    const T* __restrict__ Kg = (const T*)a.k + hoff;
    const T* __restrict__ Vg = (const T*)a.v + hoff;
    float* __restrict__ Ow = a.ow + hoff;              // running O, fp32 [N][D]
    float* __restrict__ ML = a.ml + (size_t)bh * N * 2;  // running (m, l) per row
    const int causal = a.causal;
    const float c = a.scale_log2;
    // key tiles this group needs: causal rows see keys <= row, so the last
    // query block of the group bounds the walk
    const int it_last = g + ((Tr - 1 - g) / G) * G;
    const int j_end = causal ? min(Tc, (min(it_last * BR + BR, N) - 1) / BC + 1) : Tc;

    auto load_tile = [&](int j, int buf) {
        dma_rows<T, BC, D>(sK + buf * TILE, Kg, j * BC, N, wave, lane);
        dma_rows<T, BC, D>(sV + buf * TILE, Vg, j * BC, N, wave, lane);
    };
    const TrOffsets<T, D> vto(lane);

    load_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    for (int j = 0; j < j_end; ++j) {
        if (j + 1 < j_end) load_tile(j + 1, buf ^ 1);
        const int kv0 = j * BC;
        const T* kt = sK + buf * TILE;
        const T* vt = sV + buf * TILE;
        for (int it = g; it < Tr; it += G) {
            const int qw0 = it * BR + wave * 32;
            if (qw0 >= N) break;                       // later blocks start further down
            if (causal && kv0 > qw0 + 31) continue;    // no key of tile j is visible to these rows
            const int qrow = qw0 + ln;
            const bool rok = qrow < N;
            // the 32 rows share one BC-aligned block, so one last tile
            const int j_last = causal ? qw0 / BC : Tc - 1;
            typename MM::frag qf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = rok ? load_frag<T>(Qg + (size_t)qrow * D + ks * 2 * E + hl * E) : zero_frag<T>();
            f32x16 oacc[DB];
            float m_run = -INFINITY, l_run = 0.0f;
            if (j == 0) {
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] = zero16();
            } else {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        f32x4 w = {0.0f, 0.0f, 0.0f, 0.0f};
                        if (rok) w = *reinterpret_cast<const f32x4*>(Ow + (size_t)qrow * D + db * 32 + 8 * q4 + 4 * hl);
#pragma unroll
                        for (int e = 0; e < 4; ++e) oacc[db][4 * q4 + e] = w[e];
                    }
                if (rok) {                             // each lane reads what it stored
                    m_run = ML[2 * qrow];
                    l_run = hl == 0 ? ML[2 * qrow + 1] : 0.0f;   // the pair sums its halves later
                }
            }
            // ---- S^T = K_j Q^T
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[kb] = zero16();
            lds_chain<T, KB, KS, 2>(
                s, [&](int kb, int ks) { return load_frag<T>(kt + LK::off(kb * 32 + ln, ks * 2 * E + hl * E)); },
                [&](int, int ks) { return qf[ks]; });
            if (kv0 + BC > N || (causal && kv0 + BC - 1 > qw0)) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb * 32 + hl * 16 + r;
                        if (key >= N || (causal && key > qrow)) s[kb][r] = -INFINITY;
                    }
            }
            // ---- online softmax step
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = pair_max(mx) * c;
            if (__any(mx > m_run + RESCALE)) {
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
            // ---- O^T += V_j^T P^T (bf16: high part, then the residual)
            tr_chain<T, D, KB, true, 2>(oacc, vt, vto, [&](int kb, int u) { return pack_p<T>(&p[kb][u * E]); },
                                        lane);
            if constexpr (SPLIT_P) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) p[kb][r] -= (float)(T)p[kb][r];
                tr_chain<T, D, KB, true, 2>(oacc, vt, vto,
                                            [&](int kb, int u) { return pack_p<T>(&p[kb][u * E]); }, lane);
            }
            // ---- state back to HBM, or the result
            const float l_tot = pair_sum(l_run);
            if (rok) {
                if (j == j_last) {
                    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            store4<T>((T*)a.o + hoff + (size_t)qrow * D + db * 32 + 8 * q4 + 4 * hl,
                                      oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv,
                                      oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
                    if (hl == 0)
                        a.lse[(size_t)bh * N + qrow] = l_tot > 0.0f
                                                           ? (m_run + log2f(l_tot)) * 0.69314718055994530942f
                                                           : -INFINITY;
                } else {
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            store4<float>(Ow + (size_t)qrow * D + db * 32 + 8 * q4 + 4 * hl, oacc[db][4 * q4],
                                          oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]);
                    ML[2 * qrow] = m_run;              // both lanes of the pair: same value
                    if (hl == 0) ML[2 * qrow + 1] = l_tot;
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);                 // tile j+1 has landed (this wave's part)
        __syncthreads();                               // and every wave is done with tile j
        buf ^= 1;
    }
}

namespace {
template <class T, int D, int BC>
hipError_t launch_kvo_t(const KvoArgs& a, const hipEvent_t* ev, hipStream_t s) {
    KvoArgs copy = a;
    void* args[] = {(void*)&copy};
    const dim3 grid((unsigned)((size_t)a.B * a.H * a.G));
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e != hipSuccess) return e;
    e = hipLaunchKernel((const void*)&fwd_kvo_kernel<T, D, BC>, grid, dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
    return ev ? hipEventRecord(ev[1], s) : hipSuccess;
}
template <class T, int D>
hipError_t launch_kvo_d(const KvoArgs& a, int bc, const hipEvent_t* ev, hipStream_t s) {
    return bc == 64 ? launch_kvo_t<T, D, 64>(a, ev, s) : launch_kvo_t<T, D, 128>(a, ev, s);
}
}  // namespace

hipError_t launch_kv_outer(const KvoArgs& a, fa_dtype dt, int d, int bc, const hipEvent_t* ev, hipStream_t s) {
    if (dt == FA_BF16) return d == 64 ? launch_kvo_d<bf16, 64>(a, bc, ev, s) : launch_kvo_d<bf16, 128>(a, bc, ev, s);
    return d == 64 ? launch_kvo_d<f16, 64>(a, bc, ev, s) : launch_kvo_d<f16, 128>(a, bc, ev, s);
}

}  // namespace fa
