// Backward pass of tiled exact attention for gfx950.
//
// The pages state only that the backward pass recomputes S and P on chip from
// Q, K, V and the saved softmax statistics instead of reading a stored N x N
// matrix (FlashAttention summary, xyznot.com, core ideas, recomputation;
// azimuth.plus explainer, "three ideas in one kernel", recomputation).  The
// gradients follow from the definition with the softmax Jacobian:
//     D_i = sum_k dO_ik O_ik                          pre-pass
//     P   = exp(S - LSE_i)                            recomputed per tile
//     dV_j = sum_i (P o Z s)_ij dO_i       (Z keep bits, s = 1 / P(keep))
//     dP   = (dO V^T) o Z s,   dS = P o (dP - D)
//     dK_j = scale sum_i dS_ij Q_i,  dQ_i = scale sum_j dS_ij K_j
//
// Kernels, in launch order on the caller's stream:
//   1. bwd_pre:  D = rowsum(dO o O) in fp32 (workspace).
//   2. bwd_kv:   one workgroup (8 waves) per 128 keys of one (b, h); two waves
//                per 32 keys, one holding K_j and dV_j, the other V_j and dK_j;
//                it walks the query tiles of BR rows that hold a valid pair:
//                S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q.
//   3. bwd_dq:   one workgroup (4 waves) per 128 query rows; each wave owns 32
//                rows (one per lane column, with its LSE_i and D_i in
//                registers) and walks the key tiles of 64 that hold a valid
//                pair, each as two blocks of 32 in turn (one barrier and one
//                tile load per 64 keys): S^T = K Q^T, dP^T = V dO^T,
//                dQ^T += K^T dS^T.
// dQ is therefore produced without atomics and without a dS round trip
// through memory, at the price of recomputing S and dP once more (seven
// products per pair instead of five).  Both loops prefetch the next tile into
// the LDS buffer not in use while the current one is computed (one barrier
// per tile).  Tiles are staged in their natural row-major layout with 16-byte
// global-to-LDS loads; operands that are needed transposed are read with the
// gfx950 LDS transpose read instead of being staged twice.
//
// Layouts (MI355X-specific): bwd_kv computes S with queries on the MFMA rows
// and keys on the columns (query rows staged in LDS in MFMA row order so each
// lane holds 16 consecutive queries of its key: these registers are directly
// the A operand of dV += P^T dO and dK += dS^T Q, whose B operands are the
// same Q and dO tiles read transposed).  bwd_dq is the forward kernel's
// layout: keys on the rows (K, V in MFMA row order), one query per lane, and
// the K tile read transposed for dQ^T += K^T dS^T.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

__device__ inline int clamp_len(const int32_t* key_lens, int b, int N) {
    if (!key_lens) return N;
    const int L = key_lens[b];
    return L < 0 ? 0 : (L > N ? N : L);
}

}  // namespace

// ---------------------------------------------------------------------------
// D = rowsum(dO o O) in fp32.  8 consecutive elements per lane.
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
    }
#pragma unroll
    for (int s = LPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, WAVE);
    if (row < rows && (threadIdx.x % LPR) == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: key-stationary, with specialised waves.  NW waves per workgroup,
// two per block of 32 keys (waves w and w + NW/2 share a SIMD):
//   A (w < NW/2):  holds K_j; S = Q K^T, P = exp(S - LSE) with the masks,
//                  hands P to its partner through LDS, dV_j += (P o Z s)^T dO.
//   B (w >= NW/2): holds V_j; dP = dO V^T, then with P from its partner
//                  dS = P o (dP o Z s - D), dK_j += dS^T Q.
// NW = 8 (128 keys per workgroup, one workgroup per CU) for long sequences;
// NW = 4 with 32-row query steps (64 keys, 48 KB of LDS: two workgroups per
// CU) for short ones, where a lone workgroup per CU leaves its prologue and
// epilogue latency exposed.
// Each wave keeps one operand block and one accumulator block, so two waves
// fit on a SIMD.  A and B hold the same (key, query) elements in the same
// lane and register, so the hand-off is a plain per-lane copy.
//
// B runs one query tile behind A so that the SIMD always has MFMA work:
// per step n (barriers marked |)
//   A:  S(n) MFMA     P(n) exp, hand-off      |  dV += P(n)^T dO(n) MFMA      |
//   B:  dP(n) MFMA    dK += dS(n-1)^T Q(n-1)  |  dS(n) from P(n), in regs    |
// so B's dK product overlaps A's exponentials and A's dV product overlaps
// B's dS arithmetic.  Q tiles stay in LDS one step longer (three buffers).
template <class T, int D, bool DROP, int NW, int BR>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 1 : 2) void bwd_kv_kernel(BwdArgs a) {
    typedef Mma<T> MM;
    constexpr int E = MM::E;
    constexpr int NKB = NW / 2;                   // 32-key blocks per workgroup
    constexpr int BC = 32 * NKB;                  // keys per workgroup
    constexpr int QB = BR / 32;                   // 32-row query blocks per step
    constexpr int KS = D / (2 * E);               // MFMA steps over d
    constexpr int DB = D / 32;
    constexpr int QU = 16 / E;                    // MFMA steps over 16 queries of a lane half
    constexpr int TQ = BR * D;                    // elements per staged tensor
    constexpr int NX = DROP ? 2 : 1;              // hand-off planes: P (and P o Z s)
    // The eight-wave configuration with 16-bit inputs hands P over already
    // packed as the dV operand (QU 16-byte fragments per 32-row block): half
    // the hand-off bytes in the LDS-bound long-sequence case.  The four-wave
    // one (and fp32) hands over four f32x4 chunks: there the packed form's
    // extra registers cost a wave per SIMD.
    constexpr bool PACKED = sizeof(T) == 2 && NW == 8;
    constexpr int XCH = PACKED ? QU : 4;          // 16-byte hand-off slots per lane per query block
    typedef SwzTr<T, D> LQ;    // Q, dO: BR rows (MFMA row order) x D

    __shared__ __attribute__((aligned(16))) T sQ[3 * TQ];
    __shared__ __attribute__((aligned(16))) T sdO[2 * TQ];
    __shared__ __attribute__((aligned(16))) float sLse[2 * BR];
    __shared__ __attribute__((aligned(16))) float sDel[2 * BR];
    // hand-off [key block][plane][query block][XCH slots][64 lanes] x 16 bytes
    __shared__ __attribute__((aligned(16))) f32x4 sX[NKB * NX * QB * XCH * 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane >> 5, ln = lane & 31;
    const int kb = wave % NKB;                    // key block of this wave
    const bool roleA = wave < NKB;
    const int N = a.N, H = a.H, Hkv = a.Hkv, G = H / Hkv;
    const int Tr = (N + BR - 1) / BR, Tc = (N + BC - 1) / BC;
    // key tile jt = 0 visits the most query tiles under the causal mask
    const int item = xcd_item((int)blockIdx.x, Hkv * a.B, Tc, a.mask.causal);
    if (item < 0) return;
    const int bkv = item / Tc;                    // (b, K/V head)
    const int bidx = bkv / Hkv, g = bkv % Hkv;
    const int jt = item % Tc;                     // key tile of this workgroup
    const int kbase = jt * BC, kw0 = kbase + kb * 32;
    const size_t koff = (size_t)bkv * N * D;
    const T* __restrict__ Kg = (const T*)a.k + koff;
    const T* __restrict__ Vg = (const T*)a.v + koff;
    // the G query heads that share this K/V head: dK_j, dV_j sum over all of them
    auto qhead = [&](int hh) -> size_t { return (size_t)bidx * H + (size_t)g * G + hh; };

    const int kend = clamp_len(a.mask.key_lens, bidx, N);
    const int causal = a.mask.causal;
    const bool live = kbase < kend;
    const int i_begin = (causal && live) ? kbase / BR : 0;
    const int i_end = live ? Tr : 0;
    const uint8_t* bmcol = a.mask.block_mask ? a.mask.block_mask + (kbase / MASK_TILE) : nullptr;
    auto tile_at = [&](int i) -> int {   // next visited query tile >= i, or -1
        for (; i < i_end; ++i)
            if (!bmcol || bmcol[(size_t)((i * BR) / MASK_TILE) * a.mask.mask_T]) return i;
        return -1;
    };

    auto vis_at = [&](int hh) { return a.tile_visits + qhead(hh) * Tr * (size_t)Tc + jt; };
    if (a.tile_visits)
        for (int hh = 0; hh < G; ++hh)
            for (int i = tid; i < Tr; i += NW * 64) vis_at(hh)[(size_t)i * Tc] = 0;

    const int krow = kw0 + ln;           // this lane's key
    // role A holds K_j, role B holds V_j (as the MFMA B operand of S / dP)
    typename MM::frag kvf[KS];
    {
        const T* src = roleA ? Kg : Vg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kvf[ks] = krow < N ? load_frag<T>(src + (size_t)krow * D + ks * 2 * E + hl * E) : zero_frag<T>();
        }
    }
    f32x16 acc[DB];                      // dV_j (A) or dK_j (B)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero16();

    // ---- staging of one query tile: Q, dO by global->LDS DMA; LSE, D via registers
    float lreg = 0.0f;
    auto load_tile = [&](int hh, int i, int qbuf, int obuf) {
        const int q0 = i * BR;
        const size_t qh = qhead(hh);
        dma_rows<T, BR, D, NW>(sQ + qbuf * TQ, (const T*)a.q + qh * N * D, q0, N, wave, lane);
        dma_rows<T, BR, D, NW>(sdO + obuf * TQ, (const T*)a.dout + qh * N * D, q0, N, wave, lane);
        if (tid < 2 * BR) {
            const int q = q0 + (tid % BR);
            lreg = (q < N) ? (tid < BR ? a.lse[qh * N + q] : a.delta[qh * N + q]) : (tid < BR ? INFINITY : 0.0f);
        }
    };
    auto publish_stats = [&](int obuf) {
        if (tid < BR) sLse[obuf * BR + tid] = lreg * 1.4426950408889634f;
        else if (tid < 2 * BR) sDel[obuf * BR + tid - BR] = lreg;
    };
    auto xslot = [&](int plane, int qb, int chunk) -> f32x4* {
        return &sX[(((kb * NX + plane) * QB + qb) * XCH + chunk) * 64 + lane];
    };
    auto xfrag = [&](int plane, int qb, int u) -> typename MM::frag* {
        return reinterpret_cast<typename MM::frag*>(xslot(plane, qb, u));
    };
    // B: dK_j += dS^T Q over one query tile; dS as packed A operands (query
    // block qb, 16-query step u), Q read transposed from its LDS buffer
    const TrOffsets<T, D> tro(lane);
    typename MM::frag dsf[QB][QU];
    typename MM::frag pf[QB][QU];        // A (16-bit inputs): P packed, the dV operand
    auto dk_product = [&](const T* q) __attribute__((always_inline)) {
        tr_chain<T, D, QB, false, 2>(acc, q, tro, [&](int qb, int u) { return dsf[qb][u]; }, lane);
    };

    const float c = a.scale_log2;
    // One loop per role (the role is fixed per wave), so that each is
    // register-allocated on its own; both pass the same barriers.
    auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool RA = decltype(role)::value;
    // walk over (query head hh of the group, visited query tile i); every head
    // visits the same tiles
    const int i_first = tile_at(i_begin);
    int hh = 0, i = i_first;
    auto next_step = [&](int& h2, int& i2) {
        const int t = tile_at(i2 + 1);
        if (t >= 0) i2 = t;
        else if (h2 + 1 < G) { ++h2; i2 = i_first; }
        else i2 = -1;
    };
    if (i >= 0) {
        load_tile(hh, i, 0, 0);
        publish_stats(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int qbuf = 0, obuf = 0, qprev = 0;
    bool have_prev = false;              // B holds dS of the previous step in dsf
    while (i >= 0) {
        const int q0 = i * BR;
        const uint32_t bh = (uint32_t)qhead(hh);  // query head: the dropout stream
        if (a.tile_visits && tid == 0) vis_at(hh)[(size_t)i * Tc] = 1;
        int hn = hh, in = i;
        next_step(hn, in);
        const int qnext = qbuf == 2 ? 0 : qbuf + 1;
        // lands in the other buffers during this step; the Q buffer last held
        // step n-2 (read by B before the previous step's first barrier), the
        // dO buffer step n-1 (read before the previous step's second barrier)
        if (in >= 0) load_tile(hn, in, qnext, obuf ^ 1);

        const T* q = sQ + qbuf * TQ;
        const T* o = sdO + obuf * TQ;
        const float* ls = sLse + obuf * BR;
        const float* dl = sDel + obuf * BR;
        // first product: S = Q K^T (A) or dP_hat = dO V^T (B); lane holds key krow,
        // queries q0 + 32qb + 16hl + r (operands read ahead)
        f32x16 sp[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sp[qb] = zero16();
        // this step's row statistics (A: LSE, B: D), 16 rows of the lane half
        // per query block.  Eight waves: read into registers before the first
        // chain, so the VALU phase that needs them does not start on an LDS
        // wait (dK/dV 1.4-1.9 % faster at d = 128); four waves: read where used.
        f32x4 st4[QB][4];
        auto stat4 = [&](int qb, int g) -> f32x4 {
            if constexpr (NW == 8) return st4[qb][g];
            else return *reinterpret_cast<const f32x4*>((RA ? ls : dl) + qb * 32 + hl * 16 + 4 * g);
        };
        if constexpr (NW == 8) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    st4[qb][g] = *reinterpret_cast<const f32x4*>((RA ? ls : dl) + qb * 32 + hl * 16 + 4 * g);
        }
        __builtin_amdgcn_s_setprio(1);
        {
            const T* src = RA ? q : o;
            lds_chain<T, QB, KS, BWD_PF<D>>(
                sp, [&](int qb, int ks) { return load_frag<T>(src + LQ::off(qb * 32 + ln, ks * 2 * E + hl * E)); },
                [&](int, int ks) { return kvf[ks]; });
        }
        __builtin_amdgcn_s_setprio(0);

        if constexpr (RA) {
            // P = exp(S - LSE) with the masks, handed to B (kept for dV)
            const bool edge = (causal && kw0 + 31 > q0) || (kw0 + 32 > kend) || (q0 + BR > N);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qr0 = qb * 32 + hl * 16;
                float p[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 l4 = stat4(qb, g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) p[4 * g + e] = fast_exp2(fmaf(sp[qb][4 * g + e], c, -l4[e]));
                }
                if (__builtin_expect(edge, 0)) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qq = q0 + qr0 + r;
                        if (qq >= N || krow >= kend || (causal && krow > qq)) p[r] = 0.0f;
                    }
                }
                if constexpr (PACKED) {
                    // one packing serves both the hand-off and this wave's dV operand
#pragma unroll
                    for (int u = 0; u < QU; ++u) {
                        pf[qb][u] = pack_p<T>(&p[u * E]);
                        *xfrag(0, qb, u) = pf[qb][u];
                    }
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v4 = {p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
                        *xslot(0, qb, g) = v4;
                    }
                }
                if constexpr (DROP) {
                    const uint32_t keep = keep16_quad((uint32_t)krow, (uint32_t)(q0 + qr0), (uint32_t)bh, a.drop.off,
                                                      a.drop.k0, a.drop.k1, a.drop.thr, lane);
#pragma unroll
                    for (int r = 0; r < 16; ++r) p[r] *= ((keep >> r) & 1u) ? a.drop.keep_scale : 0.0f;
                    if constexpr (PACKED) {
#pragma unroll
                        for (int u = 0; u < QU; ++u) {
                            pf[qb][u] = pack_p<T>(&p[u * E]);
                            *xfrag(1, qb, u) = pf[qb][u];
                        }
                    } else {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const f32x4 v4 = {p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
                            *xslot(1, qb, g) = v4;
                        }
                    }
                }
                if constexpr (!PACKED) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sp[qb][r] = p[r];
                }
            }
        } else if (have_prev) {
            // the previous step's dK product, while A computes P
            __builtin_amdgcn_s_setprio(1);
            dk_product(sQ + qprev * TQ);
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();   // P handed over
        if constexpr (RA) {
            // dV_j += Pd^T dO
            __builtin_amdgcn_s_setprio(1);
            tr_chain<T, D, QB, false, 2>(acc, o, tro, [&](int qb, int u) {
                if constexpr (PACKED) {
                    return pf[qb][u];
                } else {
                    float pr[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) pr[e] = sp[qb][u * E + e];
                    return pack_p<T>(pr);
                }
            }, lane);
            __builtin_amdgcn_s_setprio(0);
        } else {
            // dS = P o (dP - D), kept as packed operands for the next step
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float ds[16];
                if constexpr (PACKED) {
                    // P (and Pd = P o Z s) of the 16 queries from the packed fragments
                    float pv[16], pdv[16];
#pragma unroll
                    for (int u = 0; u < QU; ++u) {
                        const typename MM::frag f = *xfrag(0, qb, u);
#pragma unroll
                        for (int e = 0; e < E; ++e) pv[u * E + e] = (float)f[e];
                        if constexpr (DROP) {
                            const typename MM::frag fd = *xfrag(1, qb, u);
#pragma unroll
                            for (int e = 0; e < E; ++e) pdv[u * E + e] = (float)fd[e];
                        }
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 d4 = stat4(qb, g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * g + e;
                            if constexpr (DROP) ds[r] = pdv[r] * sp[qb][r] - pv[r] * d4[e];   // Pd dP_hat - P D
                            else ds[r] = pv[r] * (sp[qb][r] - d4[e]);
                        }
                    }
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 p4 = *xslot(0, qb, g);
                        const f32x4 d4 = stat4(qb, g);
                        if constexpr (DROP) {
                            // dS = P dP_hat Z s - P D = Pd dP_hat - P D
                            const f32x4 pd4 = *xslot(1, qb, g);
#pragma unroll
                            for (int e = 0; e < 4; ++e) ds[4 * g + e] = pd4[e] * sp[qb][4 * g + e] - p4[e] * d4[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) ds[4 * g + e] = p4[e] * (sp[qb][4 * g + e] - d4[e]);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < QU; ++u) dsf[qb][u] = pack_p<T>(&ds[u * E]);
            }
            have_prev = true;
        }
        if (in >= 0) publish_stats(obuf ^ 1);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA into the other buffers has landed
        __syncthreads();                 // also: the hand-off buffer may be overwritten
        qprev = qbuf;
        qbuf = qnext;
        obuf ^= 1;
        hh = hn;
        i = in;
    }
    // B: the last step's dK product (its Q tile is still in place: no DMA follows)
    if constexpr (!RA) {
        if (have_prev) dk_product(sQ + qprev * TQ);
    }
    };
    if (roleA) run(std::true_type{});
    else run(std::false_type{});

    // ---- dV_j = acc (A), dK_j = scale * acc (B); lane holds column db*32+ln, rows = keys
    T* dst = (T*)(roleA ? a.dv : a.dk) + koff;
    const float sc = roleA ? 1.0f : a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kw0 + 8 * (r / 4) + 4 * hl + (r % 4);
            if (key < N) dst[(size_t)key * D + db * 32 + ln] = (T)(acc[db][r] * sc);
        }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary.
template <class T, int D, bool DROP>
__global__ __launch_bounds__(256, sizeof(T) == 4 ? 1 : 2) void bwd_dq_kernel(BwdArgs a) {
    typedef Mma<T> MM;
    constexpr int E = MM::E;
    constexpr int BR = BWD_DQ_BR, BC = BWD_DQ_BC;   // 128 query rows, 64-key tiles
    constexpr int NSB = BC / 32;                     // 32-key blocks per staged tile, walked in turn
    constexpr int KS = D / (2 * E);
    constexpr int DB = D / 32;
    constexpr int PU = 16 / E;
    constexpr int TK = BC * D;
    typedef SwzTr<T, D> LK;    // K, V: BC rows (MFMA row order) x D

    __shared__ __attribute__((aligned(16))) T sK[2 * TK];
    __shared__ __attribute__((aligned(16))) T sV[2 * TK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ln = lane & 31;
    const int N = a.N, H = a.H;
    const int Tr = (N + BR - 1) / BR, Tc = (N + BC - 1) / BC;
    const int item = xcd_item((int)blockIdx.x, H * a.B, Tr, a.mask.causal);
    if (item < 0) return;
    const int bhi = item / Tr, r_ = item % Tr;
    const int it = a.mask.causal ? (Tr - 1 - r_) : r_;
    const int q0 = it * BR, qw0 = q0 + wave * 32;
    const size_t bh = (size_t)bhi;
    const size_t hoff = bh * (size_t)N * D;
    const size_t koff = ((size_t)(bhi / H) * a.Hkv + (bhi % H) / (H / a.Hkv)) * (size_t)N * D;
    const T* __restrict__ Qg = (const T*)a.q + hoff;
    const T* __restrict__ Kg = (const T*)a.k + koff;
    const T* __restrict__ Vg = (const T*)a.v + koff;
    const T* __restrict__ dOg = (const T*)a.dout + hoff;

    const int kend = clamp_len(a.mask.key_lens, bhi / H, N);
    const int causal = a.mask.causal;
    int j_end = min(Tc, (kend + BC - 1) / BC);
    if (causal) j_end = min(j_end, (min(q0 + BR, N) - 1) / BC + 1);
    const uint8_t* bmask = a.mask.block_mask ? a.mask.block_mask + (size_t)(q0 / MASK_TILE) * a.mask.mask_T
                                             : nullptr;
    auto tile_at = [&](int j) -> int {
        for (; j < j_end; ++j)
            if (!bmask || bmask[(j * BC) / MASK_TILE]) return j;
        return -1;
    };

    uint8_t* vis = a.tile_visits2 ? a.tile_visits2 + (bh * Tr + it) * (size_t)Tc : nullptr;
    if (vis)
        for (int j = tid; j < Tc; j += 256) vis[j] = 0;

    // this lane's query row: Q and dO rows as B operands, LSE and D as scalars
    const int qrow = qw0 + ln;
    const bool qok = qrow < N;
    typename MM::frag qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = qok ? load_frag<T>(Qg + (size_t)qrow * D + ks * 2 * E + hl * E) : zero_frag<T>();
        of[ks] = qok ? load_frag<T>(dOg + (size_t)qrow * D + ks * 2 * E + hl * E) : zero_frag<T>();
    }
    const float lse2 = qok ? a.lse[bh * N + qrow] * 1.4426950408889634f : INFINITY;
    const float del = qok ? a.delta[bh * N + qrow] : 0.0f;
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();
    const TrOffsets<T, D> tro(lane);   // transpose reads of K_j^T

    auto load_tile = [&](int j, int buf) {
        dma_rows<T, BC, D>(sK + buf * TK, Kg, j * BC, N, wave, lane);
        dma_rows<T, BC, D>(sV + buf * TK, Vg, j * BC, N, wave, lane);
    };

    const float c = a.scale_log2;
    int j = tile_at(0);
    if (j >= 0) load_tile(j, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    while (j >= 0) {
        const int kv0 = j * BC;
        if (vis && tid == 0) vis[j] = 1;
        const int jn = tile_at(j + 1);
        if (jn >= 0) load_tile(jn, buf ^ 1);

#pragma unroll 1
        for (int sb = 0; sb < NSB; ++sb) {   // in turn: the registers of one block at a time
          const int kb0 = kv0 + sb * 32;   // this 32-key block of the staged tile
          // skip blocks past the valid keys or above the diagonal for all of this wave's rows
          if (kb0 < kend && !(causal && kb0 > qw0 + 31)) {
            const T* k = sK + buf * TK + sb * 32 * D;
            const T* v = sV + buf * TK + sb * 32 * D;
            // S^T = K Q^T, dP_hat^T = V dO^T: lane holds query qrow, keys kb0 + 16hl + r
            // (chain 0: S, chain 1: dP; operands read ahead)
            f32x16 sd[2] = {zero16(), zero16()};
            __builtin_amdgcn_s_setprio(1);
            lds_chain<T, 2, KS, BWD_PF<D>>(
                sd, [&](int c, int ks) { return load_frag<T>((c ? v : k) + LK::off(ln, ks * 2 * E + hl * E)); },
                [&](int c, int ks) { return c ? of[ks] : qf[ks]; });
            __builtin_amdgcn_s_setprio(0);
            const f32x16 s = sd[0], dp = sd[1];
            const bool edge = (kb0 + 32 > kend) || (causal && kb0 + 31 > qw0);
            float ds[16];
            uint32_t keep = 0xFFFFu;
            if constexpr (DROP) {
                // keys kb0 + 16hl + r; lanes l and l ^ 1 hold rows qrow, qrow ^ 1 and share calls
                const uint32_t g0 = (uint32_t)(kb0 + hl * 16) >> 2;
                keep = keep16_row(g0, (uint32_t)qrow, (uint32_t)bh, a.drop.off, a.drop.k0, a.drop.k1, a.drop.thr);
            }
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(s[r], c, -lse2));
            if (__builtin_expect(edge, 0)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb0 + hl * 16 + r;
                    if (key >= kend || (causal && key > qrow)) p[r] = 0.0f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float dpr = dp[r];
                if constexpr (DROP) dpr *= ((keep >> r) & 1u) ? a.drop.keep_scale : 0.0f;
                ds[r] = p[r] * (dpr - del);
            }
            // dQ^T += K^T dS^T: the A operand is the K tile read transposed; k-slot
            // kk of MFMA u is key 16(kk/E) + uE + kk%E of the tile
            {
                typename MM::frag bs[PU];
#pragma unroll
                for (int u = 0; u < PU; ++u) bs[u] = pack_p<T>(&ds[u * E]);
                __builtin_amdgcn_s_setprio(1);
                tr_chain<T, D, 1, true, 2>(dq, k, tro, [&](int, int u) { return bs[u]; }, lane);
                __builtin_amdgcn_s_setprio(0);
            }
        }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA into the other buffer has landed
        __syncthreads();
        buf ^= 1;
        j = jn;
    }

    // ---- dQ = scale * dQ^T (lane holds query qrow, columns db*32 + 8(r/4) + 4hl + r%4)
    if (qok) {
        T* dQg = (T*)a.dq + hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4<T>(dQg + db * 32 + 8 * g + 4 * hl, dq[db][4 * g] * a.scale, dq[db][4 * g + 1] * a.scale,
                           dq[db][4 * g + 2] * a.scale, dq[db][4 * g + 3] * a.scale);
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
    // the dK/dV configuration: 64-key workgroups for 16-bit inputs at d = 64
    // and for causal sequences up to BWD_KV_SMALL_N, where they were measured
    // faster (a recorded tile map has that configuration's tile shape)
    const bool small = bwd_kv_small(sizeof(T) == 4 ? FA_F32 : FA_BF16, D, a.N, a.mask.causal);
    const int kbc = small ? BWD_KV_SMALL_BC : BWD_KV_BC;
    const int kv_total = ((a.N + kbc - 1) / kbc) * a.Hkv * a.B;
    const int dq_total = ((a.N + BWD_DQ_BR - 1) / BWD_DQ_BR) * a.H * a.B;
    if (a.ev_begin && (e = hipEventRecord(a.ev_begin, s)) != hipSuccess) return e;
    const dim3 kv_grid((unsigned)(8 * ((kv_total + 7) / 8)));
    const void* kv_fn = (const void*)&bwd_kv_kernel<T, D, DROP, 8, BwdTiles<T>::KV_BR>;
    if constexpr (sizeof(T) == 2) {
        if (small) kv_fn = (const void*)&bwd_kv_kernel<T, D, DROP, 4, BWD_KV_SMALL_BR>;
    }
    e = hipLaunchKernel(kv_fn, kv_grid, dim3(small ? 256 : 512), args, 0, s);
    if (e != hipSuccess) return e;
    if (a.ev_mid && (e = hipEventRecord(a.ev_mid, s)) != hipSuccess) return e;
    e = hipLaunchKernel((const void*)&bwd_dq_kernel<T, D, DROP>, dim3((unsigned)(8 * ((dq_total + 7) / 8))),
                        dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
    if (a.ev_end && (e = hipEventRecord(a.ev_end, s)) != hipSuccess) return e;
    return hipSuccess;
}

template <class T>
hipError_t launch_d(const BwdArgs& a, int d, hipStream_t s) {
    const bool drop = a.drop.on != 0;
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
