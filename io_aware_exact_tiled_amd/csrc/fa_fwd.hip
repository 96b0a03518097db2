// Forward pass of tiled exact attention for gfx950.
//
// One workgroup (4 waves) owns BR = 128 query rows of one (b, h); each wave
// owns 32 of them.  The workgroup walks the key/value tiles of BC = 64 keys
// that hold at least one valid pair (FlashAttention summary, xyznot.com,
// "Method"; the query-outer / key-inner loop order of the tutorial's section
// 12.2 pseudocode), staging K_j and V_j in LDS, and per tile:
//   S^T = K_j Q_i^T          MFMA, fp32 accumulation, one query per lane column
//   masks on edge tiles      causal j > i, key padding j >= len_b, N tail
//   m_new = max(m, rowmax)   lane-local max over 16 keys + one cross-half swap
//   P = exp2(S*scale*log2e - m_new),  l = e^{m - m_new} l + rowsum(P)
//   dropout keep bits        Philox4x32-10, one call per 4 keys x 2 rows
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
//  * K and V tiles go global -> LDS with the 16-byte direct loads (no
//    registers, no VALU), rows in MFMA row order: LDS row m of a 32-row block
//    holds key 16*((m/4)%2) + 4*(m/8) + m%4, so that lane half h of the S^T
//    accumulator holds the 16 *consecutive* keys 16h + r in registers r.
//    Those 16 values are then exactly the B operand of the P*V product (8
//    consecutive keys per MFMA per lane half), with no register shuffles.
//  * The A operand V_j^T of that product is read from the row-major V tile
//    with the gfx950 LDS transpose read.
//  * bf16 inputs: P is rounded to fp16 (11-bit significand) rather than bf16
//    (8 bits) for the P*V product, so V must be fp16 as well.  A pre-pass
//    writes V * 2^-e_bh in fp16 to the workspace once per call, with e_bh = 0
//    while the largest finite |V| of the (b, h) lies in [2^-6, 2^15) and
//    otherwise the power of two that brings it into [2^14, 2^15); the
//    epilogue multiplies O by 2^e_bh.  Every bf16 value of magnitude at
//    least 2^(e_bh - 17) converts exactly; smaller ones are off by at most
//    2^(e_bh - 25).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

// maximum over a 256-thread workgroup (every thread gets it)
__device__ inline uint32_t block_max256(uint32_t m) {
    __shared__ uint32_t red[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    return max(max(red[0], red[1]), max(red[2], red[3]));
}

}  // namespace

// ---------------------------------------------------------------------------
// bf16 V -> fp16 pre-pass: two kernels over one grid, workgroup w taking chunk
// w % nch of (b, h) = w / nch.  The first converts its chunk unscaled and, in
// the same read, records the chunk's largest finite |V| as bf16 magnitude
// bits (monotone in the value).  The second reduces the maxima of its (b, h)
// and picks the exponent e_bh: 0 while the largest |V| lies in [2^-6, 2^15)
// -- nothing overflows, and values that fp16 holds only as subnormals are
// then more than 2^8 below the largest, with absolute error <= 2^-25 --
// else the power of two that brings the largest into [2^14, 2^15).  Only
// heads with e_bh != 0 are converted again, as V * 2^-e_bh.
__device__ inline int v16_exponent(uint32_t M) {
    if (M == 0) return 0;
    const int F = (int)(M >> 7);   // bf16 exponent field: the largest is in [2^(F-127), 2^(F-126))
    if (F >= 121 && F < 142) return 0;
    return F - 141;                // F = 0 (a subnormal, >= 2^-133) included
}

__device__ inline void v16_convert_chunk(const V16Args& a, size_t bh, size_t ch, int e) {
    const size_t beg = ch * a.chunk;
    const size_t end = beg + a.chunk < a.per_head ? beg + a.chunk : a.per_head;
    const uint16_t* src = static_cast<const uint16_t*>(a.v) + bh * a.per_head;
    f16* dst = a.v16 + bh * a.per_head;
    for (size_t i = beg + (size_t)threadIdx.x * 8; i < end; i += 256 * 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + i);
        f16x8 h;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            h[2 * k] = (f16)ldexpf(__uint_as_float(w[k] << 16), -e);
            h[2 * k + 1] = (f16)ldexpf(__uint_as_float(w[k] & 0xffff0000u), -e);
        }
        *reinterpret_cast<f16x8*>(dst + i) = h;
    }
}

__global__ __launch_bounds__(256) void v16_convert_kernel(V16Args a) {
    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x / a.nch, ch = blockIdx.x % a.nch;
    const size_t beg = ch * a.chunk;
    const size_t end = beg + a.chunk < a.per_head ? beg + a.chunk : a.per_head;
    const uint16_t* src = static_cast<const uint16_t*>(a.v) + bh * a.per_head;
    f16* dst = a.v16 + bh * a.per_head;
    uint32_t m = 0;
    for (size_t i = beg + (size_t)tid * 8; i < end; i += 256 * 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + i);
        f16x8 h;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = w[k] & 0x7fffu, hi = (w[k] >> 16) & 0x7fffu;
            if (lo < 0x7f80u) m = max(m, lo);   // exponent field all ones: inf or NaN
            if (hi < 0x7f80u) m = max(m, hi);
            h[2 * k] = (f16)__uint_as_float(w[k] << 16);
            h[2 * k + 1] = (f16)__uint_as_float(w[k] & 0xffff0000u);
        }
        *reinterpret_cast<f16x8*>(dst + i) = h;
    }
    m = block_max256(m);
    if (tid == 0) a.part[bh * a.nch + ch] = m;
}

__global__ __launch_bounds__(256) void v16_rescale_kernel(V16Args a) {
    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x / a.nch, ch = blockIdx.x % a.nch;
    const int e = v16_exponent(block_max256(tid < a.nch ? a.part[bh * a.nch + tid] : 0u));
    if (ch == 0 && tid == 0) a.vexp[bh] = e;
    if (e != 0) v16_convert_chunk(a, bh, ch, e);   // else the unscaled copy stands
}

// ---------------------------------------------------------------------------
template <class T, int D, bool DROP>
__global__ __launch_bounds__(256, sizeof(T) == 4 ? 1 : 2) void fwd_kernel(FwdArgs a) {
    typedef typename PvType<T>::type TV;
    typedef Mma<T> MS;
    typedef Mma<TV> MV;
    constexpr int E = MS::E;
    constexpr int EV = MV::E;
    constexpr int BR = FWD_BR, BC = FWD_BC;
    constexpr int KS = D / (2 * E);     // MFMA steps over d in S^T
    constexpr int KB = BC / 32;         // 32-key blocks per tile
    constexpr int DB = D / 32;          // 32-wide column blocks of O
    constexpr int TILE = BC * D;        // elements of one K (or V) buffer
    constexpr float RESCALE = 8.0f;     // log2 headroom before the running max moves
    typedef SwzTr<T, D> LK;

    __shared__ __attribute__((aligned(16))) T sK[2 * TILE];
    __shared__ __attribute__((aligned(16))) TV sV[2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ln = lane & 31;
    const int N = a.N, H = a.H;
    const int Tr = (N + BR - 1) / BR, Tc = (N + BC - 1) / BC;
    // work item: contiguous head ranges per XCD; inside a head, heaviest tiles first
    const int item = xcd_item((int)blockIdx.x, H * a.B, Tr, a.mask.causal);
    if (item < 0) return;
    const int bhi = item / Tr, r_ = item % Tr;
    const int it = a.mask.causal ? (Tr - 1 - r_) : r_;
    const int q0 = it * BR, qw0 = q0 + wave * 32;
    const size_t bh = (size_t)bhi;
    const size_t hoff = bh * (size_t)N * D;
    // K/V head of this query head (grouped-query attention: H / Hkv query
    // heads share one K/V head)
    const size_t bkv = (size_t)(bhi / H) * a.Hkv + (bhi % H) / (H / a.Hkv);
    const size_t koff = bkv * (size_t)N * D;
    const T* __restrict__ Qg = (const T*)a.q + hoff;
    const T* __restrict__ Kg = (const T*)a.k + koff;
    const TV* __restrict__ Vg = (const TV*)a.v + koff;   // the fp16 copy for bf16 inputs

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

    // K_j, V_j: global -> LDS, rows past N read as zeros (masked as keys >= kend)
    auto load_tile = [&](int j, int buf) {
        dma_rows<T, BC, D>(sK + buf * TILE, Kg, j * BC, N, wave, lane);
        dma_rows<TV, BC, D>(sV + buf * TILE, Vg, j * BC, N, wave, lane);
    };

    const TrOffsets<TV, D> vto(lane);   // transpose reads of V_j^T

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = zero16();

    const float c = a.scale_log2;
    const int causal = a.mask.causal;

    int jj = tile_at(0);
    if (jj >= 0) load_tile(rev ? (j_end - 1 - jj) : jj, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    while (jj >= 0) {
        const int j = rev ? (j_end - 1 - jj) : jj;
        const int kv0 = j * BC;
        if (vis && tid == 0) vis[j] = 1;
        const int jn = tile_at(jj + 1);
        // lands in the other buffer during this tile's math; that buffer was
        // last read before the previous barrier
        if (jn >= 0) load_tile(rev ? (j_end - 1 - jn) : jn, buf ^ 1);

        // one tile of math; element masks only on tiles that straddle the
        // diagonal, the padding boundary or the N tail
        auto tile_math = [&](bool edge) {
            const T* k = sK + buf * TILE;
            const TV* v = sV + buf * TILE;
            // ---- S^T = K_j Q^T (K operands read ahead)
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[kb] = zero16();
            __builtin_amdgcn_s_setprio(1);
            lds_chain<T, KB, KS, FWD_PF<D>>(
                s, [&](int kb, int ks) { return load_frag<T>(k + LK::off(kb * 32 + ln, ks * 2 * E + hl * E)); },
                [&](int, int ks) { return qf[ks]; });
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
            mx = pair_max(mx) * c;
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
                // keys kv0 + 32kb + 16hl + r of this lane's row; rows qrow and qrow ^ 1 sit in
                // lanes l and l ^ 1 and share their generator calls
                const uint32_t g0 = (uint32_t)(kv0 + hl * 16) >> 2;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const uint32_t bits = keep16_row(g0 + kb * 8, (uint32_t)qrow, (uint32_t)bh, a.drop.off,
                                                     a.drop.k0, a.drop.k1, a.drop.thr);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (!((bits >> r) & 1u)) p[kb][r] = 0.0f;
                }
            }
            // ---- O^T += V_j^T P^T: k-slot kk of step (kb, u) is key
            // 32kb + 16(kk/EV) + u*EV + kk%EV, the lane half's own keys
            __builtin_amdgcn_s_setprio(1);
            tr_chain<TV, D, KB, true, 2>(oacc, v, vto, [&](int kb, int u) { return pack_p<TV>(&p[kb][u * EV]); },
                                         lane);
            __builtin_amdgcn_s_setprio(0);
        };
        if (!(causal && kv0 > qw0 + 31))   // else: no valid key for this wave's rows
            tile_math((kv0 + BC > kend) || (causal && kv0 + BC - 1 > qw0));
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads into the other buffer have landed
        __syncthreads();
        buf ^= 1;
        jj = jn;
    }

    // ---- epilogue: O = 2^e_bh O^T / l, LSE = m + ln l
    const float l_tot = pair_sum(l_run);
    float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if constexpr (DROP) inv *= a.drop.keep_scale;
    const int vx = a.vexp ? a.vexp[bkv] : 0;
    if (qrow < N) {
        const size_t orow = hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = db * 32 + 8 * g + 4 * hl;
                float w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = ldexpf(oacc[db][4 * g + e] * inv, vx);
                if (a.o_f32) store4<float>((float*)a.o + orow + dcol, w[0], w[1], w[2], w[3]);
                else store4<T>((T*)a.o + orow + dcol, w[0], w[1], w[2], w[3]);
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
    const bool drop = a.drop.on != 0;
    if (d == 64) return drop ? launch_t<T, 64, true>(a, s) : launch_t<T, 64, false>(a, s);
    return drop ? launch_t<T, 128, true>(a, s) : launch_t<T, 128, false>(a, s);
}
}  // namespace

hipError_t launch_fwd(FwdArgs a, fa_dtype dt, int d, void* workspace, hipStream_t s) {
    a.vexp = nullptr;
    if (dt == FA_BF16) {
        const FwdWorkspace L = fwd_workspace_layout(a.B, a.Hkv, a.N, d);   // the K/V heads' V
        char* ws = static_cast<char*>(workspace);
        V16Args p;
        p.v = a.v;
        p.v16 = reinterpret_cast<f16*>(ws + L.v16);
        p.part = reinterpret_cast<uint32_t*>(ws + L.part);
        p.vexp = reinterpret_cast<int32_t*>(ws + L.vexp);
        p.per_head = (size_t)a.N * d;
        p.nch = L.nch;
        p.chunk = L.chunk;
        void* args[] = {(void*)&p};
        const dim3 grid((unsigned)((size_t)a.B * a.Hkv * L.nch));
        hipError_t e = hipLaunchKernel((const void*)&v16_convert_kernel, grid, dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
        e = hipLaunchKernel((const void*)&v16_rescale_kernel, grid, dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
        a.v = p.v16;
        a.vexp = p.vexp;
    }
    switch (dt) {
        case FA_BF16: return launch_d<bf16>(a, d, s);
        case FA_F16: return launch_d<f16>(a, d, s);
        default: return launch_d<float>(a, d, s);
    }
}

}  // namespace fa
