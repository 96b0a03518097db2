// Host-side view of the kernels: argument blocks and launchers shared by the
// C-ABI layer (fa_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace fa {

// Tile shapes (query rows x keys).  Forward: a workgroup owns FWD_BR query
// rows (4 waves x 32) and walks key tiles of FWD_BC.  Backward dK/dV kernel: a
// workgroup owns BWD_KV_BC keys (8 waves: 4 key blocks of 32 x 2 roles) and
// walks query tiles of BwdTiles<T>::KV_BR rows -- or, for 16-bit inputs at
// d = 64 and for short causal sequences (bwd_kv_small), 4 waves owning 64
// keys that walk 32-row query tiles.  Backward dQ kernel: a workgroup owns
// BWD_DQ_BR query rows and walks key tiles of BWD_DQ_BC.  All divide the
// 128-token block-mask tile.
constexpr int MASK_TILE = 128;   // block-mask granularity (tokens)
constexpr int FWD_BR = 128;
constexpr int FWD_BC = 64;
constexpr int BWD_KV_BC = 128;
constexpr int BWD_KV_SMALL_N = 2048;      // d = 128 causal N at or below this: 64-key dK/dV workgroups
constexpr int BWD_KV_BR16 = 64;  // 16-bit inputs
constexpr int BWD_KV_BR32 = 32;  // fp32 inputs (LDS budget of the double buffer)
constexpr int BWD_DQ_BR = 128;
constexpr int BWD_DQ_BC = 64;   // staged per step; the math walks 32-key blocks
// How many MFMA steps ahead the LDS operands of the S (and dP) products are
// read.  Deeper read-ahead hides more LDS latency but costs registers: at
// d = 64 one step keeps the forward at 4 waves per SIMD and two keep the dQ
// kernel at 4 (measured faster there than deeper read-ahead at 3 waves).
template <int D> constexpr int FWD_PF = D == 64 ? 1 : 3;
template <int D> constexpr int BWD_PF = D == 64 ? 2 : 3;
template <class T> struct BwdTiles {
    static constexpr int KV_BR = sizeof(T) == 4 ? BWD_KV_BR32 : BWD_KV_BR16;
};
constexpr int BWD_KV_SMALL_BC = 64;   // keys per workgroup of the four-wave dK/dV configuration
constexpr int BWD_KV_SMALL_BR = 32;   // its query rows per step

// The dK/dV configuration fa_bwd launches: the four-wave one for 16-bit
// inputs at d = 64 and for causal d = 128 sequences up to BWD_KV_SMALL_N
// (where a lone 8-wave workgroup per CU leaves its prologue and epilogue
// exposed), else the eight-wave one.
inline bool bwd_kv_small(fa_dtype dt, int d, int N, int causal) {
    return dt != FA_F32 && (d == 64 || (causal && N <= BWD_KV_SMALL_N));
}

struct MaskArgs {
    int causal;
    const int32_t* key_lens;    // device [B] or null
    const uint8_t* block_mask;  // device [T][T] or null
    int mask_T;                 // ceil(N / 128)
};

struct DropArgs {
    uint32_t on;          // 1 iff p > 0 (kept entries scaled, mask applied)
    uint32_t thr;         // drop iff the element's 16-bit uniform u < thr
    float keep_scale;     // 2^16 / (2^16 - thr): the inverse of the keep probability
    uint32_t k0, k1;      // Philox key (seed low, high)
    uint32_t off;         // Philox counter word 3
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N;
    int Hkv;              // K/V heads; query head h reads K/V head h / (H / Hkv)
    float scale_log2;     // scale * log2(e)
    int o_f32;            // O stored as fp32 instead of the input dtype
    MaskArgs mask;
    DropArgs drop;
    uint8_t* tile_visits; // null unless recording
    int reverse_kv;
    hipEvent_t ev_begin, ev_end;   // optional profiling events around the kernel
    const int32_t* vexp;  // bf16: per-(b, h) exponent e, V operand = V * 2^-e in fp16
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Forward workspace (bf16 inputs only): V * 2^-e_bh as fp16 [B][H][N][d],
// then the per-chunk maxima of |V| and the exponents e_bh.  Each (b, h) is
// cut into nch chunks of `chunk` elements (a multiple of one 256-thread x
// 8-element pass) for the pre-pass kernels.
constexpr int V16_MAX_CHUNKS = 64;
struct FwdWorkspace {
    size_t v16, part, vexp, bytes;   // byte offsets, total
    int nch;
    size_t chunk;
};
inline FwdWorkspace fwd_workspace_layout(int B, int H, int N, int d) {
    FwdWorkspace w;
    const size_t bh = (size_t)B * H, per_head = (size_t)N * d;
    constexpr size_t GRAIN = 256 * 8;
    const size_t passes = (per_head + GRAIN - 1) / GRAIN;
    const size_t want = passes < (size_t)V16_MAX_CHUNKS ? passes : (size_t)V16_MAX_CHUNKS;
    w.chunk = ((passes + want - 1) / want) * GRAIN;
    w.nch = (int)((per_head + w.chunk - 1) / w.chunk);
    w.v16 = 0;
    w.part = align256(bh * per_head * 2);
    w.vexp = w.part + align256(bh * (size_t)w.nch * 4);
    w.bytes = w.vexp + align256(bh * 4);
    return w;
}

struct V16Args {
    const void* v;        // bf16 [B][H][N][d]
    _Float16* v16;        // fp16 [B][H][N][d]
    uint32_t* part;       // [B*H][nch] largest finite |V| per chunk (bf16 magnitude bits)
    int32_t* vexp;        // [B*H]
    size_t per_head;      // N * d
    int nch;
    size_t chunk;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;         // fp32 [B][H][N] workspace: D = rowsum(dO o O)
    int B, H, N;
    int Hkv;              // K/V heads (K, V, dK, dV are [B][Hkv][N][d])
    float scale;
    float scale_log2;
    int o_f32;
    MaskArgs mask;
    DropArgs drop;
    uint8_t* tile_visits;          // dK/dV kernel's map (or null)
    uint8_t* tile_visits2;         // dQ kernel's map (or null)
    hipEvent_t ev_begin, ev_end;   // optional profiling events around the two main kernels
    hipEvent_t ev_mid;             // optional: between the two main kernels
};

// Forward in the key/value-outer order (IO ablation): see fa_kvouter.hip.
struct KvoArgs {
    const void* q;        // [B][H][N][d]
    const void* k;
    const void* v;
    void* o;              // [B][H][N][d], input dtype
    float* lse;           // [B][H][N]
    float* ow;            // workspace [B][H][N][d]: running O between key tiles
    float* ml;            // workspace [B][H][N][2]: running (m, l)
    int B, H, N, G;       // G workgroups per head, each taking every G-th query block
    int causal;
    float scale_log2;
};
// events: null or two events (before and after the kernel)
hipError_t launch_kv_outer(const KvoArgs& a, fa_dtype dt, int d, int bc, const hipEvent_t* ev, hipStream_t s);

// Decode (split key/value cache): see fa_decode.hip.
struct DecodeArgs {
    const void* q;        // [B][H][Nq][d]
    const void* k;        // [B][Hkv][Nk][d]
    const void* v;
    void* o;              // [B][H][Nq][d]
    float* lse;           // [B][H][Nq]
    float* opart;         // workspace [B*H*Nq][S][d]: per-split O
    float* lpart;         // workspace [B*H*Nq][S]: per-split log2-sum-exp
    const int32_t* kv_lens;   // device [B] valid cache rows, or null (= Nk)
    int B, H, Hkv, Nq, Nk;
    int S, C, QBn;        // splits, cache rows per split, 32-row query blocks per K/V head
    int causal;
    float scale_log2;
};
constexpr int DECODE_TARGET_WGS = 2048;   // workgroups the split count aims for
struct DecodeSplit { int S, C, QBn; };
inline DecodeSplit decode_split(int B, int H, int Hkv, int Nq, int Nk) {
    DecodeSplit p;
    p.QBn = ((H / Hkv) * Nq + 31) / 32;
    const long base = (long)B * Hkv * p.QBn;
    long want = (DECODE_TARGET_WGS + base - 1) / base;
    const long maxs = (Nk + 127) / 128;
    want = want < 1 ? 1 : (want > maxs ? maxs : want);
    p.C = (int)((((long)Nk + want - 1) / want + 127) / 128 * 128);
    p.S = (Nk + p.C - 1) / p.C;
    return p;
}
inline size_t decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
    const DecodeSplit p = decode_split(B, H, Hkv, Nq, Nk);
    const size_t rows = (size_t)B * H * Nq;
    return align256(rows * p.S * d * 4) + align256(rows * p.S * 4);
}
// events: null or three events (before the chunk kernel, between, after the merge)
hipError_t launch_decode(const DecodeArgs& a, fa_dtype dt, int d, const hipEvent_t* ev, hipStream_t s);

// Validation and argument block shared by fa_bwd and fa_bwd_noalloc (every
// check but the workspace's; a->delta is left null), and the thread-local
// error text behind FA_ERR_HIP (fa_api.cpp).
fa_status bwd_prepare(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, int32_t B, int32_t H, int32_t N, int32_t d,
                      fa_dtype dtype, float scale, int32_t causal, float dropout_p, uint64_t seed,
                      const uint8_t* block_mask, const fa_opts* opts, BwdArgs* a);
fa_status set_hip_error(hipError_t e);

hipError_t launch_fwd(FwdArgs a, fa_dtype dt, int d, void* workspace, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, fa_dtype dt, int d, hipStream_t s);
hipError_t launch_keep_mask(uint32_t k0, uint32_t k1, uint32_t off, uint32_t thr,
                            int B, int H, int N, uint8_t* keep, hipStream_t s);

}  // namespace fa
