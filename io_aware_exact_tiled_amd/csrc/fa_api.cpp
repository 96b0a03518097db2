// C-ABI layer: host-side validation, dispatch and status reporting.
// Declarations and the contract of each entry point are in include/fa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstddef>
#include <cstring>

#include "../../include/fa.h"
#include "fa_internal.hpp"

namespace {

thread_local char g_hip_error[256] = "";

fa_status hip_fail(hipError_t e) {
    std::strncpy(g_hip_error, hipGetErrorString(e), sizeof(g_hip_error) - 1);
    g_hip_error[sizeof(g_hip_error) - 1] = 0;
    return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int dt) { return dt == FA_F32 || dt == FA_F16 || dt == FA_BF16; }

fa_status check_shape(int32_t B, int32_t H, int32_t N, int32_t d) {
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (B < 1 || H < 1 || N < 1 || B > 65535 || H > 65535) return FA_ERR_SHAPE;
    const int64_t per_head = (int64_t)N * d;
    if (per_head >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    if ((int64_t)B * H * N >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status check_common(int32_t B, int32_t H, int32_t N, int32_t d, fa_dtype dtype, float scale,
                       float dropout_p, const fa_opts* opts) {
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
    if (!std::isfinite(dropout_p) || dropout_p < 0.0f || dropout_p >= 1.0f) return FA_ERR_DROPOUT;
    if (!std::isfinite(scale) || scale <= 0.0f) return FA_ERR_SCALE;
    if (opts) {
        // the current layout, or the one before kv_heads was appended
        if (opts->struct_size != sizeof(fa_opts) && opts->struct_size != offsetof(fa_opts, kv_heads))
            return FA_ERR_OPTS;
        if (opts->flags & ~(uint32_t)(FA_FLAG_RECORD_TILES | FA_FLAG_REVERSE_KV)) return FA_ERR_OPTS;
        if ((opts->flags & FA_FLAG_RECORD_TILES) && !opts->tile_visits) return FA_ERR_NULL;
    }
    return FA_OK;
}

// K/V heads: opts->kv_heads when the caller's struct has the field and sets
// it, else H.  Returns 0 when it does not divide H.
int32_t kv_heads(int32_t H, const fa_opts* opts) {
    if (!opts || opts->struct_size < offsetof(fa_opts, kv_heads) + sizeof(int32_t) || opts->kv_heads == 0) return H;
    const int32_t k = opts->kv_heads;
    return (k >= 1 && k <= H && H % k == 0) ? k : 0;
}

// threshold on an element's 16-bit uniform: drop iff u < thr
uint32_t drop_threshold(float p) {
    const double t = std::floor((double)p * 65536.0);
    return t >= 65535.0 ? 0xFFFFu : (uint32_t)t;
}

fa::MaskArgs mask_args(int32_t N, int32_t causal, const uint8_t* block_mask, const fa_opts* opts) {
    fa::MaskArgs m;
    m.causal = causal ? 1 : 0;
    m.key_lens = opts ? opts->key_lens : nullptr;
    m.block_mask = block_mask;
    m.mask_T = (N + fa::MASK_TILE - 1) / fa::MASK_TILE;
    return m;
}

fa::DropArgs drop_args(float p, uint64_t seed, const fa_opts* opts) {
    fa::DropArgs d;
    d.on = p > 0.0f ? 1u : 0u;
    d.thr = drop_threshold(p);
    // kept entries are scaled by the inverse of the exact keep probability
    // (2^16 - thr) / 2^16, so the dropped product is unbiased
    d.keep_scale = d.on ? (float)(65536.0 / (65536.0 - (double)d.thr)) : 1.0f;
    d.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
    d.k1 = (uint32_t)(seed >> 32);
    d.off = opts ? (uint32_t)(opts->rng_offset & 0xFFFFFFFFu) : 0u;
    return d;
}

constexpr float LOG2E = 1.4426950408889634f;


}  // namespace

namespace fa {

fa_status set_hip_error(hipError_t e) { return hip_fail(e); }

// Everything fa_bwd checks except the workspace, and the argument block it
// launches with (delta left for the caller to point at D's storage).
fa_status bwd_prepare(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, int32_t B, int32_t H, int32_t N, int32_t d,
                      fa_dtype dtype, float scale, int32_t causal, float dropout_p, uint64_t seed,
                      const uint8_t* block_mask, const fa_opts* opts, BwdArgs* out) {
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULL;
    fa_status st = check_common(B, H, N, d, dtype, scale, dropout_p, opts);
    if (st != FA_OK) return st;
    if (opts && (opts->flags & FA_FLAG_REVERSE_KV)) return FA_ERR_OPTS;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
        !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
        return FA_ERR_ALIGN;
    const int32_t hkv = kv_heads(H, opts);
    if (!hkv) return FA_ERR_OPTS;
    BwdArgs& a = *out;
    a.q = Q; a.k = K; a.v = V; a.o = O; a.dout = dO; a.lse = LSE;
    a.dq = dQ; a.dk = dK; a.dv = dV;
    a.delta = nullptr;
    a.B = B; a.H = H; a.N = N; a.Hkv = hkv;
    a.scale = scale;
    a.scale_log2 = scale * LOG2E;
    a.o_f32 = (opts && opts->o_fp32) ? 1 : 0;
    a.mask = mask_args(N, causal, block_mask, opts);
    a.drop = drop_args(dropout_p, seed, opts);
    const bool rec = opts && (opts->flags & FA_FLAG_RECORD_TILES);
    a.tile_visits = rec ? opts->tile_visits : nullptr;
    a.tile_visits2 = rec ? opts->tile_visits2 : nullptr;
    a.ev_begin = (opts && opts->main_end) ? opts->main_begin : nullptr;
    a.ev_end = (opts && opts->main_begin) ? opts->main_end : nullptr;
    a.ev_mid = (a.ev_begin && a.ev_end) ? opts->main_mid : nullptr;
    return FA_OK;
}

}  // namespace fa

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(fa_status s) {
    switch (s) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1 and the tensor within limits)";
        case FA_ERR_HEAD_DIM: return "head dim must be 64 or 128";
        case FA_ERR_DTYPE: return "unsupported dtype";
        case FA_ERR_DROPOUT: return "dropout probability must be finite and in [0, 1)";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_ALIGN: return "tensor base address is not 16-byte aligned";
        case FA_ERR_WORKSPACE: return "workspace is NULL, too small or not 256-byte aligned";
        case FA_ERR_HIP: return "HIP launch failed";
        case FA_ERR_OPTS: return "invalid fa_opts (struct_size or flags)";
        case FA_ERR_SCRATCH: return "problem too large for the static scratch of fa_bwd_noalloc";
    }
    return "unknown status";
}

const char* fa_last_hip_error(void) { return g_hip_error; }

fa_status fa_tile_shape(int32_t d, fa_dtype dtype, int32_t pass, int32_t N, int32_t causal, int32_t* Br,
                        int32_t* Bc) {
    if (!Br || !Bc) return FA_ERR_NULL;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
    if (N < 1) return FA_ERR_SHAPE;
    if (pass == 0) { *Br = fa::FWD_BR; *Bc = fa::FWD_BC; return FA_OK; }
    if (pass == 1) {
        if (fa::bwd_kv_small(dtype, d, N, causal)) {
            *Br = fa::BWD_KV_SMALL_BR;
            *Bc = fa::BWD_KV_SMALL_BC;
        } else {
            *Br = dtype == FA_F32 ? fa::BWD_KV_BR32 : fa::BWD_KV_BR16;
            *Bc = fa::BWD_KV_BC;
        }
        return FA_OK;
    }
    if (pass == 2) { *Br = fa::BWD_DQ_BR; *Bc = fa::BWD_DQ_BC; return FA_OK; }
    return FA_ERR_OPTS;
}

size_t fa_fwd_workspace_bytes(int32_t B, int32_t Hkv, int32_t N, int32_t d, fa_dtype dtype) {
    if (check_shape(B, Hkv, N, d) != FA_OK || !valid_dtype(dtype)) return 0;
    return dtype == FA_BF16 ? fa::fwd_workspace_layout(B, Hkv, N, d).bytes : 0;
}

fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int32_t B, int32_t H,
                 int32_t N, int32_t d, fa_dtype dtype, float scale, int32_t causal, float dropout_p,
                 uint64_t seed, const uint8_t* block_mask, const fa_opts* opts, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
    fa_status st = check_common(B, H, N, d, dtype, scale, dropout_p, opts);
    if (st != FA_OK) return st;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
        return FA_ERR_ALIGN;
    const int32_t hkv = kv_heads(H, opts);
    if (!hkv) return FA_ERR_OPTS;
    // the bf16 V copy covers the K/V heads only
    const size_t need = fa_fwd_workspace_bytes(B, hkv, N, d, dtype);
    if (need && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return FA_ERR_WORKSPACE;
    fa::FwdArgs a;
    a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
    a.B = B; a.H = H; a.N = N; a.Hkv = hkv;
    a.scale_log2 = scale * LOG2E;
    a.o_f32 = (opts && opts->o_fp32) ? 1 : 0;
    a.mask = mask_args(N, causal, block_mask, opts);
    a.drop = drop_args(dropout_p, seed, opts);
    a.tile_visits = (opts && (opts->flags & FA_FLAG_RECORD_TILES)) ? opts->tile_visits : nullptr;
    a.reverse_kv = (opts && (opts->flags & FA_FLAG_REVERSE_KV)) ? 1 : 0;
    a.ev_begin = (opts && opts->main_end) ? opts->main_begin : nullptr;
    a.ev_end = (opts && opts->main_begin) ? opts->main_end : nullptr;
    const hipError_t e = fa::launch_fwd(a, dtype, d, workspace, stream);
    return e == hipSuccess ? FA_OK : hip_fail(e);
}

namespace {
fa_status check_decode(int32_t B, int32_t H, int32_t Hkv, int32_t Nq, int32_t Nk, int32_t d) {
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || B > 65535 || H > 65535 || H % Hkv) return FA_ERR_SHAPE;
    if ((int64_t)Nk * d >= (int64_t(1) << 31) || (int64_t)B * H * Nq >= (int64_t(1) << 31) ||
        (int64_t)B * Hkv * Nk >= (int64_t(1) << 31) || (int64_t)(H / Hkv) * Nq > 65535)
        return FA_ERR_SHAPE;
    return FA_OK;
}
}  // namespace

size_t fa_decode_workspace_bytes(int32_t B, int32_t H, int32_t Hkv, int32_t Nq, int32_t Nk, int32_t d) {
    if (check_decode(B, H, Hkv, Nq, Nk, d) != FA_OK) return 0;
    return fa::decode_workspace_bytes(B, H, Hkv, Nq, Nk, d);
}

fa_status fa_decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int32_t B, int32_t H,
                    int32_t Hkv, int32_t Nq, int32_t Nk, int32_t d, fa_dtype dtype, float scale, int32_t causal,
                    const int32_t* kv_lens, const hipEvent_t* events, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
    fa_status st = check_decode(B, H, Hkv, Nq, Nk, d);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
    if (!std::isfinite(scale) || scale <= 0.0f) return FA_ERR_SCALE;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_ALIGN;
    const size_t need = fa::decode_workspace_bytes(B, H, Hkv, Nq, Nk, d);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return FA_ERR_WORKSPACE;
    const fa::DecodeSplit sp = fa::decode_split(B, H, Hkv, Nq, Nk);
    fa::DecodeArgs a;
    a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
    const size_t rows = (size_t)B * H * Nq;
    a.opart = static_cast<float*>(workspace);
    a.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa::align256(rows * sp.S * d * 4));
    a.kv_lens = kv_lens;
    a.B = B; a.H = H; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk;
    a.S = sp.S; a.C = sp.C; a.QBn = sp.QBn;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = scale * LOG2E;
    const hipError_t e = fa::launch_decode(a, dtype, d, events, stream);
    return e == hipSuccess ? FA_OK : hip_fail(e);
}

size_t fa_fwd_kv_outer_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d) {
    if (check_shape(B, H, N, d) != FA_OK) return 0;
    const size_t rows = (size_t)B * H * N;
    return fa::align256(rows * d * sizeof(float)) + fa::align256(rows * 2 * sizeof(float));
}

fa_status fa_fwd_kv_outer(const void* Q, const void* K, const void* V, void* O, float* LSE, int32_t B, int32_t H,
                          int32_t N, int32_t d, fa_dtype dtype, float scale, int32_t causal, int32_t block_cols,
                          int32_t groups_per_head, const hipEvent_t* events, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
    if (!std::isfinite(scale) || scale <= 0.0f) return FA_ERR_SCALE;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_ALIGN;
    if (block_cols != 64 && block_cols != 128) return FA_ERR_OPTS;
    const int Tr = (N + 127) / 128;
    int G = groups_per_head;
    if (G == 0) G = std::max(1, std::min(Tr, (1024 + B * H - 1) / (B * H)));
    if (G < 1 || G > Tr || (int64_t)B * H * G >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    const size_t rows = (size_t)B * H * N;
    const size_t need = fa::align256(rows * d * sizeof(float)) + fa::align256(rows * 2 * sizeof(float));
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return FA_ERR_WORKSPACE;
    fa::KvoArgs a;
    a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
    a.ow = static_cast<float*>(workspace);
    a.ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa::align256(rows * d * sizeof(float)));
    a.B = B; a.H = H; a.N = N; a.G = G;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = scale * LOG2E;
    const hipError_t e = fa::launch_kv_outer(a, dtype, d, block_cols, events, stream);
    return e == hipSuccess ? FA_OK : hip_fail(e);
}

size_t fa_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d) {
    if (check_shape(B, H, N, d) != FA_OK) return 0;
    const size_t rows = (size_t)B * H * N;
    return fa::align256(rows * sizeof(float));
}

fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                 void* dQ, void* dK, void* dV, int32_t B, int32_t H, int32_t N, int32_t d, fa_dtype dtype,
                 float scale, int32_t causal, float dropout_p, uint64_t seed, const uint8_t* block_mask,
                 const fa_opts* opts, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    fa::BwdArgs a;
    fa_status st = fa::bwd_prepare(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, N, d, dtype, scale, causal, dropout_p,
                                   seed, block_mask, opts, &a);
    if (st != FA_OK) return st;
    const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return FA_ERR_WORKSPACE;
    a.delta = static_cast<float*>(workspace);
    const hipError_t e = fa::launch_bwd(a, dtype, d, stream);
    return e == hipSuccess ? FA_OK : hip_fail(e);
}

fa_status fa_dropout_keep_mask(uint64_t seed, uint64_t rng_offset, float dropout_p, int32_t B, int32_t H,
                               int32_t N, uint8_t* keep, hipStream_t stream) {
    if (!keep) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if ((int64_t)B * H * N >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    if (!std::isfinite(dropout_p) || dropout_p < 0.0f || dropout_p >= 1.0f) return FA_ERR_DROPOUT;
    const hipError_t e = fa::launch_keep_mask((uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32),
                                              (uint32_t)(rng_offset & 0xFFFFFFFFu), drop_threshold(dropout_p),
                                              B, H, N, keep, stream);
    return e == hipSuccess ? FA_OK : hip_fail(e);
}

}  // extern "C"
