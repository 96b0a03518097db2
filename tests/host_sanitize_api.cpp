// Host-side checks of the C-ABI layer (csrc/fa_api.cpp) built with
// AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU: the kernel
// launchers are replaced by stubs that record the argument blocks the ABI layer
// derives (sizes, workspace carving, dropout threshold and scale, split
// counts) and check them against the buffers the caller passed.  Built and run
// by tests/test_host_sanitizers.py; exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fa.h"
#include "../io_aware_exact_tiled_amd/csrc/fa_internal.hpp"

#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
            return 1;                                                        \
        }                                                                    \
    } while (0)

namespace {
hipError_t g_status = hipSuccess;   // what the stub launchers return
int g_calls = 0;
fa::FwdArgs g_fwd;
fa::BwdArgs g_bwd;
fa::DecodeArgs g_dec;
fa::KvoArgs g_kvo;
const char* g_ws_base = nullptr;    // workspace passed to the last launch
size_t g_ws_bytes = 0;
}  // namespace

extern "C" const char* hipGetErrorString(hipError_t) { return "stubbed launch failure"; }

namespace fa {
hipError_t launch_fwd(FwdArgs a, fa_dtype, int, void* ws, hipStream_t) {
    ++g_calls; g_fwd = a; g_ws_base = static_cast<const char*>(ws);
    return g_status;
}
hipError_t launch_bwd(const BwdArgs& a, fa_dtype, int, hipStream_t) { ++g_calls; g_bwd = a; return g_status; }
hipError_t launch_decode(const DecodeArgs& a, fa_dtype, int, const hipEvent_t*, hipStream_t) {
    ++g_calls; g_dec = a; return g_status;
}
hipError_t launch_kv_outer(const KvoArgs& a, fa_dtype, int, int, const hipEvent_t*, hipStream_t) {
    ++g_calls; g_kvo = a; return g_status;
}
hipError_t launch_keep_mask(uint32_t, uint32_t, uint32_t, uint32_t, int, int, int, uint8_t*, hipStream_t) {
    ++g_calls; return g_status;
}
}  // namespace fa

static bool inside(const void* p, size_t bytes, const char* base, size_t total) {
    const char* c = static_cast<const char*>(p);
    return c >= base && c + bytes <= base + total;
}

int main() {
    // real host buffers stand in for device memory: the stubs never read them,
    // but every pointer the ABI layer derives must stay inside them
    std::vector<char> big(1 << 20);
    char* base = big.data() + (256 - (reinterpret_cast<uintptr_t>(big.data()) & 255)) % 256;
    void* P = base;
    float* F = reinterpret_cast<float*>(base);
    fa_opts o;
    std::memset(&o, 0, sizeof o);
    o.struct_size = sizeof(fa_opts);

    // ---- validation rejects before any launch
    const int before = g_calls;
    CHECK(fa_fwd(nullptr, P, P, P, F, 1, 2, 256, 64, FA_BF16, 0.125f, 0, 0.f, 0, nullptr, nullptr, P, 1 << 20,
                 nullptr) == FA_ERR_NULL);
    CHECK(fa_fwd(P, P, P, P, F, 1, 2, 256, 80, FA_BF16, 0.125f, 0, 0.f, 0, nullptr, nullptr, P, 1 << 20,
                 nullptr) == FA_ERR_HEAD_DIM);
    CHECK(fa_fwd(P, P, P, P, F, 1, 2, 256, 64, (fa_dtype)9, 0.125f, 0, 0.f, 0, nullptr, nullptr, P, 1 << 20,
                 nullptr) == FA_ERR_DTYPE);
    CHECK(fa_fwd(P, P, P, P, F, 1, 2, 256, 64, FA_F16, 0.125f, 0, NAN, 0, nullptr, nullptr, P, 0, nullptr) ==
          FA_ERR_DROPOUT);
    CHECK(fa_fwd(P, P, P, P, F, 1, 2, 256, 64, FA_F16, INFINITY, 0, 0.f, 0, nullptr, nullptr, P, 0, nullptr) ==
          FA_ERR_SCALE);
    CHECK(fa_fwd(P, P, P, P, F, 65536, 2, 256, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, nullptr, P, 0, nullptr) ==
          FA_ERR_SHAPE);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 1 << 25, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, nullptr, P, 0, nullptr) ==
          FA_ERR_SHAPE);   // N * d reaches 2^31
    CHECK(fa_fwd(P, P, static_cast<char*>(P) + 8, P, F, 1, 2, 256, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, nullptr,
                 P, 0, nullptr) == FA_ERR_ALIGN);
    o.struct_size = 3;
    CHECK(fa_fwd(P, P, P, P, F, 1, 2, 256, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, &o, P, 0, nullptr) == FA_ERR_OPTS);
    o.struct_size = sizeof(fa_opts);
    o.kv_heads = 3;   // does not divide H = 8
    CHECK(fa_fwd(P, P, P, P, F, 1, 8, 256, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, &o, P, 0, nullptr) == FA_ERR_OPTS);
    o.kv_heads = 0;
    o.flags = FA_FLAG_RECORD_TILES;   // without a map
    CHECK(fa_fwd(P, P, P, P, F, 1, 2, 256, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, &o, P, 0, nullptr) == FA_ERR_NULL);
    o.flags = FA_FLAG_REVERSE_KV;     // forward only
    CHECK(fa_bwd(P, P, P, P, P, F, P, P, P, 1, 2, 256, 64, FA_BF16, 1.f, 0, 0.f, 0, nullptr, &o, P, 1 << 20,
                 nullptr) == FA_ERR_OPTS);
    o.flags = 0;
    CHECK(fa_bwd(P, P, P, P, P, F, P, P, P, 1, 2, 256, 64, FA_BF16, 1.f, 0, 0.f, 0, nullptr, nullptr, P, 16,
                 nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_decode(P, P, P, P, F, 1, 4, 3, 1, 100, 64, FA_BF16, 1.f, 0, nullptr, nullptr, P, 1 << 20, nullptr) ==
          FA_ERR_SHAPE);
    CHECK(fa_fwd_kv_outer(P, P, P, P, F, 1, 2, 300, 64, FA_BF16, 1.f, 0, 32, 0, nullptr, P, 1 << 20, nullptr) ==
          FA_ERR_OPTS);
    CHECK(fa_dropout_keep_mask(1, 0, 1.0f, 1, 1, 16, static_cast<uint8_t*>(P), nullptr) == FA_ERR_DROPOUT);
    CHECK(g_calls == before);

    // ---- forward: derived arguments, bf16 workspace carved by K/V heads
    {
        const int B = 2, H = 8, Hkv = 2, N = 1000, d = 128;
        const size_t need = fa_fwd_workspace_bytes(B, Hkv, N, d, FA_BF16);
        CHECK(need >= (size_t)B * Hkv * N * d * 2 && need % 256 == 0);
        CHECK(fa_fwd_workspace_bytes(B, H, N, d, FA_BF16) >= need);
        std::vector<char> wsv(need + 256);
        char* ws = wsv.data() + (256 - (reinterpret_cast<uintptr_t>(wsv.data()) & 255)) % 256;
        o.kv_heads = Hkv;
        o.rng_offset = 0x100000007ull;
        CHECK(fa_fwd(P, P, P, P, F, B, H, N, d, FA_BF16, 0.125f, 1, 0.1f, 0x123456789abcdefull, nullptr, &o, ws,
                     need - 1, nullptr) == FA_ERR_WORKSPACE);
        CHECK(fa_fwd(P, P, P, P, F, B, H, N, d, FA_BF16, 0.125f, 1, 0.1f, 0x123456789abcdefull, nullptr, &o, ws,
                     need, nullptr) == FA_OK);
        CHECK(g_fwd.Hkv == Hkv && g_fwd.H == H && g_fwd.B == B && g_fwd.N == N);
        CHECK(g_fwd.drop.on == 1 && g_fwd.drop.thr == 6553u);
        CHECK(g_fwd.drop.keep_scale == (float)(65536.0 / 58983.0));
        CHECK(g_fwd.drop.k0 == 0x89abcdefu && g_fwd.drop.k1 == 0x01234567u && g_fwd.drop.off == 7u);
        CHECK(g_fwd.mask.causal == 1 && g_fwd.mask.mask_T == 8);
        // the launcher's workspace layout for these K/V heads fits what was passed
        const fa::FwdWorkspace L = fa::fwd_workspace_layout(B, Hkv, N, d);
        CHECK(L.bytes == need && g_ws_base == ws);
        CHECK(inside(ws + L.v16, (size_t)B * Hkv * N * d * 2, ws, need));
        CHECK(inside(ws + L.part, (size_t)B * Hkv * L.nch * 4, ws, need));
        CHECK(inside(ws + L.vexp, (size_t)B * Hkv * 4, ws, need));
        CHECK(L.nch >= 1 && L.nch <= fa::V16_MAX_CHUNKS && (size_t)L.nch * L.chunk >= (size_t)N * d);
        o.kv_heads = 0;
        o.rng_offset = 0;
        // p at the top of its range: the threshold saturates, the scale stays finite
        CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, FA_F16, 1.f, 0, 0.99999994f, 0, nullptr, nullptr, nullptr, 0,
                     nullptr) == FA_OK);
        CHECK(g_fwd.drop.thr == 65535u && g_fwd.drop.keep_scale == 65536.0f);
        CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, nullptr, nullptr, 0, nullptr) ==
              FA_OK);
        CHECK(g_fwd.drop.on == 0 && g_fwd.drop.keep_scale == 1.0f);
    }

    // ---- workspace sizes at the largest accepted shapes do not wrap
    {
        const size_t f = fa_fwd_workspace_bytes(1, 1, (1 << 24) - 1, 128, FA_BF16);
        CHECK(f >= (size_t)((1 << 24) - 1) * 128 * 2);
        const size_t b = fa_bwd_workspace_bytes(65535, 32767, 1, 64);
        CHECK(b >= (size_t)65535 * 32767 * 4);
        CHECK(fa_bwd_workspace_bytes(65535, 32769, 1, 64) == 0);   // B * H * N passes 2^31
        CHECK(fa_fwd_kv_outer_workspace_bytes(1, 1, (1 << 24) - 1, 128) >= (size_t)((1 << 24) - 1) * 128 * 4);
    }

    // ---- decode: the split covers the cache and the partials fit the workspace
    {
        const int shapes[][6] = {{1, 1, 1, 1, 1, 64},     {16, 32, 8, 1, 16384, 128}, {2, 8, 1, 4, 700, 64},
                                 {64, 32, 8, 1, 4096, 128}, {1, 4, 1, 3, 2600, 128}, {3, 8, 2, 16, 100000, 64},
                                 {1, 64, 1, 1023, 257, 128}};
        for (const auto& s : shapes) {
            const int B = s[0], H = s[1], Hkv = s[2], Nq = s[3], Nk = s[4], d = s[5];
            const size_t need = fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d);
            CHECK(need > 0 && need % 256 == 0);
            std::vector<char> wsv(need + 256);
            char* ws = wsv.data() + (256 - (reinterpret_cast<uintptr_t>(wsv.data()) & 255)) % 256;
            CHECK(fa_decode(P, P, P, P, F, B, H, Hkv, Nq, Nk, d, FA_BF16, 0.1f, 1, nullptr, nullptr, ws, need - 1,
                            nullptr) == FA_ERR_WORKSPACE);
            CHECK(fa_decode(P, P, P, P, F, B, H, Hkv, Nq, Nk, d, FA_BF16, 0.1f, 1, nullptr, nullptr, ws, need,
                            nullptr) == FA_OK);
            const size_t rows = (size_t)B * H * Nq;
            CHECK(g_dec.S >= 1 && g_dec.C % 128 == 0 && (long)g_dec.S * g_dec.C >= Nk &&
                  (long)(g_dec.S - 1) * g_dec.C < Nk);
            CHECK(inside(g_dec.opart, rows * g_dec.S * d * 4, ws, need));
            CHECK(inside(g_dec.lpart, rows * g_dec.S * 4, ws, need));
            CHECK(g_dec.QBn * 32 >= (H / Hkv) * Nq);
        }
    }

    // ---- K/V-outer forward: group count and workspace carving
    {
        const int B = 2, H = 3, N = 1000, d = 64;
        const size_t need = fa_fwd_kv_outer_workspace_bytes(B, H, N, d);
        std::vector<char> wsv(need + 256);
        char* ws = wsv.data() + (256 - (reinterpret_cast<uintptr_t>(wsv.data()) & 255)) % 256;
        CHECK(fa_fwd_kv_outer(P, P, P, P, F, B, H, N, d, FA_F16, 1.f, 1, 64, 9, nullptr, ws, need, nullptr) ==
              FA_ERR_SHAPE);   // more groups than 128-row query blocks
        CHECK(fa_fwd_kv_outer(P, P, P, P, F, B, H, N, d, FA_F16, 1.f, 1, 64, 0, nullptr, ws, need, nullptr) == FA_OK);
        CHECK(g_kvo.G >= 1 && g_kvo.G <= (N + 127) / 128);
        CHECK(inside(g_kvo.ow, (size_t)B * H * N * d * 4, ws, need));
        CHECK(inside(g_kvo.ml, (size_t)B * H * N * 2 * 4, ws, need));
    }

    // ---- backward: D sits at the start of the workspace; tile maps pass through
    {
        const size_t need = fa_bwd_workspace_bytes(2, 4, 300, 64);
        CHECK(need == 2 * 4 * 300 * 4 + 256 - (2 * 4 * 300 * 4) % 256);
        uint8_t maps[2];
        o.flags = FA_FLAG_RECORD_TILES;
        o.tile_visits = &maps[0];
        o.tile_visits2 = &maps[1];
        CHECK(fa_bwd(P, P, P, P, P, F, P, P, P, 2, 4, 300, 64, FA_F16, 0.125f, 1, 0.f, 0, nullptr, &o, P, need,
                     nullptr) == FA_OK);
        CHECK(g_bwd.delta == F && g_bwd.tile_visits == &maps[0] && g_bwd.tile_visits2 == &maps[1]);
        o.flags = 0;
        o.tile_visits = o.tile_visits2 = nullptr;
    }

    // ---- tile shapes name the launched dK/dV configuration
    {
        int32_t br = 0, bc = 0;
        CHECK(fa_tile_shape(64, FA_BF16, 1, 16384, 0, &br, &bc) == FA_OK && br == 32 && bc == 64);
        CHECK(fa_tile_shape(128, FA_BF16, 1, 2048, 1, &br, &bc) == FA_OK && br == 32 && bc == 64);
        CHECK(fa_tile_shape(128, FA_BF16, 1, 2049, 1, &br, &bc) == FA_OK && br == 64 && bc == 128);
        CHECK(fa_tile_shape(64, FA_F32, 1, 256, 0, &br, &bc) == FA_OK && br == 32 && bc == 128);
        CHECK(fa_tile_shape(64, FA_BF16, 1, 256, 0, nullptr, &bc) == FA_ERR_NULL);
    }

    // ---- a failed launch maps to FA_ERR_HIP with its text kept per thread
    g_status = hipErrorInvalidValue;
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, FA_F16, 1.f, 0, 0.f, 0, nullptr, nullptr, nullptr, 0, nullptr) ==
          FA_ERR_HIP);
    CHECK(std::strcmp(fa_last_hip_error(), "stubbed launch failure") == 0);
    g_status = hipSuccess;
    for (int s = 1; s >= -11; --s) CHECK(fa_status_string((fa_status)s) != nullptr);

    std::printf("host sanitize ok: %d launches\n", g_calls);
    return 0;
}
