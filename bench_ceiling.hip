// MFMA ceiling probe for gfx950: how fast 32x32x16 MFMAs run when they are fed
// the way the attention kernels feed them, with the kernels' operand data.
//
// The attention forward issues, per 32x32x16 MFMA, about 1 KB of LDS reads (the
// K or V operand of a 32-row wave) and about five VALU instructions of the
// online softmax, one of them an exponential.  Each probe kernel here runs
// 8 waves per CU (one 512-thread workgroup, 96 KB of LDS so no second one fits)
// that issue a fixed number of MFMAs with four independent accumulators, in
// one of these mixes:
//   mfma            MFMA only, both operands in registers
//   mfma+lds        one 16-byte LDS read per lane (1 KB per wave) per MFMA,
//                   used as the A operand
//   mfma+lds+valu   the same, plus one v_exp_f32 and four v_fma_f32 per MFMA
// with operands that are either constants (no bit toggles between MFMAs) or
// N(0,1) values rounded to bf16 / fp16, as in the synthetic workloads.
// Under rocprofv3 --pmc (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES) it shows
// the shader clock each mix sustains and how busy the matrix cores are.
//
// Build and run (one GPU):
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         bench_ceiling.hip -o /tmp/bench_ceiling && /tmp/bench_ceiling
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

constexpr int LOOP = 4096;          // outer iterations; 8 MFMAs each
constexpr int WAVES = 8;
constexpr int LDS_VEC = 6144;       // 96 KB of 16-byte vectors
constexpr int GRID = 256;           // one workgroup per CU

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

enum Mix { MFMA = 0, MFMA_LDS = 1, MFMA_LDS_VALU = 2 };

// A 32-bit mix of i (a finaliser of the murmur3 family), then 16-bit
// floating-point words: approximately N(0,1) (sum of four uniforms, rescaled)
// rounded to bf16 or fp16, or the constant 1/16.
__device__ inline uint32_t mix32(uint32_t h) {
    h ^= h >> 16; h *= 0x85EBCA6Bu; h ^= h >> 13; h *= 0xC2B2AE35u; h ^= h >> 16;
    return h;
}
template <bool BF>
__device__ inline uint16_t word16(uint32_t i, bool gauss) {
    float x = 0.0625f;
    if (gauss) {
        const uint32_t h = mix32(i * 0x9E3779B9u + 0x7F4A7C15u);
        const float s = (float)(h & 0xFF) + (float)((h >> 8) & 0xFF) + (float)((h >> 16) & 0xFF) + (float)(h >> 24);
        x = (s - 510.0f) / 147.8f;   // four uniforms on [0, 255]: mean 510, sd 147.8
    }
    if (BF) {
        const __bf16 v = (__bf16)x;
        uint16_t u; __builtin_memcpy(&u, &v, 2); return u;
    }
    const _Float16 v = (_Float16)x;
    uint16_t u; __builtin_memcpy(&u, &v, 2); return u;
}
template <bool BF>
__device__ inline uint4 vec16(uint32_t i, bool gauss) {
    uint32_t w[4];
    for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)word16<BF>(8 * i + 2 * e, gauss) | ((uint32_t)word16<BF>(8 * i + 2 * e + 1, gauss) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool BF>
__device__ inline f16v mma(uint4 a, uint4 b, f16v c) {
    if constexpr (BF) {
        b8 x, y; __builtin_memcpy(&x, &a, 16); __builtin_memcpy(&y, &b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    } else {
        h8 x, y; __builtin_memcpy(&x, &a, 16); __builtin_memcpy(&y, &b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
    }
}

template <int MIX, bool GAUSS, bool BF>
__global__ __launch_bounds__(512, 1) void ceiling_kernel(float* out) {
    __shared__ uint4 buf[LDS_VEC];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < LDS_VEC; i += 512) buf[i] = vec16<BF>((uint32_t)i, GAUSS);
    // two register operand sets per lane, alternated between MFMAs
    const uint4 r0 = vec16<BF>((uint32_t)(LDS_VEC + 2 * tid), GAUSS);
    const uint4 r1 = vec16<BF>((uint32_t)(LDS_VEC + 2 * tid + 1), GAUSS);
    __syncthreads();
    f16v acc[4];
    for (int c = 0; c < 4; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    float x[10];
    for (int c = 0; c < 10; ++c) x[c] = 1e-3f * (float)(tid + c);
    for (int it = 0; it < LOOP; ++it) {
        // eight consecutive 1 KB blocks from a window that moves per iteration:
        // index < 64 * 15 + 64 + 7 * 64 = 1472 (of 6144); the per-read offsets
        // are immediates, so addressing costs one VALU op per eight reads
        const uint4* row = buf + lane + 64 * ((it + wave * 5) & 15);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            uint4 a = (u & 1) ? r1 : r0;
            if (MIX != MFMA) a = row[64 * u];
            acc[u & 3] = mma<BF>(a, (u & 2) ? r1 : r0, acc[u & 3]);
            if (MIX == MFMA_LDS_VALU) {
                float* y = x + (u & 1) * 5;
                y[0] = __builtin_amdgcn_exp2f(-y[0]);
#pragma unroll
                for (int c = 1; c < 5; ++c) y[c] = fmaf(y[c], 0.999f, 1e-4f);
            }
        }
    }
    float s = 0.0f;
    for (int c = 0; c < 4; ++c)
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    for (int c = 0; c < 10; ++c) s += x[c];
    out[blockIdx.x * 512 + tid] = s;
}

void check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        std::exit(1);
    }
}

template <int MIX, bool GAUSS, bool BF>
void run(const char* name, float* out) {
    const dim3 grid(GRID), block(512);
    hipLaunchKernelGGL((ceiling_kernel<MIX, GAUSS, BF>), grid, block, 0, 0, out);   // warm-up
    check(hipGetLastError(), "launch");
    hipEvent_t a, b;
    check(hipEventCreate(&a), "event");
    check(hipEventCreate(&b), "event");
    check(hipEventRecord(a, 0), "record");
    hipLaunchKernelGGL((ceiling_kernel<MIX, GAUSS, BF>), grid, block, 0, 0, out);
    check(hipGetLastError(), "launch");
    check(hipEventRecord(b, 0), "record");
    check(hipEventSynchronize(b), "sync");
    float ms = 0.0f;
    check(hipEventElapsedTime(&ms, a, b), "elapsed");
    const double flop = (double)GRID * WAVES * LOOP * 8 * 32768.0;
    const double tf = flop / (ms * 1e-3) / 1e12;
    std::printf("%-28s %8.3f ms %8.1f TFLOP/s %6.1f %% of 2500\n", name, ms, tf, 100.0 * tf / 2500.0);
    check(hipEventDestroy(a), "event");
    check(hipEventDestroy(b), "event");
}

}  // namespace

int main() {
    float* out = nullptr;
    check(hipMalloc(&out, sizeof(float) * GRID * 512), "malloc");
    run<MFMA, false, false>("fp16 const  mfma", out);
    run<MFMA, true, false>("fp16 N(0,1) mfma", out);
    run<MFMA, true, true>("bf16 N(0,1) mfma", out);
    run<MFMA_LDS, false, false>("fp16 const  mfma+lds", out);
    run<MFMA_LDS, true, false>("fp16 N(0,1) mfma+lds", out);
    run<MFMA_LDS, true, true>("bf16 N(0,1) mfma+lds", out);
    run<MFMA_LDS_VALU, false, false>("fp16 const  mfma+lds+valu", out);
    run<MFMA_LDS_VALU, true, false>("fp16 N(0,1) mfma+lds+valu", out);
    run<MFMA_LDS_VALU, true, true>("bf16 N(0,1) mfma+lds+valu", out);
    check(hipDeviceSynchronize(), "sync");
    check(hipFree(out), "free");
    return 0;
}
