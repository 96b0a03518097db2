// Dropout keep-mask export: the keep bit of every (b, h, i, j), produced by
// the same device generator (keep4) the attention kernels call, so tests can
// compare the GPU's dropout pattern bit for bit with the oracle's.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

__global__ __launch_bounds__(256) void keep_mask_kernel(uint32_t k0, uint32_t k1, uint32_t off,
                                                        uint32_t thr, int BH, int N, uint8_t* keep) {
    const size_t gpr = (size_t)(N + 3) / 4;          // 4-key groups per row
    const size_t total = (size_t)BH * N * gpr;
    for (size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += (size_t)gridDim.x * blockDim.x) {
        const size_t g = gid % gpr;
        const size_t row = gid / gpr;                 // bh * N + i
        const uint32_t i = (uint32_t)(row % N);
        const uint32_t bh = (uint32_t)(row / N);
        const uint32_t bits = keep4((uint32_t)g, i, bh, off, k0, k1, thr);
        uint8_t* dst = keep + row * N + 4 * g;
        for (int e = 0; e < 4; ++e)
            if (4 * g + e < (size_t)N) dst[e] = (uint8_t)((bits >> e) & 1u);
    }
}

hipError_t launch_keep_mask(uint32_t k0, uint32_t k1, uint32_t off, uint32_t thr, int B, int H, int N,
                            uint8_t* keep, hipStream_t s) {
    const size_t total = (size_t)B * H * N * ((N + 3) / 4);
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    int BH = B * H;
    void* args[] = {&k0, &k1, &off, &thr, &BH, &N, &keep};
    return hipLaunchKernel((const void*)&keep_mask_kernel, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

}  // namespace fa
