// Dropout keep-mask export: the keep bit of every (b, h, i, j), produced by
// the same device generator (keep8) the attention kernels call, so tests can
// compare the GPU's dropout pattern bit for bit with the oracle's.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

// one thread per generator call: key group g (keys 4g .. 4g+3) x row pair m
// (rows 2m, 2m+1) of one (b, h)
__global__ __launch_bounds__(256) void keep_mask_kernel(uint32_t k0, uint32_t k1, uint32_t off,
                                                        uint32_t thr, int BH, int N, uint8_t* keep) {
    const size_t gpr = (size_t)(N + 3) / 4;          // key groups per row pair
    const size_t pairs = (size_t)(N + 1) / 2;        // row pairs per (b, h)
    const size_t total = (size_t)BH * pairs * gpr;
    for (size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += (size_t)gridDim.x * blockDim.x) {
        const size_t g = gid % gpr;
        const size_t pm = gid / gpr;                  // bh * pairs + m
        const uint32_t m = (uint32_t)(pm % pairs);
        const uint32_t bh = (uint32_t)(pm / pairs);
        const uint32_t bits = keep8<true>((uint32_t)g, m, bh, off, k0, k1, thr);
        for (int s = 0; s < 2; ++s) {
            const size_t i = 2 * (size_t)m + s;
            if (i >= (size_t)N) break;
            uint8_t* dst = keep + ((size_t)bh * N + i) * N + 4 * g;
            for (int e = 0; e < 4; ++e)
                if (4 * g + e < (size_t)N) dst[e] = (uint8_t)((bits >> (4 * s + e)) & 1u);
        }
    }
}

hipError_t launch_keep_mask(uint32_t k0, uint32_t k1, uint32_t off, uint32_t thr, int B, int H, int N,
                            uint8_t* keep, hipStream_t s) {
    const size_t total = (size_t)B * H * ((N + 1) / 2) * ((N + 3) / 4);
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    int BH = B * H;
    void* args[] = {&k0, &k1, &off, &thr, &BH, &N, &keep};
    return hipLaunchKernel((const void*)&keep_mask_kernel, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

}  // namespace fa
