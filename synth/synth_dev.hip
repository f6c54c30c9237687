// synth_dev.hip — device twin of synth.c's matrix generator (Philox4x32-10 +
// Irwin-Hall n=8 normal deviates + seeded single-element row outliers).
// Input generation only: it fills f32 weight matrices in HBM so that the
// 16-layer workloads (tens of GB) need no host generation or upload. Every
// element it writes must equal synth_fill_matrix() on the host bit for bit;
// the integer Irwin-Hall sum and one f32 multiply make that exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t out[4])
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1; c3 = (uint32_t)p0; c0 = n0; c2 = n2;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

__global__ void fill_values(uint32_t seed, uint32_t stream, uint64_t base, uint64_t count, float c,
                            float *__restrict__ out)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint64_t n = base + i;
        uint32_t w[4];
        philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u, seed, stream, w);
        int32_t z = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z += 2 * (int32_t)(w[k] & 0xFFFFu) - 65535;
            z += 2 * (int32_t)(w[k] >> 16) - 65535;
        }
        out[i] = __fmul_rn((float)z, c);
    }
}

__global__ void apply_outliers(uint32_t seed, uint32_t stream, int64_t row0, int64_t nrows, int64_t cols,
                               uint32_t thr, float mult, float *__restrict__ out)
{
    const int64_t rr = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (rr >= nrows) return;
    const int64_t r = row0 + rr;
    uint32_t w[4];
    philox4x32_10((uint32_t)r, (uint32_t)((uint64_t)r >> 32), 1u, 0u, seed, stream, w);
    if (w[0] >= thr) return;
    const int64_t col = (int64_t)(((uint64_t)w[1] * (uint64_t)cols) >> 32);
    float *p = out + rr * cols + col;
    *p = __fmul_rn(*p, mult);
}

} // namespace

// Fills out[nrows*cols] (device memory) with rows row0..row0+nrows-1 of the
// stream. c is synth_normal_scale(sigma) and thr is floor(rate * 2^32)
// (0 disables outliers), both computed on the host. Returns 0 or a HIP error.
extern "C" int synth_dev_fill_matrix(uint32_t seed, uint32_t stream, int64_t row0, int64_t nrows,
                                     int64_t cols, float c, uint32_t thr, float mult, float *out,
                                     void *hip_stream)
{
    if (nrows <= 0 || cols <= 0 || out == nullptr) return nrows == 0 ? 0 : -1;
    hipStream_t s = (hipStream_t)hip_stream;
    const uint64_t count = (uint64_t)nrows * (uint64_t)cols;
    const uint64_t base = (uint64_t)row0 * (uint64_t)cols;
    uint64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_values, dim3((unsigned)blocks), dim3(256), 0, s, seed, stream, base, count, c, out);
    if (thr > 0) {
        const unsigned ob = (unsigned)((nrows + 255) / 256);
        hipLaunchKernelGGL(apply_outliers, dim3(ob), dim3(256), 0, s, seed, stream, row0, nrows, cols, thr, mult, out);
    }
    return (int)hipGetLastError();
}
