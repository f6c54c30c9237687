// kernels_quant.hip — Q8_0-style activation quantisation, int4 row packing,
// RMSNorm, the block-dot test hook and small utility fills.
//
// Formats and rules follow the colibri architecture overview, section 3.1
// (int4 packed two per byte with one f32 scale per row; IDOT activations
// quantised to int8) and the ai4coding.ru summary "what is implemented"
// (Q8_0-style int8 activations, 32-wide blocks with absmax/127 scales).
#include "device_common.hpp"
#include "internal.hpp"

namespace coli {
namespace {

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16)
         | ((uint32_t)(d & 0xFF) << 24);
}

// One thread per 32-wide block: absmax, d = absmax/127, codes.
__global__ void __launch_bounds__(256) k_quant_q8(const float *__restrict__ x, long nblocks,
                                                  int8_t *__restrict__ xq, float *__restrict__ xs,
                                                  int reorder)
{
    const long b = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float4 *src = reinterpret_cast<const float4 *>(x + b * QK);
    float v[QK];
#pragma unroll
    for (int i = 0; i < QK / 4; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) amax = fmaxf(amax, fabsf(v[i]));
    float d, id;
    q8_scale(amax, d, id);
    int c[QK];
#pragma unroll
    for (int i = 0; i < QK; ++i) c[i] = round_clamp(__fmul_rn(v[i], id), -127.0f, 127.0f);
    uint32_t out[8];
    if (reorder) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            out[2 * m] = pack4(c[8 * m], c[8 * m + 2], c[8 * m + 4], c[8 * m + 6]);
            out[2 * m + 1] = pack4(c[8 * m + 1], c[8 * m + 3], c[8 * m + 5], c[8 * m + 7]);
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) out[m] = pack4(c[4 * m], c[4 * m + 1], c[4 * m + 2], c[4 * m + 3]);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(xq + b * QK);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    xs[b] = d;
}

// Natural-order int8 codes to the reordered layout, one thread per 8-group.
__global__ void k_reorder_q8(const int8_t *__restrict__ src, long ngroups, int8_t *__restrict__ dst)
{
    const long g = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= ngroups) return;
    const uint2 a = *reinterpret_cast<const uint2 *>(src + 8 * g);
    const uint32_t a0 = a.x, a1 = a.y;
    const uint32_t even = (a0 & 0xFFu) | (((a0 >> 16) & 0xFFu) << 8) | ((a1 & 0xFFu) << 16)
                        | (((a1 >> 16) & 0xFFu) << 24);
    const uint32_t odd = ((a0 >> 8) & 0xFFu) | (((a0 >> 24) & 0xFFu) << 8) | (((a1 >> 8) & 0xFFu) << 16)
                       | (((a1 >> 24) & 0xFFu) << 24);
    *reinterpret_cast<uint2 *>(dst + 8 * g) = make_uint2(even, odd);
}

// One workgroup per row: absmax/7 scale, nibble codes, two per byte.
__global__ void __launch_bounds__(256) k_pack_int4(const float *__restrict__ w, int cols,
                                                   uint8_t *__restrict__ q, float *__restrict__ sc)
{
    __shared__ float red[4];
    const long row = blockIdx.x;
    const float *src = w + row * (long)cols;
    float amax = 0.0f;
    for (int c = threadIdx.x; c < cols; c += blockDim.x) amax = fmaxf(amax, fabsf(src[c]));
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) amax = fmaxf(amax, red[i]);
    const float d = __fdiv_rn(amax, 7.0f);
    const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
    uint8_t *dst = q + row * (long)(cols / 2);
    for (int j = threadIdx.x; j < cols / 2; j += blockDim.x) {
        const int lo = round_clamp(__fmul_rn(src[2 * j], id), -8.0f, 7.0f);
        const int hi = round_clamp(__fmul_rn(src[2 * j + 1], id), -8.0f, 7.0f);
        dst[j] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
    }
    if (threadIdx.x == 0) sc[row] = d;
}

// Group scales: one workgroup per row, one thread per group of G columns,
// each group packed as k_pack_int4 packs a row.
__global__ void __launch_bounds__(256) k_pack_int4_groups(const float *__restrict__ w, int cols, int G,
                                                          uint8_t *__restrict__ q, float *__restrict__ sc)
{
    const long row = blockIdx.x;
    const int ng = cols / G;
    for (int g = threadIdx.x; g < ng; g += blockDim.x) {
        const float *src = w + row * (long)cols + (long)g * G;
        float amax = 0.0f;
        for (int c = 0; c < G; ++c) amax = fmaxf(amax, fabsf(src[c]));
        const float d = __fdiv_rn(amax, 7.0f);
        const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
        uint8_t *dst = q + row * (long)(cols / 2) + (long)g * (G / 2);
        for (int j = 0; j < G / 2; ++j) {
            const int lo = round_clamp(__fmul_rn(src[2 * j], id), -8.0f, 7.0f);
            const int hi = round_clamp(__fmul_rn(src[2 * j + 1], id), -8.0f, 7.0f);
            dst[j] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
        }
        sc[row * ng + g] = d;
    }
}

// int2 rows: d = absmax/1, codes clamp(rint(w/d), -2, 1); in every aligned
// group of 16 columns byte k holds columns 2k, 2k+1, 2k+8, 2k+9 in its 2-bit
// fields 0..3 (the order the kernels read activation blocks in). One thread
// per output byte.
__global__ void __launch_bounds__(256) k_pack_int2(const float *__restrict__ w, int cols,
                                                   uint8_t *__restrict__ q, float *__restrict__ sc)
{
    __shared__ float red[4];
    const long row = blockIdx.x;
    const float *src = w + row * (long)cols;
    float amax = 0.0f;
    for (int c = threadIdx.x; c < cols; c += blockDim.x) amax = fmaxf(amax, fabsf(src[c]));
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) amax = fmaxf(amax, red[i]);
    const float d = __fdiv_rn(amax, 1.0f);
    const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
    uint8_t *dst = q + row * (long)(cols / 4);
    for (int j = threadIdx.x; j < cols / 4; j += blockDim.x) {
        const int c0 = (j >> 2) * 16 + 2 * (j & 3);
        const int cs[4] = {c0, c0 + 1, c0 + 8, c0 + 9};
        int byte = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) byte |= (round_clamp(__fmul_rn(src[cs[i]], id), -2.0f, 1.0f) & 3) << (2 * i);
        dst[j] = (uint8_t)byte;
    }
    if (threadIdx.x == 0) sc[row] = d;
}

// int8 rows: d = absmax/127, codes clamp(rint(w/d), -127, 127); within each
// group of 8 columns column c goes to byte perm8(c) (0,2,4,6 then 1,3,5,7) of
// its block, and a row holds the first 16 bytes of every block, then the
// second 16 bytes of every block.
__global__ void __launch_bounds__(256) k_pack_int8(const float *__restrict__ w, int cols,
                                                   int8_t *__restrict__ q, float *__restrict__ sc)
{
    __shared__ float red[4];
    const long row = blockIdx.x;
    const float *src = w + row * (long)cols;
    float amax = 0.0f;
    for (int c = threadIdx.x; c < cols; c += blockDim.x) amax = fmaxf(amax, fabsf(src[c]));
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) amax = fmaxf(amax, red[i]);
    const float d = __fdiv_rn(amax, 127.0f);
    const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
    int8_t *dst = q + row * (long)cols;
    const int nblk = cols / 32;
    for (int c = threadIdx.x; c < cols; c += blockDim.x) {
        const int p = (c & 31 & ~7) + perm8(c & 7);          // byte of column c in its block
        dst[(p >> 4) * 16 * nblk + (c >> 5) * 16 + (p & 15)] =
            (int8_t)round_clamp(__fmul_rn(src[c], id), -127.0f, 127.0f);
    }
    if (threadIdx.x == 0) sc[row] = d;
}

// One workgroup of RMS_BLOCK threads per token: the row's scale as
// rms_scales takes it (so a router launch that normalises its own input
// agrees with this kernel bit for bit), then the scaled row.
__global__ void __launch_bounds__(RMS_BLOCK) k_rmsnorm(const float *__restrict__ x, const float *__restrict__ g,
                                                       int H, float eps, float *__restrict__ out, int vec)
{
    __shared__ double red[RMS_BLOCK / 64];
    const long t = blockIdx.x;
    const float *xt = x + t * (long)H;
    float *ot = out + t * (long)H;
    double sc[1];
    rms_scales<1>(xt, 1, H, eps, vec != 0, red, sc);   // ends with a barrier: x is read before out is written
    for (int i = threadIdx.x; i < H; i += RMS_BLOCK) ot[i] = rms_apply(xt[i], sc[0], g[i]);
}

// S[r][b] for one (row, block) per thread with the layer's block-dot function.
__global__ void k_block_dots(const uint8_t *__restrict__ q4, const int8_t *__restrict__ q8, int rows,
                             int cols, int32_t *__restrict__ S)
{
    const int nb = cols / QK;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)rows * nb) return;
    const long r = i / nb;
    const int b = (int)(i % nb);
    Blk8 a;
    const uint32_t *nat = reinterpret_cast<const uint32_t *>(q8 + (long)b * QK);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t a0 = nat[2 * m], a1 = nat[2 * m + 1];
        a.v[2 * m] = (int)((a0 & 0xFFu) | (((a0 >> 16) & 0xFFu) << 8) | ((a1 & 0xFFu) << 16)
                           | (((a1 >> 16) & 0xFFu) << 24));
        a.v[2 * m + 1] = (int)(((a0 >> 8) & 0xFFu) | (((a0 >> 24) & 0xFFu) << 8)
                               | (((a1 >> 8) & 0xFFu) << 16) | (((a1 >> 24) & 0xFFu) << 24));
    }
    int lo[4], hi[4];
    unpack_nibbles(load_u4(q4 + r * (long)(cols / 2) + (long)b * (QK / 2)), lo, hi);
    S[i] = dot_block16(lo, hi, a) / 16;
}

__global__ void k_zero(uint4 *__restrict__ p, size_t n16, uint8_t *__restrict__ tail, size_t ntail)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

__global__ void k_copy_f32(const float *__restrict__ a, float *__restrict__ b, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) b[i] = a[i];
}

inline unsigned grid_for(long n, int bs) { return (unsigned)((n + bs - 1) / bs); }

} // namespace

hipError_t launch_quant_q8(const float *x, int T, int H, int8_t *xq, float *xs, bool reorder, hipStream_t s)
{
    const long nb = (long)T * (H / QK);
    COLI_LAUNCH(k_quant_q8, dim3(grid_for(nb, 256)), dim3(256), 0, s, x, nb, xq, xs, reorder ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_reorder_q8(const int8_t *xq_nat, int n, int8_t *xq_perm, hipStream_t s)
{
    const long ng = n / 8;
    COLI_LAUNCH(k_reorder_q8, dim3(grid_for(ng, 256)), dim3(256), 0, s, xq_nat, ng, xq_perm);
    return hipGetLastError();
}

hipError_t launch_pack_int4(const float *w, int rows, int cols, uint8_t *q, float *sc, hipStream_t s)
{
    COLI_LAUNCH(k_pack_int4, dim3(rows), dim3(256), 0, s, w, cols, q, sc);
    return hipGetLastError();
}

hipError_t launch_pack_int4_groups(const float *w, int rows, int cols, int group, uint8_t *q, float *sc, hipStream_t s)
{
    COLI_LAUNCH(k_pack_int4_groups, dim3(rows), dim3(256), 0, s, w, cols, group, q, sc);
    return hipGetLastError();
}

hipError_t launch_pack_int2(const float *w, int rows, int cols, uint8_t *q, float *sc, hipStream_t s)
{
    COLI_LAUNCH(k_pack_int2, dim3(rows), dim3(256), 0, s, w, cols, q, sc);
    return hipGetLastError();
}

hipError_t launch_pack_int8(const float *w, int rows, int cols, int8_t *q, float *sc, hipStream_t s)
{
    COLI_LAUNCH(k_pack_int8, dim3(rows), dim3(256), 0, s, w, cols, q, sc);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *x, const float *g, int T, int H, float eps, float *out, hipStream_t s)
{
    COLI_LAUNCH(k_rmsnorm, dim3(T), dim3(RMS_BLOCK), 0, s, x, g, H, eps, out, rms_vec(x, H) ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_block_dots(const uint8_t *q4, const int8_t *q8, int rows, int cols, int32_t *S, hipStream_t s)
{
    const long n = (long)rows * (cols / QK);
    COLI_LAUNCH(k_block_dots, dim3(grid_for(n, 256)), dim3(256), 0, s, q4, q8, rows, cols, S);
    return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s)
{
    const size_t n16 = bytes / 16, ntail = bytes % 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks == 0) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    COLI_LAUNCH(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint4 *>(p), n16,
                       reinterpret_cast<uint8_t *>(p) + n16 * 16, ntail);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float *src, float *dst, size_t n, hipStream_t s)
{
    size_t blocks = (n + 255) / 256;
    if (blocks == 0) return hipSuccess;
    if (blocks > 4096) blocks = 4096;
    COLI_LAUNCH(k_copy_f32, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

} // namespace coli
