// device_common.hpp — device helpers shared by every kernel of the layer.
//
// Data formats (colibri architecture overview, section 3.1):
//  * int4 rows: byte j holds element 2j in bits 0-3 and element 2j+1 in bits
//    4-7, 4-bit two's complement; one f32 scale per row.
//  * Q8 activations: 32-wide blocks, int8 codes plus one f32 scale per block.
//
// Nibble trick: for a packed dword w (elements 8m..8m+7),
//   (w << 4) & 0xF0F0F0F0  = the four even elements, each times 16, as int8;
//    w       & 0xF0F0F0F0  = the four odd elements, each times 16, as int8.
// So one 16-byte load of a row is one 32-wide block, and eight v_dot4 against
// activations stored with every 8-group reordered as (0,2,4,6,1,3,5,7) give
// 16 * S_b exactly (|16 S_b| <= 16*32*8*127 < 2^20). The factor 16 is folded
// into the block scale (an exact power-of-two multiply in f64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace coli {

// Position of element i (0..7) of an 8-group in the reordered activation layout.
__host__ __device__ constexpr int perm8(int i) { return (i & 1) ? 4 + (i >> 1) : (i >> 1); }

struct Blk8 { int v[8]; };      // one 32-wide activation block, reordered, 8 dwords

__device__ __forceinline__ void unpack_nibbles(const uint4 w, int (&lo)[4], int (&hi)[4])
{
    const uint32_t m = 0xF0F0F0F0u;
    lo[0] = (int)((w.x << 4) & m); hi[0] = (int)(w.x & m);
    lo[1] = (int)((w.y << 4) & m); hi[1] = (int)(w.y & m);
    lo[2] = (int)((w.z << 4) & m); hi[2] = (int)(w.z & m);
    lo[3] = (int)((w.w << 4) & m); hi[3] = (int)(w.w & m);
}

// 16 * S_b for one block: unpacked weight nibbles against one reordered block.
__device__ __forceinline__ int dot_block16(const int (&lo)[4], const int (&hi)[4], const Blk8 &a)
{
    int s = 0;
    s = __builtin_amdgcn_sdot4(lo[0], a.v[0], s, false);
    s = __builtin_amdgcn_sdot4(hi[0], a.v[1], s, false);
    s = __builtin_amdgcn_sdot4(lo[1], a.v[2], s, false);
    s = __builtin_amdgcn_sdot4(hi[1], a.v[3], s, false);
    s = __builtin_amdgcn_sdot4(lo[2], a.v[4], s, false);
    s = __builtin_amdgcn_sdot4(hi[2], a.v[5], s, false);
    s = __builtin_amdgcn_sdot4(lo[3], a.v[6], s, false);
    s = __builtin_amdgcn_sdot4(hi[3], a.v[7], s, false);
    return s;
}

// int8 weight block (32 codes in the activations' reordered byte order, as
// the int8 packer stores them) against a reordered activation block: 16·S_b
// is not needed here, the dot is S_b itself.
__device__ __forceinline__ int dot_block_i8(const uint4 w0, const uint4 w1, const Blk8 &a)
{
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)w0.x, a.v[0], s, false);
    s = __builtin_amdgcn_sdot4((int)w0.y, a.v[1], s, false);
    s = __builtin_amdgcn_sdot4((int)w0.z, a.v[2], s, false);
    s = __builtin_amdgcn_sdot4((int)w0.w, a.v[3], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.x, a.v[4], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.y, a.v[5], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.z, a.v[6], s, false);
    s = __builtin_amdgcn_sdot4((int)w1.w, a.v[7], s, false);
    return s;
}

// Weight formats of the token-GEMV path: bytes of one row's 32-wide block,
// the register pieces (16 bytes each; an int2 block fills half of one) and
// the factor that turns a block dot into S_b (int4 dots come out x16, int2
// dots x64).
template <int WB> struct WFmt;
template <> struct WFmt<2> { static constexpr int BLK_BYTES = 8, NP = 1; static constexpr double KSCALE = 1.0 / 64; };
template <> struct WFmt<4> { static constexpr int BLK_BYTES = 16, NP = 1; static constexpr double KSCALE = 0.0625; };
template <> struct WFmt<8> { static constexpr int BLK_BYTES = 32, NP = 2; static constexpr double KSCALE = 1.0; };

// int2 rows, in the order the activation blocks are read: in every aligned
// group of 16 columns, byte k holds columns 2k, 2k+1, 2k+8, 2k+9 in its 2-bit
// fields 0..3. Field i of the four bytes, moved to the top of each byte, is
// then the x64 code of the columns activation dword i of the group holds
// (8-groups stored as 0,2,4,6 then 1,3,5,7).
__device__ __forceinline__ int dot_block_i2(uint32_t w0, uint32_t w1, const Blk8 &a)
{
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)((w0 << 6) & 0xC0C0C0C0u), a.v[0], s, false);
    s = __builtin_amdgcn_sdot4((int)((w0 << 4) & 0xC0C0C0C0u), a.v[1], s, false);
    s = __builtin_amdgcn_sdot4((int)((w0 << 2) & 0xC0C0C0C0u), a.v[2], s, false);
    s = __builtin_amdgcn_sdot4((int)(w0 & 0xC0C0C0C0u), a.v[3], s, false);
    s = __builtin_amdgcn_sdot4((int)((w1 << 6) & 0xC0C0C0C0u), a.v[4], s, false);
    s = __builtin_amdgcn_sdot4((int)((w1 << 4) & 0xC0C0C0C0u), a.v[5], s, false);
    s = __builtin_amdgcn_sdot4((int)((w1 << 2) & 0xC0C0C0C0u), a.v[6], s, false);
    s = __builtin_amdgcn_sdot4((int)(w1 & 0xC0C0C0C0u), a.v[7], s, false);
    return s;
}

// Where a row's pieces sit: block b's piece q starts at blk_off(b) +
// piece_off(q). int8 rows keep the first 16 bytes of every block, then the
// second 16 bytes of every block (nblk blocks per row), so each piece's
// load by a wave's 64 lanes reads 1 KB contiguous; int4 and int2 blocks are
// one piece each.
template <int WB>
__device__ __forceinline__ long blk_off(int b)
{
    return WB == 8 ? 16L * b : (long)b * WFmt<WB>::BLK_BYTES;
}
template <int WB>
__device__ __forceinline__ long piece_off(int q, int nblk)
{
    return WB == 8 ? 16L * q * nblk : 16L * q;
}

// One block of one weight row times one activation block: S_b scaled by the
// format's factor applies later; w holds the block's NP pieces.
template <int WB>
__device__ __forceinline__ int dot_block_w(const uint4 (&w)[WFmt<WB>::NP], const Blk8 &a)
{
    if constexpr (WB == 8) {
        return dot_block_i8(w[0], w[1], a);
    } else if constexpr (WB == 2) {
        return dot_block_i2(w[0].x, w[0].y, a);
    } else {
        int lo[4], hi[4];
        unpack_nibbles(w[0], lo, hi);
        return dot_block16(lo, hi, a);
    }
}

__device__ __forceinline__ Blk8 load_blk8(const int8_t *p)
{
    const int4 a = *reinterpret_cast<const int4 *>(p);
    const int4 b = *reinterpret_cast<const int4 *>(p + 16);
    Blk8 r;
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    return r;
}

__device__ __forceinline__ uint4 load_u4(const uint8_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

// Streaming (use-once) 16-byte load: weights are read once per call.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_u4_stream(const uint8_t *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One register piece of a weight row block: 16 bytes, or the 8 bytes of an
// int2 block (the upper half unused).
template <int WB>
__device__ __forceinline__ uint4 load_w_stream(const uint8_t *p)
{
    if constexpr (WB == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        return make_uint4(v.x, v.y, 0u, 0u);
    } else {
        return load_u4_stream(p);
    }
}

// Device-coherent relaxed accesses for data one workgroup hands to another in
// the same launch: they reach the device coherence point without an L2-wide
// writeback or invalidate, so no agent-scope fence is needed around them.
__device__ __forceinline__ void st_dev(float *p, float v)
{
    __hip_atomic_store(reinterpret_cast<unsigned *>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(double *p, double v)
{
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), (unsigned long long)__double_as_longlong(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p)
{
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned *>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int ld_dev(const int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_dev(const double *p)
{
    return __longlong_as_double((long long)__hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Round half to even and clamp, the rule shared by both quantisers; a NaN
// product (0 * inf) gives 0.
__device__ __forceinline__ int round_clamp(float v, float lo, float hi)
{
    if (v != v) return 0;
    float r = __builtin_rintf(v);
    r = r < lo ? lo : r;
    r = r > hi ? hi : r;
    return (int)r;
}

// Scale of a Q8 block from its absmax: IEEE f32 divisions, no reciprocal
// approximation.
__device__ __forceinline__ void q8_scale(float amax, float &d, float &id)
{
    d = __fdiv_rn(amax, 127.0f);
    id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
}

// Q8 of one 32-wide activation block into registers in the reordered layout:
// the Q8_0-style rule d = absmax/127, codes rint(x * (1/d)) clamped to +-127.
__device__ __forceinline__ void q8_block_vals(const float (&v)[QK], uint32_t (&o)[8], float &dsc)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) amax = fmaxf(amax, fabsf(v[i]));
    float d, id;
    q8_scale(amax, d, id);
    int c[QK];
#pragma unroll
    for (int i = 0; i < QK; ++i) c[i] = round_clamp(__fmul_rn(v[i], id), -127.0f, 127.0f) & 0xFF;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        o[2 * m] = (uint32_t)(c[8 * m] | (c[8 * m + 2] << 8) | (c[8 * m + 4] << 16) | (c[8 * m + 6] << 24));
        o[2 * m + 1] = (uint32_t)(c[8 * m + 1] | (c[8 * m + 3] << 8) | (c[8 * m + 5] << 16) | (c[8 * m + 7] << 24));
    }
    dsc = d;
}

// The same from memory (16-byte aligned block).
__device__ __forceinline__ void q8_block_regs(const float *__restrict__ src, uint32_t (&o)[8], float &dsc)
{
    float v[QK];
#pragma unroll
    for (int i = 0; i < QK / 4; ++i) {
        const float4 f = reinterpret_cast<const float4 *>(src)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    q8_block_vals(v, o, dsc);
}

__device__ __forceinline__ void q8_block_reordered(const float *__restrict__ src, int8_t *__restrict__ dst,
                                                   float *__restrict__ dsc)
{
    uint32_t o[8];
    float d;
    q8_block_regs(src, o, d);
    reinterpret_cast<uint4 *>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4 *>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
    *dsc = d;
}

// Q8 of one 32-wide block by the 32 lanes of an aligned half-wave, lane i
// holding element v: absmax = fmaxf over 0 and every |v| (as q8_block_vals
// takes it, so NaN elements are passed over alike), the same scale and
// rounding; lane i stores its code in the reordered position and lane 0 the
// scale. Bit for bit q8_block_reordered's output.
__device__ __forceinline__ void q8_block_lanes(float v, int i, int8_t *__restrict__ dst, float *__restrict__ dsc)
{
    float a = fmaxf(0.0f, fabsf(v));
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
    float d, id;
    q8_scale(a, d, id);
    dst[(i & ~7) + perm8(i & 7)] = (int8_t)round_clamp(__fmul_rn(v, id), -127.0f, 127.0f);
    if (i == 0) *dsc = d;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v, int width = 64)
{
    for (int o = width >> 1; o > 0; o >>= 1) {
        T u = __shfl_xor(v, o, width);
        v = u > v ? u : v;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v, int width = 64)
{
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, width);
    return v;
}

// 64-bit lane exchanges built from 32-bit cross-lane primitives.
__device__ __forceinline__ int dlo(double v) { return __double2loint(v); }
__device__ __forceinline__ int dhi(double v) { return __double2hiint(v); }
__device__ __forceinline__ double dmk(int lo, int hi) { return __hiloint2double(hi, lo); }

// v_permlane32_swap on a pair of doubles: returns (a + b') where, for lanes
// 0..31, the sum is a[l] + a[l+32] and for lanes 32..63 it is b[l-32] + b[l].
__device__ __forceinline__ double swap_add32(double a, double b)
{
    const auto lo = __builtin_amdgcn_permlane32_swap(dlo(a), dlo(b), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(dhi(a), dhi(b), false, false);
    return dmk(lo[0], hi[0]) + dmk(lo[1], hi[1]);
}

// v_permlane16_swap: rows of 16 lanes; even rows get a[l] + a[l+16], odd rows
// get b[l-16] + b[l].
__device__ __forceinline__ double swap_add16(double a, double b)
{
    const auto lo = __builtin_amdgcn_permlane16_swap(dlo(a), dlo(b), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(dhi(a), dhi(b), false, false);
    return dmk(lo[0], hi[0]) + dmk(lo[1], hi[1]);
}

// DPP move of a double (both halves with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v)
{
    return dmk(__builtin_amdgcn_mov_dpp(dlo(v), CTRL, 0xF, 0xF, false),
               __builtin_amdgcn_mov_dpp(dhi(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_ROR8 = 0x128;   // row_ror:8 == lane ^ 8 inside a 16-lane row

template <int D>
__device__ __forceinline__ double xor_lane(double v)
{
    if constexpr (D == 1) return dpp_d<DPP_XOR1>(v);
    else if constexpr (D == 2) return dpp_d<DPP_XOR2>(v);
    else if constexpr (D == 8) return dpp_d<DPP_ROR8>(v);
    else return __shfl_xor(v, D);
}

// One halving step of the transposing reduction at lane distance D on N
// values: lanes with bit D clear keep the lower half, the others the upper.
template <int N, int D>
__device__ __forceinline__ void tr_step(double *v, int lane)
{
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        if constexpr (D == 32) {
            v[i] = swap_add32(v[i], v[i + N / 2]);
        } else if constexpr (D == 16) {
            v[i] = swap_add16(v[i], v[i + N / 2]);
        } else {
            const bool upper = (lane & D) != 0;
            const double lo = v[i], hi = v[i + N / 2];
            const double keep = upper ? hi : lo;
            const double send = upper ? lo : hi;
            v[i] = keep + xor_lane<D>(send);
        }
    }
}

template <int N, int D>
__device__ __forceinline__ void tr_rec(double *v, int lane)
{
    if constexpr (N > 1) {
        tr_step<N, D>(v, lane);
        tr_rec<N / 2, D / 2>(v, lane);
    } else if constexpr (D >= 1) {
        v[0] += xor_lane<D>(v[0]);
        tr_rec<1, D / 2>(v, lane);
    }
}

// Transposing reduction of N values per lane over a 64-lane wave (N a power
// of two, N <= 64): afterwards lane l holds the wave-wide sum of value
// (l >> (6 - log2 N)) & (N - 1) in v[0]. Each halving step sends the half a
// lane does not keep to its partner, so N values cost N - 1 exchanges; the
// distance-32/16 steps use the gfx950 permlane swaps, which need no select.
template <int N>
__device__ __forceinline__ void wave_transpose_reduce(double (&v)[N])
{
    tr_rec<N, 32>(v, threadIdx.x & 63);
}

template <int N>
__device__ __forceinline__ constexpr int log2i() { return N <= 1 ? 0 : 1 + log2i<N / 2>(); }

template <int N>
__device__ __forceinline__ int transpose_index(int lane) { return (lane >> (6 - log2i<N>())) & (N - 1); }

// Sigmoid-weighted linear unit on f64 inputs: silu(g) = g / (1 + exp(-g)).
__device__ __forceinline__ double silu_f64(double g) { return g / (1.0 + exp(-g)); }

// RMSNorm scales of T <= NT token rows (the chain's glue: colibri
// architecture overview, section 4, rmsnorm among the kernels). Every
// workgroup that needs a row's scale takes it in this one order, so all of
// them agree bit for bit: RMS_BLOCK threads, thread j summing the f64 squares
// of its float4s j, j + RMS_BLOCK, ... (components x, y, z, w), or of its
// elements j, j + RMS_BLOCK, ... when !vec; a wave sum; the wave sums in wave
// order. scale = 1 / sqrt(sum / H + eps) in f64, and a normalised element is
// (float)((double)x * scale * (double)gamma). vec: x 16-byte aligned and
// H % 4 == 0. All RMS_BLOCK threads call it; red holds 8 * NT doubles.
constexpr int RMS_BLOCK = 512;

template <int NT>
__device__ __forceinline__ void rms_scales(const float *__restrict__ x, int T, int H, float eps, bool vec,
                                           double *red, double (&scale)[NT])
{
    double ss[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        ss[t] = 0.0;
        if (t < T) {
            const float *xt = x + (long)t * H;
            if (vec) {
                for (int i = threadIdx.x; i < H / 4; i += RMS_BLOCK) {
                    const float4 v = reinterpret_cast<const float4 *>(xt)[i];
                    ss[t] += (double)v.x * (double)v.x;
                    ss[t] += (double)v.y * (double)v.y;
                    ss[t] += (double)v.z * (double)v.z;
                    ss[t] += (double)v.w * (double)v.w;
                }
            } else {
                for (int i = threadIdx.x; i < H; i += RMS_BLOCK) ss[t] += (double)xt[i] * (double)xt[i];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const double v = wave_sum(ss[t]);
        if ((threadIdx.x & 63) == 0) red[(threadIdx.x >> 6) * NT + t] = v;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        double v = red[t];
        for (int w = 1; w < RMS_BLOCK / 64; ++w) v += red[w * NT + t];
        scale[t] = 1.0 / sqrt(v / (double)H + (double)eps);
    }
    __syncthreads();
}

__device__ __forceinline__ float rms_apply(float x, double scale, float g)
{
    return (float)((double)x * scale * (double)g);
}

} // namespace coli
