// kernels_grouped.hip — grouped int8-MFMA expert GEMMs for large batches
// (prefill, T > 8).
//
// The same IDOT arithmetic as the GEMV path (colibri architecture overview,
// section 3.1: int4 weights dequantised on use, int8 activations, integer
// dot products), batched over the union of selected experts (colibri README
// zh-TW, "how it works": a batch reads each distinct expert once). Pairs
// (token, expert) are bucketed per expert and cut into tiles of 32 pairs.
//
// One wave computes a 32-row x 32-pair output tile. For every 32-wide block
// b it issues v_mfma_i32_32x32x32_i8 with
//   A = 32 weight rows x 32 k (lane l: row l%32, half l/32 holds 16 k),
//   B = 32 k x 32 pairs     (lane l: pair l%32, the same 16 k),
// unpacking the nibbles in registers (x16, exact), then adds
// C * (d_b/16) to an f64 accumulator per element: the block scale is per
// (token, block), so each block's int32 result is rescaled on its own.
// Both operands list their 16 k in the same order (the reordered 8-groups),
// so the product sums exactly the block's 32 k whatever order the matrix
// core uses inside a lane. Output element (row, pair) sits in lane
// pair + 32*((row/4)&1), register (row/8)*4 + row%4.
#include "device_common.hpp"
#include "internal.hpp"

namespace coli {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE_N = 32;     // pairs per tile (matches the bucket kernel)
constexpr int WAVES = 4;       // row tiles per workgroup

struct GroupedArgs {
    const uint8_t *q_a, *q_b;  // gate/up (both) or down (q_a)
    const float *s_a, *s_b;
    int H, I;
    const int8_t *act;         // gate/up: reordered Q8(x) [T][H]; down: reordered hq [pairs][I]
    const float *act_s;        // xs [T][H/32] or hs [pairs][I/32]
    const int *ctrl;
    const int2 *tiles;
    const int *expert_off, *pair_tok;
    float *h;
    int8_t *hq;
    float *hs;
    float *ye;
    int ntiles_max;            // tiles the grid covers
};

__device__ __forceinline__ v4i unpack8(uint2 w)
{
    const uint32_t m = 0xF0F0F0F0u;
    v4i a;
    a[0] = (int)((w.x << 4) & m);
    a[1] = (int)(w.x & m);
    a[2] = (int)((w.y << 4) & m);
    a[3] = (int)(w.y & m);
    return a;
}

__device__ __forceinline__ int tile_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

constexpr int PF = 4;          // 32-wide blocks loaded ahead of the MFMAs
constexpr int N_XCD = 8;       // workgroups go round-robin over the 8 XCDs by index

// Tile and row group of workgroup w. Tiles of one expert are consecutive in
// the tile list and each re-reads that expert's rows; with nrg a multiple of
// N_XCD, XCD x (w % 8 == x) owns row groups x, x + 8, ... and walks the
// tiles in order for each, so the tiles that share rows run together behind
// one L2 and the repeats hit there.
__device__ __forceinline__ void tile_rg(int w, int nrg, int ntiles, int &tile, int &rg)
{
    if (nrg % N_XCD == 0) {
        const int x = w % N_XCD, j = w / N_XCD;
        rg = (j / ntiles) * N_XCD + x;
        tile = j % ntiles;
    } else {
        tile = w / nrg;
        rg = w % nrg;
    }
}

static_assert(PF == 4, "two pairs of blocks per group: activation scales are fetched four blocks at a time");

// A pair of blocks (b, b+1) per stage: lane half h loads the 16 bytes of
// block b + h of its row (one contiguous load per row and block instead of
// two 8-byte halves), and one permlane32 swap per dword hands each half its
// 8 bytes of both blocks: afterwards A holds block b's bytes 8h..8h+7 and B
// block b+1's, the layout one MFMA per block expects.
__device__ __forceinline__ void split_pair(uint4 w, uint2 &A, uint2 &B)
{
    const auto s0 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
    A = make_uint2(s0[0], s1[0]);
    B = make_uint2(s0[1], s1[1]);
}

struct GuStage {
    uint4 wg, wu;              // 16 bytes of the gate and up rows: block b + half of the pair
    int4 xb0, xb1;             // this lane's 16 activation codes of blocks b and b+1
};

struct DnStageG {
    uint4 wd;
    int4 hb0, hb1;
};

__global__ void __launch_bounds__(256) k_gateup_mfma(GroupedArgs a)
{
    const int n_rt = a.I / QK;
    const int nrg = (n_rt + WAVES - 1) / WAVES;
    int tile, rg;
    tile_rg(blockIdx.x, nrg, a.ntiles_max, tile, rg);
    if (tile >= a.ctrl[CTRL_N_TILES_GU]) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rt = rg * WAVES + wave;
    if (rt >= n_rt) return;
    const int2 td = a.tiles[tile];
    const int e = td.x, p0 = td.y;
    const int np = min(TILE_N, a.expert_off[e + 1] - p0);
    const int n = lane & 31, half = lane >> 5;
    const bool valid = n < np;
    const int pair = p0 + n;
    const int tok = valid ? a.pair_tok[pair] : 0;
    const int nblk = a.H / QK;
    const long rowb = a.H / 2;
    const long wrow = (long)e * a.I + (long)rt * QK + n;
    const uint8_t *pg = a.q_a + wrow * rowb;
    const uint8_t *pu = a.q_b + wrow * rowb;
    const int8_t *px = a.act + (long)tok * a.H + 16 * half;
    const float *ps = a.act_s + (long)tok * nblk;

    double acc_g[16], acc_u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc_g[i] = 0.0; acc_u[i] = 0.0; }
    const v16i zero = {};

    auto mfma_block = [&](uint2 wg, uint2 wu, int4 xb, float dsc) {
        const v4i B = {xb.x, xb.y, xb.z, xb.w};
        const double d = valid ? (double)dsc * 0.0625 : 0.0;
        const v16i cg = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack8(wg), B, zero, 0, 0, 0);
        const v16i cu = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack8(wu), B, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc_g[i] = fma((double)cg[i], d, acc_g[i]);
            acc_u[i] = fma((double)cu[i], d, acc_u[i]);
        }
    };
    // two pairs of blocks in flight ahead of the MFMAs; the activation
    // scales of the four blocks of a group come as one 16-byte load
    GuStage st[2];
    auto load = [&](GuStage &g, int bp) {
        const int b = 2 * bp;
        g.wg = *reinterpret_cast<const uint4 *>(pg + 16 * (b + half));
        g.wu = *reinterpret_cast<const uint4 *>(pu + 16 * (b + half));
        g.xb0 = *reinterpret_cast<const int4 *>(px + 32 * b);   // padding lanes: token 0, scaled by zero
        g.xb1 = *reinterpret_cast<const int4 *>(px + 32 * (b + 1));
    };
    auto step = [&](const GuStage &g, float d0, float d1) {
        uint2 ga, gb, ua, ub;
        split_pair(g.wg, ga, gb);
        split_pair(g.wu, ua, ub);
        mfma_block(ga, ua, g.xb0, d0);
        mfma_block(gb, ub, g.xb1, d1);
    };
    // whole groups of two pairs: every load unconditional (past the end it
    // re-reads the last pair), so the waits count exactly the older loads
    const int npair = nblk / 2;
    const int nfull = nblk % 4 == 0 ? npair - npair % 2 : 0;   // 16-byte scale loads need 4 | nblk
    if (nfull > 0) {
        load(st[0], 0);
        float4 dcur = *reinterpret_cast<const float4 *>(ps);
        for (int p0 = 0; p0 < nfull; p0 += 2) {
            const float4 dnext = *reinterpret_cast<const float4 *>(ps + 2 * min(p0 + 2, nfull - 2));
            load(st[1], p0 + 1);
            step(st[0], dcur.x, dcur.y);
            load(st[0], min(p0 + 2, npair - 1));
            step(st[1], dcur.z, dcur.w);
            dcur = dnext;
        }
    }
    for (int bp = nfull; bp < npair; ++bp) {
        load(st[0], bp);
        step(st[0], ps[2 * bp], ps[2 * bp + 1]);
    }
    if (nblk % 2) {                              // an odd last block: each half loads its own 8 bytes
        const int b = nblk - 1;
        mfma_block(*reinterpret_cast<const uint2 *>(pg + 16 * b + 8 * half),
                   *reinterpret_cast<const uint2 *>(pu + 16 * b + 8 * half),
                   *reinterpret_cast<const int4 *>(px + 32 * b), ps[b]);
    }
    // epilogue: g, u, h = silu(g)*u, Q8 over the tile's 32 rows per pair
    float hv[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const long grow = (long)e * a.I + (long)rt * QK + tile_row(i, half);
        const float gf = (float)((double)a.s_a[grow] * acc_g[i]);
        const float uf = (float)((double)a.s_b[grow] * acc_u[i]);
        hv[i] = (float)(silu_f64((double)gf) * (double)uf);
        amax = fmaxf(amax, fabsf(hv[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (!valid) return;
    float d, id;
    q8_scale(amax, d, id);
    const long base = (long)pair * a.I + (long)rt * QK;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = tile_row(i, half);
        a.h[base + r] = hv[i];
        a.hq[base + (r & ~7) + perm8(r & 7)] = (int8_t)round_clamp(__fmul_rn(hv[i], id), -127.0f, 127.0f);
    }
    if (half == 0) a.hs[(long)pair * n_rt + rt] = d;
}

__global__ void __launch_bounds__(256) k_down_mfma(GroupedArgs a)
{
    const int n_rt = a.H / QK;
    const int nrg = (n_rt + WAVES - 1) / WAVES;
    int tile, rg;
    tile_rg(blockIdx.x, nrg, a.ntiles_max, tile, rg);
    if (tile >= a.ctrl[CTRL_N_TILES_GU]) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rt = rg * WAVES + wave;
    if (rt >= n_rt) return;
    const int2 td = a.tiles[tile];
    const int e = td.x, p0 = td.y;
    const int np = min(TILE_N, a.expert_off[e + 1] - p0);
    const int n = lane & 31, half = lane >> 5;
    const bool valid = n < np;
    const int pair = p0 + n;
    const int nblk = a.I / QK;
    const long rowb = a.I / 2;
    const long wrow = (long)e * a.H + (long)rt * QK + n;
    const uint8_t *pd = a.q_a + wrow * rowb;
    const int8_t *ph = a.act + (long)(valid ? pair : p0) * a.I + 16 * half;
    const float *ps = a.act_s + (long)(valid ? pair : p0) * nblk;

    double acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0;
    const v16i zero = {};

    auto mfma_block = [&](uint2 wd, int4 hb, float dsc) {
        const v4i B = {hb.x, hb.y, hb.z, hb.w};
        const double d = valid ? (double)dsc * 0.0625 : 0.0;
        const v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack8(wd), B, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = fma((double)c[i], d, acc[i]);
    };
    DnStageG st[2];
    auto load = [&](DnStageG &g, int bp) {
        const int b = 2 * bp;
        g.wd = *reinterpret_cast<const uint4 *>(pd + 16 * (b + half));
        g.hb0 = *reinterpret_cast<const int4 *>(ph + 32 * b);   // padding lanes: pair p0, scaled by zero
        g.hb1 = *reinterpret_cast<const int4 *>(ph + 32 * (b + 1));
    };
    auto step = [&](const DnStageG &g, float d0, float d1) {
        uint2 wa, wb;
        split_pair(g.wd, wa, wb);
        mfma_block(wa, g.hb0, d0);
        mfma_block(wb, g.hb1, d1);
    };
    const int npair = nblk / 2;
    const int nfull = nblk % 4 == 0 ? npair - npair % 2 : 0;   // 16-byte scale loads need 4 | nblk
    if (nfull > 0) {
        load(st[0], 0);
        float4 dcur = *reinterpret_cast<const float4 *>(ps);
        for (int p0 = 0; p0 < nfull; p0 += 2) {
            const float4 dnext = *reinterpret_cast<const float4 *>(ps + 2 * min(p0 + 2, nfull - 2));
            load(st[1], p0 + 1);
            step(st[0], dcur.x, dcur.y);
            load(st[0], min(p0 + 2, npair - 1));
            step(st[1], dcur.z, dcur.w);
            dcur = dnext;
        }
    }
    for (int bp = nfull; bp < npair; ++bp) {
        load(st[0], bp);
        step(st[0], ps[2 * bp], ps[2 * bp + 1]);
    }
    if (nblk % 2) {
        const int b = nblk - 1;
        mfma_block(*reinterpret_cast<const uint2 *>(pd + 16 * b + 8 * half),
                   *reinterpret_cast<const int4 *>(ph + 32 * b), ps[b]);
    }
    if (!valid) return;
    float rs[16];                                // row scales first: the stores below may not alias them
#pragma unroll
    for (int i = 0; i < 16; ++i) rs[i] = a.s_a[(long)e * a.H + (long)rt * QK + tile_row(i, half)];
    const long base = (long)pair * a.H + (long)rt * QK;
#pragma unroll
    for (int i = 0; i < 16; ++i) a.ye[base + tile_row(i, half)] = (float)((double)rs[i] * acc[i]);
}

GroupedArgs make_args(const WsLayout &lay, char *ws, const coli_moe_layer &L)
{
    GroupedArgs a;
    a.H = L.H; a.I = L.I;
    a.ctrl = reinterpret_cast<const int *>(ws + lay.ctrl);
    a.tiles = reinterpret_cast<const int2 *>(ws + lay.tiles);
    a.expert_off = reinterpret_cast<const int *>(ws + lay.expert_off);
    a.pair_tok = reinterpret_cast<const int *>(ws + lay.pair_tok);
    a.h = reinterpret_cast<float *>(ws + lay.h);
    a.hq = reinterpret_cast<int8_t *>(ws + lay.hq);
    a.hs = reinterpret_cast<float *>(ws + lay.hs);
    a.ye = reinterpret_cast<float *>(ws + lay.ye);
    return a;
}

int max_tiles(const WsLayout &lay, const coli_moe_layer &L)
{
    return (lay.n_pairs + TILE_N - 1) / TILE_N + L.E + 1;
}

} // namespace

hipError_t launch_gateup_grouped(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    (void)T;
    GroupedArgs a = make_args(lay, ws, L);
    a.ntiles_max = max_tiles(lay, L);
    a.q_a = L.gate_q; a.s_a = L.gate_s; a.q_b = L.up_q; a.s_b = L.up_s;
    a.act = reinterpret_cast<const int8_t *>(ws + lay.xq);
    a.act_s = reinterpret_cast<const float *>(ws + lay.xs);
    const int nrg = (L.I / QK + WAVES - 1) / WAVES;
    hipLaunchKernelGGL(k_gateup_mfma, dim3((unsigned)(max_tiles(lay, L) * nrg)), dim3(64 * WAVES), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_grouped(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    (void)T;
    GroupedArgs a = make_args(lay, ws, L);
    a.ntiles_max = max_tiles(lay, L);
    a.q_a = L.down_q; a.s_a = L.down_s; a.q_b = nullptr; a.s_b = nullptr;
    a.act = reinterpret_cast<const int8_t *>(ws + lay.hq);
    a.act_s = reinterpret_cast<const float *>(ws + lay.hs);
    const int nrg = (L.H / QK + WAVES - 1) / WAVES;
    hipLaunchKernelGGL(k_down_mfma, dim3((unsigned)(max_tiles(lay, L) * nrg)), dim3(64 * WAVES), 0, s, a);
    return hipGetLastError();
}

} // namespace coli
