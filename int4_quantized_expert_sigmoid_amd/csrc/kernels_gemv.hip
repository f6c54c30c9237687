// kernels_gemv.hip — the token-GEMV expert path for small batches (T <= 8).
//
// What is computed (colibri architecture overview, sections 3.1 and 5; the
// IDOT path dot_i4i8): for every item (a distinct expert of the batch, read
// once, with up to 8 token slots) and every row,
//   g_row = d_row * sum_b d_b * S_b,  S_b = sum_{k in b} code4 * q8   (int32),
// the block sum in f64; h = silu(g) * u (f64, stored f32); Q8(h) in 32-row
// blocks; then the down projection the same way.
//
// Mapping: a workgroup owns 32 consecutive output rows of one item. Every
// thread owns one 32-wide block column and streams that 16-byte piece of each
// row (lanes of a wave read 1 KB contiguous per load); the activation block of
// each token slot stays in registers. Per-row partial sums are folded with a
// transposing wave reduction, then across waves through LDS in wave order.
#include "device_common.hpp"
#include "internal.hpp"

namespace coli {
namespace {

struct GemvArgs {
    const uint8_t *q_a, *q_b;      // gate, up (gate/up kernel) or down (down kernel)
    const float *s_a, *s_b;
    int H, I;
    const int8_t *xq;              // [T][H] reordered Q8(x)
    const float *xs;               // [T][H/32]
    const int *ctrl, *item_expert, *item_ntok, *item_tok;
    float *h;                      // [pairs][I]
    int8_t *hq;                    // [pairs][I] reordered
    float *hs;                     // [pairs][I/32]
    float *ye;                     // [pairs][H]
};

template <int NT, int RC>
__global__ void __launch_bounds__(256) k_gateup_gemv(GemvArgs a)
{
    constexpr int NV = 2 * RC;                   // values per chunk: RC rows x (gate, up)
    __shared__ double red[4][NT][64];
    const int nrb = a.I / QK;
    const int item = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    if (item >= a.ctrl[CTRL_N_ITEMS]) return;
    const int e = a.item_expert[item];
    const int nt = a.item_ntok[item];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nblk = a.H / QK;
    const bool active = tid < nblk;
    const long rowb = (long)(a.H / 2);

    Blk8 act[NT];
    double dsc[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) {
        if (s < nt && active) {
            const int t = a.item_tok[item * MAX_SLOTS + s];
            act[s] = load_blk8(a.xq + (long)t * a.H + tid * QK);
            dsc[s] = (double)a.xs[(long)t * nblk + tid] * 0.0625;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) act[s].v[k] = 0;
            dsc[s] = 0.0;
        }
    }
    const long row0 = (long)e * a.I + (long)rb * QK;
    // threads past the row's last block read block 0 and multiply it by zero
    const int tb = active ? tid : 0;
    const uint8_t *pg = a.q_a + row0 * rowb + tb * 16;
    const uint8_t *pu = a.q_b + row0 * rowb + tb * 16;

    for (int c = 0; c < QK / RC; ++c) {
        uint4 wg[RC], wu[RC];
#pragma unroll
        for (int r = 0; r < RC; ++r) {
            wg[r] = load_u4_stream(pg + (long)(c * RC + r) * rowb);
            wu[r] = load_u4_stream(pu + (long)(c * RC + r) * rowb);
        }
        double v[NT][NV];
#pragma unroll
        for (int r = 0; r < RC; ++r) {
            int lo[4], hi[4];
            unpack_nibbles(wg[r], lo, hi);
#pragma unroll
            for (int s = 0; s < NT; ++s) v[s][2 * r] = (double)dot_block16(lo, hi, act[s]) * dsc[s];
            unpack_nibbles(wu[r], lo, hi);
#pragma unroll
            for (int s = 0; s < NT; ++s) v[s][2 * r + 1] = (double)dot_block16(lo, hi, act[s]) * dsc[s];
        }
        const int vi = transpose_index<NV>(lane);
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            wave_transpose_reduce<NV>(v[s]);
            if ((lane & (64 / NV - 1)) == 0) red[wave][s][2 * c * RC + vi] = v[s][0];
        }
    }
    __syncthreads();

    const int nw = blockDim.x >> 6;
    for (int i = tid; i < NT * QK; i += blockDim.x) {
        const int s = i / QK, r = i % QK;
        if (s >= nt) continue;                   // uniform over the 32 lanes of a slot
        double g = red[0][s][2 * r], u = red[0][s][2 * r + 1];
        for (int w = 1; w < nw; ++w) { g += red[w][s][2 * r]; u += red[w][s][2 * r + 1]; }
        const long grow = row0 + r;
        const float gf = (float)((double)a.s_a[grow] * g);
        const float uf = (float)((double)a.s_b[grow] * u);
        const float hv = (float)(silu_f64((double)gf) * (double)uf);
        const float amax = wave_max(fabsf(hv), 32);
        float d, id;
        q8_scale(amax, d, id);
        const int code = round_clamp(__fmul_rn(hv, id), -127.0f, 127.0f);
        const long pair = (long)item * MAX_SLOTS + s;
        const int col = rb * QK + r;
        a.h[pair * a.I + col] = hv;
        a.hq[pair * a.I + rb * QK + (r & ~7) + perm8(r & 7)] = (int8_t)code;
        if (r == 0) a.hs[pair * nrb + rb] = d;
    }
}

template <int NT, int RD>
__global__ void __launch_bounds__(256) k_down_gemv(GemvArgs a)
{
    const int ngrp = a.H / QK;
    const int item = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    if (item >= a.ctrl[CTRL_N_ITEMS]) return;
    const int e = a.item_expert[item];
    const int nt = a.item_ntok[item];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = a.I / QK;
    const bool active = lane < nblk;
    const long rowb = (long)(a.I / 2);

    Blk8 act[NT];
    double dsc[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) {
        if (s < nt && active) {
            const long pair = (long)item * MAX_SLOTS + s;
            act[s] = load_blk8(a.hq + pair * a.I + lane * QK);
            dsc[s] = (double)a.hs[pair * nblk + lane] * 0.0625;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) act[s].v[k] = 0;
            dsc[s] = 0.0;
        }
    }
    const int rows_per_wave = QK / (blockDim.x >> 6);
    const long row0 = (long)grp * QK + wave * rows_per_wave;
    const uint8_t *pd = a.q_a + ((long)e * a.H + row0) * rowb + (active ? lane : 0) * 16;
    for (int c = 0; c < rows_per_wave / RD; ++c) {
        uint4 wd[RD];
#pragma unroll
        for (int r = 0; r < RD; ++r)
            wd[r] = load_u4_stream(pd + (long)(c * RD + r) * rowb);
        double v[NT][RD];
#pragma unroll
        for (int r = 0; r < RD; ++r) {
            int lo[4], hi[4];
            unpack_nibbles(wd[r], lo, hi);
#pragma unroll
            for (int s = 0; s < NT; ++s) v[s][r] = (double)dot_block16(lo, hi, act[s]) * dsc[s];
        }
        const int vi = transpose_index<RD>(lane);
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            wave_transpose_reduce<RD>(v[s]);
            if (s < nt && (lane & (64 / RD - 1)) == 0) {
                const long row = row0 + c * RD + vi;
                const long pair = (long)item * MAX_SLOTS + s;
                a.ye[pair * a.H + row] = (float)((double)a.s_a[(long)e * a.H + row] * v[s][0]);
            }
        }
    }
}

GemvArgs make_args(const coli_moe_layer &L, const WsLayout &lay, char *ws)
{
    GemvArgs a;
    a.H = L.H; a.I = L.I;
    a.xq = reinterpret_cast<const int8_t *>(ws + lay.xq);
    a.xs = reinterpret_cast<const float *>(ws + lay.xs);
    a.ctrl = reinterpret_cast<const int *>(ws + lay.ctrl);
    a.item_expert = reinterpret_cast<const int *>(ws + lay.item_expert);
    a.item_ntok = reinterpret_cast<const int *>(ws + lay.item_ntok);
    a.item_tok = reinterpret_cast<const int *>(ws + lay.item_tok);
    a.h = reinterpret_cast<float *>(ws + lay.h);
    a.hq = reinterpret_cast<int8_t *>(ws + lay.hq);
    a.hs = reinterpret_cast<float *>(ws + lay.hs);
    a.ye = reinterpret_cast<float *>(ws + lay.ye);
    return a;
}

} // namespace

hipError_t launch_gateup_gemv(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    GemvArgs a = make_args(L, lay, ws);
    a.q_a = L.gate_q; a.s_a = L.gate_s; a.q_b = L.up_q; a.s_b = L.up_s;
    const int nblk = L.H / QK;
    const int threads = ((nblk + 63) / 64) * 64;
    const dim3 grid((unsigned)(lay.max_items * (L.I / QK)));
    if (T <= 1)
        hipLaunchKernelGGL((k_gateup_gemv<1, 8>), grid, dim3(threads), 0, s, a);
    else if (T <= 2)
        hipLaunchKernelGGL((k_gateup_gemv<2, 8>), grid, dim3(threads), 0, s, a);
    else if (T <= 4)
        hipLaunchKernelGGL((k_gateup_gemv<4, 4>), grid, dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL((k_gateup_gemv<8, 2>), grid, dim3(threads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_gemv(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    GemvArgs a = make_args(L, lay, ws);
    a.q_a = L.down_q; a.s_a = L.down_s; a.q_b = nullptr; a.s_b = nullptr;
    const dim3 grid((unsigned)(lay.max_items * (L.H / QK)));
    if (T <= 1)
        hipLaunchKernelGGL((k_down_gemv<1, 8>), grid, dim3(256), 0, s, a);
    else if (T <= 2)
        hipLaunchKernelGGL((k_down_gemv<2, 8>), grid, dim3(256), 0, s, a);
    else if (T <= 4)
        hipLaunchKernelGGL((k_down_gemv<4, 4>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_down_gemv<8, 2>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace coli
