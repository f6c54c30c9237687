// gemv_device.hpp — device bodies of the token-GEMV expert path (T <= 8),
// shared by the standalone GEMV kernels, the decode launches and the dense MLP.
//
// What is computed (colibri architecture overview, sections 3.1 and 5; the
// IDOT path dot_i4i8): for every item (a distinct expert of the batch, read
// once, with up to 8 token slots) and every row,
//   g_row = d_row * sum_b d_b * S_b,  S_b = sum_{k in b} code4 * q8   (int32),
// the block sum in f64; h = silu(g) * u (f64, stored f32); Q8(h) in 32-row
// blocks; then the down projection the same way.
//
// Gate/up mapping: a workgroup owns 32 consecutive rows of one item. Thread
// b owns the 32-wide block column b of every row and streams that 16-byte
// piece (lanes of a wave read 1 KB contiguous per load); the activation block
// of each token slot stays in registers. Rows are taken in chunks with the
// next chunk's loads in flight while the current one is reduced. Per-row
// partials are folded with a transposing wave reduction, then across waves
// through LDS in wave order.
// Down mapping: each wave owns 8 rows; lane l owns block column l.
#pragma once
#include "device_common.hpp"

namespace coli {

struct GemvArgs {
    const uint8_t *q_a, *q_b;      // gate, up (gate/up) or down (down)
    const float *s_a, *s_b;
    int H, I, E, T;
    int has_shared;                // item 0 is the shared expert (expert E, slot t = token t)
    int gsh;                       // group scales: log2(group / 32) (kernels instantiated with GS)
    int item0;                     // first item of a launch that covers items item0.. only
    const int8_t *xq;              // [T][H] reordered Q8(x)
    const float *xs;               // [T][H/32]
    const int *ctrl, *item_expert, *item_ntok, *item_tok;
    float *h;                      // [pairs][I]
    int8_t *hq;                    // [pairs][I] reordered
    float *hs;                     // [pairs][I/32]
    float *ye;                     // [pairs][H]
};

struct ItemDesc {
    int item, e, nt;
    int tok[MAX_SLOTS];
};

// An item's expert and token slots from the union tables an earlier launch
// wrote: plain loads, which the launch boundary makes coherent.
__device__ __forceinline__ ItemDesc item_from_table(const GemvArgs &a, int item)
{
    ItemDesc d;
    d.item = item;
    d.e = a.item_expert[item];
    d.nt = a.item_ntok[item];
#pragma unroll
    for (int s = 0; s < MAX_SLOTS; ++s) d.tok[s] = a.item_tok[item * MAX_SLOTS + s];
#pragma unroll
    for (int s = 0; s < MAX_SLOTS; ++s) d.tok[s] = s < d.nt ? d.tok[s] : 0;
    return d;
}

// The shared expert: item 0, slot t = token t (known before routing).
__device__ __forceinline__ ItemDesc shared_item(const GemvArgs &a)
{
    ItemDesc d;
    d.item = 0;
    d.e = a.E;
    d.nt = a.T;
#pragma unroll
    for (int s = 0; s < MAX_SLOTS; ++s) d.tok[s] = s;
    return d;
}

template <int NT>
struct GateUpShared {
    double red[4][NT][64];
};

// Gate/up rows [rb*32, rb*32+32) of one item for its token slots, SwiGLU,
// Q8(h); writes h, hq, hs of pairs item*8 + slot. All threads of the
// workgroup must call it (blockDim >= 64 * ceil(H/32/64) * RS; waves past
// that idle until the epilogue). RS > 1 splits the 32 rows into RS sets of
// waves, each streaming 32/RS rows, so fewer loads queue behind each other.
// GS: int4 rows with one scale per group of 32 << gsh columns; each block's
// term is (S_b * d_b) * s_group, so no row scale is applied at the end.
template <int NT, int RC, int RS = 1, int WB = 4, bool GS = false>
__device__ __forceinline__ void gateup_rows(const GemvArgs &a, const ItemDesc &it, int rb, GateUpShared<NT> &sh)
{
    static_assert(!GS || WB == 4, "group scales are an int4 format");
    constexpr int RG = GS ? RC : 1;              // group scales held per chunk
    constexpr int NP = WFmt<WB>::NP;     // 16-byte pieces per row block
    constexpr double KS = WFmt<WB>::KSCALE;
    constexpr int NV = 2 * RC;                   // values per chunk: RC rows x (gate, up)
    constexpr int RPS = QK / RS;                 // rows per set
    constexpr int NC = RPS / RC;                 // chunks per set
    static_assert(RPS % RC == 0, "a set covers whole chunks");
    const int nrb = a.I / QK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nblk = a.H / QK;
    const int nw = (nblk + 63) >> 6;             // waves that own block columns
    const long rowb = (long)a.H * WB / 8;
    const long row0 = (long)it.e * a.I + (long)rb * QK;
    const int set = wave / nw, wv = wave - set * nw;
    const int col = wv * 64 + lane;              // this thread's block column
    // token slots in use, as a scalar: slots past it cost no dot products
    const int ntu = __builtin_amdgcn_readfirstlane(it.nt);

    if (set < RS) {
        const bool active = col < nblk;
        Blk8 act[NT];
        double dsc[NT];
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            if (s < it.nt && active) {
                const int t = it.tok[s];
                act[s] = load_blk8(a.xq + (long)t * a.H + col * QK);
                dsc[s] = (double)a.xs[(long)t * nblk + col] * KS;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) act[s].v[k] = 0;
                dsc[s] = 0.0;
            }
        }
        // threads past the row's last block read block 0 and multiply it by zero
        const int tb = active ? col : 0;
        const uint8_t *pg = a.q_a + (row0 + set * RPS) * rowb + blk_off<WB>(tb);
        const uint8_t *pu = a.q_b + (row0 + set * RPS) * rowb + blk_off<WB>(tb);
        // group scales of this thread's block column: row stride H / group
        const long gstr = GS ? (long)(nblk >> a.gsh) : 0;
        const float *psg = GS ? a.s_a + (row0 + set * RPS) * gstr + (tb >> a.gsh) : nullptr;
        const float *psu = GS ? a.s_b + (row0 + set * RPS) * gstr + (tb >> a.gsh) : nullptr;

        uint4 wg[2][RC][NP], wu[2][RC][NP];
        float sg[2][RG], su[2][RG];
#pragma unroll
        for (int r = 0; r < RC; ++r) {
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                wg[0][r][q] = load_w_stream<WB>(pg + (long)r * rowb + piece_off<WB>(q, nblk));
                wu[0][r][q] = load_w_stream<WB>(pu + (long)r * rowb + piece_off<WB>(q, nblk));
            }
            if constexpr (GS) {
                sg[0][r] = psg[(long)r * gstr];
                su[0][r] = psu[(long)r * gstr];
            }
        }
        // chunk c computes from buffer cur (= c % 2) while chunk c + 1 loads
        // into the other; cur must fold to a constant at every call, or the
        // buffers go to scratch memory
        auto chunk = [&](int c, int cur) {
            if (c + 1 < NC) {
#pragma unroll
                for (int r = 0; r < RC; ++r) {
#pragma unroll
                    for (int q = 0; q < NP; ++q) {
                        wg[cur ^ 1][r][q] = load_w_stream<WB>(pg + (long)((c + 1) * RC + r) * rowb + piece_off<WB>(q, nblk));
                        wu[cur ^ 1][r][q] = load_w_stream<WB>(pu + (long)((c + 1) * RC + r) * rowb + piece_off<WB>(q, nblk));
                    }
                    if constexpr (GS) {
                        sg[cur ^ 1][r] = psg[(long)((c + 1) * RC + r) * gstr];
                        su[cur ^ 1][r] = psu[(long)((c + 1) * RC + r) * gstr];
                    }
                }
            }
            double v[NT][NV];
#pragma unroll
            for (int r = 0; r < RC; ++r) {
#pragma unroll
                for (int s = 0; s < NT; ++s) {
                    if (s > 0 && s >= ntu) break;    // slot 0 is always in use
                    v[s][2 * r] = (double)dot_block_w<WB>(wg[cur][r], act[s]) * dsc[s];
                    v[s][2 * r + 1] = (double)dot_block_w<WB>(wu[cur][r], act[s]) * dsc[s];
                    if constexpr (GS) {
                        v[s][2 * r] *= (double)sg[cur][r];
                        v[s][2 * r + 1] *= (double)su[cur][r];
                    }
                }
            }
            const int vi = transpose_index<NV>(lane);
#pragma unroll
            for (int s = 0; s < NT; ++s) {
                if (s > 0 && s >= ntu) break;
                wave_transpose_reduce<NV>(v[s]);
                if ((lane & (64 / NV - 1)) == 0) sh.red[wv][s][2 * (set * RPS + c * RC) + vi] = v[s][0];
            }
        };
        if constexpr (NT >= 8) {
            // 8 slots: the unrolled loop would cost more registers than
            // its loads in flight are worth, so it runs in pairs
#pragma unroll 1
            for (int c = 0; c < NC; c += 2) {
                chunk(c, 0);
                if (c + 1 < NC) chunk(c + 1, 1);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) chunk(c, c & 1);
        }
    }
    __syncthreads();

    for (int i = tid; i < NT * QK; i += blockDim.x) {
        const int s = i / QK, r = i % QK;
        if (s >= it.nt) continue;                // uniform over the 32 lanes of a slot
        double g = sh.red[0][s][2 * r], u = sh.red[0][s][2 * r + 1];
        for (int w = 1; w < nw; ++w) { g += sh.red[w][s][2 * r]; u += sh.red[w][s][2 * r + 1]; }
        const long grow = row0 + r;
        const float gf = GS ? (float)g : (float)((double)a.s_a[grow] * g);
        const float uf = GS ? (float)u : (float)((double)a.s_b[grow] * u);
        const float hv = (float)(silu_f64((double)gf) * (double)uf);
        const float amax = wave_max(fabsf(hv), 32);
        float d, id;
        q8_scale(amax, d, id);
        const int code = round_clamp(__fmul_rn(hv, id), -127.0f, 127.0f);
        const long pair = (long)it.item * MAX_SLOTS + s;
        a.h[pair * a.I + rb * QK + r] = hv;
        a.hq[pair * a.I + rb * QK + (r & ~7) + perm8(r & 7)] = (int8_t)code;
        if (r == 0) a.hs[pair * nrb + rb] = d;
    }
    __syncthreads();
}

// Down rows of one item for row group grp of 4*RPW rows (each wave RPW rows,
// lane l owns block column l; chunks of RD rows with the next chunk's loads in
// flight); writes ye of pairs item*8 + slot. blockDim = 256. GS: group
// scales, as gateup_rows.
template <int NT, int RD, int RPW, int WB = 4, bool GS = false>
__device__ __forceinline__ void down_rows(const GemvArgs &a, const ItemDesc &it, int grp)
{
    static_assert(!GS || WB == 4, "group scales are an int4 format");
    constexpr int RG = GS ? RD : 1;
    constexpr int NP = WFmt<WB>::NP;
    constexpr double KS = WFmt<WB>::KSCALE;
    constexpr int NC = RPW / RD;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = a.I / QK;
    const bool active = lane < nblk;
    const long rowb = (long)a.I * WB / 8;
    const long row0 = (long)grp * (4 * RPW) + wave * RPW;
    const int ntu = __builtin_amdgcn_readfirstlane(it.nt);
    const uint8_t *pd = a.q_a + ((long)it.e * a.H + row0) * rowb + blk_off<WB>(active ? lane : 0);
    const long gstr = GS ? (long)(nblk >> a.gsh) : 0;     // group scales per row: I / group
    const float *psd = GS ? a.s_a + ((long)it.e * a.H + row0) * gstr + ((active ? lane : 0) >> a.gsh) : nullptr;

    uint4 wd[2][RD][NP];
    float sd[2][RG];
#pragma unroll
    for (int r = 0; r < RD; ++r) {
#pragma unroll
        for (int q = 0; q < NP; ++q) wd[0][r][q] = load_w_stream<WB>(pd + (long)r * rowb + piece_off<WB>(q, nblk));
        if constexpr (GS) sd[0][r] = psd[(long)r * gstr];
    }

    Blk8 act[NT];
    double dsc[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) {
        if (s < it.nt && active) {
            const long pair = (long)it.item * MAX_SLOTS + s;
            act[s] = load_blk8(a.hq + pair * a.I + lane * QK);
            dsc[s] = (double)a.hs[pair * nblk + lane] * KS;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) act[s].v[k] = 0;
            dsc[s] = 0.0;
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int cur = c & 1;
        if (c + 1 < NC) {
#pragma unroll
            for (int r = 0; r < RD; ++r) {
#pragma unroll
                for (int q = 0; q < NP; ++q)
                    wd[cur ^ 1][r][q] = load_w_stream<WB>(pd + (long)((c + 1) * RD + r) * rowb + piece_off<WB>(q, nblk));
                if constexpr (GS) sd[cur ^ 1][r] = psd[(long)((c + 1) * RD + r) * gstr];
            }
        }
        double v[NT][RD];
#pragma unroll
        for (int r = 0; r < RD; ++r) {
#pragma unroll
            for (int s = 0; s < NT; ++s) {
                if (s > 0 && s >= ntu) break;        // slot 0 is always in use
                v[s][r] = (double)dot_block_w<WB>(wd[cur][r], act[s]) * dsc[s];
                if constexpr (GS) v[s][r] *= (double)sd[cur][r];
            }
        }
        const int vi = transpose_index<RD>(lane);
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            if (s > 0 && s >= ntu) break;
            wave_transpose_reduce<RD>(v[s]);
            if ((lane & (64 / RD - 1)) == 0) {
                const long row = row0 + c * RD + vi;
                const long pair = (long)it.item * MAX_SLOTS + s;
                const float out = GS ? (float)v[s][0] : (float)((double)a.s_a[(long)it.e * a.H + row] * v[s][0]);
                a.ye[pair * a.H + row] = out;
            }
        }
    }
}

// Gate/up chunking per token capacity: rows per chunk keep registers bounded.
template <int NT> struct GemvTune;
template <> struct GemvTune<1> { static constexpr int RC = 4, RD = 8; };
template <> struct GemvTune<2> { static constexpr int RC = 4, RD = 8; };
template <> struct GemvTune<4> { static constexpr int RC = 2, RD = 4; };
template <> struct GemvTune<8> { static constexpr int RC = 2, RD = 2; };

// The same per weight format: an int8 row block is twice the bytes, so a
// chunk holds half the rows, except with 4 or more slots, where one int8
// row per chunk leaves too few bytes in flight for the long dot-product
// work of a chunk (two rows: 68 -> 51 us per 151 MB gate/up pass at 8
// slots, dense T=4 59 -> 56 us).
template <int NT, int WB> struct GemvTuneW {
    static constexpr int RC = WB == 8 ? (NT >= 4 ? 2 : (GemvTune<NT>::RC > 1 ? GemvTune<NT>::RC / 2 : 1))
                                      : GemvTune<NT>::RC;
    static constexpr int RD = WB == 8 ? (GemvTune<NT>::RD > 1 ? GemvTune<NT>::RD / 2 : 1) : GemvTune<NT>::RD;
};

} // namespace coli
