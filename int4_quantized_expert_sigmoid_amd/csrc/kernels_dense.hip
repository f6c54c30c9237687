// kernels_dense.hip — the dense SwiGLU MLP of the first layers (colibri
// architecture overview, section 4: dense_mlp ahead of the MoE layers), with
// the experts' numerics: Q8 activations in 32-wide blocks, int4 or int8
// weight rows with one f32 scale each, exact int32 block dots summed in f64
// (section 3.1), y_t = W_down (Q8(silu(W_gate Q8(x_t)) * (W_up Q8(x_t)))).
// Every token goes through it; there is no routing.
//
// T <= 8: the token-GEMV gate/up body of the expert path (one item, the T
// tokens as its slots) and k_dense_down, a GEMV over the H down rows whose
// threads own one (or, at one slot, two) block columns of every row (up to
// 8 waves: the intermediate size can exceed one wave's 64 columns). T > 8: the grouped MFMA kernels of the expert path
// over one "expert" holding all T tokens, then k_dense_out.
#include "gemv_device.hpp"
#include "internal.hpp"

namespace coli {
namespace {

// Gate/up rows [rb*32, rb*32+32) for the T tokens + SwiGLU + Q8(h).
template <int NT, int WB>
__global__ void __launch_bounds__(256) k_dense_gateup(GemvArgs a)
{
    __shared__ GateUpShared<NT> sh;
    ItemDesc it;
    it.item = 0;
    it.e = 0;
    it.nt = a.T;
#pragma unroll
    for (int s = 0; s < MAX_SLOTS; ++s) it.tok[s] = s;
    gateup_rows<NT, GemvTuneW<NT, WB>::RC, 1, WB>(a, it, blockIdx.x, sh);
}

struct DenseDnArgs {
    const uint8_t *q;          // down rows [H][I/2] (int4) or [H][I] (int8)
    const float *s;            // [H]
    const int8_t *hq;          // [T][I] reordered Q8(h)
    const float *hs;           // [T][I/32]
    float *y;                  // [T][H]
    int H, I, T, accumulate;
};

constexpr int DD_ROWS = 8;     // down rows per workgroup
constexpr int DD_WAVES = 8;    // at most: I/32 <= 512 block columns

// Down rows [blockIdx*8, +8). Thread c owns block columns c, c + blockDim,
// ... (CPT of them) of every row, with the activations of those columns for
// the T slots in registers; rows stream in chunks of RC with the next
// chunk's loads in flight. Per-row partials: a transposing wave reduction,
// then the waves in order through LDS.
template <int NT, int WB, int CPT, int RC>
__global__ void __launch_bounds__(64 * DD_WAVES) k_dense_down(DenseDnArgs a)
{
    constexpr int NP = WFmt<WB>::BLK_BYTES / 16;
    constexpr double KS = WFmt<WB>::KSCALE;
    constexpr int NC = DD_ROWS / RC;
    static_assert(DD_ROWS % RC == 0, "whole chunks");
    __shared__ double red[DD_WAVES][NT][DD_ROWS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nblk = a.I / QK;
    const long rowb = (long)a.I * WB / 8;
    const long row0 = (long)blockIdx.x * DD_ROWS;
    const int ntu = __builtin_amdgcn_readfirstlane(a.T);

    Blk8 act[CPT][NT];
    float ds[CPT][NT];
    bool active[CPT];
    const uint8_t *pw[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int col = tid + (int)blockDim.x * k;
        active[k] = col < nblk;
        pw[k] = a.q + row0 * rowb + blk_off<WB>(active[k] ? col : 0);
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            if (s < a.T && active[k]) {
                act[k][s] = load_blk8(a.hq + (long)s * a.I + col * QK);
                ds[k][s] = a.hs[(long)s * nblk + col];
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) act[k][s].v[j] = 0;
                ds[k][s] = 0.0f;
            }
        }
    }
    uint4 w[2][RC][CPT][NP];
#pragma unroll
    for (int r = 0; r < RC; ++r)
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int q = 0; q < NP; ++q) w[0][r][k][q] = load_u4_stream(pw[k] + (long)r * rowb + piece_off<WB>(q, nblk));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int cur = c & 1;
        if (c + 1 < NC) {
#pragma unroll
            for (int r = 0; r < RC; ++r)
#pragma unroll
                for (int k = 0; k < CPT; ++k)
#pragma unroll
                    for (int q = 0; q < NP; ++q)
                        w[cur ^ 1][r][k][q] = load_u4_stream(pw[k] + (long)((c + 1) * RC + r) * rowb + piece_off<WB>(q, nblk));
        }
        double v[NT][RC];
#pragma unroll
        for (int r = 0; r < RC; ++r) {
#pragma unroll
            for (int s = 0; s < NT; ++s) {
                if (s > 0 && s >= ntu) break;            // slot 0 is always in use
                double acc = 0.0;
#pragma unroll
                for (int k = 0; k < CPT; ++k)
                    acc += (double)dot_block_w<WB>(w[cur][r][k], act[k][s]) * ((double)ds[k][s] * KS);
                v[s][r] = acc;
            }
        }
        const int vi = transpose_index<RC>(lane);
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            if (s > 0 && s >= ntu) break;
            wave_transpose_reduce<RC>(v[s]);
            if ((lane & (64 / RC - 1)) == 0) red[wave][s][c * RC + vi] = v[s][0];
        }
    }
    __syncthreads();
    const int nw = (int)(blockDim.x >> 6);      // every wave owns columns
    for (int i = tid; i < NT * DD_ROWS; i += blockDim.x) {
        const int s = i / DD_ROWS, r = i % DD_ROWS;
        if (s >= a.T) continue;
        double acc = red[0][s][r];
        for (int wv = 1; wv < nw; ++wv) acc += red[wv][s][r];
        const long row = row0 + r;
        const float out = (float)((double)a.s[row] * acc);
        const long o = (long)s * a.H + row;
        a.y[o] = a.accumulate ? __fadd_rn(a.y[o], out) : out;
    }
}

// Grouped-path bookkeeping for one expert holding all T tokens: pair p is
// token p, tiles of 32 pairs.
__global__ void k_dense_setup(int *ctrl, int2 *tiles, int *expert_off, int *pair_tok, int T)
{
    const int ntiles = (T + 31) / 32;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < T; i += gridDim.x * blockDim.x) {
        pair_tok[i] = i;
        if (i < ntiles) tiles[i] = make_int2(0, 32 * i);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctrl[CTRL_N_TILES_GU] = ntiles;
        ctrl[CTRL_N_TILES_DN] = ntiles;
        expert_off[0] = 0;
        expert_off[1] = T;
    }
}

// y = ye (or y += ye), pair p = token p.
__global__ void k_dense_out(const float *__restrict__ ye, float *__restrict__ y, long n, int accumulate)
{
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
        y[i] = accumulate ? __fadd_rn(y[i], ye[i]) : ye[i];
}

template <int NT, int WB>
void launch_dense_down_nt(const DenseDnArgs &d, hipStream_t s)
{
    const dim3 grid((unsigned)(d.H / DD_ROWS));
    const int nblk = d.I / QK;                   // <= 512 (I <= 16384)
    constexpr int RC = NT <= 2 ? 4 : (NT <= 4 ? 2 : 1);
    // one slot: four waves with a second column for the blocks past 256
    // (measured a little faster there); more slots: one column per thread,
    // as many waves as the blocks need (fewer registers per thread)
    if constexpr (NT == 1) {
        if (nblk > 256) {
            COLI_LAUNCH((k_dense_down<NT, WB, 2, RC>), grid, dim3(256), 0, s, d);
            return;
        }
    }
    COLI_LAUNCH((k_dense_down<NT, WB, 1, RC>), grid, dim3((unsigned)(64 * ((nblk + 63) / 64))), 0, s, d);
}

template <int WB>
void launch_dense_gemv_wb(const DenseLayer &M, int T, const GemvArgs &g, const DenseDnArgs &d, hipStream_t s)
{
    const dim3 grid((unsigned)(M.I / QK));
    if (T <= 1) { COLI_LAUNCH((k_dense_gateup<1, WB>), grid, dim3(256), 0, s, g); launch_dense_down_nt<1, WB>(d, s); }
    else if (T <= 2) { COLI_LAUNCH((k_dense_gateup<2, WB>), grid, dim3(256), 0, s, g); launch_dense_down_nt<2, WB>(d, s); }
    else if (T <= 4) { COLI_LAUNCH((k_dense_gateup<4, WB>), grid, dim3(256), 0, s, g); launch_dense_down_nt<4, WB>(d, s); }
    else { COLI_LAUNCH((k_dense_gateup<8, WB>), grid, dim3(256), 0, s, g); launch_dense_down_nt<8, WB>(d, s); }
}

} // namespace

hipError_t launch_dense_gemv(const DenseLayer &M, int T, int t0, const DenseLayout &lay, char *ws, float *y,
                             bool accumulate, hipStream_t s)
{
    const long t = t0;
    GemvArgs g;
    g.q_a = M.gate_q; g.s_a = M.gate_s; g.q_b = M.up_q; g.s_b = M.up_s;
    g.H = M.H; g.I = M.I; g.E = 0; g.T = T; g.has_shared = 0; g.gsh = 0; g.item0 = 0;
    g.xq = reinterpret_cast<const int8_t *>(ws + lay.xq) + t * M.H;
    g.xs = reinterpret_cast<const float *>(ws + lay.xs) + t * (M.H / QK);
    g.ctrl = nullptr; g.item_expert = nullptr; g.item_ntok = nullptr; g.item_tok = nullptr;
    g.h = reinterpret_cast<float *>(ws + lay.h) + t * M.I;
    g.hq = reinterpret_cast<int8_t *>(ws + lay.hq) + t * M.I;
    g.hs = reinterpret_cast<float *>(ws + lay.hs) + t * (M.I / QK);
    g.ye = nullptr;
    DenseDnArgs d;
    d.q = M.down_q; d.s = M.down_s;
    d.hq = g.hq; d.hs = g.hs; d.y = y + t * M.H;
    d.H = M.H; d.I = M.I; d.T = T; d.accumulate = accumulate ? 1 : 0;
    if (M.weight_bits == 8) launch_dense_gemv_wb<8>(M, T, g, d, s);
    else launch_dense_gemv_wb<4>(M, T, g, d, s);
    return hipGetLastError();
}

hipError_t launch_dense_setup(int T, const DenseLayout &lay, char *ws, hipStream_t s)
{
    COLI_LAUNCH(k_dense_setup, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s,
                reinterpret_cast<int *>(ws + lay.ctrl), reinterpret_cast<int2 *>(ws + lay.tiles),
                reinterpret_cast<int *>(ws + lay.expert_off), reinterpret_cast<int *>(ws + lay.pair_tok), T);
    return hipGetLastError();
}

hipError_t launch_dense_out(int T, int H, const DenseLayout &lay, const char *ws, float *y, bool accumulate,
                            hipStream_t s)
{
    const long n = (long)T * H;
    long blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    COLI_LAUNCH(k_dense_out, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float *>(ws + lay.ye), y,
                n, accumulate ? 1 : 0);
    return hipGetLastError();
}

} // namespace coli
