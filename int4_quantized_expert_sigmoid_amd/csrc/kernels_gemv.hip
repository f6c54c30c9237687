// kernels_gemv.hip — the standalone token-GEMV expert kernels (T <= 8): one
// launch for gate/up + SwiGLU + Q8(h), one for the down projection. The
// device bodies are in gemv_device.hpp.
#include "gemv_device.hpp"
#include "internal.hpp"

namespace coli {
namespace {

template <int NT, int WB, bool GS>
__global__ void __launch_bounds__(256) k_gateup_gemv(GemvArgs a)
{
    __shared__ GateUpShared<NT> sh;
    const int nrb = a.I / QK;
    const int item = a.item0 + (int)blockIdx.x / nrb, rb = blockIdx.x % nrb;
    // the grid covers every item a union can have, so the table entry is in
    // bounds: read it together with the item count (one round trip; the
    // empty asm keeps the compiler from sinking the entry's loads past the
    // exit test)
    const int n_items = a.ctrl[CTRL_N_ITEMS];
    const ItemDesc it = item_from_table(a, item);
    asm volatile("" ::"s"(n_items), "s"(it.e), "s"(it.nt));
    if (item >= n_items) return;
    gateup_rows<NT, GemvTuneW<NT, WB>::RC, 1, WB, GS>(a, it, rb, sh);
}

template <int NT, int WB, bool GS>
__global__ void __launch_bounds__(256) k_down_gemv(GemvArgs a)
{
    const int ngrp = a.H / QK;
    const int item = a.item0 + (int)blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    if (a.has_shared && item == 0) {            // the shared expert exists whatever the routing:
        down_rows<NT, GemvTuneW<NT, WB>::RD, 8, WB, GS>(a, shared_item(a), grp);   // no table wait
        return;
    }
    const int n_items = a.ctrl[CTRL_N_ITEMS];   // with the entry in one round trip, as above
    const ItemDesc it = item_from_table(a, item);
    asm volatile("" ::"s"(n_items), "s"(it.e), "s"(it.nt));
    if (item >= n_items) return;
    down_rows<NT, GemvTuneW<NT, WB>::RD, 8, WB, GS>(a, it, grp);
}

template <int WB, bool GS = false>
void launch_gateup_wb(int T, dim3 grid, dim3 block, const GemvArgs &a, hipStream_t s)
{
    if (T <= 1) COLI_LAUNCH((k_gateup_gemv<1, WB, GS>), grid, block, 0, s, a);
    else if (T <= 2) COLI_LAUNCH((k_gateup_gemv<2, WB, GS>), grid, block, 0, s, a);
    else if (T <= 4) COLI_LAUNCH((k_gateup_gemv<4, WB, GS>), grid, block, 0, s, a);
    else COLI_LAUNCH((k_gateup_gemv<8, WB, GS>), grid, block, 0, s, a);
}

template <int WB, bool GS = false>
void launch_down_wb(int T, dim3 grid, const GemvArgs &a, hipStream_t s)
{
    if (T <= 1) COLI_LAUNCH((k_down_gemv<1, WB, GS>), grid, dim3(256), 0, s, a);
    else if (T <= 2) COLI_LAUNCH((k_down_gemv<2, WB, GS>), grid, dim3(256), 0, s, a);
    else if (T <= 4) COLI_LAUNCH((k_down_gemv<4, WB, GS>), grid, dim3(256), 0, s, a);
    else COLI_LAUNCH((k_down_gemv<8, WB, GS>), grid, dim3(256), 0, s, a);
}

GemvArgs make_args(const coli_moe_layer &L, const WsLayout &lay, char *ws)
{
    GemvArgs a;
    a.H = L.H; a.I = L.I; a.E = L.E; a.T = lay.T; a.has_shared = L.has_shared; a.item0 = 0;
    a.gsh = group_shift(L);
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

hipError_t launch_gateup_gemv(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, int item0,
                              hipStream_t s)
{
    GemvArgs a = make_args(L, lay, ws);
    a.item0 = item0;
    a.q_a = L.gate_q; a.s_a = L.gate_s; a.q_b = L.up_q; a.s_b = L.up_s;
    const int nblk = L.H / QK;
    const int threads = ((nblk + 63) / 64) * 64;
    const dim3 grid((unsigned)((lay.max_items - item0) * (L.I / QK)));
    if (L.group_size) launch_gateup_wb<4, true>(T, grid, dim3(threads), a, s);
    else if (L.weight_bits == 2) launch_gateup_wb<2>(T, grid, dim3(threads), a, s);
    else if (L.weight_bits == 8) launch_gateup_wb<8>(T, grid, dim3(threads), a, s);
    else launch_gateup_wb<4>(T, grid, dim3(threads), a, s);
    return hipGetLastError();
}

hipError_t launch_down_gemv(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, int item0,
                            hipStream_t s)
{
    GemvArgs a = make_args(L, lay, ws);
    a.item0 = item0;
    a.q_a = L.down_q; a.s_a = L.down_s; a.q_b = nullptr; a.s_b = nullptr;
    const dim3 grid((unsigned)((lay.max_items - item0) * (L.H / QK)));
    if (L.group_size) launch_down_wb<4, true>(T, grid, a, s);
    else if (L.weight_bits == 2) launch_down_wb<2>(T, grid, a, s);
    else if (L.weight_bits == 8) launch_down_wb<8>(T, grid, a, s);
    else launch_down_wb<4>(T, grid, a, s);
    return hipGetLastError();
}

} // namespace coli
