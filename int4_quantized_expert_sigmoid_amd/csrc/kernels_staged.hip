// kernels_staged.hip — the two decode launches (T <= 8) that also carry the
// always-on shared expert (colibri architecture overview, section 5: every
// token goes through the shared expert; it needs no routing decision):
//   launch 1: router logits + Q8(x) (one workgroup per expert) and, beside
//             them, the shared expert's gate/up + SwiGLU + Q8(h), which
//             quantises x itself;
//   launch 2: top-k + batch union (one workgroup) and, beside it, the shared
//             expert's down projection.
// The routed experts then follow in their own gate/up and down launches, so
// the shared expert's 19 MB stream while the router runs.
#include "gemv_device.hpp"
#include "route_device.hpp"
#include "internal.hpp"

namespace coli {
namespace {

template <int NT>
__global__ void __launch_bounds__(256) k_route_shared_gu(const float *__restrict__ W, const float *__restrict__ x,
                                                         int T, int H, int E, double *__restrict__ z,
                                                         int8_t *__restrict__ xq, float *__restrict__ xs,
                                                         GemvArgs g)
{
    __shared__ GateUpShared<NT> sh;
    if ((int)blockIdx.x < E) {
        const long nb = (long)T * (H / QK);
        for (long b = (long)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (long)E * blockDim.x)
            q8_block_reordered(x + b * QK, xq + b * QK, xs + b);
        logits_expert<NT>(W, x, T, H, E, blockIdx.x, z, &sh.red[0][0][0]);
    } else {
        // quantising x in registers costs VGPRs: the widest slot count takes one row per chunk
        constexpr int RC = NT >= 8 ? 1 : GemvTune<NT>::RC;
        gateup_rows<NT, RC, true, false>(g, shared_item(g), (int)blockIdx.x - E, sh);
    }
}

template <int NT>
__global__ void __launch_bounds__(256) k_select_shared_dn(SelArgs a, GemvArgs g)
{
    extern __shared__ double dyn_lds[];
    if (blockIdx.x == 0) {
        char *lds = reinterpret_cast<char *>(dyn_lds);
        SelShared sh = sel_view(lds, a.T, a.E, a.top_k, a.n_group);
        UnionShared u = union_view(lds + sel_lds_bytes(a.T, a.E, a.top_k, a.n_group), a.T, a.E, a.top_k);
        select_tokens_block(a, 0, a.T, sh);
        routing_to_union(a, sh, u);
        build_union(a, u);
    } else {
        down_rows<NT, GemvTune<NT>::RD, false, 8>(g, shared_item(g), (int)blockIdx.x - 1);
    }
}

GemvArgs gemv_view(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws)
{
    GemvArgs g;
    g.H = L.H; g.I = L.I; g.E = L.E; g.T = T; g.item0 = 0; g.x = nullptr;
    g.xq = reinterpret_cast<const int8_t *>(ws + lay.xq);
    g.xs = reinterpret_cast<const float *>(ws + lay.xs);
    g.ctrl = reinterpret_cast<const int *>(ws + lay.ctrl);
    g.item_expert = reinterpret_cast<const int *>(ws + lay.item_expert);
    g.item_ntok = reinterpret_cast<const int *>(ws + lay.item_ntok);
    g.item_tok = reinterpret_cast<const int *>(ws + lay.item_tok);
    g.h = reinterpret_cast<float *>(ws + lay.h);
    g.hq = reinterpret_cast<int8_t *>(ws + lay.hq);
    g.hs = reinterpret_cast<float *>(ws + lay.hs);
    g.ye = reinterpret_cast<float *>(ws + lay.ye);
    return g;
}

} // namespace

hipError_t launch_route_shared_gateup(const coli_moe_layer &L, const float *x, int T, const WsLayout &lay,
                                      char *ws, hipStream_t s)
{
    GemvArgs g = gemv_view(L, T, lay, ws);
    g.x = x;
    g.q_a = L.gate_q; g.s_a = L.gate_s; g.q_b = L.up_q; g.s_b = L.up_s;
    double *z = reinterpret_cast<double *>(ws + lay.logits);
    int8_t *xq = reinterpret_cast<int8_t *>(ws + lay.xq);
    float *xs = reinterpret_cast<float *>(ws + lay.xs);
    const dim3 grid((unsigned)(L.E + (L.has_shared ? L.I / QK : 0)));
    if (T <= 1) hipLaunchKernelGGL(k_route_shared_gu<1>, grid, dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs, g);
    else if (T <= 2) hipLaunchKernelGGL(k_route_shared_gu<2>, grid, dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs, g);
    else if (T <= 4) hipLaunchKernelGGL(k_route_shared_gu<4>, grid, dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs, g);
    else hipLaunchKernelGGL(k_route_shared_gu<8>, grid, dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs, g);
    return hipGetLastError();
}

hipError_t launch_select_shared_down(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    GemvArgs g = gemv_view(L, T, lay, ws);
    g.q_a = L.down_q; g.s_a = L.down_s; g.q_b = nullptr; g.s_b = nullptr;
    SelArgs a;
    a.z = reinterpret_cast<const double *>(ws + lay.logits);
    a.bias = L.router_b;
    a.T = T; a.E = L.E; a.top_k = L.top_k; a.n_group = L.n_group; a.topk_group = L.topk_group;
    a.has_shared = L.has_shared; a.route_scale = L.route_scale;
    a.given_idx = nullptr; a.given_w = nullptr;
    a.idx = reinterpret_cast<int32_t *>(ws + lay.idx); a.idx_user = nullptr;
    a.w = reinterpret_cast<float *>(ws + lay.w); a.w_user = nullptr;
    a.ctrl = reinterpret_cast<int *>(ws + lay.ctrl);
    a.item_expert = reinterpret_cast<int *>(ws + lay.item_expert);
    a.item_ntok = reinterpret_cast<int *>(ws + lay.item_ntok);
    a.item_tok = reinterpret_cast<int *>(ws + lay.item_tok);
    a.pair_of = reinterpret_cast<int *>(ws + lay.pair_of);
    a.shared_pair = reinterpret_cast<int *>(ws + lay.shared_pair);
    const size_t lds = sel_lds_bytes(T, L.E, L.top_k, L.n_group) + union_lds_bytes(T, L.E, L.top_k);
    const dim3 grid((unsigned)(1 + (L.has_shared ? L.H / QK : 0)));
    if (T <= 1) hipLaunchKernelGGL(k_select_shared_dn<1>, grid, dim3(256), lds, s, a, g);
    else if (T <= 2) hipLaunchKernelGGL(k_select_shared_dn<2>, grid, dim3(256), lds, s, a, g);
    else if (T <= 4) hipLaunchKernelGGL(k_select_shared_dn<4>, grid, dim3(256), lds, s, a, g);
    else hipLaunchKernelGGL(k_select_shared_dn<8>, grid, dim3(256), lds, s, a, g);
    return hipGetLastError();
}

} // namespace coli
