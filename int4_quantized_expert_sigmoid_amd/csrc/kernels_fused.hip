// kernels_fused.hip — the whole decode/verify layer (T <= 8) in one
// persistent launch.
//
// Same arithmetic as the staged kernels (route_device.hpp, gemv_device.hpp):
// router logits and top-k with the batch union (colibri README zh-TW, "how it
// works"), the IDOT gate/up + SwiGLU + Q8(h) and down projections (colibri
// architecture overview, sections 3.1 and 5), and the combine with the shared
// expert. What changes is scheduling. The work items are numbered
//   [logits, one expert each] [shared gate/up: I/32] [shared down: H/DG]
//   [top-k + union] [routed gate/up: U*I/32] [routed down: U*H/DG]
// (U = distinct routed experts of the batch, known once the union is built;
// DG = 96 down rows per item when H allows) and workgroup w takes items w,
// w + G, w + 2G, ... in that order, so the
// shared expert streams while the router runs and no launch gaps sit between
// the stages. An item waits only for items with smaller numbers; with all G
// workgroups resident (G is sized from the occupancy of this kernel) the
// smallest unfinished item always has its inputs, so the schedule progresses.
// Waits are bounded: past the spin limit a workgroup sets the error word and
// goes on (wrong output, no hang).
//
// Every value one workgroup hands to another (logits, routing, hq/hs, ye)
// moves through device-coherent relaxed loads/stores; completion counters are
// bumped after a workgroup barrier that waits for those stores. This avoids
// agent-scope fences, whose L2 writeback/invalidate across the chip's XCDs
// costs tens of microseconds per use. Q8(x) is recomputed from x inside each
// gate/up item. The down item that completes a row group last (counted over
// all items) combines that row group for every token; the last workgroup to
// leave (counted per group of workgroups, then overall) zeroes the counters.
#include "gemv_device.hpp"
#include "route_device.hpp"
#include "sync_device.hpp"
#include "internal.hpp"

#include <algorithm>

namespace coli {
namespace {

constexpr int LOGIT_EXPERTS = 1;        // experts per logits item
constexpr int LOGIT_COUNTERS = 8;       // logits completions are counted on 8 words
constexpr int EXIT_GROUPS = 8;

struct FusedArgs {
    GemvArgs gu, dn;
    SelArgs sel;
    const float *router_w;
    double *z;
    float *y;
    int accumulate;
    FusedSync *sync;
    int T, H, I, E, top_k, has_shared;
    int nrb, ndg, dg, n_logit_items, max_items;
    int t_sgu, t_sdn, t_sel, t_rgu;
#ifdef COLI_TRACE
    unsigned long long *trace;          // [total][4]: workgroup, start, end, XCC (profiling builds only)
#endif
};

// y rows [g*dg, g*dg+dg) of every token: sum_j w_tj * ye[pair(t,j)] + ye[shared pair],
// f64 in j order. Routing words are staged in LDS first so the ye loads of
// all terms are issued together.
__device__ void combine_rows(const FusedArgs &a, int g, int *pr, float *wr)
{
    const int n = a.T * a.top_k;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        pr[i] = ld_dev(a.sel.pair_of + i);
        wr[i] = ld_dev(a.sel.w + i);
    }
    for (int t = threadIdx.x; t < a.T; t += blockDim.x) pr[n + t] = a.has_shared ? ld_dev(a.sel.shared_pair + t) : 0;
    __syncthreads();
    for (int i = threadIdx.x; i < a.T * a.dg; i += blockDim.x) {
        const int t = i / a.dg;
        const long r = (long)g * a.dg + (i % a.dg);
        float yv[COLI_MAX_TOPK + 1];
#pragma unroll
        for (int j = 0; j < COLI_MAX_TOPK; ++j)
            yv[j] = j < a.top_k ? ld_dev(a.dn.ye + (long)pr[t * a.top_k + j] * a.H + r) : 0.0f;
        yv[COLI_MAX_TOPK] = a.has_shared ? ld_dev(a.dn.ye + (long)pr[n + t] * a.H + r) : 0.0f;
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < COLI_MAX_TOPK; ++j)
            if (j < a.top_k) acc += (double)wr[t * a.top_k + j] * (double)yv[j];
        if (a.has_shared) acc += (double)yv[COLI_MAX_TOPK];
        const float out = (float)acc;
        float *dst = a.y + (long)t * a.H + r;
        *dst = a.accumulate ? __fadd_rn(*dst, out) : out;
    }
}

// Down rows of one row group (dg = 96 rows, or 32 when H is not a multiple of 96).
template <int NT>
__device__ __forceinline__ void down_group(const FusedArgs &a, const ItemDesc &it, int g)
{
    if (a.dg == 96) down_rows<NT, GemvTune<NT>::RD, true, 24>(a.dn, it, g);
    else down_rows<NT, GemvTune<NT>::RD, true, 8>(a.dn, it, g);
}

template <int NT>
__global__ void __launch_bounds__(256, NT == 1 ? 3 : 2) k_decode_fused(FusedArgs a)
{
    // phases reuse one dynamic LDS block sized at launch (fused_lds_bytes)
    extern __shared__ double dyn_lds[];
    char *lds = reinterpret_cast<char *>(dyn_lds);
    GateUpShared<NT> &lds_gu = *reinterpret_cast<GateUpShared<NT> *>(lds);
    double *lds_red = dyn_lds;
    int *cmb_pr = reinterpret_cast<int *>(lds);
    float *cmb_wr = reinterpret_cast<float *>(cmb_pr + a.T * (a.top_k + 1));
    __shared__ int flag;
    FusedSync *sy = a.sync;
    constexpr int RC = GemvTune<NT>::RC;

    int n_routed = -1;                                            // known after the union
    for (int cur = blockIdx.x;; cur += gridDim.x) {
#ifdef COLI_TRACE
        const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();
#endif
        if (cur < a.t_sgu) {                                      // router logits
            const int e0 = cur * LOGIT_EXPERTS;
            for (int e = e0; e < e0 + LOGIT_EXPERTS && e < a.E; ++e)
                logits_expert<NT>(a.router_w, a.gu.x, a.T, a.H, a.E, e, a.z, lds_red);
            signal_add(&sy->logits_done[cur % LOGIT_COUNTERS]);
        } else if (cur < a.t_sdn) {                               // shared expert gate/up
            gateup_rows<NT, RC, true, true>(a.gu, shared_item(a.gu), cur - a.t_sgu, lds_gu);
            signal_add(&sy->gu_done[0]);
        } else if (cur < a.t_sel) {                               // shared expert down
            const int g = cur - a.t_sdn;
            wait_ge(&sy->gu_done[0], (unsigned)a.nrb, &sy->err);
            down_group<NT>(a, shared_item(a.dn), g);
            const unsigned old = signal_add(&sy->dn_done[g]);
            if (threadIdx.x == 0) {
                // while the router runs, routed down items are pending: this is not the last
                const bool routed = ld_counter(&sy->select_done) != 0u;
                flag = routed && (int)(old + 1) == ld_dev(a.gu.ctrl + CTRL_N_ITEMS);
            }
            __syncthreads();
            if (flag) combine_rows(a, g, cmb_pr, cmb_wr);
        } else if (cur < a.t_rgu) {                               // top-k and union
            {
                unsigned tgt[LOGIT_COUNTERS];
#pragma unroll
                for (int c = 0; c < LOGIT_COUNTERS; ++c)
                    tgt[c] = (unsigned)((a.n_logit_items - c + LOGIT_COUNTERS - 1) / LOGIT_COUNTERS);
                wait_all_ge(sy->logits_done, tgt, LOGIT_COUNTERS, &sy->err);
            }
            SelShared ss = sel_view(lds, a.T, a.E, a.top_k, a.sel.n_group);
            UnionShared uu = union_view(lds + sel_lds_bytes(a.T, a.E, a.top_k, a.sel.n_group), a.T, a.E,
                                              a.top_k);
            select_tokens_block(a.sel, 0, a.T, ss);
            routing_to_union(a.sel, ss, uu);
            build_union(a.sel, uu);
            signal_add(&sy->select_done);
        } else {
            if (n_routed < 0) {
                wait_ge(&sy->select_done, 1u, &sy->err);
                n_routed = ld_dev(a.gu.ctrl + CTRL_N_ITEMS) - a.has_shared;
            }
            const int j = cur - a.t_rgu;
            if (j >= n_routed * (a.nrb + a.ndg)) break;
            if (j < n_routed * a.nrb) {                           // routed gate/up
                const int item = a.has_shared + j / a.nrb;
                gateup_rows<NT, RC, true, true>(a.gu, item_from_union(a.gu, item), j % a.nrb, lds_gu);
                signal_add(&sy->gu_done[item]);
            } else {                                              // routed down
                const int jd = j - n_routed * a.nrb;
                const int item = a.has_shared + jd / a.ndg, g = jd % a.ndg;
                wait_ge(&sy->gu_done[item], (unsigned)a.nrb, &sy->err);
                down_group<NT>(a, item_from_union(a.dn, item), g);
                const unsigned old = signal_add(&sy->dn_done[g]);
                if (threadIdx.x == 0) flag = (int)(old + 1) == n_routed + a.has_shared;
                __syncthreads();
                if (flag) combine_rows(a, g, cmb_pr, cmb_wr);
            }
        }
        __syncthreads();
#ifdef COLI_TRACE
        if (threadIdx.x == 0 && a.trace) {
            a.trace[4 * cur] = blockIdx.x;
            a.trace[4 * cur + 1] = t_start;
            a.trace[4 * cur + 2] = __builtin_amdgcn_s_memrealtime();
            a.trace[4 * cur + 3] = __builtin_amdgcn_s_getreg((3 << 11) | 20);   // XCC id (4 bits)
        }
#endif
    }
    // leave: the last of each group of workgroups counts the group out, the
    // last group zeroes the counters for the next call
    if (threadIdx.x == 0) {
        const int grp = blockIdx.x % EXIT_GROUPS;
        const unsigned gsize = (gridDim.x - grp + EXIT_GROUPS - 1) / EXIT_GROUPS;
        const unsigned ngroups = gridDim.x < EXIT_GROUPS ? gridDim.x : EXIT_GROUPS;
        flag = 0;
        if (__hip_atomic_fetch_add(&sy->exits[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == gsize)
            flag = __hip_atomic_fetch_add(&sy->exits_all, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1
                   == ngroups;
    }
    __syncthreads();
    if (flag) {
        const unsigned z0 = 0;
        if (threadIdx.x < EXIT_GROUPS)
            __hip_atomic_store(&sy->exits[threadIdx.x], z0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) {
            __hip_atomic_store(&sy->exits_all, z0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int c = 0; c < LOGIT_COUNTERS; ++c)
                __hip_atomic_store(&sy->logits_done[c], z0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&sy->select_done, z0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (int i = threadIdx.x; i < a.max_items; i += blockDim.x)
            __hip_atomic_store(&sy->gu_done[i], z0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = threadIdx.x; i < a.ndg; i += blockDim.x)
            __hip_atomic_store(&sy->dn_done[i], z0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Persistent grid: every workgroup resident at once (occupancy of the kernel
// instance times the compute units; both cached per device).
int grid_size(const void *kernel, int nt_slot, int total, size_t lds)
{
    static int cus[64], occ[64][4];
    static size_t occ_lds[64][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    if (occ[dev][nt_slot] == 0 || occ_lds[dev][nt_slot] != lds) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel, 256, lds) != hipSuccess || b <= 0) b = 1;
        occ[dev][nt_slot] = b;
        occ_lds[dev][nt_slot] = lds;
    }
    const int g = cus[dev] * occ[dev][nt_slot];
    return total < g ? total : g;
}

} // namespace

#ifdef COLI_TRACE
static unsigned long long *g_trace = nullptr;
extern "C" void coli_trace_set(void *p) { g_trace = static_cast<unsigned long long *>(p); }
#endif

hipError_t launch_decode_fused(const coli_moe_layer &L, const float *x, int T, const WsLayout &lay, char *ws,
                               float *y, bool accumulate, hipStream_t s)
{
    FusedArgs a;
    // gate/up and down views of the GEMV arguments
    GemvArgs g;
    g.H = L.H; g.I = L.I; g.E = L.E; g.T = T; g.has_shared = L.has_shared; g.gsh = 0; g.item0 = 0;
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
    a.gu = g; a.gu.q_a = L.gate_q; a.gu.s_a = L.gate_s; a.gu.q_b = L.up_q; a.gu.s_b = L.up_s;
    a.dn = g; a.dn.q_a = L.down_q; a.dn.s_a = L.down_s; a.dn.q_b = nullptr; a.dn.s_b = nullptr;
    SelArgs &sa = a.sel;
    sa.z = reinterpret_cast<const double *>(ws + lay.logits);
    sa.bias = L.router_b;
    sa.T = T; sa.E = L.E; sa.top_k = L.top_k; sa.n_group = L.n_group; sa.topk_group = L.topk_group;
    sa.has_shared = L.has_shared; sa.route_scale = L.route_scale;
    sa.given_idx = nullptr; sa.given_w = nullptr;
    sa.idx = reinterpret_cast<int32_t *>(ws + lay.idx); sa.idx_user = nullptr;
    sa.w = reinterpret_cast<float *>(ws + lay.w); sa.w_user = nullptr;
    sa.ctrl = reinterpret_cast<int *>(ws + lay.ctrl);
    sa.item_expert = reinterpret_cast<int *>(ws + lay.item_expert);
    sa.item_ntok = reinterpret_cast<int *>(ws + lay.item_ntok);
    sa.item_tok = reinterpret_cast<int *>(ws + lay.item_tok);
    sa.pair_of = reinterpret_cast<int *>(ws + lay.pair_of);
    sa.shared_pair = reinterpret_cast<int *>(ws + lay.shared_pair);
    a.gu.x = x; a.dn.x = x;
    a.router_w = L.router_w;
    a.z = reinterpret_cast<double *>(ws + lay.logits);
    a.y = y; a.accumulate = accumulate ? 1 : 0;
    a.sync = reinterpret_cast<FusedSync *>(ws + lay.sync);
    a.T = T; a.H = L.H; a.I = L.I; a.E = L.E; a.top_k = L.top_k; a.has_shared = L.has_shared;
    const int max_routed = T * L.top_k;
    a.dg = (L.H % 96 == 0) ? 96 : 32;
    a.nrb = L.I / QK; a.ndg = L.H / a.dg; a.max_items = lay.max_items;
    a.n_logit_items = (L.E + LOGIT_EXPERTS - 1) / LOGIT_EXPERTS;
    a.t_sgu = a.n_logit_items;
    a.t_sdn = a.t_sgu + (L.has_shared ? a.nrb : 0);
    a.t_sel = a.t_sdn + (L.has_shared ? a.ndg : 0);
    a.t_rgu = a.t_sel + 1;
    // enough workgroups for the largest possible union; the rest leave at once
    const int total = a.t_rgu + max_routed * (a.nrb + a.ndg);
#ifdef COLI_TRACE
    a.trace = g_trace;
#endif
    const int ntc = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
    size_t lds = sel_lds_bytes(T, L.E, L.top_k, L.n_group) + union_lds_bytes(T, L.E, L.top_k);
    lds = std::max(lds, (size_t)4 * 64 * ntc * 8);                      // gate/up partials
    lds = std::max(lds, (size_t)T * (L.top_k + 1) * 4 + (size_t)T * L.top_k * 4);   // combine
    lds = (lds + 15) & ~(size_t)15;
    if (T <= 1) {
        COLI_LAUNCH(k_decode_fused<1>, dim3(grid_size((const void *)k_decode_fused<1>, 0, total, lds)),
                           dim3(256), lds, s, a);
    } else if (T <= 2) {
        COLI_LAUNCH(k_decode_fused<2>, dim3(grid_size((const void *)k_decode_fused<2>, 1, total, lds)),
                           dim3(256), lds, s, a);
    } else if (T <= 4) {
        COLI_LAUNCH(k_decode_fused<4>, dim3(grid_size((const void *)k_decode_fused<4>, 2, total, lds)),
                           dim3(256), lds, s, a);
    } else {
        COLI_LAUNCH(k_decode_fused<8>, dim3(grid_size((const void *)k_decode_fused<8>, 3, total, lds)),
                           dim3(256), lds, s, a);
    }
    return hipGetLastError();
}

} // namespace coli
