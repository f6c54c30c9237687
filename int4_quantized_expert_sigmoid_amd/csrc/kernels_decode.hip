// kernels_decode.hip — the decode / verify layer (T <= 8) in three launches.
//
//   1. k_router: router logits z = W_r x, the selection keys s + b and
//      s = sigmoid(z), and Q8(x); one workgroup per expert.
//   2. k_select_gateup: the first workgroups run the shared expert's gate/up
//      + SwiGLU + Q8(h) (every token goes through it, so it needs no routing
//      decision: colibri architecture overview, section 5) and stream while
//      the others route. Each routed workgroup derives the top-k of every
//      token and the batch union from the keys (the same deterministic
//      computation in every workgroup), then runs the gate/up rows of its
//      routed expert. The first routed workgroup also publishes the routing
//      and the union for launch 3.
//   3. k_down_combine: each workgroup owns a few output rows of the down
//      projection for every item of the union (shared and routed; its waves
//      take the items round-robin), keeps the per-pair results in LDS and
//      combines them into y:
//      y_t = sum_j w_tj * y_{t,e_j} + y_{t,shared}, f64, in slot order.
//
// Batch union (colibri README zh-TW, "how it works"): every distinct expert
// of the batch is read once, for all of its tokens.
#ifdef COLI_TRACE
// selection phase marks of profiling builds: [workgroup][8] real-time stamps
__device__ unsigned long long *coli_sel_marks;
#define COLI_SEL_MARK(i)                                                                                        \
    do {                                                                                                        \
        if ((threadIdx.x & 63) == 0 && coli_sel_marks && blockIdx.x < 4096)                                     \
            coli_sel_marks[blockIdx.x * 8 + (i)] = __builtin_amdgcn_s_memrealtime();                            \
    } while (0)
#endif
#include "gemv_device.hpp"
#include "route_device.hpp"
#include "internal.hpp"

namespace coli {

#ifdef COLI_TRACE
// Profiling builds only: per-workgroup timestamps [launch][workgroup][4] =
// start, end of the first phase, end (100 MHz real-time counter), and the
// XCC id with the HW_ID register of the first wave in the upper 32 bits
// (its CU, shader array, shader engine and SIMD).
static unsigned long long *g_dec_trace = nullptr;
extern "C" void coli_trace_decode_set(void *p)
{
    g_dec_trace = static_cast<unsigned long long *>(p);
    unsigned long long *m = p ? g_dec_trace + 3 * 4096 * 4 : nullptr;   // marks follow the three launches
    (void)hipMemcpyToSymbol(HIP_SYMBOL(coli_sel_marks), &m, sizeof(m));
}
constexpr int TRACE_WG = 4096;
__device__ __forceinline__ void trace_mark(unsigned long long *tr, int launch, int slot)
{
    if (tr && threadIdx.x == 0 && blockIdx.x < TRACE_WG) {
        unsigned long long *p = tr + ((size_t)launch * TRACE_WG + blockIdx.x) * 4;
        p[slot] = __builtin_amdgcn_s_memrealtime();
        if (slot == 2)
            p[3] = (unsigned long long)__builtin_amdgcn_s_getreg((3 << 11) | 20) |
                   ((unsigned long long)__builtin_amdgcn_s_getreg((31 << 11) | 4) << 32);
    }
}
#define TRACE(args, launch, slot) trace_mark((args).trace, launch, slot)
#else
#define TRACE(args, launch, slot) ((void)0)
#endif

namespace {

// ------------------------------------------------------------ launch 1
struct RouterArgs {
    const float *W, *bias, *x;
    const float *gamma;        // RMSNorm gains of the norm-fused router (x is then the raw residual row)
    float eps;
    int vec;                   // rms_vec(x, H)
    int T, H, E;
    double *z, *key, *sig;
    int8_t *xq;
    float *xs;
#ifdef COLI_TRACE
    unsigned long long *trace;
#endif
};

template <int NT>
__global__ void __launch_bounds__(512) k_router(RouterArgs r)
{
    __shared__ double red[8 * NT];
    TRACE(r, 0, 0);
    // Q8(x): one block per half-wave, workgroup e taking blocks e, e + E, ...
    // (one each at T = 1), so no workgroup's logits wait behind all of them
    const long nb = (long)r.T * (r.H / QK);
    const int hw = (int)(threadIdx.x >> 5), hl = (int)(threadIdx.x & 31);
    for (long b = (long)blockIdx.x + (long)r.E * hw; b < nb; b += (long)r.E * (blockDim.x >> 5))
        q8_block_lanes(r.x[b * QK + hl], hl, r.xq + b * QK, r.xs + b);
    logits_expert<NT>(r.W, r.x, r.T, r.H, r.E, blockIdx.x, r.z, red, r.bias, r.key, r.sig);
    TRACE(r, 0, 2);
}

// Launch 1 with the chain's RMSNorm folded in: every workgroup takes the
// scales of the T raw rows itself (rms_scales, the order k_rmsnorm uses, so
// the normalised rows are the ones coli_rmsnorm writes), then the logits of
// its expert and its share of Q8 from the normalised rows. The workgroup's
// router row is loaded before the scales are taken, so the two loads
// overlap. Needs H <= 4 * RMS_BLOCK * 4.
constexpr int RN_PRE = 4;      // float4 of the router row per thread

template <int NT>
__global__ void __launch_bounds__(RMS_BLOCK) k_router_norm(RouterArgs r)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ double red[8 * NT];
    const int e = blockIdx.x, tid = threadIdx.x;
    TRACE(r, 0, 0);
    const int H4 = r.H / 4;
    const f32x4 *we = reinterpret_cast<const f32x4 *>(r.W + (long)e * r.H);
    f32x4 wp[RN_PRE];
#pragma unroll
    for (int j = 0; j < RN_PRE; ++j) {
        const int i = tid + j * RMS_BLOCK;
        wp[j] = i < H4 ? __builtin_nontemporal_load(&we[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double sc[NT];
    rms_scales<NT>(r.x, r.T, r.H, r.eps, r.vec != 0, red, sc);

    // Q8 of the normalised rows: one block per half-wave, workgroup e taking
    // blocks e, e + E, ... (one each at T = 1)
    const int nblk = r.H / QK;
    const long nb = (long)r.T * nblk;
    const int hw = tid >> 5, hl = tid & 31;
    for (long b = (long)e + (long)r.E * hw; b < nb; b += (long)r.E * (RMS_BLOCK >> 5)) {
        const int t = (int)(b / nblk), c0 = (int)(b % nblk) * QK;
        double st = sc[0];
#pragma unroll
        for (int k = 1; k < NT; ++k) st = t == k ? sc[k] : st;
        const float v = rms_apply(r.x[(long)t * r.H + c0 + hl], st, r.gamma[c0 + hl]);
        q8_block_lanes(v, hl, r.xq + b * QK, r.xs + b);
    }

    // logits of expert e from the normalised rows, summed in logits_expert's order
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
#pragma unroll
    for (int j = 0; j < RN_PRE; ++j) {
        const int h = tid + j * RMS_BLOCK;
        if (h < H4) {
            const float4 g = reinterpret_cast<const float4 *>(r.gamma)[h];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < r.T) {
                    const float4 xv = reinterpret_cast<const float4 *>(r.x + (long)t * r.H)[h];
                    acc[t] = fma((double)wp[j].x, (double)rms_apply(xv.x, sc[t], g.x), acc[t]);
                    acc[t] = fma((double)wp[j].y, (double)rms_apply(xv.y, sc[t], g.y), acc[t]);
                    acc[t] = fma((double)wp[j].z, (double)rms_apply(xv.z, sc[t], g.z), acc[t]);
                    acc[t] = fma((double)wp[j].w, (double)rms_apply(xv.w, sc[t], g.w), acc[t]);
                }
            }
        }
    }
    logits_finish<NT>(acc, r.T, r.E, e, r.z, red, r.bias, r.key, r.sig);
    TRACE(r, 0, 2);
}

// ------------------------------------------------------------ launch 2
struct SelGuArgs {
    const double *key, *sig;
    int T, E, top_k, n_group, topk_group, has_shared;
    float route_scale;
    // published by workgroup 0
    int32_t *idx;
    float *w;
    int *ctrl, *item_expert, *item_ntok, *item_tok, *pair_of, *shared_pair;
#ifdef COLI_TRACE
    unsigned long long *trace;
#endif
};

template <int KPL>
struct SelGuShared {
    DecUnion u;
    double kw[4][64 * KPL];    // each wave's copy of a token's keys (group scores)
};

template <int NT, int KPL, int WB, bool GS>
__global__ void __launch_bounds__(256) k_select_gateup(SelGuArgs a, GemvArgs g, int n_shared_wg, int n_routed_wg)
{
    __shared__ GateUpShared<NT> sh;
    __shared__ SelGuShared<KPL> su;
    TRACE(a, 1, 0);
    if ((int)blockIdx.x < n_shared_wg) {         // the shared expert: no routing needed
        gateup_rows<NT, GemvTuneW<NT, WB>::RC, 1, WB, GS>(g, shared_item(g), blockIdx.x, sh);
        TRACE(a, 1, 2);
        return;
    }
    const int b = (int)blockIdx.x - n_shared_wg;
    DecUnion &u = su.u;
    // only the publishing workgroup needs the routing weights
    dec_route_union<KPL>(a.key, a.sig, a.T, a.E, a.top_k, a.n_group, a.topk_group, a.route_scale, a.has_shared,
                         u, &su.kw[0][0], b == 0);
    TRACE(a, 1, 1);
    const int nrb = g.I / QK;
    const int n_items = u.n_items;
    if (b == 0) {
        const int tid = threadIdx.x, np = a.T * a.top_k;
        for (int i = tid; i < np; i += blockDim.x) {
            a.idx[i] = u.sel_e[i];
            a.w[i] = u.sel_w[i];
            a.pair_of[i] = u.pair_of[i];
        }
        for (int i = tid; i < n_items; i += blockDim.x) {
            a.item_expert[i] = u.item_e[i];
            a.item_ntok[i] = u.item_nt[i];
        }
        for (int i = tid; i < n_items * MAX_SLOTS; i += blockDim.x) {
            const int it = i / MAX_SLOTS, s = i % MAX_SLOTS;
            a.item_tok[i] = s < u.item_nt[it] ? u.item_tok[i] : 0;
        }
        if (a.has_shared)
            for (int t = tid; t < a.T; t += blockDim.x) a.shared_pair[t] = t;
        if (tid == 0) a.ctrl[CTRL_N_ITEMS] = n_items;
    }
    // The routed units (item, 32-row block) of the union, workgroup b taking
    // units b, b + n_routed_wg, ...: the grid is no larger than fits on the
    // chip at once, so no workgroup waits for another's slot, and none
    // routes only to find its item past the union (a batch of T tokens has
    // up to T * k items, usually far fewer). Uniform over the workgroup.
    const int n_units = (n_items - a.has_shared) * nrb;
    for (int un = b; un < n_units; un += n_routed_wg) {
        const int item = a.has_shared + un / nrb, rb = un % nrb;
        ItemDesc it;
        it.item = item;
        it.e = u.item_e[item];
        it.nt = u.item_nt[item];
#pragma unroll
        for (int s = 0; s < MAX_SLOTS; ++s) it.tok[s] = s < it.nt ? u.item_tok[item * MAX_SLOTS + s] : 0;
        gateup_rows<NT, GemvTuneW<NT, WB>::RC, 1, WB, GS>(g, it, rb, sh);
    }
    TRACE(a, 1, 2);
}

// ------------------------------------------------------------ launch 3
struct DnArgs {
    const uint8_t *q;          // down_q [E+shared][H][I/2] (int4), [E+shared][H][I] (int8) or [E+shared][H][I/4] (int2)
    const float *s;            // down_s [E+shared][H], or [E+shared][H][I/group] with group scales
    int H, I, E, T, top_k, has_shared;
    int gsh;                   // group scales: log2(group / 32)
    int max_items;             // entries of the item tables (<= DEC_MAX_ITEMS)
    const int *ctrl, *item_expert, *item_ntok;
    const int8_t *hq;          // [pairs][I] reordered
    const float *hs;           // [pairs][I/32]
    float *ye;                 // [pairs][H]
    const int *pair_of, *shared_pair;
    const float *w;
    float *y;
    int accumulate;
#ifdef COLI_TRACE
    unsigned long long *trace;
#endif
};

// One item's slice: the workgroup's RPU rows of the item's down matrix (lane
// l holds block column l of each row) and the activations of up to NT token
// slots; with group scales (GS) also the scale of each row's group.
template <int NT, int RPU, int WB, bool GS>
struct DnStage {
    uint4 wd[RPU][WFmt<WB>::NP];
    float sw[GS ? RPU : 1];
    Blk8 act[NT];
    float ds[NT];              // block scales as loaded (turned to f64 where used, so a load is never waited for early)
    int e, nt;
};

template <int NT, int RPU, int WB, bool GS>
__device__ __forceinline__ void dn_load_e(const DnArgs &a, int item, long row0, int lane, int e, int nt,
                                          DnStage<NT, RPU, WB, GS> &st)
{
    constexpr int NP = WFmt<WB>::NP;
    const int nblk = a.I / QK;
    const bool active = lane < nblk;
    const long rowb = (long)a.I * WB / 8;
    st.e = e;
    st.nt = nt;
    const uint8_t *pd = a.q + ((long)st.e * a.H + row0) * rowb + blk_off<WB>(active ? lane : 0);
#pragma unroll
    for (int r = 0; r < RPU; ++r)
#pragma unroll
        for (int q = 0; q < NP; ++q) st.wd[r][q] = load_w_stream<WB>(pd + (long)r * rowb + piece_off<WB>(q, nblk));
    if constexpr (GS) {
        const long gstr = nblk >> a.gsh;         // group scales per row: I / group
        const float *ps = a.s + ((long)st.e * a.H + row0) * gstr + ((active ? lane : 0) >> a.gsh);
#pragma unroll
        for (int r = 0; r < RPU; ++r) st.sw[r] = ps[(long)r * gstr];
    }
#pragma unroll
    for (int s = 0; s < NT; ++s) {
        if (s < st.nt && active) {
            const long pair = (long)item * MAX_SLOTS + s;
            st.act[s] = load_blk8(a.hq + pair * a.I + lane * QK);
            st.ds[s] = a.hs[pair * nblk + lane];
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) st.act[s].v[k] = 0;
            st.ds[s] = 0.0f;
        }
    }
}

// The same for an item of the union, its expert and token count from the
// table in LDS.
template <int NT, int RPU, int WB, bool GS>
__device__ __forceinline__ void dn_load(const DnArgs &a, int item, long row0, int lane, const int *it_e,
                                        const int *it_nt, DnStage<NT, RPU, WB, GS> &st)
{
    dn_load_e(a, item, row0, lane, it_e[item], it_nt[item], st);
}

template <int NT, int RPU, int WB, bool GS>
__device__ __forceinline__ void dn_compute(const DnArgs &a, int item, long row0, int lane,
                                           const DnStage<NT, RPU, WB, GS> &st, float *ye_l)
{
    const int ntu = __builtin_amdgcn_readfirstlane(st.nt);   // slots past it cost no dot products
    double v[NT][RPU];
#pragma unroll
    for (int r = 0; r < RPU; ++r) {
#pragma unroll
        for (int s = 0; s < NT; ++s) {
            if (s > 0 && s >= ntu) break;            // slot 0 is always in use
            v[s][r] = (double)dot_block_w<WB>(st.wd[r], st.act[s]) * ((double)st.ds[s] * WFmt<WB>::KSCALE);
            if constexpr (GS) v[s][r] *= (double)st.sw[r];
        }
    }
    const int vi = transpose_index<RPU>(lane);
#pragma unroll
    for (int s = 0; s < NT; ++s) {
        if (s > 0 && s >= ntu) break;
        wave_transpose_reduce<RPU>(v[s]);
        if ((lane & (64 / RPU - 1)) == 0) {
            const long row = row0 + vi;
            const long pair = (long)item * MAX_SLOTS + s;
            const float out = GS ? (float)v[s][0] : (float)((double)a.s[(long)st.e * a.H + row] * v[s][0]);
            a.ye[pair * a.H + row] = out;
            ye_l[pair * RPU + vi] = out;
        }
    }
}

// A workgroup owns RPU consecutive output rows. Its waves take the items of
// the union round-robin (wave w: items w, w + 4, ...), each item's RPU rows
// at once with the wave's next item already loading (wave 0 starts on the
// shared expert at once); then the per-pair row values in LDS are combined
// into y.
template <int NT, int RPU, int WB, bool GS>
__global__ void __launch_bounds__(256) k_down_combine(DnArgs a)
{
    extern __shared__ float ye_l[];              // [max pairs][RPU]
    __shared__ int it_e[DEC_MAX_ITEMS], it_nt[DEC_MAX_ITEMS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const long row0 = (long)blockIdx.x * RPU;
    TRACE(a, 2, 0);
    DnStage<NT, RPU, WB, GS> A, B;
    // the shared expert is item 0 with T token slots whatever the routing:
    // wave 0 starts loading it before the item table arrives
    const bool early = a.has_shared && wave == 0;
    if (early) dn_load_e(a, 0, row0, lane, a.E, a.T, A);
    // the whole item table up front, so no item's loads wait on a lookup;
    // every entry a union of this batch can have is read together with the
    // item count (one round trip; entries past the count go unused)
    const int n_items = min(a.ctrl[CTRL_N_ITEMS], a.max_items);
    for (int i = threadIdx.x; i < a.max_items; i += blockDim.x) {
        it_e[i] = a.item_expert[i];
        it_nt[i] = a.item_ntok[i];
    }
    __syncthreads();

    int i = wave;
    if (i < n_items && !early) dn_load(a, i, row0, lane, it_e, it_nt, A);
    for (; i < n_items; i += 2 * nwave) {
        if (i + nwave < n_items) dn_load(a, i + nwave, row0, lane, it_e, it_nt, B);
        dn_compute(a, i, row0, lane, A, ye_l);
        if (i + nwave < n_items) {
            if (i + 2 * nwave < n_items) dn_load(a, i + 2 * nwave, row0, lane, it_e, it_nt, A);
            dn_compute(a, i + nwave, row0, lane, B, ye_l);
        }
    }
    __syncthreads();
    TRACE(a, 2, 1);

    const int k = a.top_k;
    for (int j = threadIdx.x; j < a.T * RPU; j += blockDim.x) {
        const int t = j / RPU, rl = j % RPU;
        double acc = 0.0;
        for (int q = 0; q < k; ++q)
            acc += (double)a.w[t * k + q] * (double)ye_l[a.pair_of[t * k + q] * RPU + rl];
        if (a.has_shared) acc += (double)ye_l[a.shared_pair[t] * RPU + rl];
        const float out = (float)acc;
        const long o = (long)t * a.H + row0 + rl;
        a.y[o] = a.accumulate ? __fadd_rn(a.y[o], out) : out;
    }
    TRACE(a, 2, 2);
}

GemvArgs gemv_view(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws)
{
    GemvArgs g;
    g.H = L.H; g.I = L.I; g.E = L.E; g.T = T; g.has_shared = L.has_shared; g.item0 = 0;
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
    g.q_a = L.gate_q; g.s_a = L.gate_s; g.q_b = L.up_q; g.s_b = L.up_s;
    g.gsh = group_shift(L);
    return g;
}

// Routed workgroups of the gate/up launch: at most one per routed unit a
// batch can have (units_max) and, past that, no more than fit on the device
// beside the nsh shared-expert ones (res: resident workgroups, 0 unknown).
inline int sel_routed_wg(int res, int nsh, int units_max)
{
    int nrwg = units_max;
    if (res > nsh && res - nsh < nrwg) nrwg = res - nsh;
    return nrwg < 1 ? 1 : nrwg;
}

#define COLI_SEL_LAUNCH(KERN)                                                                                   \
    do {                                                                                                        \
        const int nrwg_ = sel_routed_wg(resident_wg_256(KERN), nsh, units_max);                                     \
        COLI_LAUNCH(KERN, dim3((unsigned)(nsh + nrwg_)), dim3(256), 0, s, a, g, nsh, nrwg_);                     \
        return hipGetLastError();                                                                               \
    } while (0)

// keys per lane of the selection: E <= 64 * KPL
template <int NT, int WB, bool GS = false>
hipError_t launch_sel_nt(int E, const SelGuArgs &a, const GemvArgs &g, int nsh, int units_max, hipStream_t s)
{
    if (E <= 64) COLI_SEL_LAUNCH((k_select_gateup<NT, 1, WB, GS>));
    if (E <= 128) COLI_SEL_LAUNCH((k_select_gateup<NT, 2, WB, GS>));
    if (E <= 256) COLI_SEL_LAUNCH((k_select_gateup<NT, 4, WB, GS>));
    COLI_SEL_LAUNCH((k_select_gateup<NT, 8, WB, GS>));
}

template <int NT>
hipError_t launch_sel_wb(const coli_moe_layer &L, const SelGuArgs &a, const GemvArgs &g, int nsh, int units_max,
                         hipStream_t s)
{
    if (L.group_size) return launch_sel_nt<NT, 4, true>(L.E, a, g, nsh, units_max, s);
    if (L.weight_bits == 2) return launch_sel_nt<NT, 2>(L.E, a, g, nsh, units_max, s);
    return L.weight_bits == 8 ? launch_sel_nt<NT, 8>(L.E, a, g, nsh, units_max, s)
                              : launch_sel_nt<NT, 4>(L.E, a, g, nsh, units_max, s);
}

template <int NT, int RPU, int WB, bool GS = false>
hipError_t launch_dn_nt(const coli_moe_layer &L, const WsLayout &lay, const DnArgs &a, hipStream_t s)
{
    const size_t lds = (size_t)lay.max_items * MAX_SLOTS * RPU * sizeof(float);
    COLI_LAUNCH((k_down_combine<NT, RPU, WB, GS>), dim3((unsigned)(L.H / RPU)), dim3(256), lds, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_decode_router(const coli_moe_layer &L, const float *x, int T, const WsLayout &lay, char *ws,
                                const float *gamma, float eps, hipStream_t s)
{
    RouterArgs r;
    r.W = L.router_w; r.bias = L.router_b; r.x = x;
    r.gamma = gamma; r.eps = eps; r.vec = rms_vec(x, L.H) ? 1 : 0;
    r.T = T; r.H = L.H; r.E = L.E;
    r.z = reinterpret_cast<double *>(ws + lay.logits);
    r.key = reinterpret_cast<double *>(ws + lay.keys);
    r.sig = r.key + (size_t)T * L.E;
    r.xq = reinterpret_cast<int8_t *>(ws + lay.xq);
    r.xs = reinterpret_cast<float *>(ws + lay.xs);
#ifdef COLI_TRACE
    r.trace = g_dec_trace;
#endif
    const dim3 grid((unsigned)L.E);
    if (gamma) {
        if (T <= 1) COLI_LAUNCH(k_router_norm<1>, grid, dim3(RMS_BLOCK), 0, s, r);
        else if (T <= 2) COLI_LAUNCH(k_router_norm<2>, grid, dim3(RMS_BLOCK), 0, s, r);
        else if (T <= 4) COLI_LAUNCH(k_router_norm<4>, grid, dim3(RMS_BLOCK), 0, s, r);
        else COLI_LAUNCH(k_router_norm<8>, grid, dim3(RMS_BLOCK), 0, s, r);
        return hipGetLastError();
    }
    if (T <= 1) COLI_LAUNCH(k_router<1>, grid, dim3(512), 0, s, r);
    else if (T <= 2) COLI_LAUNCH(k_router<2>, grid, dim3(512), 0, s, r);
    else if (T <= 4) COLI_LAUNCH(k_router<4>, grid, dim3(512), 0, s, r);
    else COLI_LAUNCH(k_router<8>, grid, dim3(512), 0, s, r);
    return hipGetLastError();
}

hipError_t launch_decode_select_gateup(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    SelGuArgs a;
    a.key = reinterpret_cast<const double *>(ws + lay.keys);
    a.sig = a.key + (size_t)T * L.E;
    a.T = T; a.E = L.E; a.top_k = L.top_k; a.n_group = L.n_group; a.topk_group = L.topk_group;
    a.has_shared = L.has_shared; a.route_scale = L.route_scale;
    a.idx = reinterpret_cast<int32_t *>(ws + lay.idx);
    a.w = reinterpret_cast<float *>(ws + lay.w);
    a.ctrl = reinterpret_cast<int *>(ws + lay.ctrl);
    a.item_expert = reinterpret_cast<int *>(ws + lay.item_expert);
    a.item_ntok = reinterpret_cast<int *>(ws + lay.item_ntok);
    a.item_tok = reinterpret_cast<int *>(ws + lay.item_tok);
    a.pair_of = reinterpret_cast<int *>(ws + lay.pair_of);
    a.shared_pair = reinterpret_cast<int *>(ws + lay.shared_pair);
#ifdef COLI_TRACE
    a.trace = g_dec_trace;
#endif
    GemvArgs g = gemv_view(L, T, lay, ws);
    const int nrb = L.I / QK, nsh = L.has_shared ? nrb : 0;
    const int units_max = (lay.max_items - L.has_shared) * nrb;
    if (T <= 1) return launch_sel_wb<1>(L, a, g, nsh, units_max, s);
    if (T <= 2) return launch_sel_wb<2>(L, a, g, nsh, units_max, s);
    if (T <= 4) return launch_sel_wb<4>(L, a, g, nsh, units_max, s);
    return launch_sel_wb<8>(L, a, g, nsh, units_max, s);
}

hipError_t launch_decode_down_combine(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, float *y,
                                      bool accumulate, hipStream_t s)
{
    DnArgs a;
    a.q = L.down_q; a.s = L.down_s;
    a.H = L.H; a.I = L.I; a.E = L.E; a.T = T; a.top_k = L.top_k; a.has_shared = L.has_shared;
    a.gsh = group_shift(L);
    a.max_items = lay.max_items < DEC_MAX_ITEMS ? lay.max_items : DEC_MAX_ITEMS;
    a.ctrl = reinterpret_cast<const int *>(ws + lay.ctrl);
    a.item_expert = reinterpret_cast<const int *>(ws + lay.item_expert);
    a.item_ntok = reinterpret_cast<const int *>(ws + lay.item_ntok);
    a.hq = reinterpret_cast<const int8_t *>(ws + lay.hq);
    a.hs = reinterpret_cast<const float *>(ws + lay.hs);
    a.ye = reinterpret_cast<float *>(ws + lay.ye);
    a.pair_of = reinterpret_cast<const int *>(ws + lay.pair_of);
    a.shared_pair = reinterpret_cast<const int *>(ws + lay.shared_pair);
    a.w = reinterpret_cast<const float *>(ws + lay.w);
    a.y = y;
    a.accumulate = accumulate ? 1 : 0;
#ifdef COLI_TRACE
    a.trace = g_dec_trace;
#endif
    // int8 rows are twice the bytes: half the rows per workgroup
    if (L.weight_bits == 8) {
        if (T <= 1) return launch_dn_nt<1, 4, 8>(L, lay, a, s);
        return launch_dn_nt<2, 2, 8>(L, lay, a, s);
    }
    if (L.weight_bits == 2) {
        if (T <= 1) return launch_dn_nt<1, 8, 2>(L, lay, a, s);
        return launch_dn_nt<2, 4, 2>(L, lay, a, s);
    }
    if (L.group_size) {
        if (T <= 1) return launch_dn_nt<1, 8, 4, true>(L, lay, a, s);
        return launch_dn_nt<2, 4, 4, true>(L, lay, a, s);
    }
    if (T <= 1) return launch_dn_nt<1, 8, 4>(L, lay, a, s);
    return launch_dn_nt<2, 4, 4>(L, lay, a, s);
}

} // namespace coli
