// route_device.hpp — device bodies of the router and the batch bookkeeping,
// shared by the standalone router kernels and the decode launches.
//
// Router (ai4coding.ru summary, "what is implemented"; colibri architecture
// overview, section 5): logits z = W_r x with f64 sums, s = sigmoid(z),
// key = s + bias for selection only, optional group-limited selection, the
// top_k largest keys (equal keys to the lower expert index), weights
// route_scale * s / sum(s) over the chosen experts.
//
// Batch union (colibri README zh-TW, "how it works"): a batch reads every
// distinct expert once. For T <= 8 the union is a list of items (an expert
// and up to 8 token slots). The shared expert, when present, is item 0 with
// slot t = token t, so its work never waits for the router; routed experts
// follow in order of first use.
#pragma once
#include "device_common.hpp"

// Optional timing hook of profiling builds (no-op otherwise).
#ifndef COLI_SEL_MARK
#define COLI_SEL_MARK(i) ((void)0)
#endif

namespace coli {

constexpr int MAX_E = 512;
constexpr int SEL_T = 8;            // tokens one selection workgroup handles

// The workgroup's per-thread logit partials of expert e summed: wave sums,
// then the waves in order; z (and the selection key s + b and s = sigmoid(z))
// written for each token.
template <int NT>
__device__ __forceinline__ void logits_finish(const double (&acc)[NT], int T, int E, int e, double *__restrict__ z,
                                              double *red, const float *__restrict__ bias,
                                              double *__restrict__ key, double *__restrict__ sig)
{
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const double v = wave_sum(acc[t]);
        if ((threadIdx.x & 63) == 0) red[(threadIdx.x >> 6) * NT + t] = v;
    }
    __syncthreads();
    if (threadIdx.x < (unsigned)T && threadIdx.x < NT) {
        const int t = threadIdx.x;
        double v = red[t];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v += red[w * NT + t];
        st_dev(z + (long)t * E + e, v);
        if (key) {
            // the selection key of the sigmoid router: s = sigmoid(z), key = s + b
            const double sg = 1.0 / (1.0 + exp(-v));
            st_dev(key + (long)t * E + e, sg + (double)bias[e]);
            st_dev(sig + (long)t * E + e, sg);
        }
    }
    __syncthreads();
}

// Logits of one expert for T <= NT tokens by the whole workgroup (blockDim a
// multiple of 64): float4 loads, f64 FMAs, wave sums, then the waves in
// order. Writes z[t][e] and, with key != nullptr, the selection key s + b and
// s = sigmoid(z). red must hold (blockDim / 64) * NT doubles of LDS.
template <int NT>
__device__ __forceinline__ void logits_expert(const float *__restrict__ W, const float *__restrict__ x, int T,
                                              int H, int E, int e, double *__restrict__ z, double *red,
                                              const float *__restrict__ bias = nullptr,
                                              double *__restrict__ key = nullptr, double *__restrict__ sig = nullptr)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 *we = reinterpret_cast<const f32x4 *>(W + (long)e * H);
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
    const int H4 = H / 4;
#pragma unroll 4
    for (int h = threadIdx.x; h < H4; h += blockDim.x) {
        const f32x4 wv = __builtin_nontemporal_load(&we[h]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < T) {
                const float4 xv = reinterpret_cast<const float4 *>(x + (long)t * H)[h];
                acc[t] = fma((double)wv.x, (double)xv.x, acc[t]);
                acc[t] = fma((double)wv.y, (double)xv.y, acc[t]);
                acc[t] = fma((double)wv.z, (double)xv.z, acc[t]);
                acc[t] = fma((double)wv.w, (double)xv.w, acc[t]);
            }
        }
    }
    logits_finish<NT>(acc, T, E, e, z, red, bias, key, sig);
}

struct SelShared;
struct UnionShared;

struct SelArgs {
    const double *z;           // [T][E] logits, or n_part partial sums [n_part][T][E] added in order
    int n_part = 1;
    const float *bias;
    int T, E, top_k, n_group, topk_group, has_shared;
    float route_scale;
    const int32_t *given_idx;
    const float *given_w;
    int32_t *idx, *idx_user;   // workspace copy and optional caller copy
    float *w, *w_user;
    int *ctrl;
    int *item_expert, *item_ntok, *item_tok;
    int *pair_of, *shared_pair;
};

constexpr int MAX_SPLIT = 16;       // slices of H the large-batch logits are split into, at most

// Logit z[t][e]: the partial sums over slices of H in slice order. The
// partials come from an earlier launch: every load is issued before the
// first is added, so the sum waits on one round trip, not n_part.
__device__ __forceinline__ double sel_logit(const SelArgs &a, int t, int e)
{
    const double *p = a.z + (long)t * a.E + e;
    if (a.n_part <= 1) return *p;
    const long stride = (long)a.T * a.E;
    double v[MAX_SPLIT];
#pragma unroll
    for (int s = 0; s < MAX_SPLIT; ++s) v[s] = s < a.n_part ? p[s * stride] : 0.0;
    double acc = 0.0;
#pragma unroll
    for (int s = 0; s < MAX_SPLIT; ++s)
        if (s < a.n_part) acc += v[s];
    return acc;
}

// LDS of the selection for nt tokens, carved from dynamic shared memory.
struct SelShared {
    double *key;       // [nt][E] selection keys; -inf where the group is not kept
    double *gscore;    // [nt][n_group]
    double *ssel;      // [nt][top_k]
    int *isel;         // [nt][top_k]
};

__host__ __device__ inline size_t sel_lds_bytes(int nt, int E, int k, int ng)
{
    return (size_t)8 * ((size_t)nt * E + (size_t)nt * ng + (size_t)nt * k) + (size_t)4 * nt * k;
}

__device__ inline SelShared sel_view(char *base, int nt, int E, int k, int ng)
{
    SelShared v;
    v.key = reinterpret_cast<double *>(base);
    v.gscore = v.key + (size_t)nt * E;
    v.ssel = v.gscore + (size_t)nt * ng;
    v.isel = reinterpret_cast<int *>(v.ssel + (size_t)nt * k);
    return v;
}

// Score of one group of group-limited routing: the sum of its two largest
// keys (a running top-2 in index order; the group's single key when it has
// one). The keys are read eight at a time, so the reads of a chunk are in
// flight together.
__device__ inline double group_score(const double *g, int gsize)
{
    double m1 = -INFINITY, m2 = -INFINITY;
    int j = 0;
    for (; j + 8 <= gsize; j += 8) {
        double v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = g[j + i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (v[i] > m1) { m2 = m1; m1 = v[i]; }
            else if (v[i] > m2) { m2 = v[i]; }
        }
    }
    for (; j < gsize; ++j) {
        const double v = g[j];
        if (v > m1) { m2 = m1; m1 = v; }
        else if (v > m2) { m2 = v; }
    }
    return gsize >= 2 ? m1 + m2 : m1;
}

// Top-k of nt tokens (t0 ..) by rank: expert e is chosen at position
// rank(e) = #{e' : key_e' > key_e, or key_e' == key_e and e' < e} when that
// rank is below top_k. This is the largest-first order with ties to the lower
// index; every rank is computed independently, so no serial argmax chain.
__device__ inline void select_tokens_block(const SelArgs &a, int t0, int nt, SelShared &sh)
{
    const int E = a.E, k = a.top_k;
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int i = tid; i < nt * E; i += nth) {
        const int t = i / E, e = i % E;
        const double s = 1.0 / (1.0 + exp(-sel_logit(a, t0 + t, e)));
        sh.key[t * E + e] = s + (double)a.bias[e];
    }
    __syncthreads();
    if (a.n_group > 1) {
        const int gsize = E / a.n_group;
        for (int i = tid; i < nt * a.n_group; i += nth) {
            const int t = i / a.n_group, g = i % a.n_group;
            sh.gscore[t * a.n_group + g] = group_score(sh.key + (size_t)t * E + g * gsize, gsize);
        }
        __syncthreads();
        for (int i = tid; i < nt * E; i += nth) {
            const int t = i / E, e = i % E, g = e / gsize;
            const double gs = sh.gscore[t * a.n_group + g];
            int r = 0;
            for (int g2 = 0; g2 < a.n_group; ++g2) {
                const double o = sh.gscore[t * a.n_group + g2];
                r += (o > gs) || (o == gs && g2 < g);
            }
            if (r >= a.topk_group) sh.key[t * E + e] = -INFINITY;   // keys stay finite otherwise
        }
        __syncthreads();
    }
    for (int i = tid; i < nt * E; i += nth) {
        const int t = i / E, e = i % E;
        const double ke = sh.key[t * E + e];
        if (ke == -INFINITY) continue;
        const double *kt = sh.key + (size_t)t * E;
        int r = 0;
#pragma unroll 8
        for (int e2 = 0; e2 < E; ++e2) {
            const double o = kt[e2];
            r += (o > ke) || (o == ke && e2 < e);
        }
        if (r < k) {
            sh.isel[t * k + r] = e;
            sh.ssel[t * k + r] = 1.0 / (1.0 + exp(-sel_logit(a, t0 + t, e)));
        }
    }
    __syncthreads();
    for (int i = tid; i < nt * k; i += nth) {
        const int t = i / k, j = i % k;
        double ssum = 0.0;
        for (int jj = 0; jj < k; ++jj) ssum += sh.ssel[t * k + jj];
        st_dev(a.idx + (long)(t0 + t) * k + j, sh.isel[t * k + j]);
        st_dev(a.w + (long)(t0 + t) * k + j, (float)((double)a.route_scale * sh.ssel[t * k + j] / ssum));
    }
}

// LDS of the batch union, carved from dynamic shared memory.
struct UnionShared {
    int *idx;          // [T][top_k] routing, staged by the caller
    int *item_of;      // [E + 1]
    int *slot_count;   // [T*top_k + 2]
    int *n_items;      // [1]
};

__host__ __device__ inline size_t union_lds_bytes(int T, int E, int k)
{
    return (size_t)4 * ((size_t)T * k + (E + 1) + ((size_t)T * k + 2) + 1);
}

__device__ inline UnionShared union_view(char *base, int T, int E, int k)
{
    UnionShared u;
    u.idx = reinterpret_cast<int *>(base);
    u.item_of = u.idx + (size_t)T * k;
    u.slot_count = u.item_of + (E + 1);
    u.n_items = u.slot_count + ((size_t)T * k + 2);
    return u;
}

// Batch union for T <= 8 from the routing in u.idx (filled by the caller).
// All threads of the workgroup take part.
__device__ inline void build_union(const SelArgs &a, UnionShared &u)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    for (int e = threadIdx.x; e <= a.E; e += blockDim.x) u.item_of[e] = -1;
    for (int i = threadIdx.x; i < a.T * a.top_k + 2; i += blockDim.x) u.slot_count[i] = 0;
    if (threadIdx.x == 0) *u.n_items = a.has_shared ? 1 : 0;
    if (a.has_shared) {
        for (int t = threadIdx.x; t < a.T; t += blockDim.x) {
            st_dev(a.item_tok + t, t);
            st_dev(a.shared_pair + t, t);
        }
        if (threadIdx.x == 0) {
            st_dev(a.item_expert, a.E);
            u.slot_count[0] = a.T;
        }
    }
    __syncthreads();
    // routed items in token order, each appearing at its first use
    for (int t = 0; t < a.T; ++t) {
        const int j = threadIdx.x;
        int e = -1, it = -1;
        bool is_new = false;
        if (j < a.top_k) {
            e = u.idx[t * a.top_k + j];
            if (e < 0 || e >= a.E) e = 0;        // invalid caller routing: memory-safe, result unspecified
            it = u.item_of[e];
            is_new = it < 0;
        }
        __syncthreads();
        if (wave == 0) {
            const unsigned long long mask = __ballot(is_new);
            const int rank = __popcll(mask & ((1ull << lane) - 1ull));
            const int base = *u.n_items;
            if (is_new) {
                it = base + rank;
                u.item_of[e] = it;
                st_dev(a.item_expert + it, e);
            }
            if (j < a.top_k) {
                int slot = u.slot_count[it];
                u.slot_count[it] = slot + 1;
                if (slot >= MAX_SLOTS) slot = MAX_SLOTS - 1;   // only a caller repeating an expert
                st_dev(a.item_tok + it * MAX_SLOTS + slot, t);
                st_dev(a.pair_of + t * a.top_k + j, it * MAX_SLOTS + slot);
            }
            if (lane == 0) *u.n_items = base + __popcll(mask);
        }
        __syncthreads();
    }
    const int n_items = *u.n_items;
    for (int i = threadIdx.x; i < n_items; i += blockDim.x) st_dev(a.item_ntok + i, u.slot_count[i]);
    if (threadIdx.x == 0) st_dev(a.ctrl + CTRL_N_ITEMS, n_items);
    __syncthreads();
}

// Routing of this workgroup's selection (sh.isel) into the union's LDS copy.
__device__ inline void routing_to_union(const SelArgs &a, const SelShared &sh, UnionShared &u)
{
    for (int i = threadIdx.x; i < a.T * a.top_k; i += blockDim.x) u.idx[i] = sh.isel[i];
}

// ---------------------------------------------------------------------------
// Selection and batch union inside one workgroup (decode, T <= 8). Every
// workgroup of the routed gate/up launch derives the same routing from the
// keys the router launch wrote, so no launch sits between the router and the
// experts.

constexpr int DEC_MAX_T = 8;
constexpr int DEC_MAX_ITEMS = 1 + DEC_MAX_T * COLI_MAX_TOPK;
constexpr int DEC_MAX_PAIRS = DEC_MAX_T * COLI_MAX_TOPK;

// Order-preserving map of an f64 onto u64 (-0.0 is taken as +0.0, so equal
// keys map to equal integers). A candidate of value 0 is never selected.
__device__ __forceinline__ unsigned long long order_key(double v)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(v + 0.0);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// (key, expert) candidate of the wave argmax: larger key first, equal keys to
// the lower expert index. A total order, so every lane ends with one winner.
struct Cand {
    unsigned lo, hi;
    int e;
};

__device__ __forceinline__ bool cand_beats(const Cand &a, const Cand &b)
{
    const unsigned long long ka = ((unsigned long long)a.hi << 32) | a.lo;
    const unsigned long long kb = ((unsigned long long)b.hi << 32) | b.lo;
    return ka > kb || (ka == kb && a.e < b.e);
}

template <int CTRL>
__device__ __forceinline__ void cand_dpp_step(Cand &c)
{
    Cand p;
    p.lo = (unsigned)__builtin_amdgcn_mov_dpp((int)c.lo, CTRL, 0xF, 0xF, false);
    p.hi = (unsigned)__builtin_amdgcn_mov_dpp((int)c.hi, CTRL, 0xF, 0xF, false);
    p.e = __builtin_amdgcn_mov_dpp(c.e, CTRL, 0xF, 0xF, false);
    if (cand_beats(p, c)) c = p;
}

// Both results of a permlane swap of a value with itself are {own, partner}
// in some order; the better of the two is what the all-reduce keeps.
template <bool W32>
__device__ __forceinline__ void cand_swap_step(Cand &c)
{
    Cand a, b;
    if constexpr (W32) {
        const auto l = __builtin_amdgcn_permlane32_swap(c.lo, c.lo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(c.hi, c.hi, false, false);
        const auto x = __builtin_amdgcn_permlane32_swap((unsigned)c.e, (unsigned)c.e, false, false);
        a = Cand{l[0], h[0], (int)x[0]};
        b = Cand{l[1], h[1], (int)x[1]};
    } else {
        const auto l = __builtin_amdgcn_permlane16_swap(c.lo, c.lo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(c.hi, c.hi, false, false);
        const auto x = __builtin_amdgcn_permlane16_swap((unsigned)c.e, (unsigned)c.e, false, false);
        a = Cand{l[0], h[0], (int)x[0]};
        b = Cand{l[1], h[1], (int)x[1]};
    }
    c = cand_beats(b, a) ? b : a;
}

// Wave-wide best candidate, left in every lane: quad swaps, then row
// rotations by 4 and 8 (each quad already uniform, so a rotation pairs whole
// quads), then the 16- and 32-lane swaps.
__device__ __forceinline__ Cand wave_best(Cand c)
{
    cand_dpp_step<DPP_XOR1>(c);
    cand_dpp_step<DPP_XOR2>(c);
    cand_dpp_step<0x124>(c);          // row_ror:4
    cand_dpp_step<0x128>(c);          // row_ror:8
    cand_swap_step<false>(c);
    cand_swap_step<true>(c);
    return c;
}

// Kept groups of group-limited routing for one token (one wave): a group's
// score is the sum of its two largest keys (group_score), the topk_group best
// scores are kept, equal scores to the lower group. kw holds the token's E
// keys (this wave's LDS copy); lane g scores group g. Returns a bitmask over
// groups (all ones when n_group == 1).
__device__ inline unsigned long long kept_groups(const double *kw, int E, int n_group, int topk_group)
{
    if (n_group <= 1) return ~0ull;
    const int lane = threadIdx.x & 63, gsize = E / n_group;
    double gs = -INFINITY;
    if (lane < n_group) gs = group_score(kw + lane * gsize, gsize);
    int r = 0;
    for (int g2 = 0; g2 < n_group; ++g2) {
        const double o = __shfl(gs, g2);
        r += (o > gs) || (o == gs && g2 < lane);
    }
    return __ballot(lane < n_group && r < topk_group);
}

// Wave-wide maximum of a u32, left in every lane.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v)
{
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, DPP_XOR1, 0xF, 0xF, false));
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, DPP_XOR2, 0xF, 0xF, false));
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));   // row_ror:4
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));   // row_ror:8
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(b[0], b[1]);
}

// Lane l's KPL keys and sigmoids (experts l, l+64, ...), read together. The
// keys come from an earlier launch: plain loads, so the workgroups on one
// XCD share its L2 copy instead of each reading the same lines from memory.
template <int KPL>
__device__ __forceinline__ void lane_load(const double *__restrict__ key, const double *__restrict__ sig, int E,
                                          double (&kv)[KPL], double (&sv)[KPL])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        kv[i] = e < E ? key[e] : 0.0;
        sv[i] = e < E ? sig[e] : 0.0;
    }
}

// The lane's keys as order keys (0 for experts outside the kept groups gm)
// with their experts and sigmoids, sorted by (key desc, expert asc).
template <int KPL>
__device__ __forceinline__ void lane_order(const double (&kv)[KPL], int E, int gsize, unsigned long long gm,
                                           unsigned long long (&ok)[KPL], int (&oe)[KPL], double (&sv)[KPL])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        ok[i] = (e < E && ((gm >> (e / gsize)) & 1ull)) ? order_key(kv[i]) : 0ull;
        oe[i] = e;
    }
    COLI_SEL_MARK(0);
#pragma unroll
    for (int i = 1; i < KPL; ++i) {                  // insertion sort
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = ok[j] > ok[j - 1] || (ok[j] == ok[j - 1] && oe[j] < oe[j - 1]);
            const unsigned long long tk = ok[j];
            const int te = oe[j];
            const double ts = sv[j];
            ok[j] = sw ? ok[j - 1] : ok[j];
            oe[j] = sw ? oe[j - 1] : oe[j];
            sv[j] = sw ? sv[j - 1] : sv[j];
            ok[j - 1] = sw ? tk : ok[j - 1];
            oe[j - 1] = sw ? te : oe[j - 1];
            sv[j - 1] = sw ? ts : sv[j - 1];
        }
    }
}

// The owning lane hands its best on: sel_e/sel_s of slot r, then shifts its
// sorted list.
template <int KPL>
__device__ __forceinline__ void lane_pop(int r, unsigned long long (&ok)[KPL], int (&oe)[KPL], double (&sv)[KPL],
                                         int *sel_e, double *sel_s)
{
    sel_e[r] = oe[0];
    sel_s[r] = sv[0];
#pragma unroll
    for (int i = 0; i + 1 < KPL; ++i) { ok[i] = ok[i + 1]; oe[i] = oe[i + 1]; sv[i] = sv[i + 1]; }
    ok[KPL - 1] = 0ull;
    oe[KPL - 1] = 0x7FFFFFFF;
    sv[KPL - 1] = 0.0;
}

// Top-k of one token (one wave; E <= 64 * KPL). Each of the k rounds takes
// the wave maximum of the upper 32 bits of the lanes' current best keys;
// when a single lane holds it, that lane's best is the next expert (every
// other remaining key is smaller in its upper bits). If two lanes ever tie
// there, the whole selection is taken again with the exact (key, expert)
// order in every round. Writes the experts, largest key first, and
// w_j = route_scale * s_j / sum_j s_j (s summed in slot order, f64) to LDS.
template <int KPL>
__device__ inline void wave_topk(const double *__restrict__ key, const double *__restrict__ sig, int E, int k,
                                 int n_group, int topk_group, float route_scale, int *sel_e, float *sel_w,
                                 double *sel_s, bool weights, double *kw)
{
    const int lane = threadIdx.x & 63;
    const int gsize = E / n_group;
    double kv[KPL], sv[KPL];
    lane_load<KPL>(key, sig, E, kv, sv);             // one round trip for all keys and sigmoids
    unsigned long long gm = ~0ull;
    if (n_group > 1) {                               // group scores from this wave's LDS copy of the keys
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (lane + 64 * i < E) kw[lane + 64 * i] = kv[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        gm = kept_groups(kw, E, n_group, topk_group);
    }
    unsigned long long ok[KPL];
    int oe[KPL];
    double ss[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) ss[i] = sv[i];
    lane_order<KPL>(kv, E, gsize, gm, ok, oe, ss);
    COLI_SEL_MARK(1);
    if (lane < k) { sel_e[lane] = 0; sel_s[lane] = 0.0; }   // kept only without enough finite keys
    // fast rounds on the upper 32 bits only (a valid key's are never 0)
    unsigned kh[KPL];
    int fe[KPL];
    double fs[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) { kh[i] = (unsigned)(ok[i] >> 32); fe[i] = oe[i]; fs[i] = ss[i]; }
    bool tie = false;
    for (int r = 0; r < k; ++r) {
        const unsigned long long m = __ballot(kh[0] == wave_max_u32(kh[0]));
        tie |= (m & (m - 1ull)) != 0ull;
        if (lane == __ffsll((long long)m) - 1 && kh[0] != 0u) {
            sel_e[r] = fe[0];
            sel_s[r] = fs[0];
#pragma unroll
            for (int i = 0; i + 1 < KPL; ++i) { kh[i] = kh[i + 1]; fe[i] = fe[i + 1]; fs[i] = fs[i + 1]; }
            kh[KPL - 1] = 0u;
        }
    }
    if (tie) {                                       // exact order in every round
        lane_order<KPL>(kv, E, gsize, gm, ok, oe, sv);
        if (lane < k) { sel_e[lane] = 0; sel_s[lane] = 0.0; }
        for (int r = 0; r < k; ++r) {
            Cand c{(unsigned)ok[0], (unsigned)(ok[0] >> 32), ok[0] != 0ull ? oe[0] : 0x7FFFFFFF};
            c = wave_best(c);
            if (oe[0] == c.e && ok[0] != 0ull) lane_pop<KPL>(r, ok, oe, sv, sel_e, sel_s);
        }
    }
    COLI_SEL_MARK(2);
    if (!weights) return;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < k) {
        double ssum = 0.0;
        for (int j = 0; j < k; ++j) ssum += sel_s[j];
        sel_w[lane] = (float)((double)route_scale * sel_s[lane] / ssum);
    }
    COLI_SEL_MARK(3);
}

// Routing and batch union of T <= 8 tokens held in LDS by one workgroup.
struct DecUnion {
    int sel_e[DEC_MAX_PAIRS];        // [t][j] experts
    float sel_w[DEC_MAX_PAIRS];      // [t][j] weights
    double sel_s[DEC_MAX_PAIRS];     // [t][j] sigmoid of the chosen logits
    int item_e[DEC_MAX_ITEMS];
    int item_nt[DEC_MAX_ITEMS];
    int item_tok[DEC_MAX_ITEMS * MAX_SLOTS];
    int first_item[DEC_MAX_PAIRS];   // item of a pair that opens an item
    int pair_of[DEC_MAX_PAIRS];      // item * 8 + slot
    int n_items;
};

// Selection of all T tokens (wave w takes tokens w, w + waves, ...; E <=
// 64 * KPL), then the
// union: the shared expert is item 0 (slot t = token t), routed experts follow
// in order of first use (token-major, then slot). All threads of the
// workgroup call it; blockDim >= 64. kw: LDS of 64 * KPL doubles per wave
// (the wave's copy of a token's keys while its groups are scored).
template <int KPL>
__device__ inline void dec_route_union(const double *__restrict__ key, const double *__restrict__ sig, int T, int E,
                                       int k, int n_group, int topk_group, float route_scale, int has_shared,
                                       DecUnion &u, double *kw, bool weights = true)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
    for (int t = wave; t < T; t += nwave) {
        const double *kt = key + (long)t * E, *st = sig + (long)t * E;
        int *se = u.sel_e + t * k;
        float *sw = u.sel_w + t * k;
        double *ss = u.sel_s + t * k;
        wave_topk<KPL>(kt, st, E, k, n_group, topk_group, route_scale, se, sw, ss, weights, kw + wave * 64 * KPL);
    }
    if (T == 1) {                                 // one token: item has_shared + j is its slot j
        __syncthreads();
        if (tid < k) {
            const int it = has_shared + tid;
            u.item_e[it] = u.sel_e[tid];
            u.item_nt[it] = 1;
            u.item_tok[it * MAX_SLOTS] = 0;
            u.pair_of[tid] = it * MAX_SLOTS;
        }
        if (has_shared && tid == 0) { u.item_e[0] = E; u.item_nt[0] = 1; u.item_tok[0] = 0; }
        if (tid == 0) u.n_items = has_shared + k;
        COLI_SEL_MARK(4);
        __syncthreads();
        return;
    }
    const int n_items_max = has_shared + T * k;
    for (int i = tid; i < n_items_max; i += blockDim.x) u.item_nt[i] = 0;
    if (has_shared && tid == 0) { u.item_e[0] = E; u.item_nt[0] = T; }
    if (has_shared && tid < T) u.item_tok[tid] = tid;
    __syncthreads();
    const int np = T * k;
    int running = has_shared;                     // items so far (wave 0 keeps it)
    for (int c = 0; c < np; c += 64) {
        const int p = c + lane;
        const bool valid = wave == 0 && p < np;
        int e = -1, cnt = 0, qf = -1, my_item = -1;
        if (wave == 0) {
            if (valid) e = u.sel_e[p];
            if (np <= 64) {                                 // every pair in a lane: read them by readlane
                for (int q = 0; q < np; ++q) {              // earlier pairs of the same expert
                    const int eq_e = __builtin_amdgcn_readlane(e, q);
                    const bool eq = valid && q < p && eq_e == e;
                    if (eq && qf < 0) qf = q;
                    cnt += eq ? 1 : 0;
                }
            } else {
                for (int q = 0; q < np; ++q) {
                    const bool eq = valid && q < p && u.sel_e[q] == e;
                    if (eq && qf < 0) qf = q;
                    cnt += eq ? 1 : 0;
                }
            }
            const bool is_new = valid && cnt == 0;
            const unsigned long long m = __ballot(is_new);
            my_item = running + __popcll(m & ((1ull << lane) - 1ull));
            if (is_new) { u.first_item[p] = my_item; u.item_e[my_item] = e; }
            running += __popcll(m);
        }
        __syncthreads();
        if (valid) {
            const int it = cnt == 0 ? my_item : u.first_item[qf];
            const int slot = cnt < MAX_SLOTS ? cnt : MAX_SLOTS - 1;   // repeats only from a caller's routing
            u.pair_of[p] = it * MAX_SLOTS + slot;
            u.item_tok[it * MAX_SLOTS + slot] = p / k;
            atomicAdd(&u.item_nt[it], 1);
        }
        __syncthreads();
    }
    COLI_SEL_MARK(4);
    if (tid == 0) u.n_items = running;
    __syncthreads();
}

} // namespace coli
