// route_device.hpp — device bodies of the router and the batch bookkeeping,
// shared by the standalone router kernels and the fused decode kernel.
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

namespace coli {

constexpr int MAX_E = 512;
constexpr int SEL_T = 8;            // tokens one selection workgroup handles

// Logits of one expert for T <= NT tokens by the whole workgroup (blockDim a
// multiple of 64, at most 256): float4 loads, f64 FMAs, wave sums, then the
// waves in order. Writes z[t][e]. red must hold 4 * NT doubles of LDS.
template <int NT>
__device__ __forceinline__ void logits_expert(const float *__restrict__ W, const float *__restrict__ x, int T,
                                              int H, int E, int e, double *__restrict__ z, double *red)
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
    }
    __syncthreads();
}

struct SelShared;
struct UnionShared;

struct SelArgs {
    const double *z;
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
        const double s = 1.0 / (1.0 + exp(-ld_dev(a.z + (long)(t0 + t) * E + e)));
        sh.key[t * E + e] = s + (double)a.bias[e];
    }
    __syncthreads();
    if (a.n_group > 1) {
        const int gsize = E / a.n_group;
        for (int i = tid; i < nt * a.n_group; i += nth) {
            const int t = i / a.n_group, g = i % a.n_group;
            double m1 = -INFINITY, m2 = -INFINITY;       // two largest keys, in index order
            for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
                const double v = sh.key[t * E + e];
                if (v > m1) { m2 = m1; m1 = v; }
                else if (v > m2) { m2 = v; }
            }
            sh.gscore[t * a.n_group + g] = gsize >= 2 ? m1 + m2 : m1;
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
            sh.ssel[t * k + r] = 1.0 / (1.0 + exp(-ld_dev(a.z + (long)(t0 + t) * E + e)));
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

} // namespace coli
