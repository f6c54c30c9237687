// kernels_route.hip — the DeepSeek-V3-style sigmoid router and the batch
// bookkeeping that follows it.
//
// Router (ai4coding.ru summary, "what is implemented"; colibri architecture
// overview, section 5): logits z = W_r x with f64 sums, s = sigmoid(z),
// key = s + bias for selection only, optional group-limited selection, the
// top_k largest keys (equal keys to the lower expert index), weights
// route_scale * s / sum(s) over the chosen experts.
//
// Batch union (colibri README zh-TW, "how it works"): a batch reads every
// distinct expert once. For T <= 8 the union becomes a list of items (expert,
// up to 8 token slots); for larger T the pairs are bucketed per expert and cut
// into token tiles for the grouped GEMM.
#include "device_common.hpp"
#include "internal.hpp"

namespace coli {
namespace {

constexpr int MAX_E = 1024;
constexpr int EPL = MAX_E / 64;     // experts per lane in a one-wave selection
constexpr int TILE_M = 32;          // tokens per grouped-GEMM tile

// ---------------------------------------------------------------- logits
template <int NT>
__global__ void __launch_bounds__(256) k_logits_small(const float *__restrict__ W, const float *__restrict__ x,
                                                      int T, int H, int E, double *__restrict__ z)
{
    __shared__ double red[4][NT];
    const int e = blockIdx.x;
    const float *we = W + (long)e * H;
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        const double wv = (double)we[h];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < T) acc[t] = fma(wv, (double)x[(long)t * H + h], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const double v = wave_sum(acc[t]);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < (unsigned)T && threadIdx.x < NT) {
        const int t = threadIdx.x;
        double v = red[0][t];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v += red[w][t];
        z[(long)t * E + e] = v;
    }
}

// 32 tokens x 32 experts per workgroup, 2x2 outputs per thread, f64 FMA.
__global__ void __launch_bounds__(256) k_logits_tiled(const float *__restrict__ W, const float *__restrict__ x,
                                                      int T, int H, int E, double *__restrict__ z)
{
    __shared__ float xs[32][33];
    __shared__ float ws[32][33];
    const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
    for (int k0 = 0; k0 < H; k0 += 32) {
        for (int i = threadIdx.x; i < 32 * 32; i += 256) {
            const int r = i >> 5, c = i & 31;
            xs[r][c] = (t0 + r < T) ? x[(long)(t0 + r) * H + k0 + c] : 0.0f;
            ws[r][c] = (e0 + r < E) ? W[(long)(e0 + r) * H + k0 + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < 32; ++k) {
            const double a0 = xs[ty][k], a1 = xs[ty + 16][k];
            const double b0 = ws[tx][k], b1 = ws[tx + 16][k];
            acc[0][0] = fma(a0, b0, acc[0][0]);
            acc[0][1] = fma(a0, b1, acc[0][1]);
            acc[1][0] = fma(a1, b0, acc[1][0]);
            acc[1][1] = fma(a1, b1, acc[1][1]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
            if (t < T && e < E) z[(long)t * E + e] = acc[i][j];
        }
}

// ------------------------------------------------------------- selection
struct KeyIdx { double key; int idx; };

__device__ __forceinline__ bool better(double ka, int ia, double kb, int ib)
{
    return ka > kb || (ka == kb && ia < ib);
}

// One wave selects the top_k experts of one token from its logits row.
// Writes idx/w (global) and leaves nothing else behind.
__device__ void select_topk_wave(const double *__restrict__ zt, const float *__restrict__ bias, int E,
                                 int top_k, int n_group, int topk_group, float route_scale,
                                 int32_t *__restrict__ idx_out, float *__restrict__ w_out)
{
    const int lane = threadIdx.x & 63;
    double s[EPL], key[EPL];
    bool elig[EPL];
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
        const int e = lane + 64 * m;
        elig[m] = e < E;
        if (e < E) {
            s[m] = 1.0 / (1.0 + exp(-zt[e]));
            key[m] = s[m] + (double)bias[e];
        } else {
            s[m] = 0.0; key[m] = 0.0;
        }
    }
    if (n_group > 1) {
        // group score = sum of the two largest keys of the group
        const int gsize = E / n_group;
        unsigned long long kept = 0ull;     // groups kept (n_group <= 64)
        double gscore_lane = -INFINITY;     // lane g holds the score of group g
        for (int g = 0; g < n_group; ++g) {
            double b1 = -INFINITY; int i1 = MAX_E;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int e = lane + 64 * m;
                if (e < E && e / gsize == g && better(key[m], e, b1, i1)) { b1 = key[m]; i1 = e; }
            }
            for (int o = 32; o > 0; o >>= 1) {
                const double ob = __shfl_xor(b1, o); const int oi = __shfl_xor(i1, o);
                if (better(ob, oi, b1, i1)) { b1 = ob; i1 = oi; }
            }
            double b2 = -INFINITY;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int e = lane + 64 * m;
                if (e < E && e / gsize == g && e != i1 && key[m] > b2) b2 = key[m];
            }
            b2 = wave_max(b2);
            const double score = gsize >= 2 ? b1 + b2 : b1;
            if (lane == g) gscore_lane = score;
        }
        for (int pick = 0; pick < topk_group; ++pick) {
            double bs = (lane < n_group && !((kept >> lane) & 1ull)) ? gscore_lane : -INFINITY;
            int bi = (lane < n_group && !((kept >> lane) & 1ull)) ? lane : MAX_E;
            for (int o = 32; o > 0; o >>= 1) {
                const double ob = __shfl_xor(bs, o); const int oi = __shfl_xor(bi, o);
                if (better(ob, oi, bs, bi)) { bs = ob; bi = oi; }
            }
            kept |= 1ull << bi;
        }
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            const int e = lane + 64 * m;
            if (e < E) elig[m] = (kept >> (e / gsize)) & 1ull;
        }
    }
    double ssel[COLI_MAX_TOPK];
    int isel[COLI_MAX_TOPK];
    double ssum = 0.0;
    for (int j = 0; j < top_k; ++j) {
        double bk = -INFINITY; int bi = MAX_E; double bs = 0.0;
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            const int e = lane + 64 * m;
            if (elig[m] && (bi == MAX_E || better(key[m], e, bk, bi))) { bk = key[m]; bi = e; bs = s[m]; }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const double ok = __shfl_xor(bk, o); const int oi = __shfl_xor(bi, o);
            const double os = __shfl_xor(bs, o);
            if (oi != MAX_E && (bi == MAX_E || better(ok, oi, bk, bi))) { bk = ok; bi = oi; bs = os; }
        }
#pragma unroll
        for (int m = 0; m < EPL; ++m)
            if (lane + 64 * m == bi) elig[m] = false;
        isel[j < COLI_MAX_TOPK ? j : 0] = bi;
        ssel[j < COLI_MAX_TOPK ? j : 0] = bs;
        ssum += bs;
    }
    for (int j = 0; j < top_k; ++j) {
        if (lane == j) {
            idx_out[j] = isel[j];
            w_out[j] = (float)((double)route_scale * ssel[j] / ssum);
        }
    }
}

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

// T <= 8: top-k of every token (one wave per token), then the batch union.
__global__ void __launch_bounds__(256) k_select_union(SelArgs a)
{
    __shared__ int item_of[MAX_E + 1];
    __shared__ int slot_count[8 * COLI_MAX_TOPK + 1];
    __shared__ int n_items_s;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int e = threadIdx.x; e <= a.E; e += blockDim.x) item_of[e] = -1;
    for (int i = threadIdx.x; i < 8 * COLI_MAX_TOPK + 1; i += blockDim.x) slot_count[i] = 0;
    if (threadIdx.x == 0) n_items_s = 0;
    if (a.given_idx) {
        for (int i = threadIdx.x; i < a.T * a.top_k; i += blockDim.x) {
            a.idx[i] = a.given_idx[i];
            a.w[i] = a.given_w[i];
        }
    } else {
        for (int t = wave; t < a.T; t += (int)(blockDim.x >> 6))
            select_topk_wave(a.z + (long)t * a.E, a.bias, a.E, a.top_k, a.n_group, a.topk_group,
                             a.route_scale, a.idx + t * a.top_k, a.w + t * a.top_k);
    }
    __syncthreads();
    if (a.idx_user)
        for (int i = threadIdx.x; i < a.T * a.top_k; i += blockDim.x) {
            a.idx_user[i] = a.idx[i];
            a.w_user[i] = a.w[i];
        }
    // union in token order: items appear in the order of first use
    for (int t = 0; t < a.T; ++t) {
        const int j = threadIdx.x;
        int e = -1, it = -1;
        bool is_new = false;
        if (j < a.top_k) {
            e = a.idx[t * a.top_k + j];
            if (e < 0 || e >= a.E) e = 0;        // invalid caller routing: memory-safe, result unspecified
            it = item_of[e];
            is_new = it < 0;
        }
        __syncthreads();
        if (wave == 0) {
            const unsigned long long mask = __ballot(is_new);
            const int rank = __popcll(mask & ((1ull << lane) - 1ull));
            const int base = n_items_s;
            if (is_new) {
                it = base + rank;
                item_of[e] = it;
                a.item_expert[it] = e;
            }
            if (j < a.top_k) {
                int slot = slot_count[it];
                slot_count[it] = slot + 1;
                if (slot >= MAX_SLOTS) slot = MAX_SLOTS - 1;   // only a caller repeating an expert
                a.item_tok[it * MAX_SLOTS + slot] = t;
                a.pair_of[t * a.top_k + j] = it * MAX_SLOTS + slot;
            }
            if (lane == 0) n_items_s = base + __popcll(mask);
        }
        __syncthreads();
    }
    const int n_routed = n_items_s;
    if (a.has_shared) {
        for (int t = threadIdx.x; t < a.T; t += blockDim.x) {
            a.item_tok[n_routed * MAX_SLOTS + t] = t;
            a.shared_pair[t] = n_routed * MAX_SLOTS + t;
        }
        if (threadIdx.x == 0) {
            a.item_expert[n_routed] = a.E;
            slot_count[n_routed] = a.T;
        }
    }
    __syncthreads();
    const int n_items = n_routed + (a.has_shared ? 1 : 0);
    for (int i = threadIdx.x; i < n_items; i += blockDim.x) a.item_ntok[i] = slot_count[i];
    if (threadIdx.x == 0) a.ctrl[CTRL_N_ITEMS] = n_items;
}

// T > 8: one wave per token.
__global__ void __launch_bounds__(256) k_select_tokens(SelArgs a)
{
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= a.T) return;
    if (a.given_idx) {
        for (int j = threadIdx.x & 63; j < a.top_k; j += 64) {
            a.idx[t * a.top_k + j] = a.given_idx[t * a.top_k + j];
            a.w[t * a.top_k + j] = a.given_w[t * a.top_k + j];
        }
    } else {
        select_topk_wave(a.z + (long)t * a.E, a.bias, a.E, a.top_k, a.n_group, a.topk_group,
                         a.route_scale, a.idx + t * a.top_k, a.w + t * a.top_k);
    }
    if (a.idx_user)
        for (int j = threadIdx.x & 63; j < a.top_k; j += 64) {
            a.idx_user[t * a.top_k + j] = a.idx[t * a.top_k + j];
            a.w_user[t * a.top_k + j] = a.w[t * a.top_k + j];
        }
}

struct BucketArgs {
    const int32_t *idx;
    int T, E, top_k, has_shared;
    int *ctrl;
    int *expert_off;     // [E + 2]: bucket e is pairs [off[e], off[e+1]); bucket E = shared
    int *pair_tok;       // [n_pairs] token of each pair
    int *pair_of, *shared_pair;
    int2 *tiles;         // (expert, first pair) of each TILE_M-token tile
};

// T > 8: histogram of the T*top_k choices, exclusive scan, scatter, tile list.
// Positions inside a bucket come from atomics; every pair's result is
// computed on its own, so the order inside a bucket changes no value.
__global__ void __launch_bounds__(1024) k_bucket(BucketArgs a)
{
    __shared__ int cnt[MAX_E + 1];
    __shared__ int off[MAX_E + 2];
    __shared__ int toff[MAX_E + 2];
    const int nb = a.E + (a.has_shared ? 1 : 0);
    for (int e = threadIdx.x; e <= MAX_E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int P = a.T * a.top_k;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int e = a.idx[p];
        atomicAdd(&cnt[(e < 0 || e >= a.E) ? 0 : e], 1);   // invalid caller routing: memory-safe only
    }
    if (threadIdx.x == 0 && a.has_shared) cnt[a.E] = a.T;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0, tacc = 0;
        for (int e = 0; e < nb; ++e) {
            off[e] = acc; toff[e] = tacc;
            acc += cnt[e];
            tacc += (cnt[e] + TILE_M - 1) / TILE_M;
        }
        off[nb] = acc; toff[nb] = tacc;
        a.ctrl[CTRL_N_TILES_GU] = tacc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= nb; e += blockDim.x) a.expert_off[e] = off[e];
    for (int e = threadIdx.x; e < nb; e += blockDim.x) {
        for (int tt = 0; tt < toff[e + 1] - toff[e]; ++tt)
            a.tiles[toff[e] + tt] = make_int2(e, off[e] + tt * TILE_M);
        cnt[e] = 0;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        int e = a.idx[p];
        if (e < 0 || e >= a.E) e = 0;
        const int pos = off[e] + atomicAdd(&cnt[e], 1);
        a.pair_tok[pos] = p / a.top_k;
        a.pair_of[p] = pos;
    }
    if (a.has_shared)
        for (int t = threadIdx.x; t < a.T; t += blockDim.x) {
            a.pair_tok[off[a.E] + t] = t;
            a.shared_pair[t] = off[a.E] + t;
        }
}

} // namespace

hipError_t launch_logits(const coli_moe_layer &L, const float *x, int T, double *z, hipStream_t s)
{
    if (T <= 1)
        hipLaunchKernelGGL(k_logits_small<1>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z);
    else if (T <= 2)
        hipLaunchKernelGGL(k_logits_small<2>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z);
    else if (T <= 4)
        hipLaunchKernelGGL(k_logits_small<4>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z);
    else if (T <= 8)
        hipLaunchKernelGGL(k_logits_small<8>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z);
    else
        hipLaunchKernelGGL(k_logits_tiled, dim3((T + 31) / 32, (L.E + 31) / 32), dim3(256), 0, s, L.router_w,
                           x, T, L.H, L.E, z);
    return hipGetLastError();
}

hipError_t launch_select(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws,
                         const int32_t *given_idx, const float *given_w, int32_t *idx_out, float *w_out,
                         hipStream_t s)
{
    SelArgs a;
    a.z = reinterpret_cast<const double *>(ws + lay.logits);
    a.bias = L.router_b;
    a.T = T; a.E = L.E; a.top_k = L.top_k; a.n_group = L.n_group; a.topk_group = L.topk_group;
    a.has_shared = L.has_shared; a.route_scale = L.route_scale;
    a.given_idx = given_idx; a.given_w = given_w;
    a.idx = reinterpret_cast<int32_t *>(ws + lay.idx);
    a.w = reinterpret_cast<float *>(ws + lay.w);
    a.idx_user = idx_out; a.w_user = w_out;
    a.ctrl = reinterpret_cast<int *>(ws + lay.ctrl);
    a.item_expert = reinterpret_cast<int *>(ws + lay.item_expert);
    a.item_ntok = reinterpret_cast<int *>(ws + lay.item_ntok);
    a.item_tok = reinterpret_cast<int *>(ws + lay.item_tok);
    a.pair_of = reinterpret_cast<int *>(ws + lay.pair_of);
    a.shared_pair = reinterpret_cast<int *>(ws + lay.shared_pair);
    if (lay.path == 0) {
        hipLaunchKernelGGL(k_select_union, dim3(1), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_select_tokens, dim3((T + 3) / 4), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    BucketArgs b;
    b.idx = a.idx; b.T = T; b.E = L.E; b.top_k = L.top_k; b.has_shared = L.has_shared; b.ctrl = a.ctrl;
    b.expert_off = reinterpret_cast<int *>(ws + lay.expert_off);
    b.pair_tok = reinterpret_cast<int *>(ws + lay.pair_tok);
    b.pair_of = a.pair_of; b.shared_pair = a.shared_pair;
    b.tiles = reinterpret_cast<int2 *>(ws + lay.tiles);
    hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, s, b);
    return hipGetLastError();
}

} // namespace coli
