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

constexpr int MAX_E = 512;
constexpr int SEL_T = 8;            // tokens one selection workgroup handles
constexpr int TILE_M = 32;          // tokens per grouped-GEMM tile

// ---------------------------------------------------------------- logits
// Q8 of one 32-wide activation block (reordered layout), the rule of the
// Q8_0-style quantiser: d = absmax/127, codes rint(x * (1/d)) clamped.
__device__ __forceinline__ void q8_block_reordered(const float *__restrict__ src, int8_t *__restrict__ dst,
                                                   float *__restrict__ dsc)
{
    float v[QK];
#pragma unroll
    for (int i = 0; i < QK / 4; ++i) {
        const float4 f = reinterpret_cast<const float4 *>(src)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) amax = fmaxf(amax, fabsf(v[i]));
    float d, id;
    q8_scale(amax, d, id);
    int c[QK];
#pragma unroll
    for (int i = 0; i < QK; ++i) c[i] = round_clamp(__fmul_rn(v[i], id), -127.0f, 127.0f) & 0xFF;
    uint32_t o[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        o[2 * m] = (uint32_t)(c[8 * m] | (c[8 * m + 2] << 8) | (c[8 * m + 4] << 16) | (c[8 * m + 6] << 24));
        o[2 * m + 1] = (uint32_t)(c[8 * m + 1] | (c[8 * m + 3] << 8) | (c[8 * m + 5] << 16) | (c[8 * m + 7] << 24));
    }
    reinterpret_cast<uint4 *>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4 *>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
    *dsc = d;
}

// T <= 8: one workgroup per expert computes that expert's logits for every
// token (f64 sums over float4 loads); the workgroups also share the Q8 of x.
template <int NT>
__global__ void __launch_bounds__(256) k_logits_small(const float *__restrict__ W, const float *__restrict__ x,
                                                      int T, int H, int E, double *__restrict__ z,
                                                      int8_t *__restrict__ xq, float *__restrict__ xs)
{
    __shared__ double red[4][NT];
    const int e = blockIdx.x;
    if (xq != nullptr) {
        const long nb = (long)T * (H / QK);
        for (long b = (long)e * blockDim.x + threadIdx.x; b < nb; b += (long)gridDim.x * blockDim.x)
            q8_block_reordered(x + b * QK, xq + b * QK, xs + b);
    }
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

struct SelShared {
    double key[SEL_T][MAX_E];      // selection keys; -inf where the group is not kept
    double gscore[SEL_T][64];
    double ssel[SEL_T][COLI_MAX_TOPK];
    int isel[SEL_T][COLI_MAX_TOPK];
};

// Top-k of nt tokens (t0 ..) by rank: expert e is chosen at position
// rank(e) = #{e' : key_e' > key_e, or key_e' == key_e and e' < e} when that
// rank is below top_k. This is the largest-first order with ties to the lower
// index; every rank is computed independently, so no serial argmax chain.
__device__ void select_tokens_block(const SelArgs &a, int t0, int nt, SelShared &sh)
{
    const int E = a.E, k = a.top_k;
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int i = tid; i < nt * E; i += nth) {
        const int t = i / E, e = i % E;
        const double s = 1.0 / (1.0 + exp(-a.z[(long)(t0 + t) * E + e]));
        sh.key[t][e] = s + (double)a.bias[e];
    }
    __syncthreads();
    if (a.n_group > 1) {
        const int gsize = E / a.n_group;
        for (int i = tid; i < nt * a.n_group; i += nth) {
            const int t = i / a.n_group, g = i % a.n_group;
            double m1 = -INFINITY, m2 = -INFINITY;       // two largest keys, in index order
            for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
                const double v = sh.key[t][e];
                if (v > m1) { m2 = m1; m1 = v; }
                else if (v > m2) { m2 = v; }
            }
            sh.gscore[t][g] = gsize >= 2 ? m1 + m2 : m1;
        }
        __syncthreads();
        for (int i = tid; i < nt * E; i += nth) {
            const int t = i / E, e = i % E, g = e / gsize;
            const double gs = sh.gscore[t][g];
            int r = 0;
            for (int g2 = 0; g2 < a.n_group; ++g2) {
                const double o = sh.gscore[t][g2];
                r += (o > gs) || (o == gs && g2 < g);
            }
            if (r >= a.topk_group) sh.key[t][e] = -INFINITY;   // keys stay finite otherwise
        }
        __syncthreads();
    }
    for (int i = tid; i < nt * E; i += nth) {
        const int t = i / E, e = i % E;
        const double ke = sh.key[t][e];
        if (ke == -INFINITY) continue;
        int r = 0;
        for (int e2 = 0; e2 < E; ++e2) {
            const double o = sh.key[t][e2];
            r += (o > ke) || (o == ke && e2 < e);
        }
        if (r < k) {
            sh.isel[t][r] = e;
            sh.ssel[t][r] = 1.0 / (1.0 + exp(-a.z[(long)(t0 + t) * E + e]));
        }
    }
    __syncthreads();
    for (int i = tid; i < nt * k; i += nth) {
        const int t = i / k, j = i % k;
        double ssum = 0.0;
        for (int jj = 0; jj < k; ++jj) ssum += sh.ssel[t][jj];
        a.idx[(long)(t0 + t) * k + j] = sh.isel[t][j];
        a.w[(long)(t0 + t) * k + j] = (float)((double)a.route_scale * sh.ssel[t][j] / ssum);
    }
}

// T <= 8: top-k of every token, then the batch union.
__global__ void __launch_bounds__(1024) k_select_union(SelArgs a)
{
    __shared__ SelShared sh;
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
        select_tokens_block(a, 0, a.T, sh);
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

// T > 8: one workgroup per token.
__global__ void __launch_bounds__(256) k_select_tokens(SelArgs a)
{
    __shared__ SelShared sh;
    const int t = blockIdx.x;
    if (a.given_idx) {
        for (int j = threadIdx.x; j < a.top_k; j += blockDim.x) {
            a.idx[t * a.top_k + j] = a.given_idx[t * a.top_k + j];
            a.w[t * a.top_k + j] = a.given_w[t * a.top_k + j];
        }
        __syncthreads();
    } else {
        select_tokens_block(a, t, 1, sh);
    }
    if (a.idx_user)
        for (int j = threadIdx.x; j < a.top_k; j += blockDim.x) {
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

hipError_t launch_logits(const coli_moe_layer &L, const float *x, int T, double *z, int8_t *xq, float *xs,
                         hipStream_t s)
{
    if (T > 8) {
        if (xq) {
            hipError_t e = launch_quant_q8(x, T, L.H, xq, xs, true, s);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_logits_tiled, dim3((T + 31) / 32, (L.E + 31) / 32), dim3(256), 0, s, L.router_w,
                           x, T, L.H, L.E, z);
    } else if (T <= 1) {
        hipLaunchKernelGGL(k_logits_small<1>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    } else if (T <= 2) {
        hipLaunchKernelGGL(k_logits_small<2>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    } else if (T <= 4) {
        hipLaunchKernelGGL(k_logits_small<4>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    } else {
        hipLaunchKernelGGL(k_logits_small<8>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    }
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
        hipLaunchKernelGGL(k_select_union, dim3(1), dim3(1024), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_select_tokens, dim3(T), dim3(256), 0, s, a);
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
