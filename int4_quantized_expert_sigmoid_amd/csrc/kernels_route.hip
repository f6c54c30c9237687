// kernels_route.hip — router kernels: logits (with Q8 of x), top-k
// selection and the batch union (T <= 8) or per-expert buckets (T > 8).
// The device bodies live in route_device.hpp.
#include "route_device.hpp"
#include "internal.hpp"

namespace coli {
namespace {

constexpr int TILE_M = 32;          // tokens per grouped-GEMM tile

// T <= 8: one workgroup per expert computes that expert's logits for every
// token; the workgroups also share the Q8 of x.
template <int NT>
__global__ void __launch_bounds__(256) k_logits_small(const float *__restrict__ W, const float *__restrict__ x,
                                                      int T, int H, int E, double *__restrict__ z,
                                                      int8_t *__restrict__ xq, float *__restrict__ xs)
{
    __shared__ double red[4 * NT];
    if (xq != nullptr) {
        const long nb = (long)T * (H / QK);
        for (long b = (long)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (long)gridDim.x * blockDim.x)
            q8_block_reordered(x + b * QK, xq + b * QK, xs + b);
    }
    logits_expert<NT>(W, x, T, H, E, blockIdx.x, z, red);
}

// Large batches: 64 tokens x 64 experts per workgroup over one slice of H
// (blockIdx.z of n_split equal slices, each a whole number of 32-column
// chunks), on the f64 matrix cores: wave w owns the 32 x 32 quarter
// (w >> 1, w & 1) as 2 x 2 tiles of v_mfma_f64_16x16x4f64. The f32 inputs and
// their products are exact in f64; the sums are f64. Within a chunk the
// MFMA's k index q (lane / 16) takes columns 8q .. 8q+7 in turn, so a lane's
// values of a row are two float4 loads and nothing is staged in LDS. The
// next chunk's loads are in flight while the current one is multiplied.
// Slice s writes its partial sums to part[s][t][e] and the selection adds
// the slices in order.
constexpr int LG_T = 64, LG_E = 64, LG_K = 32;
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f4_at(const float4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__global__ void __launch_bounds__(256) k_logits_split(const float *__restrict__ W, const float *__restrict__ x,
                                                      int T, int H, int E, int kspan, double *__restrict__ part)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int t0 = blockIdx.x * LG_T + (wave >> 1) * 32, e0 = blockIdx.y * LG_E + (wave & 1) * 32;
    const long k0 = (long)blockIdx.z * kspan + 8 * q;
    // the lane's rows: tokens t0 + r and t0 + 16 + r, experts e0 + r and e0 + 16 + r.
    // A row past T (or E) reads row 0 instead: it only feeds output rows (or
    // columns) that are never stored, so every load is unconditional.
    const float *px[2], *pw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = t0 + 16 * i + r, e = e0 + 16 * i + r;
        px[i] = x + (long)(t < T ? t : 0) * H + k0;
        pw[i] = W + (long)(e < E ? e : 0) * H + k0;
    }
    float4 ax[2][2], aw[2][2], bx[2][2], bw[2][2];   // two chunks: [row block][half of the lane's 8 columns]
    auto load = [&](int kc, float4 (&lx)[2][2], float4 (&lw)[2][2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                lx[i][h] = *reinterpret_cast<const float4 *>(px[i] + kc + 4 * h);
                lw[i][h] = *reinterpret_cast<const float4 *>(pw[i] + kc + 4 * h);
            }
    };
    f64x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    auto mult = [&](const float4 (&lx)[2][2], const float4 (&lw)[2][2]) {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            double a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = (double)f4_at(lx[i][st >> 2], st & 3);
                b[i] = (double)f4_at(lw[i][st >> 2], st & 3);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    // chunks alternate between the two buffers, the next one loading while
    // the current one is multiplied. The loop body is one straight block
    // (two chunks, no exits) and every load in it is issued (past the
    // slice's end it reads the last chunk again, unused), so each wait is for
    // the current chunk only; the scheduling barriers keep the loads ahead of
    // the products instead of next to their uses.
    const int nch = kspan / LG_K, last = kspan - LG_K;
    load(0, ax, aw);
    int c = 0;
    for (; c + 2 <= nch; c += 2) {
        load((c + 1) * LG_K, bx, bw);
        __builtin_amdgcn_sched_barrier(0);
        mult(ax, aw);
        load(min((c + 2) * LG_K, last), ax, aw);
        __builtin_amdgcn_sched_barrier(0);
        mult(bx, bw);
    }
    if (c < nch) mult(ax, aw);                       // an odd last chunk
    // lane (r, q) holds rows q, q + 4, q + 8, q + 12 (tokens) of column r (expert) of each tile
    double *out = part + (long)blockIdx.z * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int t = t0 + 16 * i + 4 * m + q, e = e0 + 16 * j + r;
                if (t < T && e < E) out[(long)t * E + e] = acc[i][j][m];
            }
}

// T <= 8: top-k of every token, then the batch union.
__global__ void __launch_bounds__(1024) k_select_union(SelArgs a)
{
    extern __shared__ double dyn_lds[];
    char *lds = reinterpret_cast<char *>(dyn_lds);
    SelShared sh = sel_view(lds, a.T, a.E, a.top_k, a.n_group);
    UnionShared u = union_view(lds + sel_lds_bytes(a.T, a.E, a.top_k, a.n_group), a.T, a.E, a.top_k);
    if (a.given_idx) {
        for (int i = threadIdx.x; i < a.T * a.top_k; i += blockDim.x) {
            st_dev(a.idx + i, a.given_idx[i]);
            st_dev(a.w + i, a.given_w[i]);
            u.idx[i] = a.given_idx[i];
        }
    } else {
        select_tokens_block(a, 0, a.T, sh);
        routing_to_union(a, sh, u);
    }
    __syncthreads();
    if (a.idx_user)
        for (int i = threadIdx.x; i < a.T * a.top_k; i += blockDim.x) {
            a.idx_user[i] = ld_dev(a.idx + i);
            a.w_user[i] = ld_dev(a.w + i);
        }
    build_union(a, u);
}

// T > 8: one workgroup per token.
__global__ void __launch_bounds__(256) k_select_tokens(SelArgs a)
{
    extern __shared__ double dyn_lds[];
    SelShared sh = sel_view(reinterpret_cast<char *>(dyn_lds), 1, a.E, a.top_k, a.n_group);
    const int t = blockIdx.x;
    if (a.given_idx) {
        for (int j = threadIdx.x; j < a.top_k; j += blockDim.x) {
            st_dev(a.idx + t * a.top_k + j, a.given_idx[t * a.top_k + j]);
            st_dev(a.w + t * a.top_k + j, a.given_w[t * a.top_k + j]);
        }
        __syncthreads();
    } else {
        select_tokens_block(a, t, 1, sh);
    }
    if (a.idx_user)
        for (int j = threadIdx.x; j < a.top_k; j += blockDim.x) {
            a.idx_user[t * a.top_k + j] = ld_dev(a.idx + t * a.top_k + j);
            a.w_user[t * a.top_k + j] = ld_dev(a.w + t * a.top_k + j);
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
    {
        // exclusive scans of the pair and tile counts over buckets 0..nb
        // (thread e holds bucket e; entry nb, of count 0, gets the totals):
        // wave scans, then the wave totals, then both added together
        __shared__ int wsum[2][16];
        const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
        const int c = e < nb ? cnt[e] : 0, tc = (c + TILE_M - 1) / TILE_M;
        int ic = c, it = tc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int oc = __shfl_up(ic, d), ot = __shfl_up(it, d);
            if (lane >= d) { ic += oc; it += ot; }
        }
        if (lane == 63) { wsum[0][wave] = ic; wsum[1][wave] = it; }
        __syncthreads();
        int bc = 0, bt = 0;
        for (int w = 0; w < wave; ++w) { bc += wsum[0][w]; bt += wsum[1][w]; }
        if (e <= nb) { off[e] = bc + ic - c; toff[e] = bt + it - tc; }
        __syncthreads();
        if (e == 0) a.ctrl[CTRL_N_TILES_GU] = toff[nb];
    }
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

int logits_splits(int T, int E, int H)
{
    const long tiles = (long)((T + LG_T - 1) / LG_T) * ((E + LG_E - 1) / LG_E);
    const int nchunk = H / LG_K;
    int ns = 1;
    while (ns * 2 <= MAX_SPLIT && tiles * ns * 2 <= 1024 && nchunk % (ns * 2) == 0) ns *= 2;
    return ns;
}

hipError_t launch_logits(const coli_moe_layer &L, const float *x, int T, double *z, int8_t *xq, float *xs,
                         bool split, hipStream_t s)
{
    if (split) {
        if (xq) {
            hipError_t e = launch_quant_q8(x, T, L.H, xq, xs, true, s);
            if (e != hipSuccess) return e;
        }
        const int ns = logits_splits(T, L.E, L.H);
        COLI_LAUNCH(k_logits_split, dim3((T + LG_T - 1) / LG_T, (L.E + LG_E - 1) / LG_E, ns), dim3(256), 0,
                           s, L.router_w, x, T, L.H, L.E, L.H / ns, z);
    } else if (T <= 1) {
        COLI_LAUNCH(k_logits_small<1>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    } else if (T <= 2) {
        COLI_LAUNCH(k_logits_small<2>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    } else if (T <= 4) {
        COLI_LAUNCH(k_logits_small<4>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    } else {
        COLI_LAUNCH(k_logits_small<8>, dim3(L.E), dim3(256), 0, s, L.router_w, x, T, L.H, L.E, z, xq, xs);
    }
    return hipGetLastError();
}

hipError_t launch_select(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws,
                         const int32_t *given_idx, const float *given_w, int32_t *idx_out, float *w_out,
                         hipStream_t s)
{
    SelArgs a;
    a.z = reinterpret_cast<const double *>(ws + lay.logits);
    a.n_part = lay.path == 1 ? logits_splits(T, L.E, L.H) : 1;
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
        const size_t lds = sel_lds_bytes(T, L.E, L.top_k, L.n_group) + union_lds_bytes(T, L.E, L.top_k);
        COLI_LAUNCH(k_select_union, dim3(1), dim3(1024), lds, s, a);
        return hipGetLastError();
    }
    COLI_LAUNCH(k_select_tokens, dim3(T), dim3(256), sel_lds_bytes(1, L.E, L.top_k, L.n_group), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    BucketArgs b;
    b.idx = a.idx; b.T = T; b.E = L.E; b.top_k = L.top_k; b.has_shared = L.has_shared; b.ctrl = a.ctrl;
    b.expert_off = reinterpret_cast<int *>(ws + lay.expert_off);
    b.pair_tok = reinterpret_cast<int *>(ws + lay.pair_tok);
    b.pair_of = a.pair_of; b.shared_pair = a.shared_pair;
    b.tiles = reinterpret_cast<int2 *>(ws + lay.tiles);
    COLI_LAUNCH(k_bucket, dim3(1), dim3(1024), 0, s, b);
    return hipGetLastError();
}

} // namespace coli
