// kernels_combine.hip — routing-weighted combine with the always-on shared
// expert (colibri architecture overview, section 5; ai4coding.ru summary,
// "what is implemented"):
//   y_t = sum_j w_tj * y_{t,e_j} + y_{t,shared},
// summed in f64 in the token's top-k order with the shared expert last, so
// every output element is one deterministic sum (no atomics).
#include "device_common.hpp"
#include "internal.hpp"

namespace coli {
namespace {

// One workgroup covers 4 * 256 consecutive outputs of one token, four per
// thread: the token's routing is uniform over the workgroup (scalar loads),
// and every term's 16-byte load is issued before the sums, which then run
// per element in slot order, the shared expert last.
constexpr int CMB_THREADS = 256, CMB_VEC = 4;

__global__ void __launch_bounds__(CMB_THREADS) k_combine(const float *__restrict__ ye, const int *__restrict__ pair_of,
                                                         const int *__restrict__ shared_pair,
                                                         const float *__restrict__ w, int T, int H, int top_k,
                                                         int has_shared, float *__restrict__ y, int accumulate)
{
    const int chunks = (H + CMB_THREADS * CMB_VEC - 1) / (CMB_THREADS * CMB_VEC);
    const int t = (int)blockIdx.x / chunks;
    const int r = ((int)blockIdx.x % chunks) * CMB_THREADS * CMB_VEC + (int)threadIdx.x * CMB_VEC;
    if (t >= T || r >= H) return;
    float4 v[COLI_MAX_TOPK + 1];
    float wt[COLI_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < COLI_MAX_TOPK; ++j) {
        if (j < top_k) {
            wt[j] = w[t * top_k + j];
            v[j] = *reinterpret_cast<const float4 *>(ye + (long)pair_of[t * top_k + j] * H + r);
        }
    }
    if (has_shared) v[COLI_MAX_TOPK] = *reinterpret_cast<const float4 *>(ye + (long)shared_pair[t] * H + r);
    double acc[CMB_VEC] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < COLI_MAX_TOPK; ++j) {
        if (j < top_k) {
            const double wj = (double)wt[j];
            acc[0] += wj * (double)v[j].x;
            acc[1] += wj * (double)v[j].y;
            acc[2] += wj * (double)v[j].z;
            acc[3] += wj * (double)v[j].w;
        }
    }
    if (has_shared) {
        acc[0] += (double)v[COLI_MAX_TOPK].x;
        acc[1] += (double)v[COLI_MAX_TOPK].y;
        acc[2] += (double)v[COLI_MAX_TOPK].z;
        acc[3] += (double)v[COLI_MAX_TOPK].w;
    }
    float4 out = make_float4((float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]);
    float4 *dst = reinterpret_cast<float4 *>(y + (long)t * H + r);
    if (accumulate) {
        const float4 o = *dst;
        out = make_float4(__fadd_rn(o.x, out.x), __fadd_rn(o.y, out.y), __fadd_rn(o.z, out.z), __fadd_rn(o.w, out.w));
    }
    *dst = out;
}

} // namespace

hipError_t launch_combine(const coli_moe_layer &L, int T, const WsLayout &lay, const char *ws, const float *w,
                          float *y, bool accumulate, hipStream_t s)
{
    // H % 32 == 0 and 16-byte aligned rows (workspace regions are 256-byte
    // aligned; y is 16-byte aligned), so every float4 is whole
    const long chunks = (L.H + CMB_THREADS * CMB_VEC - 1) / (CMB_THREADS * CMB_VEC);
    COLI_LAUNCH(k_combine, dim3((unsigned)(T * chunks)), dim3(CMB_THREADS), 0, s,
                       reinterpret_cast<const float *>(ws + lay.ye), reinterpret_cast<const int *>(ws + lay.pair_of),
                       reinterpret_cast<const int *>(ws + lay.shared_pair), w, T, L.H, L.top_k, L.has_shared, y,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

} // namespace coli
