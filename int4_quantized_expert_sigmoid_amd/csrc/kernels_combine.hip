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

__global__ void __launch_bounds__(256) k_combine(const float *__restrict__ ye, const int *__restrict__ pair_of,
                                                 const int *__restrict__ shared_pair, const float *__restrict__ w,
                                                 int T, int H, int top_k, int has_shared, float *__restrict__ y,
                                                 int accumulate)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)T * H) return;
    const int t = (int)(i / H), r = (int)(i % H);
    double acc = 0.0;
    for (int j = 0; j < top_k; ++j)
        acc += (double)w[t * top_k + j] * (double)ye[(long)pair_of[t * top_k + j] * H + r];
    if (has_shared) acc += (double)ye[(long)shared_pair[t] * H + r];
    const float out = (float)acc;
    y[i] = accumulate ? __fadd_rn(y[i], out) : out;
}

} // namespace

hipError_t launch_combine(const coli_moe_layer &L, int T, const WsLayout &lay, const char *ws, const float *w,
                          float *y, bool accumulate, hipStream_t s)
{
    const long n = (long)T * L.H;
    COLI_LAUNCH(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float *>(ws + lay.ye), reinterpret_cast<const int *>(ws + lay.pair_of),
                       reinterpret_cast<const int *>(ws + lay.shared_pair), w, T, L.H, L.top_k, L.has_shared, y,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

} // namespace coli
