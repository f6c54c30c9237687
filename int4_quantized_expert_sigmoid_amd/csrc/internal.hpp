// internal.hpp — kernel launchers of the layer and the workspace layout.
// Host-side declarations only; every launcher enqueues on `s` and returns
// the HIP status of its launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "../../include/coli_moe.h"

namespace coli {

// Kernel-exact timing of one layer call (coli_moe_forward_timed): while a
// timer is installed on the calling thread, every launch records its own
// start and stop (the kernel packet's timestamps) in the next event pair.
struct KernelTimer {
    const hipEvent_t *start, *stop;
    const char **names;          // optional: the kernel expression of each launch
    int n, next;                 // event pairs; launches so far (past n: untimed)
};
KernelTimer *&kernel_timer();    // this thread's timer, nullptr outside a timed call

#define COLI_LAUNCH(kernel, grid, block, shmem, stream, ...)                                               \
    do {                                                                                                    \
        ::coli::KernelTimer *kt_ = ::coli::kernel_timer();                                                  \
        const int i_ = kt_ ? kt_->next++ : 0;                                                               \
        if (kt_ && i_ < kt_->n) {                                                                           \
            if (kt_->names) kt_->names[i_] = #kernel;                                                       \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, kt_->start[i_], kt_->stop[i_], 0,     \
                                  __VA_ARGS__);                                                             \
        } else {                                                                                            \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                            \
        }                                                                                                   \
    } while (0)

// Workgroups of 256 threads of one kernel that fit on the current device at
// once (its occupancy per CU times the CUs), queried once per (device,
// kernel); 0 if the query fails.
template <typename K>
int resident_wg_256(K kernel)
{
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const auto key = std::make_pair(dev, reinterpret_cast<const void *>(kernel));
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int ncu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || ncu <= 0 || per_cu <= 0)
        return 0;
    cache[key] = ncu * per_cu;
    return ncu * per_cu;
}

constexpr int QK = 32;          // activation block width (Q8_0-style)
constexpr int MAX_SLOTS = 8;    // token slots of one expert item on the GEMV path

// Byte offsets of every workspace region for one (layer, T, path).
struct WsLayout {
    int path;            // 0 GEMV, 1 grouped
    int T, max_items, n_pairs;
    size_t ctrl, xq, xs, logits, keys, idx, w;   // keys: [2][T][E] f64 (key, sigmoid), GEMV path
    size_t item_expert, item_ntok, item_tok;     // GEMV path items
    size_t pair_of, shared_pair;
    size_t pair_tok, expert_off, tiles;          // grouped path buckets and tile list
    size_t h, hq, hs, ye;
    size_t xn;                                   // [T][H] f32: the RMSNorm of raw rows (coli_moe_forward_rms off the decode launches)
    size_t total;
};

WsLayout make_layout(const coli_moe_layer &L, int T, int path);

// Control words at the start of the workspace.
enum CtrlWord { CTRL_N_ITEMS = 0, CTRL_N_TILES_GU = 1, CTRL_N_TILES_DN = 2, CTRL_WORDS = 64 };

// ---- quantisation, packing, norms (kernels_quant.hip)
hipError_t launch_quant_q8(const float *x, int T, int H, int8_t *xq, float *xs, bool reorder, hipStream_t s);
hipError_t launch_reorder_q8(const int8_t *xq_nat, int n, int8_t *xq_perm, hipStream_t s);
// log2(group / 32) of a layer with group scales (0 without them).
inline int group_shift(const coli_moe_layer &L)
{
    int sh = 0;
    while (L.group_size > 0 && (QK << sh) < L.group_size) ++sh;
    return sh;
}

hipError_t launch_pack_int4(const float *w, int rows, int cols, uint8_t *q, float *sc, hipStream_t s);
hipError_t launch_pack_int8(const float *w, int rows, int cols, int8_t *q, float *sc, hipStream_t s);
hipError_t launch_pack_int2(const float *w, int rows, int cols, uint8_t *q, float *sc, hipStream_t s);
hipError_t launch_pack_int4_groups(const float *w, int rows, int cols, int group, uint8_t *q, float *sc, hipStream_t s);
hipError_t launch_rmsnorm(const float *x, const float *g, int T, int H, float eps, float *out, hipStream_t s);
// The float4 order of the RMSNorm sums (x 16-byte aligned, H % 4 == 0): the
// same rule wherever a row's scale is taken.
inline bool rms_vec(const float *x, int H) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && H % 4 == 0; }
hipError_t launch_block_dots(const uint8_t *q4, const int8_t *q8, int rows, int cols, int32_t *S, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_copy_f32(const float *src, float *dst, size_t n, hipStream_t s);

// ---- router (kernels_route.hip)
// Slices of H the large-batch logits are split into (their partial sums are
// [slices][T][E] f64 at z and are added in order by the selection).
int logits_splits(int T, int E, int H);
// Router logits z [T][E] (f64; with split, as logits_splits() partial sums);
// with xq != nullptr also Q8(x) in the reordered layout.
hipError_t launch_logits(const coli_moe_layer &L, const float *x, int T, double *z, int8_t *xq, float *xs,
                         bool split, hipStream_t s);   // split: the grouped-path layout (lay.path == 1)
// Top-k of every token from logits (or, with given_idx, from the caller's
// routing), then the batch union of experts (GEMV path) or the per-expert
// buckets and tile lists (grouped path).
hipError_t launch_select(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws,
                         const int32_t *given_idx, const float *given_w,
                         int32_t *idx_out, float *w_out, hipStream_t s);

// ---- experts, GEMV path (kernels_gemv.hip)
// Items item0.. of the union (item0 = 1 skips the shared expert, item 0).
hipError_t launch_gateup_gemv(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, int item0,
                              hipStream_t s);
hipError_t launch_down_gemv(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, int item0,
                            hipStream_t s);

// ---- decode / verify layer in three launches (kernels_decode.hip), T <= 8:
// router logits + keys + Q8(x); shared gate/up beside per-workgroup
// top-k/union + routed gate/up; down of every item + combine into y.
// gamma != nullptr: x holds raw rows and the launch takes their RMSNorm
// (gains gamma, eps) first (H <= 8192).
hipError_t launch_decode_router(const coli_moe_layer &L, const float *x, int T, const WsLayout &lay, char *ws,
                                const float *gamma, float eps, hipStream_t s);
hipError_t launch_decode_select_gateup(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s);
hipError_t launch_decode_down_combine(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, float *y,
                                      bool accumulate, hipStream_t s);   // T <= 2
// ---- experts, grouped int8-MFMA path (kernels_grouped.hip)
hipError_t launch_gateup_grouped(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s);
hipError_t launch_down_grouped(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s);

// ---- dense MLP (kernels_dense.hip); its workspace uses the WsLayout fields
// ctrl, xq, xs, h, hq, hs, ye, xn, tiles, expert_off, pair_tok (pair p = token p)
typedef coli_dense_mlp DenseLayer;
typedef WsLayout DenseLayout;
WsLayout make_dense_layout(const coli_dense_mlp &M, int T);
// T <= 8 tokens from token t0 on (their Q8(x), h, hq, hs and y rows)
hipError_t launch_dense_gemv(const DenseLayer &M, int T, int t0, const DenseLayout &lay, char *ws, float *y, bool accumulate,
                             hipStream_t s);
hipError_t launch_dense_setup(int T, const DenseLayout &lay, char *ws, hipStream_t s);
hipError_t launch_dense_out(int T, int H, const DenseLayout &lay, const char *ws, float *y, bool accumulate,
                            hipStream_t s);

// ---- combine (kernels_combine.hip)
hipError_t launch_combine(const coli_moe_layer &L, int T, const WsLayout &lay, const char *ws,
                          const float *w, float *y, bool accumulate, hipStream_t s);

} // namespace coli
