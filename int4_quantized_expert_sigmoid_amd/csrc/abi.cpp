// abi.cpp — the C ABI of include/coli_moe.h: argument validation, workspace
// layout, path dispatch and the host int4 packer. No C++ exception crosses
// the boundary; every failure is a status code returned before any launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "internal.hpp"

namespace coli {

KernelTimer *&kernel_timer()
{
    static thread_local KernelTimer *t = nullptr;
    return t;
}

namespace {

constexpr size_t ALIGN = 256;
inline size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
inline bool al16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Group scales: int4 only; the group is whole 32-wide blocks, a power of two
// of them, and divides both row lengths.
bool group_ok(int G, int H, int I, int wbits)
{
    if (wbits == 8 || wbits == 2 || G < QK || G > 4096 || G % QK) return false;
    const int nb = G / QK;
    if (nb & (nb - 1)) return false;
    return H % G == 0 && I % G == 0;
}

bool layer_ok(const coli_moe_layer *L)
{
    if (!L) return false;
    if (L->H <= 0 || L->I <= 0 || L->H % 32 || L->I % 32 || L->H > 65536 || L->I > 65536) return false;
    if (L->E < 1 || L->E > 512) return false;
    if (L->top_k < 1 || L->top_k > COLI_MAX_TOPK || L->top_k > L->E) return false;
    if (L->n_group < 1 || L->n_group > 64 || L->E % L->n_group) return false;
    if (L->topk_group < 1 || L->topk_group > L->n_group) return false;
    if (L->n_group > 1 && L->top_k > L->topk_group * (L->E / L->n_group)) return false;
    if (L->has_shared != 0 && L->has_shared != 1) return false;
    if (!std::isfinite(L->route_scale)) return false;
    if (L->weight_bits != 0 && L->weight_bits != 2 && L->weight_bits != 4 && L->weight_bits != 8) return false;
    if (L->group_size != 0 && !group_ok(L->group_size, L->H, L->I, L->weight_bits)) return false;
    if (!al4(L->router_w) || !al4(L->router_b)) return false;
    if (!al16(L->gate_q) || !al16(L->up_q) || !al16(L->down_q)) return false;
    if (!al4(L->gate_s) || !al4(L->up_s) || !al4(L->down_s)) return false;
    return true;
}

bool gemv_shape_ok(const coli_moe_layer &L) { return L.H <= 8192 && L.I <= 2048; }

bool dense_ok(const coli_dense_mlp *M)
{
    if (!M) return false;
    if (M->H <= 0 || M->I <= 0 || M->H % 32 || M->I % 32 || M->H > 8192 || M->I > 16384) return false;
    if (M->weight_bits != 0 && M->weight_bits != 4 && M->weight_bits != 8) return false;
    if (!al16(M->gate_q) || !al16(M->up_q) || !al16(M->down_q)) return false;
    if (!al4(M->gate_s) || !al4(M->up_s) || !al4(M->down_s)) return false;
    return true;
}

constexpr int KNOWN_FLAGS = COLI_ACCUMULATE | COLI_PATH_GEMV | COLI_PATH_GROUPED;

int choose_path(const coli_moe_layer &L, int T, int flags)
{
    if (flags & COLI_PATH_GROUPED) return 1;
    if (flags & COLI_PATH_GEMV) return 0;
    return (T <= COLI_GEMV_MAX_T && gemv_shape_ok(L)) ? 0 : 1;
}

int status(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_EDEVICE; }

} // namespace

WsLayout make_layout(const coli_moe_layer &L, int T, int path)
{
    WsLayout o;
    std::memset(&o, 0, sizeof(o));
    o.path = path;
    o.T = T;
    const size_t H = (size_t)L.H, I = (size_t)L.I, k = (size_t)L.top_k, E = (size_t)L.E, t = (size_t)T;
    size_t n_pairs, n_tiles = 0;
    if (path == 0) {
        o.max_items = (int)(t * k + (size_t)L.has_shared);
        n_pairs = (size_t)o.max_items * MAX_SLOTS;
    } else {
        o.max_items = 0;
        n_pairs = t * k + t * (size_t)L.has_shared;
        n_tiles = (n_pairs + 31) / 32 + E + 1;
    }
    o.n_pairs = (int)n_pairs;
    size_t p = 0;
    o.ctrl = p; p = up(p + CTRL_WORDS * 4);
    o.xq = p; p = up(p + t * H);
    o.xs = p; p = up(p + t * (H / 32) * 4);
    o.logits = p; p = up(p + t * E * 8 * (size_t)(path == 1 ? logits_splits(T, L.E, L.H) : 1));
    o.keys = p; p = up(p + (path == 0 ? 2 * t * E * 8 : 0));
    o.idx = p; p = up(p + t * k * 4);
    o.w = p; p = up(p + t * k * 4);
    o.item_expert = p; p = up(p + (size_t)o.max_items * 4);
    o.item_ntok = p; p = up(p + (size_t)o.max_items * 4);
    o.item_tok = p; p = up(p + (size_t)o.max_items * MAX_SLOTS * 4);
    o.pair_of = p; p = up(p + t * k * 4);
    o.shared_pair = p; p = up(p + t * 4);
    o.pair_tok = p; p = up(p + (path == 1 ? n_pairs * 4 : 0));
    o.expert_off = p; p = up(p + (path == 1 ? (E + 2) * 4 : 0));
    o.tiles = p; p = up(p + n_tiles * 8);
    o.h = p; p = up(p + n_pairs * I * 4);
    o.hq = p; p = up(p + n_pairs * I);
    o.hs = p; p = up(p + n_pairs * (I / 32) * 4);
    o.ye = p; p = up(p + n_pairs * H * 4);
    o.xn = p; p = up(p + t * H * 4);
    o.total = p;
    return o;
}

WsLayout make_dense_layout(const coli_dense_mlp &M, int T)
{
    WsLayout o;
    std::memset(&o, 0, sizeof(o));
    const size_t H = (size_t)M.H, I = (size_t)M.I, t = (size_t)T;
    o.path = T <= COLI_GEMV_MAX_T ? 0 : 1;
    o.T = T;
    o.n_pairs = T;
    const size_t pairs = t < MAX_SLOTS ? MAX_SLOTS : t;   // the GEMV body indexes item 0's slots
    size_t p = 0;
    o.ctrl = p; p = up(p + CTRL_WORDS * 4);
    o.xn = p; p = up(p + t * H * 4);
    o.xq = p; p = up(p + t * H);
    o.xs = p; p = up(p + t * (H / 32) * 4);
    o.h = p; p = up(p + pairs * I * 4);
    o.hq = p; p = up(p + pairs * I);
    o.hs = p; p = up(p + pairs * (I / 32) * 4);
    o.ye = p; p = up(p + t * H * 4);
    o.tiles = p; p = up(p + ((t + 31) / 32) * 8);
    o.expert_off = p; p = up(p + 2 * 4);
    o.pair_tok = p; p = up(p + t * 4);
    o.total = p;
    return o;
}

} // namespace coli

using namespace coli;

extern "C" {

const char *coli_version(void) { return "coli-moe-mi355x 0.1 (gfx950)"; }

int coli_quant_act_q8(const float *x, int T, int H, int8_t *xq, float *xs, void *stream)
{
    if (T < 1 || T > COLI_MAX_T || H <= 0 || H % 32 || !al16(x) || !al16(xq) || !al4(xs)) return COLI_EINVAL;
    return status(launch_quant_q8(x, T, H, xq, xs, false, (hipStream_t)stream));
}

size_t coli_moe_workspace_bytes(const coli_moe_layer *L, int T)
{
    if (!layer_ok(L) || T < 1 || T > COLI_MAX_T) return 0;
    size_t b = make_layout(*L, T, 1).total;
    if (T <= COLI_GEMV_MAX_T && gemv_shape_ok(*L)) {
        const size_t g = make_layout(*L, T, 0).total;
        if (g > b) b = g;
    }
    return b;
}

int coli_moe_workspace_init(void *ws, size_t ws_bytes, void *stream)
{
    if (!al16(ws) || ws_bytes == 0) return COLI_EINVAL;
    return status(launch_zero(ws, ws_bytes, (hipStream_t)stream));
}

int coli_moe_workspace_layout(const coli_moe_layer *L, int T, int flags, coli_moe_ws_layout *out)
{
    if (!layer_ok(L) || T < 1 || T > COLI_MAX_T || !out) return COLI_EINVAL;
    if (flags & ~KNOWN_FLAGS) return COLI_EINVAL;
    const int path = choose_path(*L, T, flags);
    const WsLayout l = make_layout(*L, T, path);
    out->xq = l.xq; out->xs = l.xs; out->idx = l.idx; out->w = l.w;
    out->pair_of = l.pair_of; out->shared_pair = l.shared_pair;
    out->h = l.h; out->hq = l.hq; out->hs = l.hs; out->ye = l.ye;
    out->n_pairs_max = (size_t)l.n_pairs;
    out->path = path;
    return COLI_OK;
}

static int check_common(const coli_moe_layer *L, int T, int flags, void *ws, size_t ws_bytes, int &path,
                        WsLayout &lay)
{
    if (!layer_ok(L) || T < 1 || T > COLI_MAX_T) return COLI_EINVAL;
    if (flags & ~KNOWN_FLAGS) return COLI_EINVAL;
    if ((flags & COLI_PATH_GEMV) && (flags & COLI_PATH_GROUPED)) return COLI_EINVAL;
    if ((flags & COLI_PATH_GEMV) && (T > COLI_GEMV_MAX_T || !gemv_shape_ok(*L))) return COLI_EINVAL;
    if (!al16(ws)) return COLI_EINVAL;
    path = choose_path(*L, T, flags);
    lay = make_layout(*L, T, path);
    if (ws_bytes < lay.total) return COLI_EWORKSPACE;
    return COLI_OK;
}

static int record(void *const *ev, int i, hipStream_t s)
{
    if (!ev) return COLI_OK;
    return hipEventRecord((hipEvent_t)ev[i], s) == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

// Expert launches from item0 on (item0 = 1: the shared expert already ran).
static int run_experts(const coli_moe_layer *L, int T, const WsLayout &lay, char *ws, float *y, int flags,
                       int item0, hipStream_t s, void *const *ev)
{
    hipError_t e;
    if (lay.path == 0) {
        if ((e = launch_gateup_gemv(*L, T, lay, ws, item0, s)) != hipSuccess) return COLI_EDEVICE;
        if (record(ev, 3, s)) return COLI_EDEVICE;
        if ((e = launch_down_gemv(*L, T, lay, ws, item0, s)) != hipSuccess) return COLI_EDEVICE;
        if (record(ev, 4, s)) return COLI_EDEVICE;
    } else {
        if ((e = launch_gateup_grouped(*L, T, lay, ws, s)) != hipSuccess) return COLI_EDEVICE;
        if (record(ev, 3, s)) return COLI_EDEVICE;
        if ((e = launch_down_grouped(*L, T, lay, ws, s)) != hipSuccess) return COLI_EDEVICE;
        if (record(ev, 4, s)) return COLI_EDEVICE;
    }
    e = launch_combine(*L, T, lay, ws, reinterpret_cast<const float *>(ws + lay.w), y,
                       (flags & COLI_ACCUMULATE) != 0, s);
    if (e != hipSuccess) return COLI_EDEVICE;
    return record(ev, 5, s);
}

// gamma != nullptr: x holds raw rows, and the layer's input is their
// RMSNorm with gains gamma and eps. The decode launches take it inside the
// router launch; the other paths run coli_rmsnorm's kernel into the
// workspace first.
static int forward_impl(const coli_moe_layer *L, const float *x, int T, float *y, int flags, void *ws,
                        size_t ws_bytes, void *stream, void *const *ev, const float *gamma = nullptr,
                        float eps = 0.0f)
{
    int path;
    WsLayout lay;
    int rc = check_common(L, T, flags, ws, ws_bytes, path, lay);
    if (rc != COLI_OK) return rc;
    if (!al16(x) || !al16(y)) return COLI_EINVAL;
    if (gamma && (!al16(gamma) || !(eps >= 0.0f) || !std::isfinite(eps))) return COLI_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    char *base = static_cast<char *>(ws);
    if (record(ev, 0, s)) return COLI_EDEVICE;
    const bool norm_in_router = gamma && path == 0;
    if (gamma && !norm_in_router) {
        float *xn = reinterpret_cast<float *>(base + lay.xn);
        if (launch_rmsnorm(x, gamma, T, L->H, eps, xn, s) != hipSuccess) return COLI_EDEVICE;
        x = xn;
    }
    if (path == 0) {
        // router (+ the shared expert's gate/up), routed gate/up, down + combine
        if (launch_decode_router(*L, x, T, lay, base, norm_in_router ? gamma : nullptr, eps, s) != hipSuccess)
            return COLI_EDEVICE;
        if (record(ev, 1, s)) return COLI_EDEVICE;
        if (launch_decode_select_gateup(*L, T, lay, base, s) != hipSuccess) return COLI_EDEVICE;
        if (record(ev, 2, s)) return COLI_EDEVICE;
        if (T <= 2) {
            if (launch_decode_down_combine(*L, T, lay, base, y, (flags & COLI_ACCUMULATE) != 0, s) != hipSuccess)
                return COLI_EDEVICE;
        } else {
            // wider batches: item-major down projection (activations of all
            // slots loaded once per 32 rows), then the combine
            if (launch_down_gemv(*L, T, lay, base, 0, s) != hipSuccess) return COLI_EDEVICE;
            if (launch_combine(*L, T, lay, base, reinterpret_cast<const float *>(base + lay.w), y,
                               (flags & COLI_ACCUMULATE) != 0, s) != hipSuccess)
                return COLI_EDEVICE;
        }
        for (int i = 3; i < COLI_PROFILE_EVENTS; ++i)
            if (record(ev, i, s)) return COLI_EDEVICE;
        return COLI_OK;
    }
    if (launch_logits(*L, x, T, reinterpret_cast<double *>(base + lay.logits),
                      reinterpret_cast<int8_t *>(base + lay.xq), reinterpret_cast<float *>(base + lay.xs),
                      lay.path == 1, s) != hipSuccess)
        return COLI_EDEVICE;
    if (record(ev, 1, s)) return COLI_EDEVICE;
    if (launch_select(*L, T, lay, base, nullptr, nullptr, nullptr, nullptr, s) != hipSuccess) return COLI_EDEVICE;
    if (record(ev, 2, s)) return COLI_EDEVICE;
    return run_experts(L, T, lay, base, y, flags, 0, s, ev);
}

int coli_moe_route(const coli_moe_layer *L, const float *x, int T, int32_t *idx, float *w, void *ws,
                   size_t ws_bytes, void *stream)
{
    int path;
    WsLayout lay;
    int rc = check_common(L, T, 0, ws, ws_bytes, path, lay);
    if (rc != COLI_OK) return rc;
    if (!al16(x) || !al4(idx) || !al4(w)) return COLI_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    char *base = static_cast<char *>(ws);
    if (launch_logits(*L, x, T, reinterpret_cast<double *>(base + lay.logits), nullptr, nullptr, lay.path == 1,
                      s) != hipSuccess)
        return COLI_EDEVICE;
    return status(launch_select(*L, T, lay, base, nullptr, nullptr, idx, w, s));
}

int coli_moe_forward(const coli_moe_layer *L, const float *x, int T, float *y, int flags, void *ws,
                     size_t ws_bytes, void *stream)
{
    return forward_impl(L, x, T, y, flags, ws, ws_bytes, stream, nullptr);
}

int coli_moe_forward_rms(const coli_moe_layer *L, const float *x, const float *gamma, float eps, int T, float *y,
                         int flags, void *ws, size_t ws_bytes, void *stream)
{
    if (!gamma) return COLI_EINVAL;
    return forward_impl(L, x, T, y, flags, ws, ws_bytes, stream, nullptr, gamma, eps);
}

// ---- coli_moe_forward_noalloc: the library's own device scratch in place
// of a caller workspace, for callers that cannot allocate. One copy of the
// array per GPU, alive until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): it uses the device address hipGetSymbolAddress returns, taken
// once per device with that device current.
static __device__ __align__(256) unsigned char scratch[COLI_NOALLOC_MAX_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES];     // device address of `scratch` on each device
bool g_scratch_zeroed[SCRATCH_MAX_DEVICES];   // zero-filled, and no call failed since

// The current device's scratch address (taken on its first call), or null
// when the runtime cannot give it.
void *scratch_of_current_device(int &dev)
{
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
        g_scratch_zeroed[dev] = false;
    }
    return g_scratch_ptr[dev];
}
} // namespace

int coli_moe_forward_noalloc(const coli_moe_layer *L, const float *x, int T, float *y, int flags, void *stream)
{
    int path;
    WsLayout lay;
    int dev = -1;
    // the size check needs no device: a call past the limit is refused first
    int rc = check_common(L, T, flags, reinterpret_cast<void *>(ALIGN), COLI_NOALLOC_MAX_BYTES, path, lay);
    if (rc != COLI_OK) return rc;
    void *ws = scratch_of_current_device(dev);
    if (!ws) return COLI_EDEVICE;
    hipStream_t s = (hipStream_t)stream;
    bool zeroed;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        zeroed = g_scratch_zeroed[dev];
    }
    // the workspace contract: zero-filled before the first use and after a
    // failed call (a fill kernel, not a memset)
    if (!zeroed) {
        if (launch_zero(ws, COLI_NOALLOC_MAX_BYTES, s) != hipSuccess) return COLI_EDEVICE;
    }
    rc = forward_impl(L, x, T, y, flags, ws, COLI_NOALLOC_MAX_BYTES, stream, nullptr);
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        g_scratch_zeroed[dev] = rc == COLI_OK || (rc != COLI_EDEVICE && zeroed);
    }
    return rc;
}

int coli_timer_begin(void *const *start, void *const *stop, int n_pairs, const char **names)
{
    if (n_pairs < 1 || !start || !stop) return COLI_EINVAL;
    for (int i = 0; i < n_pairs; ++i)
        if (!start[i] || !stop[i]) return COLI_EINVAL;
    KernelTimer *&slot = kernel_timer();
    if (slot) return COLI_EINVAL;                // one open scope per thread
    static thread_local KernelTimer scope;
    scope = KernelTimer{reinterpret_cast<const hipEvent_t *>(start), reinterpret_cast<const hipEvent_t *>(stop),
                        names, n_pairs, 0};
    slot = &scope;
    return COLI_OK;
}

int coli_timer_end(int *n_launches)
{
    KernelTimer *&slot = kernel_timer();
    if (!slot || !n_launches) return COLI_EINVAL;
    *n_launches = slot->next;
    slot = nullptr;
    return COLI_OK;
}

size_t coli_dense_workspace_bytes(const coli_dense_mlp *M, int T)
{
    if (!dense_ok(M) || T < 1 || T > COLI_MAX_T) return 0;
    return make_dense_layout(*M, T).total;
}

int coli_dense_forward(const coli_dense_mlp *M, const float *x, const float *gamma, float eps, int T, float *y,
                       int flags, void *ws, size_t ws_bytes, void *stream)
{
    if (!dense_ok(M) || T < 1 || T > COLI_MAX_T) return COLI_EINVAL;
    if (flags & ~(COLI_ACCUMULATE | COLI_PATH_GEMV | COLI_PATH_GROUPED)) return COLI_EINVAL;
    if ((flags & COLI_PATH_GEMV) && (flags & COLI_PATH_GROUPED)) return COLI_EINVAL;
    if ((flags & COLI_PATH_GEMV) && T > COLI_GEMV_MAX_T) return COLI_EINVAL;
    if (!al16(x) || !al16(y) || !al16(ws)) return COLI_EINVAL;
    if (gamma && (!al16(gamma) || !(eps >= 0.0f) || !std::isfinite(eps))) return COLI_EINVAL;
    const WsLayout lay = make_dense_layout(*M, T);
    if (ws_bytes < lay.total) return COLI_EWORKSPACE;
    const bool grouped = (flags & COLI_PATH_GROUPED) || (!(flags & COLI_PATH_GEMV) && T > COLI_GEMV_MAX_T);
    hipStream_t s = (hipStream_t)stream;
    char *base = static_cast<char *>(ws);
    const bool acc = (flags & COLI_ACCUMULATE) != 0;
    if (gamma) {
        float *xn = reinterpret_cast<float *>(base + lay.xn);
        if (launch_rmsnorm(x, gamma, T, M->H, eps, xn, s) != hipSuccess) return COLI_EDEVICE;
        x = xn;
    }
    if (launch_quant_q8(x, T, M->H, reinterpret_cast<int8_t *>(base + lay.xq), reinterpret_cast<float *>(base + lay.xs),
                        true, s) != hipSuccess)
        return COLI_EDEVICE;
    if (!grouped) return status(launch_dense_gemv(*M, T, 0, lay, base, y, acc, s));
    // one expert holding every token on the grouped kernels of the expert path
    coli_moe_layer L;
    std::memset(&L, 0, sizeof(L));
    L.H = M->H; L.I = M->I; L.E = 1; L.top_k = 1; L.n_group = 1; L.topk_group = 1; L.has_shared = 0;
    L.route_scale = 1.0f; L.weight_bits = M->weight_bits == 8 ? 8 : 4;
    L.gate_q = M->gate_q; L.up_q = M->up_q; L.down_q = M->down_q;
    L.gate_s = M->gate_s; L.up_s = M->up_s; L.down_s = M->down_s;
    WsLayout gl = lay;
    gl.path = 1;
    if (launch_dense_setup(T, lay, base, s) != hipSuccess) return COLI_EDEVICE;
    if (launch_gateup_grouped(L, T, gl, base, s) != hipSuccess) return COLI_EDEVICE;
    if (launch_down_grouped(L, T, gl, base, s) != hipSuccess) return COLI_EDEVICE;
    return status(launch_dense_out(T, M->H, lay, base, y, acc, s));
}

int coli_moe_forward_profiled(const coli_moe_layer *L, const float *x, int T, float *y, int flags, void *ws,
                              size_t ws_bytes, void *stream, void *const *events, int n_events)
{
    if (!events || n_events < COLI_PROFILE_EVENTS) return COLI_EINVAL;
    for (int i = 0; i < COLI_PROFILE_EVENTS; ++i)
        if (!events[i]) return COLI_EINVAL;
    return forward_impl(L, x, T, y, flags, ws, ws_bytes, stream, events);
}

int coli_moe_forward_timed(const coli_moe_layer *L, const float *x, const float *gamma, float eps, int T, float *y,
                           int flags, void *ws, size_t ws_bytes, void *stream, void *const *start,
                           void *const *stop, int n_pairs, int *n_launches, const char **names)
{
    if (!n_launches || n_pairs < 0 || (n_pairs > 0 && (!start || !stop))) return COLI_EINVAL;
    for (int i = 0; i < n_pairs; ++i)
        if (!start[i] || !stop[i]) return COLI_EINVAL;
    KernelTimer kt{reinterpret_cast<const hipEvent_t *>(start), reinterpret_cast<const hipEvent_t *>(stop), names,
                   n_pairs, 0};
    KernelTimer *&slot = kernel_timer();
    if (slot) return COLI_EINVAL;                // inside an open coli_timer_begin scope
    KernelTimer *const prev = slot;
    slot = &kt;
    const int rc = forward_impl(L, x, T, y, flags, ws, ws_bytes, stream, nullptr, gamma, eps);
    slot = prev;
    *n_launches = kt.next;
    return rc;
}

int coli_moe_experts(const coli_moe_layer *L, const int8_t *xq, const float *xs, const int32_t *idx,
                     const float *w, int T, float *y, int flags, void *ws, size_t ws_bytes, void *stream)
{
    int path;
    WsLayout lay;
    int rc = check_common(L, T, flags, ws, ws_bytes, path, lay);
    if (rc != COLI_OK) return rc;
    if (!al16(xq) || !al4(xs) || !al4(idx) || !al4(w) || !al16(y)) return COLI_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    char *base = static_cast<char *>(ws);
    if (launch_reorder_q8(xq, T * L->H, reinterpret_cast<int8_t *>(base + lay.xq), s) != hipSuccess)
        return COLI_EDEVICE;
    if (launch_copy_f32(xs, reinterpret_cast<float *>(base + lay.xs), (size_t)T * (L->H / 32), s) != hipSuccess)
        return COLI_EDEVICE;
    if (launch_select(*L, T, lay, base, idx, w, nullptr, nullptr, s) != hipSuccess) return COLI_EDEVICE;
    return run_experts(L, T, lay, base, y, flags, 0, s, nullptr);
}

int coli_rmsnorm(const float *x, const float *gamma, int T, int H, float eps, float *out, void *stream)
{
    if (T < 1 || T > COLI_MAX_T || H <= 0 || !al4(x) || !al4(gamma) || !al4(out)) return COLI_EINVAL;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return COLI_EINVAL;
    return status(launch_rmsnorm(x, gamma, T, H, eps, out, (hipStream_t)stream));
}

int coli_pack_int4_rows(const float *w, int rows, int cols, uint8_t *q, float *s)
{
    if (!w || !q || !s || rows < 1 || cols < 2 || (cols & 1)) return COLI_EINVAL;
    for (int r = 0; r < rows; ++r) {
        const float *src = w + (size_t)r * cols;
        float amax = 0.0f;
        for (int c = 0; c < cols; ++c) amax = std::fmax(amax, std::fabs(src[c]));
        const float d = amax / 7.0f;
        const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        s[r] = d;
        uint8_t *dst = q + (size_t)r * (cols / 2);
        for (int j = 0; j < cols / 2; ++j) {
            int code[2];
            for (int h = 0; h < 2; ++h) {
                const float v = src[2 * j + h] * id;
                float rv = std::isnan(v) ? 0.0f : std::rint(v);
                rv = rv < -8.0f ? -8.0f : (rv > 7.0f ? 7.0f : rv);
                code[h] = (int)rv;
            }
            dst[j] = (uint8_t)((code[0] & 0xF) | ((code[1] & 0xF) << 4));
        }
    }
    return COLI_OK;
}

int coli_pack_int4_rows_dev(const float *w, int rows, int cols, uint8_t *q, float *s, void *stream)
{
    if (!al4(w) || !q || !al4(s) || rows < 1 || cols < 2 || (cols & 1)) return COLI_EINVAL;
    return status(launch_pack_int4(w, rows, cols, q, s, (hipStream_t)stream));
}

int coli_pack_int2_rows_dev(const float *w, int rows, int cols, uint8_t *q, float *s, void *stream)
{
    if (!al4(w) || !al16(q) || !al4(s) || rows < 1 || cols < 32 || cols % 32) return COLI_EINVAL;
    return status(launch_pack_int2(w, rows, cols, q, s, (hipStream_t)stream));
}

int coli_pack_int4_groups_dev(const float *w, int rows, int cols, int group, uint8_t *q, float *s, void *stream)
{
    if (!al4(w) || !q || !al4(s) || rows < 1 || group < 2 || group > 4096 || (group & 1) || cols < group ||
        cols % group)
        return COLI_EINVAL;
    return status(launch_pack_int4_groups(w, rows, cols, group, q, s, (hipStream_t)stream));
}

int coli_pack_int8_rows(const float *w, int rows, int cols, int8_t *q, float *s)
{
    if (!w || !q || !s || rows < 1 || cols < 32 || (cols % 32)) return COLI_EINVAL;
    for (int r = 0; r < rows; ++r) {
        const float *src = w + (size_t)r * cols;
        float amax = 0.0f;
        for (int c = 0; c < cols; ++c) amax = std::fmax(amax, std::fabs(src[c]));
        const float d = amax / 127.0f;
        const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        s[r] = d;
        int8_t *dst = q + (size_t)r * cols;
        for (int c = 0; c < cols; ++c) {
            const float v = src[c] * id;
            float rv = std::isnan(v) ? 0.0f : std::rint(v);
            rv = rv < -127.0f ? -127.0f : (rv > 127.0f ? 127.0f : rv);
            const int j = c & 7;                 // byte of column j in its group of 8
            const int p = (c & 31 & ~7) + ((j & 1) ? 4 + (j >> 1) : (j >> 1));   // byte in its block
            dst[(p >> 4) * 16 * (cols / 32) + (c >> 5) * 16 + (p & 15)] = (int8_t)rv;
        }
    }
    return COLI_OK;
}

int coli_pack_int8_rows_dev(const float *w, int rows, int cols, int8_t *q, float *s, void *stream)
{
    if (!al4(w) || !al16(q) || !al4(s) || rows < 1 || cols < 32 || cols % 32) return COLI_EINVAL;
    return status(launch_pack_int8(w, rows, cols, q, s, (hipStream_t)stream));
}

int coli_debug_block_dots(const uint8_t *q4, const int8_t *q8, int rows, int cols, int32_t *S, void *stream)
{
    if (!al16(q4) || !al16(q8) || !al4(S) || rows < 1 || cols < 32 || cols % 32) return COLI_EINVAL;
    return status(launch_block_dots(q4, q8, rows, cols, S, (hipStream_t)stream));
}

} // extern "C"
