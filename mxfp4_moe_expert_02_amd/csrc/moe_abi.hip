// moe_abi.hip -- the C ABI (include/moe_mxfp4.h): validation, the per-device
// workspace, and the launch sequence of one MoE expert layer.
//
// Launch sequence of a forward on `stream` (no host synchronisation):
//   route (top-k + stable sort by expert + active-expert lists)
//   -> gate_up GEMM with the SiLU * up epilogue -> down GEMM -> combine
// (with a shared expert, its gate_up and down kernels run ahead of the
// routed ones in the same stages, and the combine adds its rows)
// (on the matrix-core paths the combine is its own kernel, or the
// last-finisher step of the single-launch layer; the VALU path combines by
// last finisher inside its down kernel).  Layers of at most 16 tokens on
// the bf16 matrix-core path skip the route: their GEMM workgroups rank
// their own experts (the self-routed layer).
// Every expert that received no token is absent from the active lists and
// costs no weight bytes: the layer reads only the experts its tokens use,
// the property the pages build the 4-bit expert format around (bjdmk.com.cn
// news page, co-design section).
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_mxfp4.h"
#include "moe_internal.h"

namespace {

using moe::Workspace;

constexpr int kMaxDevices = 64;
Workspace* g_ws[kMaxDevices] = {};
int g_num_ws = 0;  // number of live workspaces (0: nothing initialised)
std::mutex g_mu;
thread_local char g_hip_msg[256] = "";

int hip_fail(hipError_t err, const char* what) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s: %s (%d)", what, hipGetErrorString(err), (int)err);
    return MOE_E_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Lay the workspace out in one allocation (256-byte aligned sub-buffers).
size_t layout(Workspace* ws, char* base) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = round_up(off + bytes, 256);
        return p;
    };
    const size_t S = (size_t)ws->max_tokens * ws->kmax;
    ws->ids = (int32_t*)take(S * 4);
    ws->wts = (float*)take(S * 4);
    ws->counts = (int32_t*)take(ws->E * 4);
    ws->offsets = (int32_t*)take((ws->E + 1) * 4);
    ws->sorted = (int32_t*)take(S * 4);
    ws->pos = (int32_t*)take(S * 4);
    ws->gemv_list = (int32_t*)take(ws->E * 4);
    ws->mfma_list = (int32_t*)take(ws->E * 4);
    ws->mfma_items = (int4*)take((ws->E + S / moe::kMfmaTok + 1) * sizeof(int4));
    ws->meta = (int32_t*)take(moe::kMetaWords * 4);
    ws->col_tiles = (int)(ws->H / moe::kColTile);
    ws->tile_done = (int32_t*)take((size_t)ws->max_tokens * (ws->H / moe::kMfmaDownRows) * 4);
    ws->bhist = (int32_t*)take((S + moe::kRouteSlotBlock - 1) / moe::kRouteSlotBlock * ws->E * 4);
    ws->max_items = (int)(ws->E + S / moe::kMfmaTok + 1);
    ws->queue = (int32_t*)take(moe::kQueueWords * 4);
    ws->gu_done = (int32_t*)take((size_t)ws->max_items * moe::kLineInts * 4);
    ws->slot_lists = (int32_t*)take((size_t)ws->E * moe::kSlotListInts * 4);
    ws->flags = (int32_t*)take((size_t)moe::self_flag_words(ws->E) * 4);
    const size_t TE = (size_t)ws->max_tokens * ws->E;
    const size_t split_te = TE < (size_t)moe::kRouterWaves * 512 ? TE : (size_t)moe::kRouterWaves * 512;
    ws->logits = (float*)take(TE * 4);
    ws->router_partial = (float*)take((size_t)moe::kRouterMaxSplit * split_te * 4);
    ws->router_cnt = (int32_t*)take((size_t)2 * moe::kRouterWaves * 4);
    const size_t R = S + (size_t)ws->max_tokens;  // routed rows, then the shared expert's
    ws->h = (uint16_t*)take(R * ws->I * 4);  // bf16 hi/lo pairs (GEMV path)
    ws->h3q = (uint8_t*)take(R * ws->I * 3);  // three MXFP8 terms (matrix-core paths)
    ws->h3s = (uint8_t*)take(R * moe::h3s_stride(ws->I));
    ws->y = (float*)take(R * ws->H * 4);
    ws->x_codes = (uint8_t*)take((size_t)ws->max_tokens * ws->H);
    ws->x_scales = (uint8_t*)take((size_t)ws->max_tokens * (ws->H / 32));
    ws->h_codes = (uint8_t*)take(R * ws->I);
    ws->h_scales = (uint8_t*)take(R * (ws->I / 32));
    return off;
}

void free_ws(Workspace* ws) {
    if (!ws) return;
    if (ws->base) {  // best effort: nothing to report to from here
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(ws->device);
        (void)hipDeviceSynchronize();
        (void)hipFree(ws->base);
        (void)hipSetDevice(cur);
    }
    delete ws;
}

// Workspace of the current device, or null (without any HIP call when no
// device has been initialised).
Workspace* current_ws() {
    if (g_num_ws == 0) return nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    return g_ws[dev];
}

// ---- the allocation-free verify layer (moe_mxfp4_forward_noalloc): the
// self-routed layer of at most kNaMaxTokens tokens, its working set in one
// file-scope device array instead of a workspace.  Byte offsets of its
// pieces, each sized for the largest accepted layer (rows = tokens x top_k,
// row strides those of the call):
constexpr int64_t kNaMaxTokens = 16, kNaMaxExperts = 256, kNaMaxTopK = 8;
constexpr int64_t kNaMaxHidden = 8192, kNaMaxInter = 4096;
constexpr size_t kNaRows = (size_t)(kNaMaxTokens * kNaMaxTopK);
constexpr size_t kNaLists = 0;  // [E][kSlotListInts] int32: per-expert slot lists
constexpr size_t kNaIds = kNaLists + (size_t)kNaMaxExperts * moe::kSlotListInts * 4;  // [T*k] int32
constexpr size_t kNaWts = kNaIds + kNaRows * 4;                                       // [T*k] fp32
constexpr size_t kNaH3q = kNaWts + kNaRows * 4;                          // [T*k][3I] h's term codes
constexpr size_t kNaH3s = kNaH3q + kNaRows * 3 * (size_t)kNaMaxInter;      // [T*k][h3s_stride(I)] their scales
constexpr size_t kNaY = kNaH3s + kNaRows * (size_t)moe::h3s_stride(kNaMaxInter);  // [T*k][H] fp32
constexpr size_t kNaBytes = kNaY + kNaRows * (size_t)kNaMaxHidden * 4;     // 5.6 MB
static_assert(kNaH3q % 256 == 0 && kNaH3s % 256 == 0 && kNaY % 256 == 0, "aligned pieces");

// per device: the device address of `scratch`, taken once
void* g_na_scratch[kMaxDevices] = {};
std::mutex g_na_mu;

}  // namespace

// The allocation-free entry point's working set (see kNaBytes).  Host code
// uses its device address from hipGetSymbolAddress, never this name.
static __device__ __align__(256) uint8_t scratch[kNaBytes];

namespace {

// The current device's address of `scratch` (taken on its first call there)
hipError_t na_scratch(uint8_t** p) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_na_mu);
    if (!g_na_scratch[dev]) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        g_na_scratch[dev] = ptr;
    }
    *p = (uint8_t*)g_na_scratch[dev];
    return hipSuccess;
}

}  // namespace

namespace moe {

hipError_t resident_grid(const void* kernel, int block, int* grid) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
    if (err != hipSuccess) return err;
    *grid = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    return hipSuccess;
}

}  // namespace moe

extern "C" {

int moe_mxfp4_init(int64_t max_tokens, int64_t num_experts, int64_t hidden, int64_t inter,
                   int32_t max_top_k) {
    if (max_tokens < 1 || max_tokens > (1 << 20)) return MOE_E_SHAPE;
    if (num_experts < 1 || num_experts > moe::kMaxExperts) return MOE_E_SHAPE;
    if (hidden < 128 || hidden > 16384 || hidden % 128) return MOE_E_SHAPE;
    if (inter < 128 || inter > 16384 || inter % 128) return MOE_E_SHAPE;
    if (max_top_k < 1 || max_top_k > moe::kMaxTopK || max_top_k > num_experts) return MOE_E_TOPK;
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice, "device index");
    Workspace* ws = new Workspace();
    ws->device = dev;
    ws->max_tokens = max_tokens;
    ws->E = num_experts;
    ws->H = hidden;
    ws->I = inter;
    ws->kmax = max_top_k;
    ws->bytes = layout(ws, nullptr);
    err = hipMalloc(&ws->base, ws->bytes);
    if (err != hipSuccess) {
        ws->base = nullptr;
        delete ws;
        return hip_fail(err, "hipMalloc(workspace)");
    }
    layout(ws, (char*)ws->base);
    err = hipMemset(ws->base, 0, ws->bytes);
    if (err != hipSuccess) {
        free_ws(ws);
        return hip_fail(err, "hipMemset(workspace)");
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ws[dev]) {
        free_ws(g_ws[dev]);
        g_num_ws--;
    }
    g_ws[dev] = ws;
    g_num_ws++;
    return MOE_OK;
}

void moe_mxfp4_finalize(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (int d = 0; d < kMaxDevices; d++) {
        if (g_ws[d]) {
            free_ws(g_ws[d]);
            g_ws[d] = nullptr;
        }
    }
    g_num_ws = 0;
}

namespace {

// A descriptor of rank `ndim`, element type `dtype` and extents `shape`
// (MOE_E_NULL / MOE_E_DTYPE / MOE_E_SHAPE otherwise).
int check_tensor(const moe_tensor* t, int32_t dtype, int32_t ndim, const int64_t* shape) {
    if (!t || !t->data) return MOE_E_NULL;
    if (t->dtype != dtype) return MOE_E_DTYPE;
    if (t->ndim != ndim) return MOE_E_SHAPE;
    for (int i = 0; i < ndim; i++)
        if (t->shape[i] != shape[i]) return MOE_E_SHAPE;
    return MOE_OK;
}

}  // namespace

int moe_mxfp4_forward_t(const moe_tensor* x, const moe_tensor* router_logits, int32_t top_k,
                        const moe_tensor* W_gate_up, const moe_tensor* W_down,
                        const moe_tensor* scales, const moe_tensor* out, void* stream,
                        const moe_mxfp4_options* opt) {
    if (!x || !W_gate_up || !W_down || !scales || !out) return MOE_E_NULL;
    if (!x->data || !W_gate_up->data) return MOE_E_NULL;
    if (x->dtype != MOE_DT_BF16 || W_gate_up->dtype != MOE_DT_U8) return MOE_E_DTYPE;
    // the sizes, from the descriptors: T, H from x; E, 2I from W_gate_up
    if (x->ndim != 2 || W_gate_up->ndim != 3) return MOE_E_SHAPE;
    const int64_t T = x->shape[0], H = x->shape[1];
    const int64_t E = W_gate_up->shape[0], I2 = W_gate_up->shape[1];
    if (T < 0 || H <= 0 || E <= 0 || I2 <= 0 || H % 2 || I2 % 4) return MOE_E_SHAPE;
    const int64_t I = I2 / 2;
    const int64_t sx[2] = {T, H}, sl[2] = {T, E};
    const int64_t sgu[3] = {E, I2, H / 2}, sdn[3] = {E, H, I / 2};
    const int64_t ssg[3] = {E, I2, H / 32}, ssd[3] = {E, H, I / 32};
    int rc;
    if ((rc = check_tensor(x, MOE_DT_BF16, 2, sx)) != MOE_OK) return rc;
    const bool computed = opt && opt->router_weight;  // logits computed in the layer
    if (!(computed && (!router_logits || !router_logits->data)) &&
        (rc = check_tensor(router_logits, MOE_DT_F32, 2, sl)) != MOE_OK)
        return rc;
    if ((rc = check_tensor(W_gate_up, MOE_DT_U8, 3, sgu)) != MOE_OK) return rc;
    if ((rc = check_tensor(W_down, MOE_DT_U8, 3, sdn)) != MOE_OK) return rc;
    if ((rc = check_tensor(&scales[0], MOE_DT_U8, 3, ssg)) != MOE_OK) return rc;
    if ((rc = check_tensor(&scales[1], MOE_DT_U8, 3, ssd)) != MOE_OK) return rc;
    if ((rc = check_tensor(out, MOE_DT_BF16, 2, sx)) != MOE_OK) return rc;
    // the layer's own sizes must be the workspace's (forward_ex reports a
    // missing workspace, after its option checks)
    if (T > 0) {
        const Workspace* ws = current_ws();
        if (ws && (E != ws->E || H != ws->H || I != ws->I)) return MOE_E_SHAPE;
    }
    const moe_mxfp4_scales sc = {(const uint8_t*)scales[0].data, (const uint8_t*)scales[1].data};
    return moe_mxfp4_forward_ex(x->data, computed && (!router_logits || !router_logits->data)
                                             ? nullptr : (const float*)router_logits->data,
                                T, top_k, (const uint8_t*)W_gate_up->data,
                                (const uint8_t*)W_down->data, &sc, out->data, stream, opt);
}

int moe_mxfp4_forward_ex(const void* x, const float* router_logits, int64_t num_tokens,
                         int32_t top_k, const uint8_t* W_gate_up, const uint8_t* W_down,
                         const moe_mxfp4_scales* scales, void* out, void* stream,
                         const moe_mxfp4_options* opt) {
    moe_mxfp4_options o;
    memset(&o, 0, sizeof(o));
    if (opt) o = *opt;
    // context-free checks first
    if (num_tokens < 0) return MOE_E_SHAPE;
    if (o.act_format != MOE_ACT_BF16 && o.act_format != MOE_ACT_MXFP8) return MOE_E_OPTION;
    if (o.weight_layout != MOE_LAYOUT_ROWS && o.weight_layout != MOE_LAYOUT_TILES)
        return MOE_E_OPTION;
    // the GEMV path reads row-major weights, the MFMA path the tile layout
    if (o.gemm_path == MOE_PATH_GEMV && o.weight_layout != MOE_LAYOUT_ROWS) return MOE_E_OPTION;
    if (o.gemm_path == MOE_PATH_MFMA && o.weight_layout != MOE_LAYOUT_TILES) return MOE_E_OPTION;
    if (o.gemm_path != MOE_PATH_AUTO && o.gemm_path != MOE_PATH_GEMV &&
        o.gemm_path != MOE_PATH_MFMA)
        return MOE_E_OPTION;
    // MXFP8 activations run on the scaled matrix cores over the tile layout
    if (o.act_format == MOE_ACT_MXFP8 &&
        (o.weight_layout != MOE_LAYOUT_TILES || o.gemm_path == MOE_PATH_GEMV))
        return MOE_E_OPTION;
    if (o.num_events < 0 || o.num_events > 4 || (o.num_events > 0 && !o.events))
        return MOE_E_OPTION;
    if (o.launch != MOE_LAUNCH_AUTO && o.launch != MOE_LAUNCH_SPLIT && o.launch != MOE_LAUNCH_FUSED &&
        o.launch != MOE_LAUNCH_SELF_ROUTED && o.launch != MOE_LAUNCH_QUEUE)
        return MOE_E_OPTION;
    if (num_tokens == 0) return MOE_OK;
    if (o.router_weight) router_logits = nullptr;  // ignored: the layer computes the logits
    if (!x || (!router_logits && !o.router_weight) || !W_gate_up || !W_down || !scales || !out)
        return MOE_E_NULL;
    if (!scales->gate_up || !scales->down) return MOE_E_NULL;
    if (top_k < 1) return MOE_E_TOPK;
    // the shared expert comes whole or not at all
    const bool shared = o.shared_gate_up || o.shared_gate_up_scales || o.shared_down ||
                        o.shared_down_scales;
    if (shared && !(o.shared_gate_up && o.shared_gate_up_scales && o.shared_down &&
                    o.shared_down_scales))
        return MOE_E_NULL;
    if (!aligned16(o.shared_gate_up) || !aligned16(o.shared_gate_up_scales) ||
        !aligned16(o.shared_down) || !aligned16(o.shared_down_scales))
        return MOE_E_ALIGN;
    if (!aligned16(x) || !aligned16(router_logits) || !aligned16(o.router_weight) ||
        !aligned16(W_gate_up) ||
        !aligned16(W_down) || !aligned16(scales->gate_up) || !aligned16(scales->down) ||
        !aligned16(out))
        return MOE_E_ALIGN;
    Workspace* ws = current_ws();
    if (!ws) return MOE_E_NOT_INIT;
    if (num_tokens > ws->max_tokens) return MOE_E_TOKENS;
    if (top_k > ws->kmax || top_k > ws->E) return MOE_E_TOPK;

    hipStream_t st = (hipStream_t)stream;
    auto mark = [&](int i) -> hipError_t {
        if (i < o.num_events && o.events[i]) return hipEventRecord((hipEvent_t)o.events[i], st);
        return hipSuccess;
    };
    const int T = (int)num_tokens, k = top_k;
    const int E = (int)ws->E, H = (int)ws->H, I = (int)ws->I;
    const int S = T * k;
    const int max_active = S < E ? S : E;
    hipError_t err;

    const int path = o.weight_layout == MOE_LAYOUT_TILES ? MOE_PATH_MFMA : MOE_PATH_GEMV;
    const bool mx8 = o.act_format == MOE_ACT_MXFP8;
    // bf16 MFMA items of the routed launch: 16 tokens, or up to 64 when the
    // experts average >= kMfmaWideMeanTok tokens (four quads per workgroup
    // then share the item's staged activations, and an expert's weights are
    // read once per 64 tokens)
    const bool wide = (int64_t)T * k >= (int64_t)moe::kMfmaWideMeanTok * E;
    const int item_tok = mx8 ? moe::kMx8Tok : wide ? moe::kMfmaItemTok : moe::kMfmaTok;
    // The self-routed layer (no sorting pass: the GEMM workgroups find their
    // experts' tokens themselves) covers the bf16 matrix-core path with
    // single-tile items of at most kSelfMaxTok tokens; AUTO takes it
    // wherever it applies.
    const bool self_ok = !mx8 && path == MOE_PATH_MFMA && T <= moe::kSelfMaxTok &&
                         (int64_t)T * E <= moe::kSelfMaxPairs &&
                         (int64_t)T * k < (int64_t)moe::kSelfMaxMeanTok * E;
    // (decided before anything is enqueued: a rejected call enqueues nothing)
    if (o.launch == MOE_LAUNCH_SELF_ROUTED && !self_ok) return MOE_E_OPTION;
    // FUSED on such a layer: the whole layer in one launch
    const bool self_fused = self_ok && o.launch == MOE_LAUNCH_FUSED;
    const bool self = self_ok && (o.launch == MOE_LAUNCH_SELF_ROUTED || o.launch == MOE_LAUNCH_AUTO ||
                                  self_fused);
    // The routed bf16 matrix-core GEMMs as one launch of one workgroup per
    // unit; AUTO takes it for wide layers without a shared expert (whose
    // blocks the split kernels run beside the routed ones).  On such layers
    // a split gate_up workgroup streams a whole 256-row block over K, and
    // the last, partly filled round of them leaves most of the GPU idle,
    // which down units of finished items fill here.
    const bool queue = !mx8 && !self && path == MOE_PATH_MFMA &&
                       (o.launch == MOE_LAUNCH_QUEUE || (o.launch == MOE_LAUNCH_AUTO && wide && !shared));

    if ((err = mark(0)) != hipSuccess) return hip_fail(err, "hipEventRecord");
    if (o.router_weight) {  // the router linear layer, ahead of the routing
        err = moe::launch_router_gemm((const uint16_t*)x, (const uint16_t*)o.router_weight, T, E, H,
                                      *ws, ws->logits, st);
        if (err != hipSuccess) return hip_fail(err, "router");
        router_logits = ws->logits;
    }
    // the routing pass also runs for a self-routed layer when its results
    // are asked for (it writes the same ids and weights the layer uses)
    const bool want_route = o.ids || o.weights || o.counts || o.offsets || o.sorted;
    if (mx8) {  // x is encoded in the routing stage (events [0]..[1])
        err = moe::launch_quantize_x_mxfp8((const uint16_t*)x, T, H, ws->x_codes, ws->x_scales, st);
        if (err != hipSuccess) return hip_fail(err, "quantize x");
    }
    if (!self || want_route) {
        err = moe::launch_route(router_logits, T, E, k, *ws, 1 << 30, path, item_tok, st);
        if (err != hipSuccess) return hip_fail(err, "route");
    }
    // a large self-routed layer ranks each expert once, in a pre-pass (the
    // single launch writes the lists in its own first units)
    const bool lists = self && !self_fused && (int64_t)E * (I / 32 + H / 128) >= moe::kSelfListUnits;
    moe::GemmArgs a;
    a.logits = router_logits;
    a.T = T;
    a.E = E;
    a.k = k;
    a.slot_lists = ws->slot_lists;
    if (lists) {
        err = moe::launch_slot_lists(a, st);
        if (err != hipSuccess) return hip_fail(err, "slot lists");
    }
    if ((err = mark(1)) != hipSuccess) return hip_fail(err, "hipEventRecord");

    a.x = (const uint16_t*)x;
    a.wgu = W_gate_up;
    a.sgu = scales->gate_up;
    a.wdn = W_down;
    a.sdn = scales->down;
    a.counts = ws->counts;
    a.offsets = ws->offsets;
    a.sorted = ws->sorted;
    a.list = ws->gemv_list;
    a.meta = ws->meta;
    a.list_meta = moe::kMetaNumGemv;
    a.h = ws->h;
    a.h3q = ws->h3q;
    a.h3s = ws->h3s;
    a.y = ws->y;
    a.H = H;
    a.I = I;
    a.tile_done = ws->tile_done;
    a.items = ws->mfma_items;
    a.wts = ws->wts;
    a.pos = ws->pos;
    a.out = (uint16_t*)out;
    a.col_tiles = ws->col_tiles;
    a.xq = ws->x_codes;
    a.xs = ws->x_scales;
    a.hq = ws->h_codes;
    a.hs = ws->h_scales;
    a.queue = ws->queue;
    a.gu_done = ws->gu_done;
    a.route_ids = ws->ids;
    a.route_wts = ws->wts;
    a.sh_wgu = shared ? o.shared_gate_up : nullptr;
    a.sh_sgu = o.shared_gate_up_scales;
    a.sh_wdn = o.shared_down;
    a.sh_sdn = o.shared_down_scales;
    a.sh_row0 = S;
    int32_t* self_misc = ws->flags + moe::self_misc_word(E);
    // The shared expert needs no routing: its gate_up runs ahead of the
    // routed gate_up, its down ahead of the routed down (which, on the VALU
    // path and in the single-launch layer, also combines), both in the
    // stages of the routed ones.  The matrix-core GEMM kernels of the split
    // launch run its workgroups themselves, ahead of the routed ones; the
    // VALU path and the single-launch layer launch them on their own.
    const bool shared_inside =
        path == MOE_PATH_MFMA && (mx8 || (o.launch != MOE_LAUNCH_FUSED && !queue) || self_fused);
    auto shared_gate_up = [&]() -> hipError_t {
        return shared && !shared_inside ? moe::launch_shared_gate_up(a, st) : hipSuccess;
    };
    auto shared_down = [&]() -> hipError_t {
        return shared && !shared_inside ? moe::launch_shared_down(a, st) : hipSuccess;
    };
    if ((err = shared_gate_up()) != hipSuccess) return hip_fail(err, "shared gate_up");
    if (self_fused) {
        a.pos = nullptr;  // h and y rows are the slots
        err = moe::launch_self_fused(a, ws->flags, st);
        if (err != hipSuccess) return hip_fail(err, "self-routed single launch");
        if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
    } else if (self) {
        a.pos = nullptr;  // h and y rows are the slots
        err = moe::launch_self_gate_up(a, lists, st);
        if (err != hipSuccess) return hip_fail(err, "gate_up");
        if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
        if ((err = shared_down()) != hipSuccess) return hip_fail(err, "shared down");
        err = moe::launch_self_down(a, lists, st);
        if (err != hipSuccess) return hip_fail(err, "down");
        err = moe::launch_combine(a, st);
        if (err != hipSuccess) return hip_fail(err, "combine");
    } else if (mx8) {
        const int max_items = max_active + S / moe::kMx8Tok + 1;
        err = moe::launch_mx8_gate_up(a, max_items, st);
        if (err != hipSuccess) return hip_fail(err, "gate_up");
        if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
        if ((err = shared_down()) != hipSuccess) return hip_fail(err, "shared down");
        err = moe::launch_mx8_down(a, max_items, st);
        if (err != hipSuccess) return hip_fail(err, "down");
        err = moe::launch_combine(a, st);
        if (err != hipSuccess) return hip_fail(err, "combine");
    } else if (path == MOE_PATH_GEMV) {
        err = moe::launch_gemv_gate_up(a, max_active, st);
        if (err != hipSuccess) return hip_fail(err, "gate_up");
        if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
        if ((err = shared_down()) != hipSuccess) return hip_fail(err, "shared down");
        err = moe::launch_gemv_down(a, max_active, st);
        if (err != hipSuccess) return hip_fail(err, "down");
    } else {
        a.list = ws->mfma_list;
        a.list_meta = moe::kMetaNumMfma;
        const int max_items = max_active + S / item_tok + 1;
        if (o.launch == MOE_LAUNCH_FUSED) {
            // one kernel: event [2] marks its end as well as [3]
            if ((err = shared_down()) != hipSuccess) return hip_fail(err, "shared down");
            err = wide ? moe::launch_wide_fused(a, max_items, st)
                       : moe::launch_mfma_fused(a, max_items, st);
            if (err != hipSuccess) return hip_fail(err, "fused expert layer");
            if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
        } else if (queue) {
            // one kernel for both GEMMs: event [2] marks its end
            err = wide ? moe::launch_wide_queue(a, max_items, st) : moe::launch_mfma_queue(a, max_items, st);
            if (err != hipSuccess) return hip_fail(err, "expert GEMMs");
            if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
            if ((err = shared_down()) != hipSuccess) return hip_fail(err, "shared down");
            err = moe::launch_combine(a, st);
            if (err != hipSuccess) return hip_fail(err, "combine");
        } else {
            err = wide ? moe::launch_wide_gate_up(a, max_items, st)
                       : moe::launch_mfma_gate_up(a, max_items, st);
            if (err != hipSuccess) return hip_fail(err, "gate_up");
            if ((err = mark(2)) != hipSuccess) return hip_fail(err, "hipEventRecord");
            if ((err = shared_down()) != hipSuccess) return hip_fail(err, "shared down");
            err = wide ? moe::launch_wide_down(a, max_items, st) : moe::launch_mfma_down(a, max_items, st);
            if (err != hipSuccess) return hip_fail(err, "down");
            err = moe::launch_combine(a, st);
            if (err != hipSuccess) return hip_fail(err, "combine");
        }
    }
    if ((err = mark(3)) != hipSuccess) return hip_fail(err, "hipEventRecord");

    // optional copies of the routing result
    struct {
        void* dst;
        const void* src;
        size_t bytes;
    } copies[] = {
        {o.ids, ws->ids, (size_t)S * 4},         {o.weights, ws->wts, (size_t)S * 4},
        {o.counts, ws->counts, (size_t)E * 4},   {o.offsets, ws->offsets, (size_t)(E + 1) * 4},
        {o.sorted, ws->sorted, (size_t)S * 4},
        {mx8 ? o.x_codes : nullptr, ws->x_codes, (size_t)T * H},
        {mx8 ? o.x_scales : nullptr, ws->x_scales, (size_t)T * (H / 32)},
        {mx8 ? o.h_codes : nullptr, ws->h_codes, (size_t)S * I},
        {mx8 ? o.h_scales : nullptr, ws->h_scales, (size_t)S * (I / 32)},
        {o.wait_error, self_fused ? self_misc + moe::kSelfErrorOut : ws->queue + moe::kQueueError, 4},
        {o.logits_out, router_logits, (size_t)T * E * 4},
    };
    for (auto& c : copies) {
        if (!c.dst) continue;
        err = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, st);
        if (err != hipSuccess) return hip_fail(err, "hipMemcpyAsync(debug output)");
    }
    return MOE_OK;
}

int moe_mxfp4_forward(const void* x, const float* router_logits, int64_t num_tokens,
                      int32_t top_k, const uint8_t* W_gate_up, const uint8_t* W_down,
                      const moe_mxfp4_scales* scales, void* out, void* stream) {
    return moe_mxfp4_forward_ex(x, router_logits, num_tokens, top_k, W_gate_up, W_down, scales,
                                out, stream, nullptr);
}

int moe_mxfp8_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes,
                       uint8_t* scales, void* stream) {
    if (rows < 0 || cols < 0 || cols % 32) return MOE_E_SHAPE;
    if (rows == 0 || cols == 0) return MOE_OK;
    if (!w || !codes || !scales) return MOE_E_NULL;
    if (!aligned16(w) || !aligned16(codes)) return MOE_E_ALIGN;
    hipError_t err = moe::launch_quantize_mxfp8(w, rows, cols, codes, scales, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "quantize");
    return MOE_OK;
}

int moe_mxfp4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* packed,
                       uint8_t* scales, void* stream) {
    if (rows < 0 || cols < 0 || cols % 32) return MOE_E_SHAPE;
    if (rows == 0 || cols == 0) return MOE_OK;
    if (!w || !packed || !scales) return MOE_E_NULL;
    if (!aligned16(w) || !aligned16(packed)) return MOE_E_ALIGN;
    hipError_t err = moe::launch_quantize_mxfp4(w, rows, cols, packed, scales, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "quantize");
    return MOE_OK;
}

int moe_mxfp4_forward_noalloc(const void* x, const float* router_logits, int64_t num_tokens,
                              int32_t top_k, int64_t num_experts, int64_t hidden, int64_t inter,
                              const uint8_t* W_gate_up, const uint8_t* W_down,
                              const moe_mxfp4_scales* scales, void* out, void* stream) {
    if (num_tokens < 0) return MOE_E_SHAPE;
    if (num_tokens == 0) return MOE_OK;
    if (num_experts < 1 || hidden < 128 || hidden % 128 || inter < 128 || inter % 128)
        return MOE_E_SHAPE;
    if (top_k < 1 || top_k > num_experts) return MOE_E_TOPK;
    // the fixed scratch limits, and the self-routed layer's own bounds
    if (num_tokens > kNaMaxTokens || num_experts > kNaMaxExperts || top_k > kNaMaxTopK ||
        hidden > kNaMaxHidden || inter > kNaMaxInter || num_tokens * num_experts > moe::kSelfMaxPairs ||
        num_tokens * top_k >= (int64_t)moe::kSelfMaxMeanTok * num_experts)
        return MOE_E_LIMIT;
    if (!x || !router_logits || !W_gate_up || !W_down || !scales || !out) return MOE_E_NULL;
    if (!scales->gate_up || !scales->down) return MOE_E_NULL;
    if (!aligned16(x) || !aligned16(router_logits) || !aligned16(W_gate_up) || !aligned16(W_down) ||
        !aligned16(scales->gate_up) || !aligned16(scales->down) || !aligned16(out))
        return MOE_E_ALIGN;
    uint8_t* base = nullptr;
    hipError_t err = na_scratch(&base);
    if (err != hipSuccess) return hip_fail(err, "hipGetSymbolAddress(scratch)");
    hipStream_t st = (hipStream_t)stream;
    const int T = (int)num_tokens, E = (int)num_experts, H = (int)hidden, I = (int)inter;
    moe::GemmArgs a{};
    a.x = (const uint16_t*)x;
    a.logits = router_logits;
    a.T = T;
    a.E = E;
    a.k = top_k;
    a.H = H;
    a.I = I;
    a.wgu = W_gate_up;
    a.sgu = scales->gate_up;
    a.wdn = W_down;
    a.sdn = scales->down;
    a.slot_lists = (int32_t*)(base + kNaLists);
    a.route_ids = (int32_t*)(base + kNaIds);
    a.route_wts = (float*)(base + kNaWts);
    a.wts = a.route_wts;
    a.pos = nullptr;  // h and y rows are the slots
    a.h3q = base + kNaH3q;
    a.h3s = base + kNaH3s;
    a.y = (float*)(base + kNaY);
    a.out = (uint16_t*)out;
    // every piece is written before it is read (lists, routing weights, the
    // h and y rows of every slot): nothing needs clearing between calls
    const bool lists = (int64_t)E * (I / 32 + H / 128) >= moe::kSelfListUnits;
    if (lists && (err = moe::launch_slot_lists(a, st)) != hipSuccess) return hip_fail(err, "slot lists");
    if ((err = moe::launch_self_gate_up(a, lists, st)) != hipSuccess) return hip_fail(err, "gate_up");
    if ((err = moe::launch_self_down(a, lists, st)) != hipSuccess) return hip_fail(err, "down");
    if ((err = moe::launch_combine(a, st)) != hipSuccess) return hip_fail(err, "combine");
    return MOE_OK;
}

const char* moe_mxfp4_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_E_NULL: return "a required pointer is NULL";
        case MOE_E_SHAPE: return "a size is out of range or not a required multiple";
        case MOE_E_ALIGN: return "a device pointer is not 16-byte aligned";
        case MOE_E_TOPK: return "top_k out of range";
        case MOE_E_TOKENS: return "num_tokens exceeds max_tokens of moe_mxfp4_init";
        case MOE_E_NOT_INIT: return "moe_mxfp4_init was not called for the current device";
        case MOE_E_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
        case MOE_E_OPTION: return "an option value is not recognised";
        case MOE_E_DTYPE: return "a tensor's element type is not the one required";
        case MOE_E_LIMIT:
            return "the layer exceeds the fixed limits of moe_mxfp4_forward_noalloc (at most 16 tokens, "
                   "256 experts, top-8, hidden 8192, inter 4096; T*E <= 4096, T*top_k < 8*E)";
        default: return "unknown status";
    }
}

}  // extern "C"
