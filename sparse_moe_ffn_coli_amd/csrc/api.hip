// api.hip -- the C ABI of include/coli_moe.h: argument validation, workspace
// layout and kernel launches.  Every check runs on the host before anything
// is enqueued, so a rejected call touches no output.  Invalid input is an
// error status, never a silent fallback (the pages' loader fails a load
// outright when data is missing: "Add GLM-5.3-Flash (glm5next) support with
// ROCmFP mix qtypes (105/106)", section "Loader").
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/coli_moe.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---- shape checks -----------------------------------------------------------
coli_status check_shape(const coli_moe_shape *s)
{
    if (!s) return COLI_E_NULL;
    if (s->dtype != COLI_F32 && s->dtype != COLI_BF16) return COLI_E_DTYPE;
    if (s->T < 0 || s->K < 1 || s->K > 8 || s->E < s->K || s->E > 1024) return COLI_E_SHAPE;
    if (s->D <= 0 || s->F <= 0 || s->D % 64 || s->F % 64 || s->D > 16384 || s->F > 16384)
        return COLI_E_SHAPE;
    // every row index of the routed/shared buffers fits in int32
    const int64_t rows = (int64_t)s->T * (s->K + 1);
    if (rows > INT32_MAX / 2) return COLI_E_SHAPE;
    return COLI_OK;
}

struct RouteWs {
    size_t z, tile_count, total;
};
struct FfnWs {
    size_t h, o, sx, list_gu, list_dn, n_items, x16, total;
    int bm;
};

RouteWs route_ws(const coli_moe_shape *s)
{
    RouteWs w{};
    const size_t T = (size_t)s->T, E = (size_t)s->E;
    const size_t ntiles = (size_t)coli::perm_tiles(s->T);
    w.z = 0;
    w.tile_count = align_up(w.z + (size_t)coli::router_splits(s->T, s->D) * T * E * 4);
    w.total = align_up(w.tile_count + ntiles * E * 4);
    return w;
}

FfnWs ffn_ws(const coli_moe_shape *s, int quant)
{
    FfnWs w{};
    const size_t T = (size_t)s->T, K = (size_t)s->K, D = (size_t)s->D, F = (size_t)s->F;
    const size_t R = T * K;
    const size_t elt = (s->dtype == COLI_F32) ? 4 : 2;
    w.bm = coli::ffn_tile_rows(s->T, s->E, s->K, quant);
    w.h = 0;
    w.o = align_up(w.h + (R + T) * F * elt);
    w.sx = align_up(w.o + R * D * elt);
    const size_t max_tiles = (size_t)coli::ffn_max_tiles(s->T, s->E, s->K, w.bm);
    w.list_gu = align_up(w.sx + T * D * 4);
    w.list_dn = align_up(w.list_gu + max_tiles * (size_t)coli::ffn_col_tiles_gu(s->F) * 16);
    w.n_items = align_up(w.list_dn + max_tiles * (size_t)coli::ffn_col_tiles_dn(s->D) * 16);
    w.x16 = align_up(w.n_items + 20 * 4);
    w.total = quant ? align_up(w.x16 + T * D * 2) : w.x16;
    return w;
}

// ---- device check: the kernels are built for gfx950 only ---------------------
coli_status check_device()
{
    static int verdict[64];   // 0 unknown, 1 gfx950, 2 other; a benign cache
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return COLI_E_DEVICE;
    if (dev < 0) return COLI_E_DEVICE;
    if (dev < 64 && verdict[dev]) return verdict[dev] == 1 ? COLI_OK : COLI_E_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return COLI_E_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) verdict[dev] = ok ? 1 : 2;
    return ok ? COLI_OK : COLI_E_DEVICE;
}

bool overlaps(const void *a, size_t an, const void *b, size_t bn)
{
    if (!a || !b || !an || !bn) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// With T = 0 the per-assignment arrays are empty and may be NULL; count and
// offset always exist.
coli_status check_routing(const coli_moe_routing *r, int32_t T)
{
    if (!r) return COLI_E_NULL;
    if (!r->count || !r->offset) return COLI_E_NULL;
    if (T > 0 && (!r->ids || !r->w || !r->perm || !r->inv)) return COLI_E_NULL;
    if (!aligned16(r->ids) || !aligned16(r->w) || !aligned16(r->count) || !aligned16(r->offset) ||
        !aligned16(r->perm) || !aligned16(r->inv))
        return COLI_E_ALIGN;
    return COLI_OK;
}

}  // namespace

extern "C" {

int32_t coli_moe_version(void) { return 100; }

const char *coli_moe_status_str(coli_status st)
{
    switch (st) {
    case COLI_OK: return "ok";
    case COLI_E_NULL: return "a required pointer is NULL";
    case COLI_E_SHAPE: return "shape out of the supported range";
    case COLI_E_DTYPE: return "unknown element type";
    case COLI_E_ALIGN: return "pointer not 16-byte aligned";
    case COLI_E_WORKSPACE: return "workspace too small";
    case COLI_E_DEVICE: return "current device is not gfx950";
    case COLI_E_LAUNCH: return "kernel launch failed";
    case COLI_E_ALIAS: return "an output overlaps an input";
    }
    return "unknown status";
}

size_t coli_moe_workspace_bytes(const coli_moe_shape *s, int int4)
{
    if (check_shape(s) != COLI_OK) return 0;
    const size_t a = route_ws(s).total, b = ffn_ws(s, int4).total;
    const size_t n = a > b ? a : b;
    return n > 256 ? n : 256;       // never 0, which reports an invalid shape
}

coli_status coli_moe_route(const coli_moe_shape *s, const void *x, const void *w_router,
                           const float *bias, const coli_moe_routing *out, void *ws,
                           size_t ws_bytes, void *stream)
{
    return coli_moe_route_timed(s, x, w_router, bias, out, ws, ws_bytes, stream, nullptr, 0);
}

coli_status coli_moe_route_timed(const coli_moe_shape *s, const void *x, const void *w_router,
                                 const float *bias, const coli_moe_routing *out, void *ws,
                                 size_t ws_bytes, void *stream, void *const *events,
                                 int32_t n_events)
{
    coli_status st = check_shape(s);
    if (st != COLI_OK) return st;
    if ((st = check_routing(out, s->T)) != COLI_OK) return st;
    if (s->T > 0 && (!x || !w_router || !bias || !ws)) return COLI_E_NULL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(bias) || !aligned16(ws)) return COLI_E_ALIGN;
    const RouteWs L = route_ws(s);
    if (s->T > 0 && ws_bytes < L.total) return COLI_E_WORKSPACE;
    if ((st = check_device()) != COLI_OK) return st;

    coli::RouteLaunch a{};
    a.T = s->T; a.D = s->D; a.E = s->E; a.K = s->K;
    a.bf16 = s->dtype == COLI_BF16;
    a.x = x; a.wr = w_router; a.bias = bias;
    char *base = (char *)ws;
    a.z = (float *)(base + L.z);
    a.tile_count = (int32_t *)(base + L.tile_count);
    a.ids = out->ids; a.w = out->w; a.count = out->count; a.offset = out->offset;
    a.perm = out->perm; a.inv = out->inv;
    coli::StageMarks marks{events, n_events, 0};
    a.marks = &marks;
    return coli::launch_route(a, (hipStream_t)stream) == hipSuccess ? COLI_OK : COLI_E_LAUNCH;
}

static coli_status ffn_common_checks(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                                     const float *residual, float *y, void *y_bf16, void *ws,
                                     size_t ws_bytes, size_t need)
{
    coli_status st;
    if ((st = check_routing(r, s->T)) != COLI_OK) return st;
    if (!x || !y || !ws) return COLI_E_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(ws) || (residual && !aligned16(residual)) ||
        (y_bf16 && !aligned16(y_bf16)))
        return COLI_E_ALIGN;
    if (y_bf16 && s->dtype != COLI_BF16) return COLI_E_DTYPE;
    const size_t TD = (size_t)s->T * s->D;
    const size_t xb = TD * (s->dtype == COLI_F32 ? 4 : 2);
    if (overlaps(x, xb, y, TD * 4) || overlaps(x, xb, y_bf16, TD * 2) ||
        overlaps(y, TD * 4, y_bf16, TD * 2) || overlaps(ws, ws_bytes, y, TD * 4) ||
        overlaps(ws, ws_bytes, x, xb))
        return COLI_E_ALIAS;
    if (residual && residual != y && overlaps(residual, TD * 4, y, TD * 4)) return COLI_E_ALIAS;
    if (ws_bytes < need) return COLI_E_WORKSPACE;
    return check_device();
}

coli_status coli_moe_ffn(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                         const coli_moe_weights *w, const float *residual, float *y, void *y_bf16,
                         void *ws, size_t ws_bytes, void *stream)
{
    return coli_moe_ffn_timed(s, x, r, w, residual, y, y_bf16, ws, ws_bytes, stream, nullptr, 0);
}

coli_status coli_moe_ffn_timed(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                               const coli_moe_weights *w, const float *residual, float *y,
                               void *y_bf16, void *ws, size_t ws_bytes, void *stream,
                               void *const *events, int32_t n_events)
{
    coli_status st = check_shape(s);
    if (st != COLI_OK) return st;
    if (s->T == 0) return check_device();
    if (!w) return COLI_E_NULL;
    if (!w->gate || !w->up || !w->down || !w->s_gate || !w->s_up || !w->s_down) return COLI_E_NULL;
    if (!aligned16(w->gate) || !aligned16(w->up) || !aligned16(w->down) || !aligned16(w->s_gate) ||
        !aligned16(w->s_up) || !aligned16(w->s_down))
        return COLI_E_ALIGN;
    const FfnWs L = ffn_ws(s, 0);
    if ((st = ffn_common_checks(s, x, r, residual, y, y_bf16, ws, ws_bytes, L.total)) != COLI_OK)
        return st;

    coli::FfnLaunch a{};
    a.T = s->T; a.D = s->D; a.E = s->E; a.K = s->K; a.F = s->F;
    a.bf16 = s->dtype == COLI_BF16;
    a.bm = L.bm;
    a.x = x;
    a.ids = r->ids; a.w = r->w; a.count = r->count; a.perm = r->perm;
    a.inv = r->inv;
    a.gate = w->gate; a.up = w->up; a.down = w->down;
    a.s_gate = w->s_gate; a.s_up = w->s_up; a.s_down = w->s_down;
    a.residual = residual; a.y = y; a.y_bf16 = y_bf16;
    char *base = (char *)ws;
    a.h = base + L.h; a.o = base + L.o;
    a.sx = (float *)(base + L.sx);
    a.list_gu = (int4 *)(base + L.list_gu);
    a.list_dn = (int4 *)(base + L.list_dn);
    a.n_items = (int32_t *)(base + L.n_items);
    coli::StageMarks marks{events, n_events, 0};
    a.marks = &marks;
    return coli::launch_ffn(a, (hipStream_t)stream) == hipSuccess ? COLI_OK : COLI_E_LAUNCH;
}

coli_status coli_moe_ffn_int4(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                              const coli_moe_weights_int4 *w, const float *residual, float *y,
                              void *y_bf16, void *ws, size_t ws_bytes, void *stream)
{
    return coli_moe_ffn_int4_timed(s, x, r, w, residual, y, y_bf16, ws, ws_bytes, stream, nullptr,
                                   0);
}

coli_status coli_moe_ffn_int4_timed(const coli_moe_shape *s, const void *x,
                                    const coli_moe_routing *r, const coli_moe_weights_int4 *w,
                                    const float *residual, float *y, void *y_bf16, void *ws,
                                    size_t ws_bytes, void *stream, void *const *events,
                                    int32_t n_events)
{
    coli_status st = check_shape(s);
    if (st != COLI_OK) return st;
    if (!w) return COLI_E_NULL;
    if (s->dtype != COLI_BF16) return COLI_E_DTYPE;
    if (w->group <= 0 || w->group % 32 || s->D % w->group || s->F % w->group) return COLI_E_SHAPE;
    if (s->T == 0) return check_device();
    if (!w->gate_q || !w->up_q || !w->down_q || !w->gate_s || !w->up_s || !w->down_s || !w->s_gate ||
        !w->s_up || !w->s_down)
        return COLI_E_NULL;
    if (!aligned16(w->gate_q) || !aligned16(w->up_q) || !aligned16(w->down_q) || !aligned16(w->gate_s) ||
        !aligned16(w->up_s) || !aligned16(w->down_s) || !aligned16(w->s_gate) || !aligned16(w->s_up) ||
        !aligned16(w->s_down))
        return COLI_E_ALIGN;
    const FfnWs L = ffn_ws(s, 1);
    if ((st = ffn_common_checks(s, x, r, residual, y, y_bf16, ws, ws_bytes, L.total)) != COLI_OK)
        return st;

    coli::FfnLaunch a{};
    a.T = s->T; a.D = s->D; a.E = s->E; a.K = s->K; a.F = s->F;
    a.bf16 = true;
    a.bm = L.bm;
    a.x = x;
    a.ids = r->ids; a.w = r->w; a.count = r->count; a.perm = r->perm;
    a.inv = r->inv;
    a.use_int4 = true;
    a.gate_q = w->gate_q; a.up_q = w->up_q; a.down_q = w->down_q;
    a.gate_s = w->gate_s; a.up_s = w->up_s; a.down_s = w->down_s;
    a.group = w->group;
    a.s_gate = w->s_gate; a.s_up = w->s_up; a.s_down = w->s_down;
    a.residual = residual; a.y = y; a.y_bf16 = y_bf16;
    char *base = (char *)ws;
    a.h = base + L.h; a.o = base + L.o;
    a.sx = (float *)(base + L.sx);
    a.list_gu = (int4 *)(base + L.list_gu);
    a.list_dn = (int4 *)(base + L.list_dn);
    a.n_items = (int32_t *)(base + L.n_items);
    a.x16 = (uint16_t *)(base + L.x16);
    coli::StageMarks marks{events, n_events, 0};
    a.marks = &marks;
    return coli::launch_ffn(a, (hipStream_t)stream) == hipSuccess ? COLI_OK : COLI_E_LAUNCH;
}

}  // extern "C"
