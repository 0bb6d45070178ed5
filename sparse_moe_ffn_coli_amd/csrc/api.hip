// api.hip -- the C ABI of include/coli_moe.h: argument validation, workspace
// layout and kernel launches.  Every check runs on the host before anything
// is enqueued, so a rejected call touches no output.  Invalid input is an
// error status, never a silent fallback (the pages' loader fails a load
// outright when data is missing: "Add GLM-5.3-Flash (glm5next) support with
// ROCmFP mix qtypes (105/106)", section "Loader").
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

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
    size_t z, tile_count, done, total;
};
struct FfnWs {
    size_t h, o, sx, list_gu, list_dn, n_items, x16, total;
    int bm, ksplit;
};

RouteWs route_ws(const coli_moe_shape *s)
{
    RouteWs w{};
    const size_t T = (size_t)s->T, E = (size_t)s->E;
    const size_t ntiles = (size_t)coli::perm_tiles(s->T);
    w.z = 0;
    w.tile_count = align_up(w.z + (size_t)coli::router_splits(s->T, s->D) * T * E * 4);
    w.done = align_up(w.tile_count + ntiles * E * 4);
    w.total = align_up(w.done + 4);
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
    w.ksplit = (s->dtype == COLI_BF16 && !quant) ? coli::ffn_down_splits(s->T, s->E, s->D, s->F, w.bm) : 1;
    const size_t max_tiles = (size_t)coli::ffn_max_tiles(s->T, s->E, s->K, w.bm);
    w.list_gu = align_up(w.sx + T * D * 4 * (size_t)w.ksplit);
    w.list_dn = align_up(w.list_gu + max_tiles * (size_t)coli::ffn_col_tiles_gu(s->F) * 16);
    // the down list holds every column tile once per part of the reduction
    w.n_items = align_up(w.list_dn + max_tiles * (size_t)coli::ffn_col_tiles_dn(s->D) * (size_t)w.ksplit * 16);
    w.x16 = align_up(w.n_items + 20 * 4);
    w.total = quant ? align_up(w.x16 + T * D * 2) : w.x16;
    return w;
}

// ---- device check: the kernels are built for gfx950 only ---------------------
// The answer per device is cached (the property query is slow): the
// library's only process-wide state.  Each entry goes from 0 (unknown) to a
// fixed verdict (1 gfx950, 2 other) once; racing writers store the same value.
coli_status check_device()
{
    static std::atomic<int> verdict[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return COLI_E_DEVICE;
    if (dev < 0) return COLI_E_DEVICE;
    const int known = dev < 64 ? verdict[dev].load(std::memory_order_relaxed) : 0;
    if (known) return known == 1 ? COLI_OK : COLI_E_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return COLI_E_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) verdict[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? COLI_OK : COLI_E_DEVICE;
}

bool overlaps(const void *a, size_t an, const void *b, size_t bn)
{
    if (!a || !b || !an || !bn) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// A buffer a call reads or writes: its first byte and its size in bytes.
struct Region {
    const void *p;
    size_t n;
};

// True when a written region overlaps any other region of the call (read or
// written).  outs[i] == ins[j] with the same size is allowed only where the
// caller passes it as `same_ok` (an in-place update of that buffer).
bool any_overlap(const Region *outs, int n_out, const Region *ins, int n_in, const void *same_ok = nullptr)
{
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return true;
        for (int j = 0; j < n_in; ++j) {
            if (same_ok && outs[i].p == same_ok && ins[j].p == same_ok && outs[i].n == ins[j].n) continue;
            if (overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return true;
        }
    }
    return false;
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

// A dense layer is the FFN with no routed experts: E = K = 0 inside.
coli_status check_dense_shape(const coli_moe_shape *s, coli_moe_shape *inner)
{
    if (!s) return COLI_E_NULL;
    if (s->dtype != COLI_F32 && s->dtype != COLI_BF16) return COLI_E_DTYPE;
    if (s->T < 0 || s->D <= 0 || s->F <= 0 || s->D % 64 || s->F % 64 || s->D > 16384 || s->F > 32768)
        return COLI_E_SHAPE;
    if ((int64_t)s->T * s->F > INT32_MAX / 2) return COLI_E_SHAPE;
    *inner = *s;
    inner->E = 0;
    inner->K = 0;
    return COLI_OK;
}

// Kind of memory behind a pointer: 1 device, 2 pinned (registered or
// hipHostMalloc) host memory, 0 anything else (pageable host memory, or a
// pointer the runtime does not know).
int memory_kind(const void *p)
{
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();                  // clear the sticky error of an unknown pointer
        return 0;
    }
    if (at.type == hipMemoryTypeDevice) return 1;
    if (at.type == hipMemoryTypeHost) return 2;
    return 0;
}

// ---- the scratch array of coli_moe_ffn_noalloc --------------------------------
// Callers that cannot allocate get the FFN workspace from this array: one
// copy per GPU, held until the process ends.  In host code `scratch` is only
// a handle: its device address is looked up once per device (with that
// device current) and kept in scratch_ptr, which is what kernels receive.
static __device__ __attribute__((aligned(256))) char scratch[COLI_NOALLOC_SCRATCH_BYTES];

std::mutex scratch_mu;
void *scratch_ptr[64];

coli_status scratch_for_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return COLI_E_DEVICE;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return COLI_E_DEVICE;
        }
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
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
    case COLI_E_MEMORY: return "pointer is not the required kind of memory (device / pinned host)";
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
    {
        const size_t TK4 = (size_t)s->T * s->K * 4, E4 = (size_t)s->E * 4;
        const size_t elt = s->dtype == COLI_F32 ? 4 : 2;
        const Region outs[] = {{out->ids, TK4}, {out->w, TK4}, {out->count, E4}, {out->offset, E4 + 4},
                               {out->perm, TK4}, {out->inv, TK4}, {ws, s->T > 0 ? L.total : 0}};
        const Region ins[] = {{x, (size_t)s->T * s->D * elt}, {w_router, (size_t)s->E * s->D * elt},
                              {bias, E4}};
        if (any_overlap(outs, 7, ins, 3)) return COLI_E_ALIAS;
    }
    if ((st = check_device()) != COLI_OK) return st;

    coli::RouteLaunch a{};
    a.T = s->T; a.D = s->D; a.E = s->E; a.K = s->K;
    a.bf16 = s->dtype == COLI_BF16;
    a.x = x; a.wr = w_router; a.bias = bias;
    char *base = (char *)ws;
    a.z = (float *)(base + L.z);
    a.tile_count = (int32_t *)(base + L.tile_count);
    a.done = (int32_t *)(base + L.done);
    a.ids = out->ids; a.w = out->w; a.count = out->count; a.offset = out->offset;
    a.perm = out->perm; a.inv = out->inv;
    coli::StageMarks marks{events, n_events, 0};
    a.marks = &marks;
    return coli::launch_route(a, (hipStream_t)stream) == hipSuccess ? COLI_OK : COLI_E_LAUNCH;
}

static coli_status ffn_common_checks(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                                     const float *residual, float *y, void *y_bf16, void *ws,
                                     size_t ws_bytes, size_t need, const Region *weights, int n_weights)
{
    coli_status st;
    if ((st = check_routing(r, s->T)) != COLI_OK) return st;
    if (!x || !y || !ws) return COLI_E_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(ws) || (residual && !aligned16(residual)) ||
        (y_bf16 && !aligned16(y_bf16)))
        return COLI_E_ALIGN;
    if (y_bf16 && s->dtype != COLI_BF16) return COLI_E_DTYPE;
    if (ws_bytes < need) return COLI_E_WORKSPACE;
    // outputs (y, y_bf16, the workspace) against each other and against every
    // input; residual may be y itself (in-place residual stream)
    const size_t TD = (size_t)s->T * s->D, TK4 = (size_t)s->T * s->K * 4;
    const size_t xb = TD * (s->dtype == COLI_F32 ? 4 : 2);
    const Region outs[] = {{y, TD * 4}, {y_bf16, TD * 2}, {ws, need}};
    constexpr int kMaxWeights = 9;
    if (n_weights > kMaxWeights) return COLI_E_SHAPE;
    Region ins[7 + kMaxWeights] = {{x, xb},          {residual, TD * 4}, {r->ids, TK4},
                                   {r->w, TK4},      {r->count, (size_t)s->E * 4},
                                   {r->perm, TK4},   {r->inv, TK4}};
    int n_in = 7;
    for (int i = 0; i < n_weights; ++i) ins[n_in++] = weights[i];
    if (any_overlap(outs, 3, ins, n_in, residual == y ? (const void *)y : nullptr)) return COLI_E_ALIAS;
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
    const size_t elt = s->dtype == COLI_F32 ? 4 : 2;
    const size_t mat = (size_t)s->F * s->D * elt;
    const Region wr[] = {{w->gate, mat * s->E}, {w->up, mat * s->E}, {w->down, mat * s->E},
                         {w->s_gate, mat},      {w->s_up, mat},      {w->s_down, mat}};
    if ((st = ffn_common_checks(s, x, r, residual, y, y_bf16, ws, ws_bytes, L.total, wr, 6)) != COLI_OK)
        return st;

    coli::FfnLaunch a{};
    a.T = s->T; a.D = s->D; a.E = s->E; a.K = s->K; a.F = s->F;
    a.bf16 = s->dtype == COLI_BF16;
    a.bm = L.bm;
    a.ksplit = L.ksplit;
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
    const size_t q = (size_t)s->E * s->F * s->D / 2, sc = (size_t)s->E * s->F * s->D / w->group * 2;
    const size_t mat = (size_t)s->F * s->D * 2;
    const Region wr[] = {{w->gate_q, q},  {w->up_q, q},   {w->down_q, q}, {w->gate_s, sc}, {w->up_s, sc},
                         {w->down_s, sc}, {w->s_gate, mat}, {w->s_up, mat}, {w->s_down, mat}};
    if ((st = ffn_common_checks(s, x, r, residual, y, y_bf16, ws, ws_bytes, L.total, wr, 9)) != COLI_OK)
        return st;

    coli::FfnLaunch a{};
    a.T = s->T; a.D = s->D; a.E = s->E; a.K = s->K; a.F = s->F;
    a.bf16 = true;
    a.bm = L.bm;
    a.ksplit = L.ksplit;
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

size_t coli_moe_dense_workspace_bytes(const coli_moe_shape *s)
{
    coli_moe_shape in;
    if (check_dense_shape(s, &in) != COLI_OK) return 0;
    const size_t n = ffn_ws(&in, 0).total;
    return n > 256 ? n : 256;
}

coli_status coli_moe_dense_ffn(const coli_moe_shape *s, const void *x, const coli_moe_dense_weights *w,
                                          const float *residual, float *y, void *y_bf16, void *ws,
                                          size_t ws_bytes, void *stream)
{
    coli_moe_shape in;
    coli_status st = check_dense_shape(s, &in);
    if (st != COLI_OK) return st;
    if (s->T == 0) return check_device();
    if (!w || !x || !y || !ws) return COLI_E_NULL;
    if (!w->gate || !w->up || !w->down) return COLI_E_NULL;
    if (!aligned16(w->gate) || !aligned16(w->up) || !aligned16(w->down) || !aligned16(x) || !aligned16(y) ||
        !aligned16(ws) || (residual && !aligned16(residual)) || (y_bf16 && !aligned16(y_bf16)))
        return COLI_E_ALIGN;
    if (y_bf16 && s->dtype != COLI_BF16) return COLI_E_DTYPE;
    const FfnWs L = ffn_ws(&in, 0);
    if (ws_bytes < L.total) return COLI_E_WORKSPACE;
    const size_t elt = s->dtype == COLI_F32 ? 4 : 2;
    const size_t TD = (size_t)s->T * s->D, mat = (size_t)s->F * s->D * elt;
    const Region outs[] = {{y, TD * 4}, {y_bf16, TD * 2}, {ws, L.total}};
    const Region ins[] = {{x, TD * elt}, {residual, TD * 4}, {w->gate, mat}, {w->up, mat}, {w->down, mat}};
    if (any_overlap(outs, 3, ins, 5, residual == y ? (const void *)y : nullptr)) return COLI_E_ALIAS;
    if ((st = check_device()) != COLI_OK) return st;

    coli::FfnLaunch a{};
    a.T = s->T; a.D = s->D; a.E = 0; a.K = 0; a.F = s->F;
    a.bf16 = s->dtype == COLI_BF16;
    a.bm = L.bm;
    a.ksplit = L.ksplit;
    a.x = x;
    a.s_gate = w->gate; a.s_up = w->up; a.s_down = w->down;
    a.residual = residual; a.y = y; a.y_bf16 = y_bf16;
    char *base = (char *)ws;
    a.h = base + L.h; a.o = base + L.o;
    a.sx = (float *)(base + L.sx);
    a.list_gu = (int4 *)(base + L.list_gu);
    a.list_dn = (int4 *)(base + L.list_dn);
    a.n_items = (int32_t *)(base + L.n_items);
    return coli::launch_ffn(a, (hipStream_t)stream) == hipSuccess ? COLI_OK : COLI_E_LAUNCH;
}


coli_status coli_moe_bank_fill(const coli_moe_shape *s, int32_t int4, int32_t group, const void *const *host,
                               void *const *bank, const int32_t *experts, int32_t n_experts, void *copy_stream,
                               void *wait_event, void *ready_event)
{
    coli_status st = check_shape(s);
    if (st != COLI_OK) return st;
    if (!host || !bank) return COLI_E_NULL;
    if (int4) {
        if (s->dtype != COLI_BF16) return COLI_E_DTYPE;
        if (group <= 0 || group % 32 || s->D % group || s->F % group) return COLI_E_SHAPE;
    }
    if (experts && (n_experts < 0 || n_experts > s->E)) return COLI_E_SHAPE;
    const int n_t = int4 ? 6 : 3;
    // bytes of one expert's slice of tensor i
    const size_t elt = s->dtype == COLI_F32 ? 4 : 2, DF = (size_t)s->D * s->F;
    size_t per[6];
    if (int4) {
        per[0] = per[1] = per[2] = DF / 2;
        per[3] = per[4] = per[5] = DF / (size_t)group * 2;
    } else {
        per[0] = per[1] = per[2] = DF * elt;
    }
    for (int i = 0; i < n_t; ++i) {
        if (!host[i] || !bank[i]) return COLI_E_NULL;
        if (!aligned16(host[i]) || !aligned16(bank[i])) return COLI_E_ALIGN;
    }
    // every expert id once, in range (a host-side check of the caller's list)
    if (experts) {
        uint64_t seen[1024 / 64] = {};
        for (int32_t j = 0; j < n_experts; ++j) {
            const int32_t e = experts[j];
            if (e < 0 || e >= s->E || (seen[e >> 6] >> (e & 63) & 1)) return COLI_E_SHAPE;
            seen[e >> 6] |= 1ull << (e & 63);
        }
    }
    {
        Region outs[6], ins[6];
        for (int i = 0; i < n_t; ++i) {
            outs[i] = Region{bank[i], per[i] * s->E};
            ins[i] = Region{host[i], per[i] * s->E};
        }
        if (any_overlap(outs, n_t, ins, n_t)) return COLI_E_ALIAS;
    }
    if ((st = check_device()) != COLI_OK) return st;
    for (int i = 0; i < n_t; ++i)
        if (memory_kind(host[i]) != 2 || memory_kind(bank[i]) != 1) return COLI_E_MEMORY;

    hipStream_t cs = (hipStream_t)copy_stream;
    if (wait_event && hipStreamWaitEvent(cs, (hipEvent_t)wait_event, 0) != hipSuccess) return COLI_E_LAUNCH;
    const int32_t n = experts ? n_experts : s->E;
    for (int32_t j = 0; j < n;) {
        // a run of consecutive ids e0, e0 + 1, ... goes as one copy per tensor
        const int32_t e0 = experts ? experts[j] : j;
        int32_t len = 1;
        while (j + len < n && (experts ? experts[j + len] : j + len) == e0 + len) ++len;
        for (int i = 0; i < n_t; ++i) {
            const size_t off = per[i] * (size_t)e0;
            if (hipMemcpyAsync((char *)bank[i] + off, (const char *)host[i] + off, per[i] * (size_t)len,
                               hipMemcpyHostToDevice, cs) != hipSuccess)
                return COLI_E_LAUNCH;
        }
        j += len;
    }
    if (ready_event && hipEventRecord((hipEvent_t)ready_event, cs) != hipSuccess) return COLI_E_LAUNCH;
    return COLI_OK;
}

coli_status coli_moe_bank_acquire(void *compute_stream, void *ready_event)
{
    if (!ready_event) return COLI_E_NULL;
    return hipStreamWaitEvent((hipStream_t)compute_stream, (hipEvent_t)ready_event, 0) == hipSuccess
               ? COLI_OK
               : COLI_E_LAUNCH;
}

coli_status coli_moe_bank_release(void *compute_stream, void *free_event)
{
    if (!free_event) return COLI_E_NULL;
    return hipEventRecord((hipEvent_t)free_event, (hipStream_t)compute_stream) == hipSuccess ? COLI_OK
                                                                                           : COLI_E_LAUNCH;
}

size_t coli_index_topk_workspace_bytes(int32_t rows, int32_t L, int32_t k)
{
    if (rows < 0 || L < 0 || L > (1 << 24) || k < 1 || k > 4096) return 0;
    return 256;                                   // one workgroup per row keeps everything on chip
}

coli_status coli_index_topk(const float *scores, int32_t rows, int32_t L, int64_t ld, const int32_t *lens,
                            int32_t k, int32_t tail, int32_t *idx, void *ws, size_t ws_bytes, void *stream)
{
    if (rows < 0 || L < 0 || L > (1 << 24) || k < 1 || k > 4096 || tail < 0 || ld < L || ld % 4)
        return COLI_E_SHAPE;
    if (rows == 0) return check_device();
    if (!idx || (L > 0 && !scores)) return COLI_E_NULL;
    if (!aligned16(scores) || !aligned16(idx) || !aligned16(lens)) return COLI_E_ALIGN;
    (void)ws;
    (void)ws_bytes;
    const Region outs[] = {{idx, (size_t)rows * k * 4}};
    const Region ins[] = {{scores, ((size_t)(rows - 1) * ld + L) * 4}, {lens, lens ? (size_t)rows * 4 : 0}};
    if (any_overlap(outs, 1, ins, 2)) return COLI_E_ALIAS;
    coli_status st = check_device();
    if (st != COLI_OK) return st;
    return coli::launch_index_topk(scores, rows, L, (long)ld, lens, k, tail, idx, (hipStream_t)stream) == hipSuccess
               ? COLI_OK
               : COLI_E_LAUNCH;
}

coli_status coli_moe_ffn_noalloc(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                                 const coli_moe_weights *w, const float *residual, float *y, void *y_bf16,
                                 void *stream)
{
    coli_status st = check_shape(s);
    if (st != COLI_OK) return st;
    if (ffn_ws(s, 0).total > (size_t)COLI_NOALLOC_SCRATCH_BYTES) return COLI_E_WORKSPACE;
    if ((st = check_device()) != COLI_OK) return st;
    void *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != COLI_OK) return st;
    return coli_moe_ffn(s, x, r, w, residual, y, y_bf16, ws, COLI_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
