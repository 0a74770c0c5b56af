// api.hip -- the C ABI declared in include/moe.h: argument checks, the
// workspace layout, and the kernel sequence on the caller's stream.
#include <math.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/moe.h"
#include "internal.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Workspace carve_workspace(const Shape &s, void *base)
{
    Workspace w;
    memset(&w, 0, sizeof w);
    const int64_t S = s.S();
    const int64_t nchunks = num_chunks(s);
    size_t off = 0;
    char *b = static_cast<char *>(base);
    auto take = [&](size_t bytes) -> void * {
        void *p = b ? b + off : nullptr;
        off += align256(bytes);
        return p;
    };
    w.scores = (float *)take(sizeof(float) * (size_t)router_splits(s) * s.T * s.E);
    w.ids = (int32_t *)take(sizeof(int32_t) * (size_t)S);
    w.wts = (float *)take(sizeof(float) * (size_t)S);
    w.masks = (uint64_t *)take(sizeof(uint64_t) * (size_t)(nchunks * s.E));
    w.chunk_base = (int32_t *)take(sizeof(int32_t) * (size_t)(nchunks * s.E));
    w.counts = (int32_t *)take(sizeof(int32_t) * (size_t)s.E);
    w.offsets = (int32_t *)take(sizeof(int32_t) * (size_t)(s.E + 1));
    w.perm = (int32_t *)take(sizeof(int32_t) * (size_t)S);
    w.inv = (int32_t *)take(sizeof(int32_t) * (size_t)S);
    w.tiles = (Tile *)take(sizeof(Tile) * (size_t)max_tiles(s, 1));
    w.ntiles = (int32_t *)take(sizeof(int32_t) * 4);
    if (make_plan(s).tiled) w.sched = (SchedItem *)take(sizeof(SchedItem) * (size_t)sched_entries(s));
    w.h = (uint16_t *)take(sizeof(uint16_t) * (size_t)S * s.F);
    w.o = (uint16_t *)take(sizeof(uint16_t) * (size_t)S * s.d);
    w.ssq = (float *)take(sizeof(float) * (size_t)S * (s.d / 64));
    // one region per split: FP8 parts and scales, or the FP6 records
    auto split_region = [&](int64_t rows, int K, uint8_t *&hi, uint8_t *&lo, uint8_t *&shi,
                            uint8_t *&slo, uint8_t *&a6) {
        const size_t part = align256((size_t)rows * K), sc = align256((size_t)rows * K / 32);
        const size_t fp8 = 2 * part + 2 * sc;
        const size_t fp6 = (size_t)rows * (K / 128) * kA6Bytes;
        uint8_t *r = (uint8_t *)take(fp8 > fp6 ? fp8 : fp6);
        hi = r;
        lo = r ? r + part : nullptr;
        shi = r ? r + 2 * part : nullptr;
        slo = r ? r + 2 * part + sc : nullptr;
        a6 = r;
    };
    split_region(s.T, s.d, w.xhi, w.xlo, w.xshi, w.xslo, w.xa6);
    split_region(S, s.F, w.hhi, w.hlo, w.hshi, w.hslo, w.ha6);
    w.bytes = off;
    return w;
}

// Shape limits: every index fits int32 where the kernels use int32.
static bool shape_ok(const moe_dims_t *dm, int32_t k)
{
    if (dm->T < 0 || dm->d <= 0 || dm->F <= 0 || dm->E < 1 || dm->E > 1024) return false;
    if (dm->d % 256 || dm->F % 128) return false;
    if (k < 1 || k > dm->E) return false;
    if (!(dm->eps >= 0.0f) || !isfinite(dm->eps)) return false;
    const int64_t S = (int64_t)dm->T * k;
    if (S > INT32_MAX / 2) return false;
    if (S * (int64_t)dm->F > ((int64_t)1 << 40) || S * (int64_t)dm->d > ((int64_t)1 << 40))
        return false;
    return true;
}

static Shape to_shape(const moe_dims_t *dm, int32_t k)
{
    Shape s;
    s.T = dm->T;
    s.d = dm->d;
    s.E = dm->E;
    s.F = dm->F;
    s.k = k;
    s.eps = dm->eps;
    return s;
}

// The current device must be gfx950 (GFX 9.5), the only target the library
// is built for.  Two attribute queries per call; nothing is cached.
static int check_arch()
{
    int dev = 0, major = 0, minor = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (hipDeviceGetAttribute(&major, hipDeviceAttributeComputeCapabilityMajor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&minor, hipDeviceAttributeComputeCapabilityMinor, dev) != hipSuccess)
        return MOE_ERR_HIP;
    return major == 9 && minor == 5 ? MOE_OK : MOE_ERR_ARCH;
}

// Caller's event for the begin or end of a stage (null when absent).
static hipEvent_t stage_event(const moe_debug_t *debug, int stage, bool begin)
{
    if (!debug) return nullptr;
    return static_cast<hipEvent_t>(begin ? debug->stage_begin[stage] : debug->stage_end[stage]);
}

// The routing copies a caller asked for in `debug` (device to device, async).
static hipError_t copy_debug(const moe_debug_t *debug, const Workspace &ws, const Shape &s,
                             hipStream_t st)
{
    const size_t S4 = sizeof(int32_t) * (size_t)s.S();
    const struct {
        void *dst;
        const void *src;
        size_t n;
    } cp[5] = {{debug->ids, ws.ids, S4},
               {debug->weights, ws.wts, S4},
               {debug->offsets, ws.offsets, sizeof(int32_t) * (size_t)(s.E + 1)},
               {debug->perm, ws.perm, S4},
               {debug->inv, ws.inv, S4}};
    for (const auto &c : cp)
        if (c.dst) {
            const hipError_t e = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

static bool aligned16(std::initializer_list<const void *> ptrs)
{
    for (const void *p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) & 15) return false;
    return true;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_layer_workspace_size(const moe_dims_t *dims, int32_t k)
{
    if (!dims || !shape_ok(dims, k)) return 0;
    return carve_workspace(to_shape(dims, k), nullptr).bytes;
}

namespace moe {

// The layer's kernel sequence on a checked shape and a workspace that is
// large enough and 256-byte aligned.
static int layer_forward(const Shape &s, const void *x, const float *router_w,
                         const uint8_t *expert_w_packed, const uint8_t *scales, const float *alpha,
                         const float *beta, void *s_out, void *workspace, void *stream,
                         const moe_debug_t *debug)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Workspace ws = carve_workspace(s, workspace);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    (void)hipGetLastError();  // start from a clean error state

    auto mark = [&](void *const *evs, int stage) -> bool {
        if (!debug || !evs[stage]) return true;
        return hipEventRecord(static_cast<hipEvent_t>(evs[stage]), st) == hipSuccess;
    };
    auto stage = [&](int id, auto &&fn) -> bool {
        if (!mark(debug ? debug->stage_begin : nullptr, id)) return false;
        if (fn() != hipSuccess) return false;
        return mark(debug ? debug->stage_end : nullptr, id);
    };
    auto launch_ok = [](hipError_t e) { return e == hipSuccess; };
    uint16_t *out = static_cast<uint16_t *>(s_out);
    const Plan p = make_plan(s);
    if (!stage(MOE_STAGE_ROUTER, [&] { return launch_router(s, p, ws, xb, router_w, st); }) ||
        !stage(MOE_STAGE_TOPK, [&] { return launch_topk(s, p, ws, st); }) ||
        !stage(MOE_STAGE_GROUP, [&] { return launch_group(s, p, ws, st); }) ||
        !launch_ok(launch_gemm1(s, p, ws, xb, expert_w_packed, scales, st,
                                stage_event(debug, MOE_STAGE_GEMM1, true),
                                stage_event(debug, MOE_STAGE_GEMM1, false))) ||
        !stage(MOE_STAGE_GEMM2, [&] { return launch_gemm2(s, p, ws, expert_w_packed, scales, st); }) ||
        !stage(MOE_STAGE_COMBINE,
               [&] { return launch_combine(s, p, ws, xb, alpha, beta, out, st); }))
        return MOE_ERR_HIP;

    if (debug && copy_debug(debug, ws, s, st) != hipSuccess) return MOE_ERR_HIP;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Argument checks of moe_layer_forward except the workspace's.
static int layer_args_ok(const moe_dims_t *dims, const void *x, const float *router_w,
                         const uint8_t *expert_w_packed, const uint8_t *scales, const float *alpha,
                         const float *beta, int32_t k, void *s_out)
{
    if (!dims) return MOE_ERR_NULL;
    if (!shape_ok(dims, k)) return MOE_ERR_SHAPE;
    if (dims->T == 0) return MOE_OK;
    if (!x || !router_w || !expert_w_packed || !scales || !alpha || !beta || !s_out)
        return MOE_ERR_NULL;
    if (!aligned16({x, router_w, expert_w_packed, scales, alpha, beta, s_out}))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_layer_forward(const moe_dims_t *dims, const void *x, const float *router_w,
                                 const uint8_t *expert_w_packed, const uint8_t *scales,
                                 const float *alpha, const float *beta, int32_t k, void *s_out,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const moe_debug_t *debug)
{
    int rc = layer_args_ok(dims, x, router_w, expert_w_packed, scales, alpha, beta, k, s_out);
    if (rc != MOE_OK || dims->T == 0) return rc;
    if (!workspace) return MOE_ERR_NULL;
    const Shape s = to_shape(dims, k);
    if (workspace_bytes < carve_workspace(s, nullptr).bytes) return MOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return MOE_ERR_WORKSPACE;
    rc = check_arch();
    if (rc != MOE_OK) return rc;
    return layer_forward(s, x, router_w, expert_w_packed, scales, alpha, beta, s_out, workspace,
                         stream, debug);
}

// ---- the variant without a workspace argument ---------------------------------

namespace moe {

// The scratch memory of moe_layer_forward_noalloc: one array per GPU, part
// of the library's device code object, held until the process ends.  Host
// code never uses this name as an address (on the host it is a stand-in
// symbol); it uses the device address scratch_address() looked up once per
// device.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up at the first
// call on that device, with it current), or NULL with *err set.
static void *scratch_address(int *err)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        *err = MOE_ERR_HIP;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = MOE_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            *err = MOE_ERR_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace moe

extern "C" int moe_layer_forward_noalloc(const moe_dims_t *dims, const void *x,
                                         const float *router_w, const uint8_t *expert_w_packed,
                                         const uint8_t *scales, const float *alpha,
                                         const float *beta, int32_t k, void *s_out, void *stream,
                                         const moe_debug_t *debug)
{
    int rc = layer_args_ok(dims, x, router_w, expert_w_packed, scales, alpha, beta, k, s_out);
    if (rc != MOE_OK || dims->T == 0) return rc;
    const Shape s = to_shape(dims, k);
    if (carve_workspace(s, nullptr).bytes > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    rc = check_arch();
    if (rc != MOE_OK) return rc;
    void *ws = scratch_address(&rc);
    if (!ws) return rc;
    return layer_forward(s, x, router_w, expert_w_packed, scales, alpha, beta, s_out, ws, stream,
                         debug);
}

// ---- latent-width variant ---------------------------------------------------

namespace moe {

// Routing at the token width D, experts at width d.
struct LatentShapes {
    Shape route, expert;
};

static bool latent_ok(const moe_latent_dims_t *dm, int32_t k)
{
    if (dm->D <= 0 || dm->D % 256) return false;
    const moe_dims_t e{dm->T, dm->d, dm->E, dm->F, dm->eps};
    const moe_dims_t r{dm->T, dm->D, dm->E, dm->F, dm->eps};
    return shape_ok(&e, k) && shape_ok(&r, k);
}

static LatentShapes latent_shapes(const moe_latent_dims_t *dm, int32_t k)
{
    const moe_dims_t e{dm->T, dm->d, dm->E, dm->F, dm->eps};
    const moe_dims_t r{dm->T, dm->D, dm->E, dm->F, dm->eps};
    return LatentShapes{to_shape(&r, k), to_shape(&e, k)};
}

// The expert path's workspace, then the router's score planes at width D,
// z and y (bf16 [T][d]) and f (fp32 [T][D]).
struct LatentWorkspace {
    Workspace ws;
    float *scores_r;
    uint16_t *z, *y;
    size_t bytes;
};

static LatentWorkspace carve_latent(const LatentShapes &ls, void *base)
{
    LatentWorkspace L;
    L.ws = carve_workspace(ls.expert, base);
    size_t off = L.ws.bytes;
    char *b = static_cast<char *>(base);
    auto take = [&](size_t bytes) -> void * {
        void *p = b ? b + off : nullptr;
        off += align256(bytes);
        return p;
    };
    const Shape &r = ls.route, &e = ls.expert;
    L.scores_r = (float *)take(sizeof(float) * (size_t)router_splits(r) * r.T * r.E);
    L.z = (uint16_t *)take(sizeof(uint16_t) * (size_t)e.T * e.d);
    L.y = (uint16_t *)take(sizeof(uint16_t) * (size_t)e.T * e.d);
    L.bytes = off;
    return L;
}

}  // namespace moe

extern "C" size_t moe_latent_workspace_size(const moe_latent_dims_t *dims, int32_t k)
{
    if (!dims || !latent_ok(dims, k)) return 0;
    return carve_latent(latent_shapes(dims, k), nullptr).bytes;
}

extern "C" int moe_latent_forward(const moe_latent_dims_t *dims, const void *x,
                                  const float *router_w, const void *w_narrow,
                                  const uint8_t *expert_w_packed, const uint8_t *scales,
                                  const void *w_widen, const float *alpha, const float *beta,
                                  int32_t k, void *s_out, void *workspace, size_t workspace_bytes,
                                  void *stream, const moe_debug_t *debug)
{
    if (!dims) return MOE_ERR_NULL;
    if (!latent_ok(dims, k)) return MOE_ERR_SHAPE;
    if (dims->T == 0) return MOE_OK;
    if (!x || !router_w || !w_narrow || !expert_w_packed || !scales || !w_widen || !alpha ||
        !beta || !s_out || !workspace)
        return MOE_ERR_NULL;
    if (!aligned16({x, router_w, w_narrow, expert_w_packed, scales, w_widen, alpha, beta, s_out}))
        return MOE_ERR_ALIGN;
    const LatentShapes ls = latent_shapes(dims, k);
    if (workspace_bytes < carve_latent(ls, nullptr).bytes) return MOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return MOE_ERR_WORKSPACE;
    int rc = check_arch();
    if (rc != MOE_OK) return rc;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const LatentWorkspace L = carve_latent(ls, workspace);
    const Shape &sr = ls.route, &se = ls.expert;
    const Plan p = make_plan(se);
    // routing reads the full-width token: its own score planes, and no split
    // of x (the experts read z)
    Workspace wr = L.ws;
    wr.scores = L.scores_r;
    // the gate/up kernel reads the router's scores when it routes itself
    Workspace we = L.ws;
    we.scores = L.scores_r;
    Plan pr = p;
    pr.stream = pr.tiled = false;
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    (void)hipGetLastError();

    auto mark = [&](void *const *evs, int stage) -> bool {
        if (!debug || !evs[stage]) return true;
        return hipEventRecord(static_cast<hipEvent_t>(evs[stage]), st) == hipSuccess;
    };
    auto stage = [&](int id, auto &&fn) -> bool {
        if (!mark(debug ? debug->stage_begin : nullptr, id)) return false;
        if (fn() != hipSuccess) return false;
        return mark(debug ? debug->stage_end : nullptr, id);
    };
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    auto narrow = [&]() -> hipError_t {
        hipError_t e = launch_dense(xb, static_cast<const uint16_t *>(w_narrow), L.z, kDenseBf16, sr.T,
                                    se.d, sr.d, st);
        if (e != hipSuccess) return e;
        if (p.stream) return launch_split_x_fp8(se, L.ws, L.z, st);
        if (p.tiled) return launch_split_x(se, L.ws, L.z, st);
        return hipSuccess;
    };
    auto widen = [&]() -> hipError_t {
        hipError_t e = launch_combine_sum(se, p, L.ws, L.y, st);
        if (e != hipSuccess) return e;
        // the widening product stores the gated residual itself
        return launch_dense(L.y, static_cast<const uint16_t *>(w_widen), s_out, kDenseGate, sr.T, sr.d,
                            se.d, st, DenseGate{xb, alpha, beta});
    };
    if (!stage(MOE_STAGE_ROUTER, [&] { return launch_router(sr, pr, wr, xb, router_w, st); }) ||
        !stage(MOE_STAGE_TOPK, [&] { return launch_topk(sr, p, wr, st); }) ||
        !stage(MOE_STAGE_GROUP, [&] { return launch_group(sr, p, wr, st); }) || !ok(narrow()) ||
        !ok(launch_gemm1(se, p, we, L.z, expert_w_packed, scales, st,
                         stage_event(debug, MOE_STAGE_GEMM1, true),
                         stage_event(debug, MOE_STAGE_GEMM1, false))) ||
        !stage(MOE_STAGE_GEMM2, [&] { return launch_gemm2(se, p, L.ws, expert_w_packed, scales, st); }) ||
        !stage(MOE_STAGE_COMBINE, widen))
        return MOE_ERR_HIP;

    if (debug && copy_debug(debug, L.ws, se, st) != hipSuccess) return MOE_ERR_HIP;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---- the block with its stream norms -------------------------------------------

namespace moe {

// The layer's workspace, then x_n (bf16 [T][d]) and y (fp32 [T][d]).
struct BlockWorkspace {
    Workspace ws;
    uint16_t *xn;
    float *y;
    size_t bytes;
};

static BlockWorkspace carve_block(const Shape &s, void *base)
{
    BlockWorkspace B;
    B.ws = carve_workspace(s, base);
    size_t off = B.ws.bytes;
    char *b = static_cast<char *>(base);
    B.xn = (uint16_t *)(b ? b + off : nullptr);
    off += align256(sizeof(uint16_t) * (size_t)s.T * s.d);
    B.y = (float *)(b ? b + off : nullptr);
    off += align256(sizeof(float) * (size_t)s.T * s.d);
    B.bytes = off;
    return B;
}

}  // namespace moe

extern "C" size_t moe_block_workspace_size(const moe_dims_t *dims, int32_t k)
{
    if (!dims || !shape_ok(dims, k)) return 0;
    return carve_block(to_shape(dims, k), nullptr).bytes;
}

extern "C" int moe_block_forward(const moe_dims_t *dims, const void *x, const float *gamma_pre,
                                 const float *router_w, const uint8_t *expert_w_packed,
                                 const uint8_t *scales, const float *gamma_post, const float *alpha,
                                 const float *beta, int32_t k, void *s_out, void *workspace,
                                 size_t workspace_bytes, void *stream, const moe_debug_t *debug)
{
    if (!dims) return MOE_ERR_NULL;
    if (!shape_ok(dims, k)) return MOE_ERR_SHAPE;
    if (dims->T == 0) return MOE_OK;
    if (!x || !gamma_pre || !router_w || !expert_w_packed || !scales || !gamma_post || !alpha ||
        !beta || !s_out || !workspace)
        return MOE_ERR_NULL;
    if (!aligned16({x, gamma_pre, router_w, expert_w_packed, scales, gamma_post, alpha, beta, s_out}))
        return MOE_ERR_ALIGN;
    const Shape s = to_shape(dims, k);
    if (workspace_bytes < carve_block(s, nullptr).bytes) return MOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return MOE_ERR_WORKSPACE;
    int rc = check_arch();
    if (rc != MOE_OK) return rc;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const BlockWorkspace B = carve_block(s, workspace);
    const Plan p = make_plan(s);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    (void)hipGetLastError();

    auto mark = [&](void *const *evs, int stage) -> bool {
        if (!debug || !evs[stage]) return true;
        return hipEventRecord(static_cast<hipEvent_t>(evs[stage]), st) == hipSuccess;
    };
    auto stage = [&](int id, auto &&fn) -> bool {
        if (!mark(debug ? debug->stage_begin : nullptr, id)) return false;
        if (fn() != hipSuccess) return false;
        return mark(debug ? debug->stage_end : nullptr, id);
    };
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    // the router reads (and, per plan, splits) the normalised copy
    auto route = [&]() -> hipError_t {
        hipError_t e = launch_prenorm(xb, gamma_pre, B.xn, s.T, s.d, s.eps, st);
        if (e != hipSuccess) return e;
        return launch_router(s, p, B.ws, B.xn, router_w, st);
    };
    auto finish = [&]() -> hipError_t {
        // one kernel (one workgroup per row) for rows that fit it; wider
        // rows or more slots: fp32 y, then the norm and gate
        if (s.d <= kBlockFusedMaxD && s.k <= kBlockFusedMaxK)
            return launch_combine_postnorm(s, p, B.ws, xb, gamma_post, alpha, beta,
                                           static_cast<uint16_t *>(s_out), st);
        hipError_t e = launch_combine_sum_f32(s, p, B.ws, B.y, st);
        if (e != hipSuccess) return e;
        return launch_postnorm_gate(xb, B.y, gamma_post, alpha, beta, static_cast<uint16_t *>(s_out),
                                    s.T, s.d, s.eps, st);
    };
    if (!stage(MOE_STAGE_ROUTER, route) ||
        !stage(MOE_STAGE_TOPK, [&] { return launch_topk(s, p, B.ws, st); }) ||
        !stage(MOE_STAGE_GROUP, [&] { return launch_group(s, p, B.ws, st); }) ||
        !ok(launch_gemm1(s, p, B.ws, B.xn, expert_w_packed, scales, st,
                         stage_event(debug, MOE_STAGE_GEMM1, true),
                         stage_event(debug, MOE_STAGE_GEMM1, false))) ||
        !stage(MOE_STAGE_GEMM2, [&] { return launch_gemm2(s, p, B.ws, expert_w_packed, scales, st); }) ||
        !stage(MOE_STAGE_COMBINE, finish))
        return MOE_ERR_HIP;

    if (debug && copy_debug(debug, B.ws, s, st) != hipSuccess) return MOE_ERR_HIP;
    if (debug && debug->xn &&
        hipMemcpyAsync(debug->xn, B.xn, sizeof(uint16_t) * (size_t)s.T * s.d, hipMemcpyDeviceToDevice,
                       st) != hipSuccess)
        return MOE_ERR_HIP;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int moe_pack_weights(const moe_dims_t *dims, const uint8_t *codes, const uint8_t *scales,
                                uint8_t *codes_packed, uint8_t *scales_packed, void *stream)
{
    if (!dims) return MOE_ERR_NULL;
    if (dims->d <= 0 || dims->F <= 0 || dims->d % 256 || dims->F % 128 || dims->E < 1 ||
        dims->E > 1024)
        return MOE_ERR_SHAPE;
    if ((int64_t)dims->E * 3 * dims->d * (int64_t)dims->F / 32 >= ((int64_t)1 << 40))
        return MOE_ERR_SHAPE;
    if (!codes || !scales || !codes_packed || !scales_packed) return MOE_ERR_NULL;
    if (!aligned16({codes, scales, codes_packed, scales_packed})) return MOE_ERR_ALIGN;
    int rc = check_arch();
    if (rc != MOE_OK) return rc;
    (void)hipGetLastError();
    if (launch_pack(codes, scales, dims->E, dims->d, dims->F, codes_packed, scales_packed,
                    static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

extern "C" int moe_pack_weights_nvfp4(const moe_dims_t *dims, const uint8_t *codes,
                                      const uint8_t *scales16, uint8_t *codes_packed,
                                      uint8_t *scales_packed, void *stream)
{
    if (!dims) return MOE_ERR_NULL;
    if (dims->d <= 0 || dims->F <= 0 || dims->d % 256 || dims->F % 128 || dims->E < 1 ||
        dims->E > 1024)
        return MOE_ERR_SHAPE;
    if ((int64_t)dims->E * 3 * dims->d * (int64_t)dims->F / 16 >= ((int64_t)1 << 40))
        return MOE_ERR_SHAPE;
    if (!codes || !scales16 || !codes_packed || !scales_packed) return MOE_ERR_NULL;
    if (!aligned16({codes, scales16, codes_packed, scales_packed})) return MOE_ERR_ALIGN;
    int rc = check_arch();
    if (rc != MOE_OK) return rc;
    (void)hipGetLastError();
    if (launch_pack_nv(codes, scales16, dims->E, dims->d, dims->F, codes_packed, scales_packed,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

extern "C" int moe_layer_forward_nvfp4(const moe_dims_t *dims, const void *x, const float *router_w,
                                       const uint8_t *expert_w_packed, const uint8_t *scales16,
                                       const float *gscale, const float *alpha, const float *beta,
                                       int32_t k, void *s_out, void *workspace,
                                       size_t workspace_bytes, void *stream,
                                       const moe_debug_t *debug)
{
    if (!dims) return MOE_ERR_NULL;
    if (!shape_ok(dims, k)) return MOE_ERR_SHAPE;
    if (dims->T == 0) return MOE_OK;
    if (!x || !router_w || !expert_w_packed || !scales16 || !gscale || !alpha || !beta || !s_out ||
        !workspace)
        return MOE_ERR_NULL;
    if (!aligned16({x, router_w, expert_w_packed, scales16, gscale, alpha, beta, s_out}))
        return MOE_ERR_ALIGN;
    const Shape s = to_shape(dims, k);
    if (workspace_bytes < carve_workspace(s, nullptr).bytes) return MOE_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return MOE_ERR_WORKSPACE;
    int rc = check_arch();
    if (rc != MOE_OK) return rc;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const Workspace ws = carve_workspace(s, workspace);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    (void)hipGetLastError();

    auto mark = [&](void *const *evs, int stage) -> bool {
        if (!debug || !evs[stage]) return true;
        return hipEventRecord(static_cast<hipEvent_t>(evs[stage]), st) == hipSuccess;
    };
    auto stage = [&](int id, auto &&fn) -> bool {
        if (!mark(debug ? debug->stage_begin : nullptr, id)) return false;
        if (fn() != hipSuccess) return false;
        return mark(debug ? debug->stage_end : nullptr, id);
    };
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    // the 16-block kernels: tiled (kNvTileRows-row tiles), streaming or
    // 16-row tiles as the plan says; the router does not split x, x is
    // converted to fp16 instead
    Plan p = make_plan(s);
    nv_plan(s, p);
    Plan pr = p;
    pr.tiled = pr.stream = false;
    auto route = [&]() -> hipError_t {
        hipError_t e = launch_router(s, pr, ws, xb, router_w, st);
        if (e != hipSuccess || p.stream) return e;  // the streaming kernel converts x itself
        return launch_f16_rows(xb, s.T, s.d, reinterpret_cast<uint16_t *>(ws.xhi),
                               reinterpret_cast<float *>(ws.xshi), st);
    };
    if (!stage(MOE_STAGE_ROUTER, route) ||
        !stage(MOE_STAGE_TOPK, [&] { return launch_topk(s, p, ws, st); }) ||
        !stage(MOE_STAGE_GROUP, [&] { return launch_group(s, p, ws, st); }) ||
        !ok(launch_gemm1_nv(s, p, ws, xb, expert_w_packed, scales16, gscale, st,
                            stage_event(debug, MOE_STAGE_GEMM1, true),
                            stage_event(debug, MOE_STAGE_GEMM1, false))) ||
        !stage(MOE_STAGE_GEMM2,
               [&] { return launch_gemm2_nv(s, p, ws, expert_w_packed, scales16, gscale, st); }) ||
        !stage(MOE_STAGE_COMBINE, [&] {
            return launch_combine(s, p, ws, xb, alpha, beta, static_cast<uint16_t *>(s_out), st);
        }))
        return MOE_ERR_HIP;
    if (debug && copy_debug(debug, ws, s, st) != hipSuccess) return MOE_ERR_HIP;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int moe_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                 int32_t K, void *out_bf16, void *stream)
{
    if (!codes || !scales || !out_bf16) return rows == 0 ? MOE_OK : MOE_ERR_NULL;
    if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    int rc = check_arch();
    if (rc != MOE_OK) return rc;
    (void)hipGetLastError();
    if (launch_dequant(codes, scales, rows, K, static_cast<uint16_t *>(out_bf16),
                       static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

extern "C" const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid sizes (T, d, E, F, k or eps)";
    case MOE_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case MOE_ERR_ARCH: return "current device is not gfx950";
    case MOE_ERR_HIP: return "HIP runtime or kernel launch error";
    case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MOE_ERR_SCRATCH:
        return "the sizes need more scratch than the library's static scratch holds "
               "(MOE_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}
