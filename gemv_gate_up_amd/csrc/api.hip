// api.hip -- the exported C ABI: argument checks, the M-based dispatcher,
// workspace layout and the launches of the hot path.
//
// Dispatcher: few rows go to the split-over-weights kernels (the narrow-
// matrix kernel of "Où part le temps d'un token" serves any product whose
// left operand has at most 16 rows; ours extends it to 64 rows by giving
// each wave up to four 16-row MFMA tiles); more rows go to the fused MFMA
// GEMM ("Tile-Level Activation Overlap for Efficient LLM Inference" picks
// between its two kernels by batch size in the same way).  fp32, FP8 and
// MXFP4 weights always take the split-over-weights kernels.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "launch.h"
#include "swiglu.h"

struct swiglu_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

namespace swg {
namespace {

constexpr int64_t MAX_DIM = (int64_t)1 << 20;
constexpr int64_t MAX_M = (int64_t)1 << 18;
// skinny/wide crossover, measured with both paths forced: skinny wins up to
// 80 rows on the 8B-class shape, wide from 64 rows on the 72B-class shape;
// above it the wide path still needs enough workgroups (resolve_path)
constexpr int64_t SKINNY_MAX_M_BF16 = 64;
constexpr int TARGET_CUS = 256;   // MI355X compute units: split-K planning target
// From 256 rows on the wide path wins with fewer workgroups (see resolve_path)
constexpr int64_t WIDE_MIN_TILES_256 = 48;
constexpr size_t WS_ALIGN = 256;

size_t align_up(size_t v) { return (v + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_sizes(int64_t M, int64_t d, int64_t dff, int dtype)
{
    if (dtype != SWIGLU_F32 && dtype != SWIGLU_BF16 && dtype != SWIGLU_BF16_FP8W &&
        dtype != SWIGLU_BF16_MXFP4W)
        return SWIGLU_ERR_UNSUPPORTED;
    if (M < 0 || d <= 0 || dff <= 0)
        return SWIGLU_ERR_INVALID_ARG;
    const int ve = act_vec_elems(dtype);
    if (d % ve != 0 || dff % ve != 0 || d > MAX_DIM || dff > MAX_DIM || M > MAX_M)
        return SWIGLU_ERR_UNSUPPORTED;
    return SWIGLU_OK;
}

int check_path(int path)
{
    return (path == SWIGLU_PATH_AUTO || path == SWIGLU_PATH_SKINNY || path == SWIGLU_PATH_WIDE ||
            path == SWIGLU_PATH_WIDE_PHASED || path == SWIGLU_PATH_FUSED_DOWN)
               ? SWIGLU_OK
               : SWIGLU_ERR_UNSUPPORTED;
}

// One product of the path, before a workspace is attached.
GemmArgs up_args(int64_t M, int64_t d, int64_t dff, int dt, bool padded_out)
{
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.geom = gateup_geom(d, dff, dt);
    g.lda = d;
    g.M = M;
    g.epi = EPI_SWIGLU;
    g.dt = dt;
    g.ldo = padded_out ? g.geom.padded_cols() : dff;
    g.ncols_out = g.ldo;
    return g;
}

GemmArgs down_args(int64_t M, int64_t d, int64_t dff, int dt)
{
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.geom = down_geom(d, dff, dt);
    g.lda = gateup_geom(d, dff, dt).padded_cols();
    g.M = M;
    g.epi = EPI_PLAIN;
    g.dt = dt;
    g.ldo = d;
    g.ncols_out = d;
    return g;
}

// Resolves the path of one product: SKINNY, WIDE or WIDE_PHASED, or an
// error.  The two-pass schedule exists for the gate/up pair only; a plain
// product asked for it takes the one-pass kernel.
int resolve_path(const GemmArgs& g, int path)
{
    if (path == SWIGLU_PATH_FUSED_DOWN)   // the MLP's fused kernel (make_plan)
        return SWIGLU_ERR_UNSUPPORTED;
    if (path == SWIGLU_PATH_WIDE_PHASED && g.epi == EPI_PLAIN)
        path = SWIGLU_PATH_WIDE;
    if (path == SWIGLU_PATH_WIDE_PHASED)
        return wide_supported(g) ? SWIGLU_PATH_WIDE_PHASED : SWIGLU_ERR_UNSUPPORTED;
    if (path == SWIGLU_PATH_WIDE)
        return wide_supported(g) ? SWIGLU_PATH_WIDE : SWIGLU_ERR_UNSUPPORTED;
    if (path == SWIGLU_PATH_SKINNY)
        return SWIGLU_PATH_SKINNY;
    if (g.dt == DT_BF16 && g.M > SKINNY_MAX_M_BF16 && wide_supported(g)) {
        // The wide path needs a grid that keeps the chip busy.  A small
        // matrix gives it few tiles (the 0.5B-class gate/up product 76 up
        // to 256 rows, a down product into d = 896 only 8 to 16), and the
        // split-over-weights kernels, which re-read the weights once per 64
        // rows, are then faster: forced-path sweeps over 0.5B-, 1.5B-, 3B-
        // and 8B-class shapes and a 72B tensor-parallel shard, 80 to 1024
        // rows, found the wide path faster wherever its grid held at least
        // 128 workgroups, or at least 48 from 256 rows on, and slower
        // elsewhere but for one case (the shard's down product at 128 rows).
        const int64_t tiles = wide_grid_tiles(g);
        if (tiles >= TARGET_CUS / 2 || (g.M >= 256 && tiles >= WIDE_MIN_TILES_256))
            return SWIGLU_PATH_WIDE;
    }
    return SWIGLU_PATH_SKINNY;
}

size_t partial_bytes(const GemmArgs& g, int path)
{
    if (path != SWIGLU_PATH_SKINNY)
        return 0;
    return skinny_partial_bytes(g, plan_skinny(g, TARGET_CUS));
}

bool is_wide(int path) { return path == SWIGLU_PATH_WIDE || path == SWIGLU_PATH_WIDE_PHASED; }

size_t h_bytes(int64_t M, int64_t d, int64_t dff, int dt)
{
    return align_up((size_t)M * (size_t)gateup_geom(d, dff, dt).padded_cols() * elem_bytes(dt));
}

// Launch plan and workspace regions of one call.  With the full workspace
// ("packed" mode, when the gate/up product takes the MFMA path) the
// activations go to that kernel in the packed layout of geometry.h: x is
// packed into the workspace first (region xp), and h is written packed when
// the down product also takes the MFMA path.  A workspace of at least the
// minimum size runs the same kernels on row-major activations instead.
struct Plan {
    GemmArgs u, dn;       // the products (dn: with_down only)
    int pu, pd;           // their paths (pd: with_down only); both FUSED_DOWN for the fused MLP
    bool packed;
    size_t h, xp, part;   // region sizes: h, packed activations, split-K partials
    FusedPlan fu;         // the fused MLP's slices (pu == FUSED_DOWN)
    size_t need() const { return h + xp + part; }
};

// Plan for a call, or a negative status in rc.
Plan make_plan(int64_t M, int64_t d, int64_t dff, int dt, int with_down, int path, bool want_packed,
               int* rc)
{
    Plan p;
    memset(&p, 0, sizeof p);
    p.u = up_args(M, d, dff, dt, with_down != 0);
    if (path == SWIGLU_PATH_FUSED_DOWN) {
        // the fused MLP: bf16 with the down projection only; its workspace
        // holds the slices' partial y (no h, no packed activations)
        *rc = (with_down && dt == DT_BF16) ? SWIGLU_OK : SWIGLU_ERR_UNSUPPORTED;
        if (*rc != SWIGLU_OK)
            return p;
        p.dn = down_args(M, d, dff, dt);
        p.pu = p.pd = SWIGLU_PATH_FUSED_DOWN;
        p.fu = plan_fused(p.u, p.dn);
        p.part = align_up(fused_partial_bytes(p.dn, p.fu));
        return p;
    }
    p.pu = resolve_path(p.u, path);
    *rc = p.pu < 0 ? p.pu : SWIGLU_OK;
    size_t part = p.pu < 0 ? 0 : partial_bytes(p.u, p.pu);
    if (with_down) {
        p.dn = down_args(M, d, dff, dt);
        p.pd = resolve_path(p.dn, path);
        if (*rc == SWIGLU_OK && p.pd < 0)
            *rc = p.pd;
        const size_t pb = p.pd < 0 ? 0 : partial_bytes(p.dn, p.pd);
        part = part > pb ? part : pb;
    }
    if (*rc != SWIGLU_OK)
        return p;
    p.packed = want_packed && is_wide(p.pu);
    p.part = align_up(part);
    if (p.packed)
        p.xp = align_up((size_t)act_packed_bytes(M, p.u.geom.nkc));
    if (with_down)
        p.h = p.packed && p.pd == SWIGLU_PATH_WIDE
                  ? align_up((size_t)act_packed_bytes(M, p.dn.geom.nkc))
                  : h_bytes(M, d, dff, dt);
    return p;
}

// The packed plan when the workspace holds it, else the minimum plan, else
// SWIGLU_ERR_WORKSPACE (also when a workspace is needed and ws is null).
int choose_plan(int64_t M, int64_t d, int64_t dff, int dt, int with_down, int path, const void* ws,
                size_t ws_bytes, Plan* out)
{
    int rc;
    for (int packed = 1; packed >= 0; --packed) {
        *out = make_plan(M, d, dff, dt, with_down, path, packed != 0, &rc);
        if (rc != SWIGLU_OK)
            return rc;
        if (out->need() <= ws_bytes && (out->need() == 0 || ws))
            return SWIGLU_OK;
    }
    return SWIGLU_ERR_WORKSPACE;
}

// Workspace size that enables the packed plan, or a negative status.
int64_t workspace_need(int64_t M, int64_t d, int64_t dff, int dt, int with_down, int path)
{
    int rc;
    const Plan p = make_plan(M, d, dff, dt, with_down, path, true, &rc);
    return rc != SWIGLU_OK ? rc : (int64_t)p.need();
}

int run(const GemmArgs& g, int path, void* partial, hipStream_t s)
{
    hipError_t e;
    if (path == SWIGLU_PATH_WIDE)
        e = launch_wide(g, s);
    else if (path == SWIGLU_PATH_WIDE_PHASED)
        e = launch_wide_phased(g, s);
    else
        e = launch_skinny(g, plan_skinny(g, TARGET_CUS), (float*)partial, s);
    return e == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_HIP;
}

// The gate/up product of a plan on activations x (row-major, or already
// packed when x_packed), writing out; in the packed plan a row-major x is
// packed into xp first.
int run_up(GemmArgs u, int pu, bool packed, const void* x, bool x_packed, void* xp, void* out,
           void* partial, hipStream_t s)
{
    u.a = x;
    if (packed) {
        if (!x_packed) {
            if (launch_pack_act(x, u.lda, u.M, u.geom.K, u.geom.nkc, xp, s) != hipSuccess)
                return SWIGLU_ERR_HIP;
            u.a = xp;
        }
        u.a_packed = 1;
    }
    u.out = out;
    return run(u, pu, partial, s);
}

// do_up / do_mlp check every argument, then launch unless `launch` is
// false (the graph-creation calls validate before touching HIP).
int do_up(const void* x, const void* wp, void* out, int64_t M, int64_t d, int64_t dff, int dtype,
          void* ws, size_t ws_bytes, hipStream_t s, int path, bool launch = true)
{
    int rc = check_sizes(M, d, dff, dtype);
    if (rc == SWIGLU_OK)
        rc = check_path(path);
    if (rc != SWIGLU_OK || M == 0)
        return rc;
    if (!x || !wp || !out)
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(wp) || !aligned16(out) || (ws && !aligned16(ws)))
        return SWIGLU_ERR_MISALIGNED;
    Plan p;
    rc = choose_plan(M, d, dff, dtype, 0, path, ws, ws_bytes, &p);
    if (rc != SWIGLU_OK || !launch)
        return rc;
    p.u.w = wp;
    uint8_t* xp = (uint8_t*)ws;
    return run_up(p.u, p.pu, p.packed, x, false, xp, out, xp + p.xp, s);
}

// Launches of the MLP on a checked plan: h = silu(x.Wg) * (x.Wu) into the
// workspace, then y = h.Wd (+ bias) (+ resid).
int run_mlp(Plan p, const void* x, bool x_packed, const void* wp, const void* wdp, void* y,
            void* h, void* xp, void* partial, hipStream_t s, const void* resid, const void* bias)
{
    if (p.pu == SWIGLU_PATH_FUSED_DOWN) {
        p.u.a = x;
        p.u.w = wp;
        p.dn.w = wdp;
        p.dn.out = y;
        p.dn.resid = resid;
        p.dn.ldr = p.dn.ldo;
        p.dn.bias = bias;
        return launch_fused(p.u, p.dn, p.fu, (float*)partial, s) == hipSuccess ? SWIGLU_OK
                                                                              : SWIGLU_ERR_HIP;
    }
    p.u.w = wp;
    const bool h_packed = p.packed && p.pd == SWIGLU_PATH_WIDE;
    if (h_packed)
        p.u.out_nkc = p.dn.geom.nkc;
    int rc = run_up(p.u, p.pu, p.packed, x, x_packed, xp, h, partial, s);
    if (rc != SWIGLU_OK)
        return rc;
    p.dn.a = h;
    p.dn.a_packed = h_packed;
    p.dn.w = wdp;
    p.dn.out = y;
    p.dn.resid = resid;
    p.dn.ldr = p.dn.ldo;
    p.dn.bias = bias;
    return run(p.dn, p.pd, partial, s);
}

int do_mlp(const void* x, const void* wp, const void* wdp, void* y, int64_t M, int64_t d,
           int64_t dff, int dtype, void* ws, size_t ws_bytes, hipStream_t s, int path,
           bool launch = true)
{
    int rc = check_sizes(M, d, dff, dtype);
    if (rc == SWIGLU_OK)
        rc = check_path(path);
    if (rc != SWIGLU_OK || M == 0)
        return rc;
    if (!x || !wp || !wdp || !y || !ws)
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(wp) || !aligned16(wdp) || !aligned16(y) || !aligned16(ws))
        return SWIGLU_ERR_MISALIGNED;
    Plan p;
    rc = choose_plan(M, d, dff, dtype, 1, path, ws, ws_bytes, &p);
    if (rc != SWIGLU_OK || !launch)
        return rc;
    uint8_t* h = (uint8_t*)ws;
    return run_mlp(p, x, false, wp, wdp, y, h, h + p.h, h + p.h + p.xp, s, nullptr, nullptr);
}

// The MLP block: out = r + MLP(rmsnorm(r)) (+ bias).  Workspace: the
// normalised rows n, then h and the partials.  In the packed plan RMSNorm
// writes n directly in the packed layout (n takes the place of xp).
size_t n_bytes(int64_t M, int64_t d, int dt) { return align_up((size_t)M * d * elem_bytes(dt)); }

size_t block_need(const Plan& p, int64_t M, int64_t d, int dt)
{
    return p.packed ? p.need() : n_bytes(M, d, dt) + p.need();
}

int choose_block_plan(int64_t M, int64_t d, int64_t dff, int dt, int path, size_t ws_bytes,
                      Plan* out)
{
    int rc;
    for (int packed = 1; packed >= 0; --packed) {
        *out = make_plan(M, d, dff, dt, 1, path, packed != 0, &rc);
        if (rc != SWIGLU_OK)
            return rc;
        if (block_need(*out, M, d, dt) <= ws_bytes)
            return SWIGLU_OK;
    }
    return SWIGLU_ERR_WORKSPACE;
}

int64_t block_workspace_need(int64_t M, int64_t d, int64_t dff, int dt, int path)
{
    int rc;
    const Plan p = make_plan(M, d, dff, dt, 1, path, true, &rc);
    return rc != SWIGLU_OK ? rc : (int64_t)block_need(p, M, d, dt);
}

int do_block(const void* r, const void* gamma, float eps, const void* wp, const void* wdp,
             const void* bias, void* out, int64_t M, int64_t d, int64_t dff, int dtype, void* ws,
             size_t ws_bytes, hipStream_t s, int path, bool launch = true)
{
    int rc = check_sizes(M, d, dff, dtype);
    if (rc == SWIGLU_OK)
        rc = check_path(path);
    if (rc != SWIGLU_OK || M == 0)
        return rc;
    if (!r || !gamma || !wp || !wdp || !out || !ws || !(eps >= 0.0f) || !(eps <= 3.4e38f))
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned16(r) || !aligned16(gamma) || !aligned16(wp) || !aligned16(wdp) ||
        !aligned16(out) || !aligned16(ws) || ((uintptr_t)bias % elem_bytes(dtype)) != 0)
        return SWIGLU_ERR_MISALIGNED;
    Plan p;
    rc = choose_block_plan(M, d, dff, dtype, path, ws_bytes, &p);
    if (rc != SWIGLU_OK || !launch)
        return rc;
    uint8_t* n = (uint8_t*)ws;
    const size_t nb = p.packed ? p.xp : n_bytes(M, d, dtype);
    if (launch_rmsnorm(r, gamma, eps, M, d, dtype, n, p.packed ? p.u.geom.nkc : 0, s) !=
        hipSuccess)
        return SWIGLU_ERR_HIP;
    uint8_t* h = n + nb;
    return run_mlp(p, n, p.packed, wp, wdp, out, h, nullptr, h + p.h, s, r, bias);
}

// Records one call (`call(stream, launch)` returns a status) on a private
// stream and instantiates it.  The arguments are checked first, without any
// HIP call; the launch attributes are set before the capture so that the
// recording holds kernel launches only.
template <class Call>
int record_graph(Call&& call, swiglu_graph_t* out)
{
    if (!out)
        return SWIGLU_ERR_INVALID_ARG;
    *out = nullptr;
    int rc = call(nullptr, false);
    if (rc != SWIGLU_OK)
        return rc;
    if (wide_prepare() != hipSuccess)
        return SWIGLU_ERR_HIP;
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess)
        return SWIGLU_ERR_HIP;
    rc = SWIGLU_ERR_HIP;
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) == hipSuccess) {
        rc = call(s, true);
        // the capture is always ended, also when the call was rejected
        if (hipStreamEndCapture(s, &graph) != hipSuccess && rc == SWIGLU_OK)
            rc = SWIGLU_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    if (rc == SWIGLU_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
        rc = SWIGLU_ERR_HIP;
    (void)hipStreamDestroy(s);
    swiglu_graph_s* h = nullptr;
    if (rc == SWIGLU_OK) {
        h = new (std::nothrow) swiglu_graph_s{graph, exec};
        if (!h) {
            (void)hipGraphExecDestroy(exec);
            rc = SWIGLU_ERR_HIP;
        }
    }
    if (rc != SWIGLU_OK) {
        if (graph)
            (void)hipGraphDestroy(graph);
        return rc;
    }
    *out = h;
    return SWIGLU_OK;
}

// ---- the entry point that allocates nothing (swiglu_up_noalloc)
// Its workspace is this fixed array: every GPU the library runs on holds a
// copy of it until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the array's address on a device
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to kernels.
constexpr size_t SCRATCH_BYTES = SWIGLU_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;
static_assert(SCRATCH_BYTES % WS_ALIGN == 0, "whole allocation units");

__device__ __attribute__((aligned(256))) uint8_t scratch[SCRATCH_BYTES];

std::atomic<void*> scratch_addr[MAX_DEVICES];
std::mutex scratch_mutex;

// The device address of the current device's copy of the array, looked up
// on the device's first call and kept.
int scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return SWIGLU_ERR_HIP;
    if (dev < 0 || dev >= MAX_DEVICES)
        return SWIGLU_ERR_UNSUPPORTED;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return SWIGLU_ERR_HIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SWIGLU_OK;
}

// swiglu_up on the automatic path with the array as its workspace: the
// packed plan when packed x fits, else x read in place; split-K partials
// always fit (at most 16 MiB for any shape within the limits).  The
// arguments and the plan are checked first, without any HIP call; a plan
// that needs more than the array is SWIGLU_ERR_SCRATCH.  Nothing in the
// array needs to start at zero: the kernels write every byte they read
// (partials, and packed x with its zero padding) earlier in the same call.
int do_up_noalloc(const void* x, const void* wp, void* out, int64_t M, int64_t d, int64_t dff,
                  int dtype, hipStream_t s)
{
    // a placeholder address (aligned, never dereferenced) while validating
    void* const placeholder = (void*)(uintptr_t)WS_ALIGN;
    int rc = do_up(x, wp, out, M, d, dff, dtype, placeholder, SCRATCH_BYTES, s, SWIGLU_PATH_AUTO,
                   false);
    if (rc == SWIGLU_ERR_WORKSPACE)
        return SWIGLU_ERR_SCRATCH;
    if (rc != SWIGLU_OK || M == 0)
        return rc;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != SWIGLU_OK)
        return rc;
    rc = do_up(x, wp, out, M, d, dff, dtype, ws, SCRATCH_BYTES, s, SWIGLU_PATH_AUTO);
    return rc == SWIGLU_ERR_WORKSPACE ? SWIGLU_ERR_SCRATCH : rc;
}

int do_pack(const void* src0, const void* src1, void* dst, const PackGeom& g, int plain,
            hipStream_t s)
{
    hipError_t e = launch_pack(src0, src1, dst, g, plain, s);
    return e == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_HIP;
}

}  // namespace
}  // namespace swg

using namespace swg;

extern "C" {

const char* swiglu_status_string(int status)
{
    switch (status) {
    case SWIGLU_OK: return "ok";
    case SWIGLU_ERR_INVALID_ARG: return "invalid argument";
    case SWIGLU_ERR_UNSUPPORTED: return "unsupported dtype, shape or path";
    case SWIGLU_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case SWIGLU_ERR_WORKSPACE: return "workspace too small";
    case SWIGLU_ERR_HIP: return "HIP launch error";
    case SWIGLU_ERR_SCRATCH: return "call needs more than the fixed scratch array";
    default: return "unknown status";
    }
}

int swiglu_version(void) { return 1; }

size_t swiglu_packed_bytes(int64_t d, int64_t dff, int dtype)
{
    if (check_sizes(0, d, dff, dtype) != SWIGLU_OK)
        return 0;
    return (size_t)gateup_geom(d, dff, dtype).bytes();
}

size_t swiglu_down_packed_bytes(int64_t d, int64_t dff, int dtype)
{
    if (check_sizes(0, d, dff, dtype) != SWIGLU_OK)
        return 0;
    return (size_t)down_geom(d, dff, dtype).bytes();
}

size_t swiglu_workspace_bytes_ex(int64_t M, int64_t d, int64_t dff, int dtype, int with_down,
                                 int path)
{
    if (check_sizes(M, d, dff, dtype) != SWIGLU_OK || check_path(path) != SWIGLU_OK || M == 0)
        return 0;
    int64_t need = workspace_need(M, d, dff, dtype, with_down ? 1 : 0, path);
    return need < 0 ? 0 : (size_t)need;
}

size_t swiglu_workspace_bytes(int64_t M, int64_t d, int64_t dff, int dtype, int with_down)
{
    return swiglu_workspace_bytes_ex(M, d, dff, dtype, with_down, SWIGLU_PATH_AUTO);
}

int swiglu_select_path(int64_t M, int64_t d, int64_t dff, int dtype)
{
    int rc = check_sizes(M, d, dff, dtype);
    if (rc != SWIGLU_OK)
        return rc;
    return resolve_path(up_args(M, d, dff, dtype, false), SWIGLU_PATH_AUTO);
}

int swiglu_pack_weights(const void* Wgate, const void* Wup, void* Wpacked, int64_t d, int64_t dff,
                        int dtype, hipStream_t stream)
{
    int rc = check_sizes(0, d, dff, dtype);
    if (rc != SWIGLU_OK)
        return rc;
    if (!Wgate || !Wup || !Wpacked)
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned16(Wgate) || !aligned16(Wup) || !aligned16(Wpacked))
        return SWIGLU_ERR_MISALIGNED;
    return do_pack(Wgate, Wup, Wpacked, gateup_geom(d, dff, dtype), 0, stream);
}

int swiglu_pack_down(const void* Wdown, void* Wdpacked, int64_t d, int64_t dff, int dtype,
                     hipStream_t stream)
{
    int rc = check_sizes(0, d, dff, dtype);
    if (rc != SWIGLU_OK)
        return rc;
    if (!Wdown || !Wdpacked)
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned16(Wdown) || !aligned16(Wdpacked))
        return SWIGLU_ERR_MISALIGNED;
    return do_pack(Wdown, Wdown, Wdpacked, down_geom(d, dff, dtype), 1, stream);
}

int swiglu_up(const void* x, const void* Wpacked, void* out, int64_t M, int64_t d, int64_t dff,
              int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return do_up(x, Wpacked, out, M, d, dff, dtype, workspace, workspace_bytes, stream,
                 SWIGLU_PATH_AUTO);
}

int swiglu_up_ex(const void* x, const void* Wpacked, void* out, int64_t M, int64_t d, int64_t dff,
                 int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream, int path)
{
    return do_up(x, Wpacked, out, M, d, dff, dtype, workspace, workspace_bytes, stream, path);
}

int swiglu_up_noalloc(const void* x, const void* Wpacked, void* out, int64_t M, int64_t d,
                      int64_t dff, int dtype, hipStream_t stream)
{
    return do_up_noalloc(x, Wpacked, out, M, d, dff, dtype, stream);
}

int mlp_forward(const void* x, const void* Wpacked, const void* Wdpacked, void* y, int64_t M,
                int64_t d, int64_t dff, int dtype, void* workspace, size_t workspace_bytes,
                hipStream_t stream)
{
    return do_mlp(x, Wpacked, Wdpacked, y, M, d, dff, dtype, workspace, workspace_bytes, stream,
                  SWIGLU_PATH_AUTO);
}

int mlp_forward_ex(const void* x, const void* Wpacked, const void* Wdpacked, void* y, int64_t M,
                   int64_t d, int64_t dff, int dtype, void* workspace, size_t workspace_bytes,
                   hipStream_t stream, int path)
{
    return do_mlp(x, Wpacked, Wdpacked, y, M, d, dff, dtype, workspace, workspace_bytes, stream,
                  path);
}

size_t mlp_block_workspace_bytes_ex(int64_t M, int64_t d, int64_t dff, int dtype, int path)
{
    if (check_sizes(M, d, dff, dtype) != SWIGLU_OK || check_path(path) != SWIGLU_OK || M == 0)
        return 0;
    const int64_t need = block_workspace_need(M, d, dff, dtype, path);
    return need < 0 ? 0 : (size_t)need;
}

size_t mlp_block_workspace_bytes(int64_t M, int64_t d, int64_t dff, int dtype)
{
    return mlp_block_workspace_bytes_ex(M, d, dff, dtype, SWIGLU_PATH_AUTO);
}

int mlp_block_forward(const void* r, const void* gamma, float eps, const void* Wpacked,
                      const void* Wdpacked, const void* bias, void* out, int64_t M, int64_t d,
                      int64_t dff, int dtype, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    return do_block(r, gamma, eps, Wpacked, Wdpacked, bias, out, M, d, dff, dtype, workspace,
                    workspace_bytes, stream, SWIGLU_PATH_AUTO);
}

int mlp_block_forward_ex(const void* r, const void* gamma, float eps, const void* Wpacked,
                         const void* Wdpacked, const void* bias, void* out, int64_t M, int64_t d,
                         int64_t dff, int dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, int path)
{
    return do_block(r, gamma, eps, Wpacked, Wdpacked, bias, out, M, d, dff, dtype, workspace,
                    workspace_bytes, stream, path);
}

int swiglu_up_graph_create(const void* x, const void* Wpacked, void* out, int64_t M, int64_t d,
                           int64_t dff, int dtype, void* workspace, size_t workspace_bytes,
                           int path, swiglu_graph_t* graph)
{
    return record_graph(
        [&](hipStream_t s, bool launch) {
            return do_up(x, Wpacked, out, M, d, dff, dtype, workspace, workspace_bytes, s, path,
                         launch);
        },
        graph);
}

int mlp_forward_graph_create(const void* x, const void* Wpacked, const void* Wdpacked, void* y,
                             int64_t M, int64_t d, int64_t dff, int dtype, void* workspace,
                             size_t workspace_bytes, int path, swiglu_graph_t* graph)
{
    return record_graph(
        [&](hipStream_t s, bool launch) {
            return do_mlp(x, Wpacked, Wdpacked, y, M, d, dff, dtype, workspace, workspace_bytes, s,
                          path, launch);
        },
        graph);
}

int mlp_block_graph_create(const void* r, const void* gamma, float eps, const void* Wpacked,
                           const void* Wdpacked, const void* bias, void* out, int64_t M, int64_t d,
                           int64_t dff, int dtype, void* workspace, size_t workspace_bytes,
                           int path, swiglu_graph_t* graph)
{
    return record_graph(
        [&](hipStream_t s, bool launch) {
            return do_block(r, gamma, eps, Wpacked, Wdpacked, bias, out, M, d, dff, dtype,
                            workspace, workspace_bytes, s, path, launch);
        },
        graph);
}

int swiglu_graph_launch(swiglu_graph_t graph, hipStream_t stream)
{
    if (!graph)
        return SWIGLU_ERR_INVALID_ARG;
    return hipGraphLaunch(graph->exec, stream) == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_HIP;
}

int swiglu_graph_destroy(swiglu_graph_t graph)
{
    if (!graph)
        return SWIGLU_OK;
    (void)hipGraphExecDestroy(graph->exec);
    (void)hipGraphDestroy(graph->graph);
    delete graph;
    return SWIGLU_OK;
}

}  // extern "C"
