// api.hip -- host side of libapmoe: argument validation, the weight page table
// with stream-ordered commits, and the launches of every layer step.
//
// Page-table semantics follow PagedWeight (arXiv:2607.16184), Section 3.1: each
// linear-block row holds the committed bitwidth q_i used by inference, the
// desired bitwidth d_i, and per-plane residency; offload lowers q_i before planes
// leave and reload raises it only once they are resident; Section 3.3: changes
// take effect only at safe boundaries -- here, between two launches on a stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "internal.h"

using apmoe::DevBlock;

namespace {

thread_local std::string g_last_error;

apmoe_status fail(apmoe_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

apmoe_status ok()
{
    return APMOE_OK;
}

apmoe_status hip_fail(hipError_t e, const char *what)
{
    return fail(APMOE_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

struct apmoe_ctx {
    int device;
    int cus;
    char arch[64];
    apmoe::SideStream side;  // runs a short tile launch beside the decode and mid launches
    void *scratch = nullptr;  // this device's copy of the static scratch array (allocation-free entry point)
    // Completion counters of the fused launches, zero between calls (each launch sets
    // the ones it counted on back to zero): [0] the route, [16, 16 + kLsWords) the
    // one-launch decode layer's work list, then kCombineCounters for the output
    // accumulation fused into the down product, then the one-launch layer's 16
    // per-expert counts.
    int32_t *sync = nullptr;
    bool fuse = true;  // APMOE_UNFUSED=1 at apmoe_create: every layer step in its own launches
    // APMOE_LAYER_KERNEL=1 at apmoe_create: gate_up and down of a small batch in one
    // launch (the one-launch decode layer) instead of two
    bool layer_kernel = false;
};

static constexpr int kRouteCounter = 0;
static constexpr int kLayerSync = 16;
static_assert(kLayerSync + apmoe::kLsWords <= 64, "layer counters below the combine counters");
static constexpr int kCombineCounter0 = 64;
static constexpr int kCombineCounters = 32 * 1024;  // tokens x 64-column blocks of one fused down call
// the one-launch layer's per-expert counts, 4 KB apart, after the combine counters
static constexpr int kLayerDone = (kCombineCounter0 + kCombineCounters + 1023) / 1024 * 1024;
static constexpr size_t kSyncBytes =
    (size_t)(kLayerDone + 16 * apmoe::kLsDoneStride) * sizeof(int32_t);
// Largest assignment count (T * (topk + n_shared)) routed in one fused launch: the last
// workgroup groups them with 256 threads, one chunk.  (At 512 assignments, two chunks,
// the fused launch took 21.6 us against 17.7 us for the two launches; at 64, 13.5
// against 14.3.)
static constexpr int kFusedRouteMax = 256;

// Workspace of apmoe_moe_forward_noalloc: a static device array.  Every device the
// library runs on holds its own copy from the code object's load until the process
// ends.  In host code its name is only a stand-in: apmoe_create takes the device's
// address with hipGetSymbolAddress and every use goes through that address.
static constexpr size_t kScratchBytes = (size_t)APMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

struct apmoe_table {
    int L, E;
    std::vector<apmoe_block_desc> staged;
    std::vector<uint8_t> staged_present;
    // committed shadow (host view of what the last commit published)
    std::vector<int32_t> cq, cn, ck;
    std::vector<uint8_t> cpresent;
    bool committed_once = false;
    // device table and pinned snapshots (a ring, so commits never overwrite a
    // snapshot whose copy is still pending)
    int device = -1;
    DevBlock *d_table = nullptr;
    static constexpr int kSlots = 4;
    DevBlock *h_snap[kSlots] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t ev[kSlots] = {nullptr, nullptr, nullptr, nullptr};
    bool ev_pending[kSlots] = {false, false, false, false};
    int slot = 0;

    size_t entries() const { return (size_t)L * E * 2; }
    size_t index(int l, int e, int u) const { return ((size_t)l * E + e) * 2 + u; }
};

namespace {

apmoe_status check_ctx(apmoe_ctx *ctx)
{
    if (!ctx)
        return fail(APMOE_INVALID_ARG, "ctx is NULL");
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (cur != ctx->device) {
        e = hipSetDevice(ctx->device);
        if (e != hipSuccess)
            return hip_fail(e, "hipSetDevice");
    }
    return ok();
}

apmoe_status check_index(const apmoe_table *t, int layer, int expert, int kind)
{
    if (!t)
        return fail(APMOE_INVALID_ARG, "table is NULL");
    if (layer < 0 || layer >= t->L)
        return fail(APMOE_INVALID_ARG, "layer %d out of range [0, %d)", layer, t->L);
    if (expert < 0 || expert >= t->E)
        return fail(APMOE_INVALID_ARG, "expert %d out of range [0, %d)", expert, t->E);
    if (kind != APMOE_GATE_UP && kind != APMOE_DOWN)
        return fail(APMOE_INVALID_ARG, "kind %d is neither gate_up (0) nor down (1)", kind);
    return ok();
}

// Validation of one staged entry (Section 3.1: q may only name resident planes).
apmoe_status validate_entry(const apmoe_block_desc &d, int l, int e, int u)
{
    if (d.n < 1 || d.k < 128 || d.k % 128 != 0)
        return fail(APMOE_INVALID_ARG, "block (%d,%d,%d): n=%d k=%d (need n>=1, k%%128==0)", l, e, u, d.n, d.k);
    if (d.q < APMOE_MIN_BITS || d.q > APMOE_MAX_BITS)
        return fail(APMOE_UNSUPPORTED, "block (%d,%d,%d): q=%d outside 3..8", l, e, u, d.q);
    for (int p = 0; p < d.q; ++p) {
        if (!((d.resident_mask >> p) & 1u) || !d.plane[p])
            return fail(APMOE_NOT_RESIDENT, "block (%d,%d,%d): plane %d needed by q=%d is not resident", l, e, u,
                        p, d.q);
        if (!aligned16(d.plane[p]))
            return fail(APMOE_INVALID_ARG, "block (%d,%d,%d): plane %d not 16-byte aligned", l, e, u, p);
    }
    if (!d.lut[d.q])
        return fail(APMOE_NOT_RESIDENT, "block (%d,%d,%d): LUT level %d is NULL", l, e, u, d.q);
    if (!aligned16(d.lut[d.q]))
        return fail(APMOE_INVALID_ARG, "block (%d,%d,%d): LUT level %d not 16-byte aligned", l, e, u, d.q);
    return ok();
}

apmoe_status validate_table(const apmoe_table *t)
{
    for (int l = 0; l < t->L; ++l)
        for (int u = 0; u < 2; ++u) {
            int n = -1, k = -1;
            for (int e = 0; e < t->E; ++e) {
                const size_t i = t->index(l, e, u);
                if (!t->staged_present[i])
                    continue;
                const apmoe_block_desc &d = t->staged[i];
                apmoe_status s = validate_entry(d, l, e, u);
                if (s != APMOE_OK)
                    return s;
                if (n < 0) {
                    n = d.n;
                    k = d.k;
                } else if (d.n != n || d.k != k) {
                    return fail(APMOE_INVALID_ARG, "layer %d kind %d: experts disagree on shape (%dx%d vs %dx%d)", l,
                                u, d.n, d.k, n, k);
                }
            }
        }
    return ok();
}

}  // namespace

extern "C" {

const char *apmoe_status_string(apmoe_status s)
{
    switch (s) {
    case APMOE_OK: return "ok";
    case APMOE_INVALID_ARG: return "invalid argument";
    case APMOE_UNSUPPORTED: return "unsupported";
    case APMOE_NOT_RESIDENT: return "not resident";
    case APMOE_HIP_ERROR: return "HIP error";
    case APMOE_OUT_OF_MEMORY: return "out of memory";
    default: return "unknown status";
    }
}

const char *apmoe_last_error(void) { return g_last_error.c_str(); }

int32_t apmoe_version(void) { return 100; }

apmoe_status apmoe_create(apmoe_ctx **out, int device)
{
    if (!out)
        return fail(APMOE_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= count)
        return fail(APMOE_INVALID_ARG, "device %d out of range [0, %d)", device, count);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDeviceProperties");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(APMOE_UNSUPPORTED, "device %d is %s; libapmoe is built for gfx950 only", device,
                    prop.gcnArchName);
    apmoe_ctx *c = new (std::nothrow) apmoe_ctx;
    if (!c)
        return fail(APMOE_OUT_OF_MEMORY, "context allocation");
    c->device = device;
    c->cus = prop.multiProcessorCount;
    snprintf(c->arch, sizeof(c->arch), "%s", prop.gcnArchName);
    // side stream (default priority) and its events, created on `device`
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device)
        e = hipSetDevice(device);
    if (e == hipSuccess)
        e = hipStreamCreateWithFlags(&c->side.stream, hipStreamNonBlocking);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&c->side.fork, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&c->side.join, hipEventDisableTiming);
    const hipError_t e_side = e;
    // this device's address of the static scratch array (device current)
    if (e == hipSuccess)
        e = hipGetSymbolAddress(&c->scratch, HIP_SYMBOL(scratch));
    // completion counters of the fused launches, zeroed once here
    if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&c->sync), kSyncBytes);
    if (e == hipSuccess)
        e = hipMemset(c->sync, 0, kSyncBytes);
    const char *unfused = getenv("APMOE_UNFUSED");
    c->fuse = !(unfused && unfused[0] == '1');
    const char *one = getenv("APMOE_LAYER_KERNEL");
    c->layer_kernel = c->fuse && one && one[0] == '1';
    if (cur >= 0 && cur != device)
        hipSetDevice(cur);
    if (e != hipSuccess) {
        apmoe_destroy(c);
        return hip_fail(e, e_side != hipSuccess ? "side stream of the context"
                                                : "static scratch address or counters of the context");
    }
    *out = c;
    return ok();
}

apmoe_status apmoe_destroy(apmoe_ctx *ctx)
{
    if (ctx) {
        if (ctx->side.stream)
            hipStreamDestroy(ctx->side.stream);
        if (ctx->side.fork)
            hipEventDestroy(ctx->side.fork);
        if (ctx->side.join)
            hipEventDestroy(ctx->side.join);
        if (ctx->sync)
            hipFree(ctx->sync);
    }
    delete ctx;
    return ok();
}

apmoe_status apmoe_ctx_faults(apmoe_ctx *ctx, int32_t *flags)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (!flags)
        return fail(APMOE_INVALID_ARG, "flags is NULL");
    hipError_t e = hipDeviceSynchronize();
    int32_t v = 0;
    if (e == hipSuccess)
        e = hipMemcpy(&v, ctx->sync + kLayerSync + apmoe::kLsFault, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e, "reading the fault flags");
    *flags = v ? APMOE_FAULT_LAYER_WAIT : 0;
    return ok();
}

int64_t apmoe_block_bytes(int32_t n, int32_t k, int32_t b)
{
    if (n < 0 || k < 0 || b < 1 || b > APMOE_MAX_BITS)
        return -1;
    return (int64_t)n * b * k / 8 + (int64_t)n * ((int64_t)1 << b) * 2;
}

// ----------------------------------------------------------------------------
// table
// ----------------------------------------------------------------------------

apmoe_status apmoe_table_create(int32_t n_layers, int32_t n_experts, apmoe_table **out)
{
    if (!out)
        return fail(APMOE_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (n_layers < 1 || n_experts < 1 || n_experts > APMOE_MAX_EXPERTS)
        return fail(APMOE_INVALID_ARG, "n_layers=%d n_experts=%d (need >=1, experts <= %d)", n_layers, n_experts,
                    APMOE_MAX_EXPERTS);
    apmoe_table *t = new (std::nothrow) apmoe_table;
    if (!t)
        return fail(APMOE_OUT_OF_MEMORY, "table allocation");
    try {
        t->L = n_layers;
        t->E = n_experts;
        apmoe_block_desc z;
        memset(&z, 0, sizeof(z));
        t->staged.assign(t->entries(), z);
        t->staged_present.assign(t->entries(), 0);
        t->cq.assign(t->entries(), 0);
        t->cn.assign(t->entries(), 0);
        t->ck.assign(t->entries(), 0);
        t->cpresent.assign(t->entries(), 0);
    } catch (...) {
        delete t;
        return fail(APMOE_OUT_OF_MEMORY, "table staging allocation");
    }
    *out = t;
    return ok();
}

apmoe_status apmoe_table_destroy(apmoe_table *t)
{
    if (!t)
        return ok();
    apmoe_status st = APMOE_OK;
    if (t->device >= 0) {
        int cur = -1;
        hipGetDevice(&cur);
        hipSetDevice(t->device);
        for (int i = 0; i < apmoe_table::kSlots; ++i) {
            if (t->ev[i]) {
                if (t->ev_pending[i] && hipEventSynchronize(t->ev[i]) != hipSuccess)
                    st = fail(APMOE_HIP_ERROR, "pending commit failed while destroying the table");
                hipEventDestroy(t->ev[i]);
            }
            if (t->h_snap[i])
                hipHostFree(t->h_snap[i]);
        }
        if (t->d_table)
            hipFree(t->d_table);
        if (cur >= 0)
            hipSetDevice(cur);
    }
    delete t;
    return st;
}

apmoe_status apmoe_table_set_block(apmoe_table *t, int32_t layer, int32_t expert, int32_t kind,
                                   const apmoe_block_desc *desc)
{
    apmoe_status s = check_index(t, layer, expert, kind);
    if (s != APMOE_OK)
        return s;
    if (!desc)
        return fail(APMOE_INVALID_ARG, "desc is NULL");
    const size_t i = t->index(layer, expert, kind);
    t->staged[i] = *desc;
    t->staged_present[i] = 1;
    return ok();
}

apmoe_status apmoe_table_set_bits(apmoe_table *t, int32_t layer, int32_t expert, int32_t kind, int32_t q)
{
    apmoe_status s = check_index(t, layer, expert, kind);
    if (s != APMOE_OK)
        return s;
    const size_t i = t->index(layer, expert, kind);
    if (!t->staged_present[i])
        return fail(APMOE_INVALID_ARG, "block (%d,%d,%d) was never set", layer, expert, kind);
    if (q < APMOE_MIN_BITS || q > APMOE_MAX_BITS)
        return fail(APMOE_UNSUPPORTED, "q=%d outside 3..8", q);
    t->staged[i].q = q;
    return ok();
}

apmoe_status apmoe_table_set_plane(apmoe_table *t, int32_t layer, int32_t expert, int32_t kind, int32_t p,
                                   const uint32_t *plane, int32_t resident)
{
    apmoe_status s = check_index(t, layer, expert, kind);
    if (s != APMOE_OK)
        return s;
    const size_t i = t->index(layer, expert, kind);
    if (!t->staged_present[i])
        return fail(APMOE_INVALID_ARG, "block (%d,%d,%d) was never set", layer, expert, kind);
    if (p < 0 || p >= APMOE_PLANES)
        return fail(APMOE_INVALID_ARG, "plane %d out of range", p);
    t->staged[i].plane[p] = plane;
    if (resident)
        t->staged[i].resident_mask |= 1u << p;
    else
        t->staged[i].resident_mask &= ~(1u << p);
    return ok();
}

apmoe_status apmoe_table_validate(const apmoe_table *t)
{
    if (!t)
        return fail(APMOE_INVALID_ARG, "table is NULL");
    return validate_table(t);
}

apmoe_status apmoe_table_committed_bits(const apmoe_table *t, int32_t layer, int32_t expert, int32_t kind,
                                        int32_t *q)
{
    apmoe_status s = check_index(t, layer, expert, kind);
    if (s != APMOE_OK)
        return s;
    if (!q)
        return fail(APMOE_INVALID_ARG, "q is NULL");
    const size_t i = t->index(layer, expert, kind);
    *q = t->cpresent[i] ? t->cq[i] : 0;
    return ok();
}

apmoe_status apmoe_table_commit(apmoe_ctx *ctx, apmoe_table *t, void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (!t)
        return fail(APMOE_INVALID_ARG, "table is NULL");
    s = validate_table(t);
    if (s != APMOE_OK)
        return s;
    if (t->device >= 0 && t->device != ctx->device)
        return fail(APMOE_INVALID_ARG, "table lives on device %d, ctx on %d", t->device, ctx->device);
    const size_t bytes = t->entries() * sizeof(DevBlock);
    hipError_t e;
    if (!t->d_table) {
        e = hipMalloc(&t->d_table, bytes);
        if (e != hipSuccess) {
            t->d_table = nullptr;
            return fail(APMOE_OUT_OF_MEMORY, "device table (%zu bytes): %s", bytes, hipGetErrorString(e));
        }
        for (int i = 0; i < apmoe_table::kSlots; ++i) {
            e = hipHostMalloc(reinterpret_cast<void **>(&t->h_snap[i]), bytes, hipHostMallocDefault);
            if (e == hipSuccess)
                e = hipEventCreateWithFlags(&t->ev[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                for (int j = 0; j <= i; ++j) {
                    if (t->h_snap[j])
                        hipHostFree(t->h_snap[j]);
                    if (t->ev[j])
                        hipEventDestroy(t->ev[j]);
                    t->h_snap[j] = nullptr;
                    t->ev[j] = nullptr;
                }
                hipFree(t->d_table);
                t->d_table = nullptr;
                return fail(APMOE_OUT_OF_MEMORY, "pinned table snapshot: %s", hipGetErrorString(e));
            }
        }
        t->device = ctx->device;
    }
    const int slot = t->slot;
    if (t->ev_pending[slot]) {
        e = hipEventSynchronize(t->ev[slot]);
        if (e != hipSuccess)
            return hip_fail(e, "waiting for an earlier commit");
        t->ev_pending[slot] = false;
    }
    DevBlock *snap = t->h_snap[slot];
    for (size_t i = 0; i < t->entries(); ++i) {
        DevBlock b;
        memset(&b, 0, sizeof(b));
        if (t->staged_present[i]) {
            const apmoe_block_desc &d = t->staged[i];
            for (int p = 0; p < APMOE_PLANES; ++p)
                b.plane[p] = p < d.q ? d.plane[p] : nullptr;
            b.lut = d.lut[d.q];
            b.q = d.q;
            b.n = d.n;
            b.k = d.k;
            b.present = 1;
        }
        snap[i] = b;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(t->d_table, snap, bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess)
        return hip_fail(e, "table copy");
    e = hipEventRecord(t->ev[slot], st);
    if (e != hipSuccess)
        return hip_fail(e, "table event");
    t->ev_pending[slot] = true;
    t->slot = (slot + 1) % apmoe_table::kSlots;
    for (size_t i = 0; i < t->entries(); ++i) {
        t->cpresent[i] = t->staged_present[i];
        t->cq[i] = t->staged[i].q;
        t->cn[i] = t->staged[i].n;
        t->ck[i] = t->staged[i].k;
    }
    t->committed_once = true;
    return ok();
}

// ----------------------------------------------------------------------------
// format tools
// ----------------------------------------------------------------------------

apmoe_status apmoe_lut_build(apmoe_ctx *ctx, const uint16_t *parent, int32_t n, uint16_t *const *levels,
                             void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (!parent || !levels)
        return fail(APMOE_INVALID_ARG, "parent / levels is NULL");
    if (n < 0)
        return fail(APMOE_INVALID_ARG, "n=%d", n);
    if (!aligned16(parent))
        return fail(APMOE_INVALID_ARG, "parent not 16-byte aligned");
    hipError_t e = apmoe::launch_lut_build(parent, n, levels, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "lut_build launch");
}

int64_t apmoe_tiled_plane_words(int32_t n, int32_t k)
{
    if (n < 1 || k < 128 || k % 128 != 0)
        return -1;
    return (int64_t)apmoe::tiled_plane_words(n, k);
}

apmoe_status apmoe_tile_planes(apmoe_ctx *ctx, const uint32_t *canonical, int32_t n, int32_t k, uint32_t *tiled,
                               void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (!canonical || !tiled)
        return fail(APMOE_INVALID_ARG, "canonical / tiled is NULL");
    if (n < 1 || k < 128 || k % 128 != 0)
        return fail(APMOE_INVALID_ARG, "n=%d k=%d (need n>=1, k%%128==0)", n, k);
    hipError_t e = apmoe::launch_tile_planes(canonical, n, k, tiled, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "tile_planes launch");
}

apmoe_status apmoe_pack_planes(apmoe_ctx *ctx, const uint8_t *codes, int32_t n, int32_t k, uint32_t *planes,
                               void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (!codes || !planes)
        return fail(APMOE_INVALID_ARG, "codes / planes is NULL");
    if (n < 0 || k < 0 || k % 32 != 0)
        return fail(APMOE_INVALID_ARG, "n=%d k=%d (k %% 32 must be 0)", n, k);
    hipError_t e = apmoe::launch_pack_planes(codes, n, k, planes, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "pack_planes launch");
}

// ----------------------------------------------------------------------------
// layer steps
// ----------------------------------------------------------------------------

apmoe_status apmoe_route(apmoe_ctx *ctx, const uint16_t *x, const uint16_t *w_router, const float *bias, int32_t T,
                         int32_t H, int32_t E, int32_t topk, int32_t n_shared, int32_t renormalize,
                         int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets, int32_t *perm,
                         int32_t *inv_perm, void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (T < 0 || H < 8 || H % 8 != 0)
        return fail(APMOE_INVALID_ARG, "T=%d H=%d (need T>=0, H%%8==0)", T, H);
    if (E < 1 || E > APMOE_MAX_EXPERTS)
        return fail(APMOE_INVALID_ARG, "E=%d outside 1..%d", E, APMOE_MAX_EXPERTS);
    if (topk < 1 || topk > E || topk > APMOE_MAX_TOPK)
        return fail(APMOE_INVALID_ARG, "topk=%d (need 1..min(E,%d))", topk, APMOE_MAX_TOPK);
    if (n_shared < 0 || n_shared > APMOE_MAX_SHARED || E + n_shared > APMOE_MAX_EXPERTS)
        return fail(APMOE_INVALID_ARG, "n_shared=%d (need 0..%d and E + n_shared <= %d)", n_shared, APMOE_MAX_SHARED,
                    APMOE_MAX_EXPERTS);
    if (!counts || !offsets)
        return fail(APMOE_INVALID_ARG, "counts / offsets is NULL");
    if (T > 0 && (!x || !w_router || !topk_ids || !topk_w || !perm || !inv_perm))
        return fail(APMOE_INVALID_ARG, "a required pointer is NULL");
    if (T > 0 && (!aligned16(x) || !aligned16(w_router)))
        return fail(APMOE_INVALID_ARG, "x / w_router not 16-byte aligned");
    const int kt = topk + n_shared;
    if ((int64_t)T * kt > (int64_t)1 << 30)
        return fail(APMOE_INVALID_ARG, "T*topk too large");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (ctx->fuse && T > 0 && T * kt <= kFusedRouteMax) {
        hipError_t e = apmoe::launch_route_fused(x, w_router, bias, T, H, E, topk, n_shared, renormalize, topk_ids,
                                                 topk_w, counts, offsets, perm, inv_perm, ctx->sync + kRouteCounter, st);
        return e == hipSuccess ? ok() : hip_fail(e, "route launch");
    }
    hipError_t e =
        apmoe::launch_route_topk(x, w_router, bias, T, H, E, topk, n_shared, renormalize, topk_ids, topk_w, st);
    if (e != hipSuccess)
        return hip_fail(e, "route_topk launch");
    e = apmoe::launch_route_sort(topk_ids, T * kt, E + n_shared, counts, offsets, perm, inv_perm, st);
    if (e != hipSuccess)
        return hip_fail(e, "route_sort launch");
    return ok();
}

apmoe_status apmoe_route_workspace(apmoe_ctx *ctx, int32_t T, int32_t E, int32_t topk, int32_t n_shared,
                                   size_t *bytes)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (!bytes)
        return fail(APMOE_INVALID_ARG, "bytes is NULL");
    if (T < 0 || E < 1 || E > APMOE_MAX_EXPERTS || topk < 1 || topk > E || topk > APMOE_MAX_TOPK || n_shared < 0 ||
        n_shared > APMOE_MAX_SHARED || E + n_shared > APMOE_MAX_EXPERTS)
        return fail(APMOE_INVALID_ARG, "T=%d E=%d topk=%d n_shared=%d", T, E, topk, n_shared);
    // the selection runs in one workgroup per token and the grouping sort in the LDS
    // of one workgroup: the route writes only its outputs
    *bytes = 0;
    return ok();
}

// ---- page movement ----------------------------------------------------------------

static apmoe_status page_common(apmoe_ctx *ctx, apmoe_table *t, int32_t layer, int32_t expert, int32_t kind,
                                size_t *idx)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    s = check_index(t, layer, expert, kind);
    if (s != APMOE_OK)
        return s;
    if (!t->committed_once)
        return fail(APMOE_NOT_RESIDENT, "table was never committed");
    if (t->device != ctx->device)
        return fail(APMOE_INVALID_ARG, "table lives on device %d, ctx on %d", t->device, ctx->device);
    const size_t i = t->index(layer, expert, kind);
    if (!t->staged_present[i] || !t->cpresent[i])
        return fail(APMOE_INVALID_ARG, "block (%d,%d,%d) was never committed", layer, expert, kind);
    if (t->staged[i].q != t->cq[i])
        return fail(APMOE_INVALID_ARG, "block (%d,%d,%d) has an uncommitted bitwidth change", layer, expert, kind);
    *idx = i;
    return APMOE_OK;
}

apmoe_status apmoe_page_out(apmoe_ctx *ctx, apmoe_table *t, int32_t layer, int32_t expert, int32_t kind,
                            int32_t q_new, void *const *host_planes, void *stream, void *copy_stream,
                            void *done_event)
{
    size_t i = 0;
    apmoe_status s = page_common(ctx, t, layer, expert, kind, &i);
    if (s != APMOE_OK)
        return s;
    apmoe_block_desc &d = t->staged[i];
    const int q_old = d.q;
    if (q_new < APMOE_MIN_BITS || q_new >= q_old)
        return fail(APMOE_INVALID_ARG, "page-out to q=%d from q=%d (need %d <= q_new < q_old)", q_new, q_old,
                    APMOE_MIN_BITS);
    if (!host_planes || !done_event)
        return fail(APMOE_INVALID_ARG, "host_planes / done_event is NULL");
    for (int p = q_new; p < q_old; ++p)
        if (!host_planes[p] || !d.plane[p])
            return fail(APMOE_INVALID_ARG, "plane %d: host buffer or device plane is NULL", p);
    // lower q first (stream-ordered commit): launches after it never read planes >= q_new
    const apmoe_block_desc saved = d;
    d.q = q_new;
    s = apmoe_table_commit(ctx, t, stream);
    if (s != APMOE_OK) {
        d = saved;
        return s;
    }
    const size_t bytes = apmoe::tiled_plane_words(d.n, d.k) * 4;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream), cs = reinterpret_cast<hipStream_t>(copy_stream);
    hipEvent_t done = reinterpret_cast<hipEvent_t>(done_event);
    // The copies start at the commit point of `stream` (every earlier write to the
    // planes and every launch that may read them have finished) and overlap the
    // launches enqueued after it; done is recorded after the copies.
    hipError_t e = hipEventRecord(done, st);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(cs, done, 0);
    for (int p = q_new; p < q_old && e == hipSuccess; ++p)
        e = hipMemcpyAsync(host_planes[p], d.plane[p], bytes, hipMemcpyDeviceToHost, cs);
    if (e == hipSuccess)
        e = hipEventRecord(done, cs);
    if (e != hipSuccess)
        return hip_fail(e, "page-out copies");
    for (int p = q_new; p < q_old; ++p) {  // no longer resident once `done` has passed
        d.plane[p] = nullptr;
        d.resident_mask &= ~(1u << p);
    }
    return ok();
}

apmoe_status apmoe_page_in(apmoe_ctx *ctx, apmoe_table *t, int32_t layer, int32_t expert, int32_t kind,
                           int32_t q_new, void *const *host_planes, uint32_t *const *dev_planes, void *stream,
                           void *copy_stream, void *copied_event)
{
    size_t i = 0;
    apmoe_status s = page_common(ctx, t, layer, expert, kind, &i);
    if (s != APMOE_OK)
        return s;
    apmoe_block_desc &d = t->staged[i];
    const int q_old = d.q;
    if (q_new <= q_old || q_new > APMOE_MAX_BITS)
        return fail(APMOE_INVALID_ARG, "page-in to q=%d from q=%d (need q_old < q_new <= %d)", q_new, q_old,
                    APMOE_MAX_BITS);
    if (!host_planes || !dev_planes || !copied_event)
        return fail(APMOE_INVALID_ARG, "host_planes / dev_planes / copied_event is NULL");
    for (int p = q_old; p < q_new; ++p) {
        if (!host_planes[p] || !dev_planes[p])
            return fail(APMOE_INVALID_ARG, "plane %d: host buffer or device plane is NULL", p);
        if (!aligned16(dev_planes[p]))
            return fail(APMOE_INVALID_ARG, "device plane %d not 16-byte aligned", p);
    }
    // stage the new planes and q, and check the result before anything is enqueued
    const apmoe_block_desc saved = d;
    for (int p = q_old; p < q_new; ++p) {
        d.plane[p] = dev_planes[p];
        d.resident_mask |= 1u << p;
    }
    d.q = q_new;
    s = validate_table(t);
    if (s != APMOE_OK) {
        d = saved;
        return s;
    }
    const size_t bytes = apmoe::tiled_plane_words(d.n, d.k) * 4;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream), cs = reinterpret_cast<hipStream_t>(copy_stream);
    hipEvent_t copied = reinterpret_cast<hipEvent_t>(copied_event);
    hipError_t e = hipSuccess;
    for (int p = q_old; p < q_new && e == hipSuccess; ++p)
        e = hipMemcpyAsync(dev_planes[p], host_planes[p], bytes, hipMemcpyHostToDevice, cs);
    // raise q last: the commit on `stream` waits for the copies
    if (e == hipSuccess)
        e = hipEventRecord(copied, cs);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(st, copied, 0);
    if (e != hipSuccess) {
        d = saved;
        return hip_fail(e, "page-in copies");
    }
    s = apmoe_table_commit(ctx, t, stream);
    if (s != APMOE_OK)
        d = saved;
    return s;
}

apmoe_status apmoe_route_stats(apmoe_ctx *ctx, const float *topk_w, const int32_t *perm, const int32_t *offsets,
                               int32_t T, int32_t topk, int32_t E, double *mass, double *total, int64_t *selections,
                               void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (T < 0)
        return fail(APMOE_INVALID_ARG, "T=%d", T);
    if (E < 1 || E > APMOE_MAX_EXPERTS)
        return fail(APMOE_INVALID_ARG, "E=%d outside 1..%d", E, APMOE_MAX_EXPERTS);
    if (topk < 1 || topk > APMOE_MAX_ASSIGN)
        return fail(APMOE_INVALID_ARG, "topk=%d (need 1..%d)", topk, APMOE_MAX_ASSIGN);
    if ((int64_t)T * topk > (int64_t)1 << 30)
        return fail(APMOE_INVALID_ARG, "T*topk too large");
    if (!mass || !total || !selections)
        return fail(APMOE_INVALID_ARG, "mass / total / selections is NULL");
    if (T == 0)
        return ok();
    if (!topk_w || !perm || !offsets)
        return fail(APMOE_INVALID_ARG, "topk_w / perm / offsets is NULL");
    if ((reinterpret_cast<uintptr_t>(mass) | reinterpret_cast<uintptr_t>(total) |
         reinterpret_cast<uintptr_t>(selections)) % 8 != 0)
        return fail(APMOE_INVALID_ARG, "accumulators not 8-byte aligned");
    hipError_t e = apmoe::launch_route_stats(topk_w, perm, offsets, E, mass, total, selections,
                                             reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "route_stats launch");
}

static apmoe_status layer_shape(const apmoe_table *t, int layer, int kind, int *N, int *K, int *max_q)
{
    *N = *K = -1;
    *max_q = 0;
    for (int e = 0; e < t->E; ++e) {
        const size_t i = t->index(layer, e, kind);
        if (!t->cpresent[i])
            return fail(APMOE_NOT_RESIDENT, "block (%d,%d,%d) has no committed entry", layer, e, kind);
        if (*N < 0) {
            *N = t->cn[i];
            *K = t->ck[i];
        }
        if (t->cq[i] > *max_q)
            *max_q = t->cq[i];
    }
    return ok();
}

// Size limits of one product call (every buffer a kernel addresses through a 32-bit
// buffer offset stays below 2 GiB); checked before anything is enqueued.
static apmoe_status gemm_limits(const apmoe_table *tbl, int layer, int kind, int T, int topk, int gather, int act,
                                int *N, int *K, int *max_q, size_t *in_bytes)
{
    apmoe_status s = layer_shape(tbl, layer, kind, N, K, max_q);
    if (s != APMOE_OK)
        return s;
    if (act && (*N % 128 != 0))
        return fail(APMOE_INVALID_ARG, "gate_up has %d rows: the fused activation needs F = N/2 a multiple of 64", *N);
    const size_t in_rows = gather ? (size_t)T : (size_t)T * topk;
    *in_bytes = in_rows * (size_t)*K * 2;
    const size_t plane_bytes = apmoe::tiled_plane_words(*N, *K) * 4;
    if (*in_bytes >= ((size_t)1 << 31) || plane_bytes >= ((size_t)1 << 31) ||
        ((size_t)*N << (*max_q + 1)) >= ((size_t)1 << 31))
        return fail(APMOE_INVALID_ARG, "operands above 2 GiB per buffer are not supported (in %zu B, plane %zu B)",
                    *in_bytes, plane_bytes);
    return ok();
}

static apmoe_status gemm_common(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, int32_t kind,
                                const uint16_t *in, int32_t gather, const int32_t *perm, const int32_t *offsets,
                                int32_t T, int32_t topk, void *out, int32_t out_dtype, int act, void *stream,
                                const apmoe::CombineArgs *comb = nullptr)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    s = check_index(tbl, layer, 0, kind);
    if (s != APMOE_OK)
        return s;
    if (!tbl->committed_once || !tbl->d_table)
        return fail(APMOE_NOT_RESIDENT, "table was never committed");
    if (tbl->device != ctx->device)
        return fail(APMOE_INVALID_ARG, "table lives on device %d, ctx on %d", tbl->device, ctx->device);
    if (T < 0 || topk < 1 || topk > APMOE_MAX_ASSIGN)
        return fail(APMOE_INVALID_ARG, "T=%d topk=%d", T, topk);
    if (out_dtype != APMOE_F16 && out_dtype != APMOE_F32)
        return fail(APMOE_UNSUPPORTED, "out_dtype %d", out_dtype);
    if (!offsets)
        return fail(APMOE_INVALID_ARG, "offsets is NULL");
    if (T == 0)
        return ok();
    if (!in || !out || (gather && !perm))
        return fail(APMOE_INVALID_ARG, "in / out / perm is NULL");
    if (!aligned16(in) || !aligned16(out))
        return fail(APMOE_INVALID_ARG, "in / out not 16-byte aligned");
    int N, K, max_q;
    size_t in_bytes;
    s = gemm_limits(tbl, layer, kind, T, topk, gather, act, &N, &K, &max_q, &in_bytes);
    if (s != APMOE_OK)
        return s;
    const DevBlock *slice = tbl->d_table + tbl->index(layer, 0, 0);
    // experts by committed q, highest first (stable): the order in which the decode and mid
    // products start them when the layer has more than 16 experts (a scheduling hint)
    uint8_t order[APMOE_MAX_EXPERTS];
    int n = 0;
    for (int q = APMOE_MAX_BITS; q >= 0; --q)
        for (int e = 0; e < tbl->E; ++e)
            if (tbl->cq[tbl->index(layer, e, kind)] == q)
                order[n++] = (uint8_t)e;
    if (n != tbl->E)  // unreachable: commit keeps every q in 3..8
        for (n = 0; n < tbl->E; ++n)
            order[n] = (uint8_t)n;
    hipError_t e = apmoe::launch_gemm(slice, kind, tbl->E, N, K, max_q, order, in, in_bytes, gather, perm, offsets,
                                      topk, T * topk, out, out_dtype == APMOE_F32, act, comb,
                                      reinterpret_cast<hipStream_t>(stream), ctx->cus, ctx->side);
    return e == hipSuccess ? ok() : hip_fail(e, "gemm launch");
}

apmoe_status apmoe_gemm(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, int32_t kind, const uint16_t *in,
                        int32_t gather, const int32_t *perm, const int32_t *offsets, int32_t T, int32_t topk,
                        void *out, int32_t out_dtype, void *stream)
{
    return gemm_common(ctx, tbl, layer, kind, in, gather, perm, offsets, T, topk, out, out_dtype, 0, stream);
}

apmoe_status apmoe_gemm_act(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, const uint16_t *x,
                            int32_t gather, const int32_t *perm, const int32_t *offsets, int32_t T, int32_t topk,
                            uint16_t *a, void *stream)
{
    return gemm_common(ctx, tbl, layer, APMOE_GATE_UP, x, gather, perm, offsets, T, topk, a, APMOE_F16, 1, stream);
}

apmoe_status apmoe_act(apmoe_ctx *ctx, const uint16_t *h, int32_t R, int32_t F, uint16_t *a, void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (R < 0 || F < 8 || F % 8 != 0)
        return fail(APMOE_INVALID_ARG, "R=%d F=%d (need F%%8==0)", R, F);
    if (R > 0 && (!h || !a || !aligned16(h) || !aligned16(a)))
        return fail(APMOE_INVALID_ARG, "h / a NULL or not 16-byte aligned");
    hipError_t e = apmoe::launch_act(h, R, F, a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "act launch");
}

apmoe_status apmoe_combine(apmoe_ctx *ctx, const void *y, int32_t y_dtype, const float *topk_w,
                           const int32_t *inv_perm, int32_t T, int32_t topk, int32_t H, uint16_t *out, void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    if (T < 0 || topk < 1 || topk > APMOE_MAX_ASSIGN || H < 8 || H % 8 != 0)
        return fail(APMOE_INVALID_ARG, "T=%d topk=%d H=%d", T, topk, H);
    if (y_dtype != APMOE_F16 && y_dtype != APMOE_F32)
        return fail(APMOE_UNSUPPORTED, "y_dtype %d", y_dtype);
    if (T > 0 && (!y || !topk_w || !inv_perm || !out || !aligned16(y) || !aligned16(out)))
        return fail(APMOE_INVALID_ARG, "NULL or misaligned pointer");
    hipError_t e = apmoe::launch_combine(y, y_dtype == APMOE_F32, topk_w, inv_perm, T, topk, H, out,
                                         reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "combine launch");
}

// ----------------------------------------------------------------------------
// whole layer
// ----------------------------------------------------------------------------

namespace {
struct WsLayout {
    size_t ids, w, counts, offsets, perm, inv_perm, a, y, total;
};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int T, int topk, int E, int H, int F)
{
    WsLayout L;
    const size_t R = (size_t)T * topk;
    size_t o = 0;
    L.ids = o;
    o = up256(o + R * 4);
    L.w = o;
    o = up256(o + R * 4);
    L.counts = o;
    o = up256(o + (size_t)E * 4);
    L.offsets = o;
    o = up256(o + ((size_t)E + 1) * 4);
    L.perm = o;
    o = up256(o + R * 4);
    L.inv_perm = o;
    o = up256(o + R * 4);
    L.a = o;
    o = up256(o + R * F * 2);
    L.y = o;
    o = up256(o + R * H * 4);
    L.total = o;
    return L;
}
}  // namespace

apmoe_status apmoe_moe_workspace(const apmoe_table *tbl, int32_t layer, int32_t T, int32_t topk, int32_t n_shared,
                                 size_t *bytes)
{
    apmoe_status s = check_index(tbl, layer, 0, 0);
    if (s != APMOE_OK)
        return s;
    if (!bytes || T < 0 || topk < 1 || n_shared < 0 || n_shared >= tbl->E)
        return fail(APMOE_INVALID_ARG, "bytes NULL or T/topk/n_shared invalid");
    int N0, K0, q0, N1, K1, q1;
    s = layer_shape(tbl, layer, APMOE_GATE_UP, &N0, &K0, &q0);
    if (s != APMOE_OK)
        return s;
    s = layer_shape(tbl, layer, APMOE_DOWN, &N1, &K1, &q1);
    if (s != APMOE_OK)
        return s;
    *bytes = ws_layout(T, topk + n_shared, tbl->E, K0, K1).total;
    return ok();
}

apmoe_status apmoe_moe_forward(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, const uint16_t *x,
                               const uint16_t *w_router, const float *bias, int32_t T, int32_t topk,
                               int32_t n_shared, int32_t renormalize, void *ws, size_t ws_bytes, uint16_t *out,
                               void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    s = check_index(tbl, layer, 0, 0);
    if (s != APMOE_OK)
        return s;
    int N0, K0, q0, N1, K1, q1;
    s = layer_shape(tbl, layer, APMOE_GATE_UP, &N0, &K0, &q0);
    if (s != APMOE_OK)
        return s;
    s = layer_shape(tbl, layer, APMOE_DOWN, &N1, &K1, &q1);
    if (s != APMOE_OK)
        return s;
    const int H = K0, F = K1;
    if (N0 != 2 * F || N1 != H)
        return fail(APMOE_INVALID_ARG, "layer %d shapes: gate_up %dx%d, down %dx%d are not [2F x H], [H x F]",
                    layer, N0, K0, N1, K1);
    if (n_shared < 0 || n_shared >= tbl->E)
        return fail(APMOE_INVALID_ARG, "n_shared=%d with %d experts in the table", n_shared, tbl->E);
    const int kt = topk + n_shared;  // assignments per token
    // every limit of the four steps is checked before the first launch, so a refused
    // call enqueues nothing
    if (T < 0 || topk < 1 || topk > tbl->E - n_shared || topk > APMOE_MAX_TOPK || H % 8 != 0)
        return fail(APMOE_INVALID_ARG, "T=%d topk=%d H=%d", T, topk, H);
    if ((int64_t)T * kt > (int64_t)1 << 30)
        return fail(APMOE_INVALID_ARG, "T*topk too large");
    const WsLayout L = ws_layout(T, kt, tbl->E, H, F);
    if (!ws || ws_bytes < L.total || ((uintptr_t)ws & 255u))
        return fail(APMOE_INVALID_ARG, "workspace NULL, unaligned or smaller than %zu bytes", L.total);
    if (T > 0 && (!out || !aligned16(out)))
        return fail(APMOE_INVALID_ARG, "out NULL or misaligned");
    if (T > 0 && (!x || !w_router || !aligned16(x) || !aligned16(w_router)))
        return fail(APMOE_INVALID_ARG, "x / w_router NULL or not 16-byte aligned");
    if (T > 0) {
        if (!tbl->committed_once || !tbl->d_table)
            return fail(APMOE_NOT_RESIDENT, "table was never committed");
        if (tbl->device != ctx->device)
            return fail(APMOE_INVALID_ARG, "table lives on device %d, ctx on %d", tbl->device, ctx->device);
        int n_, k_, q_;
        size_t b_;
        s = gemm_limits(tbl, layer, APMOE_GATE_UP, T, kt, 1, 1, &n_, &k_, &q_, &b_);
        if (s != APMOE_OK)
            return s;
        s = gemm_limits(tbl, layer, APMOE_DOWN, T, kt, 0, 0, &n_, &k_, &q_, &b_);
        if (s != APMOE_OK)
            return s;
    }
    char *w = reinterpret_cast<char *>(ws);
    int32_t *ids = reinterpret_cast<int32_t *>(w + L.ids);
    float *tw = reinterpret_cast<float *>(w + L.w);
    int32_t *counts = reinterpret_cast<int32_t *>(w + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(w + L.offsets);
    int32_t *perm = reinterpret_cast<int32_t *>(w + L.perm);
    int32_t *inv = reinterpret_cast<int32_t *>(w + L.inv_perm);
    uint16_t *a = reinterpret_cast<uint16_t *>(w + L.a);
    float *y = reinterpret_cast<float *>(w + L.y);
    s = apmoe_route(ctx, x, w_router, bias, T, H, tbl->E - n_shared, topk, n_shared, renormalize, ids, tw, counts,
                    offsets, perm, inv, stream);
    if (s != APMOE_OK || T == 0)
        return s;
    // With at most kDecodeMaxRows tokens every expert takes the decode product, and the
    // output accumulation runs in the down product's epilogue (same bits as the separate
    // launch); where the shapes allow, gate_up and down then run as one launch (same bits).
    const int nb = (H + 63) / 64;
    const bool fuse_comb = ctx->fuse && T <= apmoe::kDecodeMaxRows && (int64_t)T * nb <= kCombineCounters;
    apmoe::CombineArgs comb;
    comb.w = tw;
    comb.inv_perm = inv;
    comb.out = out;
    comb.cnt = ctx->sync + kCombineCounter0;
    if (fuse_comb && ctx->layer_kernel && apmoe::layer_launch_fits(tbl->E, H, F, T)) {
        const DevBlock *slice = tbl->d_table + tbl->index(layer, 0, 0);
        hipError_t e = apmoe::launch_layer(slice, tbl->E, H, F, x, perm, offsets, kt, T, a, y, comb,
                                           ctx->sync + kLayerSync, ctx->sync + kLayerDone,
                                           reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? ok() : hip_fail(e, "layer launch");
    }
    // gate_up with SiLU(gate) * up in its epilogue (F = K of down is a multiple of 128)
    s = apmoe_gemm_act(ctx, tbl, layer, x, 1, perm, offsets, T, kt, a, stream);
    if (s != APMOE_OK)
        return s;
    if (fuse_comb)
        return gemm_common(ctx, tbl, layer, APMOE_DOWN, a, 0, perm, offsets, T, kt, y, APMOE_F32, 0, stream, &comb);
    s = apmoe_gemm(ctx, tbl, layer, APMOE_DOWN, a, 0, perm, offsets, T, kt, y, APMOE_F32, stream);
    if (s != APMOE_OK)
        return s;
    return apmoe_combine(ctx, y, APMOE_F32, tw, inv, T, kt, H, out, stream);
}

apmoe_status apmoe_moe_forward_noalloc(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, const uint16_t *x,
                                       const uint16_t *w_router, const float *bias, int32_t T, int32_t topk,
                                       int32_t n_shared, int32_t renormalize, uint16_t *out, void *stream)
{
    apmoe_status s = check_ctx(ctx);
    if (s != APMOE_OK)
        return s;
    size_t need = 0;
    s = apmoe_moe_workspace(tbl, layer, T, topk, n_shared, &need);
    if (s != APMOE_OK)
        return s;
    if (need > kScratchBytes)
        return fail(APMOE_INVALID_ARG,
                    "layer %d at T=%d needs %zu bytes of workspace, above the %zu-byte static scratch of the "
                    "allocation-free entry point",
                    layer, T, need, kScratchBytes);
    if (!ctx->scratch)
        return fail(APMOE_HIP_ERROR, "the context has no address of the static scratch");
    // the same launches as apmoe_moe_forward, with this device's scratch as the workspace
    return apmoe_moe_forward(ctx, tbl, layer, x, w_router, bias, T, topk, n_shared, renormalize, ctx->scratch,
                             kScratchBytes, out, stream);
}

}  // extern "C"
