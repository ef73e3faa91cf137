// api.hip -- the C ABI of libgdn.so (declared in include/gdn.h): host-side
// validation of every argument, then asynchronous launches on the caller's
// stream.  Nothing is allocated and nothing is enqueued on a validation error.
#include <cmath>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

thread_local char g_err[320];

gdn_status fail(gdn_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

gdn_status ok() {
    g_err[0] = 0;
    return GDN_OK;
}

struct Span {
    const char *name;
    const void *p;
    size_t bytes;
};

bool overlap(const Span &x, const Span &y) {
    if (!x.p || !y.p || !x.bytes || !y.bytes) return false;
    const uintptr_t a0 = (uintptr_t)x.p, a1 = a0 + x.bytes;
    const uintptr_t b0 = (uintptr_t)y.p, b1 = b0 + y.bytes;
    return a0 < b1 && b0 < a1;
}

gdn_status need(const Span &s, size_t align) {
    if (s.bytes == 0) return GDN_OK;  // empty tensor: pointer unused
    if (!s.p) return fail(GDN_ERR_NULL, "%s is NULL", s.name);
    if ((uintptr_t)s.p % align)
        return fail(GDN_ERR_ALIGN, "%s is not %zu-byte aligned", s.name, align);
    return GDN_OK;
}

gdn_status check_dims(const gdn_dims *d, bool prefill) {
    if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
    if (d->B < 0) return fail(GDN_ERR_SHAPE, "B = %d < 0", d->B);
    if (prefill && d->T < 0) return fail(GDN_ERR_SHAPE, "T = %d < 0", d->T);
    if (d->Hk < 1 || d->Hv < 1) return fail(GDN_ERR_SHAPE, "Hk = %d, Hv = %d: need >= 1", d->Hk, d->Hv);
    if (d->Hv % d->Hk) return fail(GDN_ERR_SHAPE, "Hv = %d is not a multiple of Hk = %d", d->Hv, d->Hk);
    if (d->Dk != 64 && d->Dk != 128) return fail(GDN_ERR_UNSUPPORTED, "Dk = %d: supported 64, 128", d->Dk);
    if (d->Dv != 64 && d->Dv != 128) return fail(GDN_ERR_UNSUPPORTED, "Dv = %d: supported 64, 128", d->Dv);
    if (prefill && d->chunk != 64) return fail(GDN_ERR_UNSUPPORTED, "chunk = %d: supported 64", d->chunk);
    if (d->dtype != GDN_F32 && d->dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "dtype = %d: supported GDN_F32, GDN_BF16", d->dtype);
    if (!isfinite(d->scale)) return fail(GDN_ERR_SHAPE, "scale is not finite");
    // launch-grid limits
    const long long units = (long long)d->B * d->Hv;
    if (units > 0x7fffffffLL / 2) return fail(GDN_ERR_SHAPE, "B * Hv = %lld too large", units);
    if (prefill) {
        const long long nc = ((long long)d->T + 63) / 64;
        if (d->Hk > 65535 || d->B > 65535)
            return fail(GDN_ERR_SHAPE, "Hk = %d, B = %d: grid limit 65535", d->Hk, d->B);
        if (units * nc > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "B * Hv * ceil(T/64) too large");
        // one sequence of v / out is addressed with 32-bit byte offsets
        const long long seq_bytes = (((long long)d->T + 63) / 64 * 64) * d->Hv * d->Dv *
                                    (d->dtype == GDN_F32 ? 4 : 2);
        if (seq_bytes > 0x7fffffffLL)
            return fail(GDN_ERR_UNSUPPORTED, "T * Hv * Dv * element size = %lld bytes per sequence: limit 2^31",
                        seq_bytes);
    }
    return GDN_OK;
}

size_t esize(const gdn_dims *d) { return d->dtype == GDN_F32 ? 4 : 2; }

}  // namespace

extern "C" {

const char *gdn_status_str(int s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
        default: return "GDN_ERR_UNKNOWN";
    }
}

const char *gdn_last_error(void) { return g_err; }

size_t gdn_chunk_fwd_workspace_bytes(const gdn_dims *d) {
    if (check_dims(d, true) != GDN_OK) return 0;
    if (d->B == 0 || d->T == 0) return 0;
    return gdn::prefill_workspace_layout(d->B, d->T, d->Hk, d->Hv, d->Dk, d->dtype == GDN_F32, nullptr,
                                         nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Device scratch of gdn_chunk_fwd_noalloc: the prefill workspace in a
// file-scope device array instead of caller memory.  Each GPU the library runs
// on holds its own copy (allocated with the code object, kept until the
// process ends).  In host code `scratch` names a host-side stand-in, not a
// device address: its address on a device is resolved once per device with
// hipGetSymbolAddress (with that device current) and only that pointer is
// ever handed to a kernel.  Calls on one GPU share the array; the prefill
// kernels write every workspace byte they read, so nothing is cleared.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_MAX_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (nullptr: not resolved yet)

// Device address of `scratch` on the device that runs `stream`.
gdn_status scratch_on(hipStream_t stream, void **ptr) {
    int cur = -1, dev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    dev = cur;
    if (stream) {
        hipDevice_t sd;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(GDN_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess && e2 != hipSuccess) e = e2;
        }
        if (e != hipSuccess || !p)
            return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GDN_OK;
}

// The chunked prefill: validation, then the launches.  With noalloc the
// workspace arguments are ignored and the device scratch is used (the size
// limit is checked with the other arguments, before any HIP call).
gdn_status prefill(const gdn_dims *d, const void *q, const void *k, const void *v, const float *a,
                   const float *b, const float *A_log, const float *dt_bias, const float *initial_state,
                   void *out, float *final_state, void *workspace, size_t workspace_bytes, void *stream,
                   void *const *stage_events, bool noalloc) {
    gdn_status st = check_dims(d, true);
    if (st != GDN_OK) return st;
    if (noalloc) {
        const size_t wneed = gdn_chunk_fwd_workspace_bytes(d);
        if (wneed > GDN_NOALLOC_MAX_WORKSPACE_BYTES)
            return fail(GDN_ERR_WORKSPACE,
                        "these dims need %zu bytes of scratch, more than the %zu bytes gdn_chunk_fwd_noalloc "
                        "holds: call gdn_chunk_fwd with a workspace",
                        wneed, (size_t)GDN_NOALLOC_MAX_WORKSPACE_BYTES);
        workspace = nullptr;
        workspace_bytes = 0;
    }
    const size_t B = d->B, T = d->T, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv, es = esize(d);
    const Span sq{"q", q, B * T * Hk * Dk * es}, sk{"k", k, B * T * Hk * Dk * es};
    const Span sv{"v", v, B * T * Hv * Dv * es};
    const Span sa{"a", a, B * T * Hv * 4}, sb{"b", b, B * T * Hv * 4};
    const Span sal{"A_log", A_log, Hv * 4}, sdt{"dt_bias", dt_bias, Hv * 4};
    const Span s0{"initial_state", initial_state, initial_state ? B * Hv * Dk * Dv * 4 : 0};
    const Span so{"out", out, B * T * Hv * Dv * es};
    const Span sf{"final_state", final_state, final_state ? B * Hv * Dk * Dv * 4 : 0};
    const size_t wneed = gdn_chunk_fwd_workspace_bytes(d);
    const Span sw{"workspace", workspace, wneed};
    for (const Span *s : {&sq, &sk, &sv, &so, &s0, &sf})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    for (const Span *s : {&sa, &sb, &sal, &sdt})
        if ((st = need(*s, 4)) != GDN_OK) return st;
    if (wneed && !noalloc) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", wneed);
        if (workspace_bytes < wneed)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, wneed);
        if ((uintptr_t)workspace % 256) return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    }
    for (const Span *s : {&sq, &sk, &sv, &sa, &sb, &sal, &sdt, &s0, &sf, &sw})
        if (overlap(so, *s)) return fail(GDN_ERR_ALIAS, "out overlaps %s", s->name);
    for (const Span *s : {&sq, &sk, &sv, &sa, &sb, &sal, &sdt, &sw})
        if (overlap(sf, *s)) return fail(GDN_ERR_ALIAS, "final_state overlaps %s", s->name);
    if (overlap(sf, s0) && final_state != initial_state)
        return fail(GDN_ERR_ALIAS, "final_state partly overlaps initial_state");
    for (const Span *s : {&sq, &sk, &sv, &sa, &sb, &sal, &sdt, &s0})
        if (overlap(sw, *s)) return fail(GDN_ERR_ALIAS, "workspace overlaps %s", s->name);
    ok();
    if (B == 0) return GDN_OK;

    hipStream_t hs = (hipStream_t)stream;
    gdn::PrefillArgs p;
    p.B = d->B; p.T = d->T; p.Hk = d->Hk; p.Hv = d->Hv; p.Dk = d->Dk; p.Dv = d->Dv;
    p.f32 = d->dtype == GDN_F32;
    p.scale = d->scale;
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.A_log = A_log; p.dt_bias = dt_bias;
    p.S0 = initial_state; p.out = out; p.ST = final_state;
    hipEvent_t const *ev = (hipEvent_t const *)stage_events;
    auto rec = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], hs) : hipSuccess; };
    hipError_t e = hipSuccess;
    if (T == 0) {
        if (final_state && final_state != initial_state) e = gdn::launch_state_copy(p, hs);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
        return GDN_OK;
    }
    if (noalloc && (st = scratch_on(hs, &workspace)) != GDN_OK) return st;
    gdn::PrefillWorkspace ws;
    gdn::prefill_workspace_layout(d->B, d->T, d->Hk, d->Hv, d->Dk, p.f32, workspace, &ws);
    if (e == hipSuccess) e = rec(0);
    if (e == hipSuccess) e = gdn::launch_chunk_local(p, ws, hs);
    if (e == hipSuccess) e = rec(1);
    if (e == hipSuccess) e = gdn::launch_state_scan(p, ws, hs);
    if (e == hipSuccess) e = rec(2);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd_timed(const gdn_dims *d, const void *q, const void *k, const void *v,
                               const float *a, const float *b, const float *A_log,
                               const float *dt_bias, const float *initial_state, void *out,
                               float *final_state, void *workspace, size_t workspace_bytes,
                               void *stream, void *const *stage_events) {
    return prefill(d, q, k, v, a, b, A_log, dt_bias, initial_state, out, final_state, workspace,
                   workspace_bytes, stream, stage_events, false);
}

gdn_status gdn_chunk_fwd(const gdn_dims *d, const void *q, const void *k, const void *v,
                         const float *a, const float *b, const float *A_log, const float *dt_bias,
                         const float *initial_state, void *out, float *final_state, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return prefill(d, q, k, v, a, b, A_log, dt_bias, initial_state, out, final_state, workspace,
                   workspace_bytes, stream, nullptr, false);
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_dims *d, const void *q, const void *k, const void *v,
                                 const float *a, const float *b, const float *A_log,
                                 const float *dt_bias, const float *initial_state, void *out,
                                 float *final_state, void *stream) {
    return prefill(d, q, k, v, a, b, A_log, dt_bias, initial_state, out, final_state, nullptr, 0, stream,
                   nullptr, true);
}

size_t gdn2_chunk_fwd_workspace_bytes(const gdn_dims *d) {
    if (check_dims(d, true) != GDN_OK) return 0;
    if (d->B == 0 || d->T == 0) return 0;
    return gdn::gdn2_workspace_layout(d->B, d->T, d->Hv, d->Dk, d->Dv, d->dtype == GDN_F32, nullptr, nullptr);
}

gdn_status gdn2_chunk_fwd(const gdn_dims *d, const void *q, const void *k, const void *v, const void *a,
                          const float *A_log, const void *erase, const void *write,
                          const float *initial_state, void *out, float *final_state, void *workspace,
                          size_t workspace_bytes, void *stream) {
    gdn_status st = check_dims(d, true);
    if (st != GDN_OK) return st;
    const size_t B = d->B, T = d->T, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv, es = esize(d);
    const Span sq{"q", q, B * T * Hk * Dk * es}, sk{"k", k, B * T * Hk * Dk * es};
    const Span sv{"v", v, B * T * Hv * Dv * es};
    const Span sa{"a", a, B * T * Hv * Dk * es}, se{"erase", erase, B * T * Hv * Dk * es};
    const Span swr{"write", write, B * T * Hv * Dv * es};
    const Span sal{"A_log", A_log, Hv * Dk * 4};
    const Span s0{"initial_state", initial_state, initial_state ? B * Hv * Dk * Dv * 4 : 0};
    const Span so{"out", out, B * T * Hv * Dv * es};
    const Span sf{"final_state", final_state, final_state ? B * Hv * Dk * Dv * 4 : 0};
    const size_t wneed = gdn2_chunk_fwd_workspace_bytes(d);
    const Span sw{"workspace", workspace, wneed};
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &so, &s0, &sf})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    if ((st = need(sal, 4)) != GDN_OK) return st;
    if (wneed) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", wneed);
        if (workspace_bytes < wneed)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, wneed);
        if ((uintptr_t)workspace % 256) return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    }
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &sal, &s0, &sf, &sw})
        if (overlap(so, *s)) return fail(GDN_ERR_ALIAS, "out overlaps %s", s->name);
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &sal, &sw})
        if (overlap(sf, *s)) return fail(GDN_ERR_ALIAS, "final_state overlaps %s", s->name);
    if (overlap(sf, s0) && final_state != initial_state)
        return fail(GDN_ERR_ALIAS, "final_state partly overlaps initial_state");
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &sal, &s0})
        if (overlap(sw, *s)) return fail(GDN_ERR_ALIAS, "workspace overlaps %s", s->name);
    ok();
    if (B == 0) return GDN_OK;

    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (T == 0) {
        gdn::PrefillArgs p{};
        p.B = d->B; p.Hv = d->Hv; p.Dk = d->Dk; p.Dv = d->Dv; p.S0 = initial_state; p.ST = final_state;
        if (final_state && final_state != initial_state) e = gdn::launch_state_copy(p, hs);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
        return GDN_OK;
    }
    gdn::Gdn2Args p;
    p.B = d->B; p.T = d->T; p.Hk = d->Hk; p.Hv = d->Hv; p.Dk = d->Dk; p.Dv = d->Dv;
    p.f32 = d->dtype == GDN_F32;
    p.scale = d->scale;
    p.q = q; p.k = k; p.v = v; p.a = a; p.erase = erase; p.write = write; p.A_log = A_log;
    p.S0 = initial_state; p.out = out; p.ST = final_state;
    gdn::Gdn2Workspace ws;
    gdn::gdn2_workspace_layout(d->B, d->T, d->Hv, d->Dk, d->Dv, p.f32, workspace, &ws);
    e = gdn::launch_chunk_local2(p, ws, hs);
    if (e == hipSuccess) e = gdn::launch_state_scan2(p, ws, hs);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

size_t gdn2_chunk_bwd_workspace_bytes(const gdn_dims *d) {
    if (check_dims(d, true) != GDN_OK) return 0;
    if (d->B == 0 || d->T == 0) return 0;
    return gdn::bwd2_workspace_layout(d->B, d->T, d->Hv, d->Dk, d->Dv, nullptr, nullptr);
}

gdn_status gdn2_chunk_bwd_timed(const gdn_dims *d, const void *q, const void *k, const void *v,
                                const void *a, const float *A_log, const void *erase, const void *write,
                                const float *initial_state, const void *d_out, const float *d_final_state,
                                float *dq, float *dk, float *dv, float *da, float *d_erase, float *d_write,
                                float *dA_log, float *d_initial_state, void *workspace,
                                size_t workspace_bytes, void *stream, void *const *stage_events) {
    gdn_status st = check_dims(d, true);
    if (st != GDN_OK) return st;
    const size_t B = d->B, T = d->T, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv, es = esize(d);
    const Span sq{"q", q, B * T * Hk * Dk * es}, sk{"k", k, B * T * Hk * Dk * es};
    const Span sv{"v", v, B * T * Hv * Dv * es};
    const Span sa{"a", a, B * T * Hv * Dk * es}, se{"erase", erase, B * T * Hv * Dk * es};
    const Span swr{"write", write, B * T * Hv * Dv * es};
    const Span sal{"A_log", A_log, Hv * Dk * 4};
    const Span s0{"initial_state", initial_state, initial_state ? B * Hv * Dk * Dv * 4 : 0};
    const Span sdo{"d_out", d_out, B * T * Hv * Dv * es};
    const Span sdf{"d_final_state", d_final_state, d_final_state ? B * Hv * Dk * Dv * 4 : 0};
    const Span gq{"dq", dq, B * T * Hk * Dk * 4}, gk{"dk", dk, B * T * Hk * Dk * 4};
    const Span gv{"dv", dv, B * T * Hv * Dv * 4}, gw{"d_write", d_write, B * T * Hv * Dv * 4};
    const Span ga{"da", da, B * T * Hv * Dk * 4}, ge{"d_erase", d_erase, B * T * Hv * Dk * 4};
    const Span gal{"dA_log", dA_log, Hv * Dk * 4};
    const Span g0{"d_initial_state", d_initial_state, d_initial_state ? B * Hv * Dk * Dv * 4 : 0};
    const size_t wneed = gdn2_chunk_bwd_workspace_bytes(d);
    const Span sw{"workspace", workspace, wneed};
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &s0, &sdo, &sdf, &gq, &gk, &gv, &gw, &ga, &ge, &g0})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    for (const Span *s : {&sal, &gal})
        if ((st = need(*s, 4)) != GDN_OK) return st;
    if (wneed) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", wneed);
        if (workspace_bytes < wneed)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, wneed);
        if ((uintptr_t)workspace % 256) return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    }
    const Span *ins[] = {&sq, &sk, &sv, &sa, &se, &swr, &sal, &s0, &sdo, &sdf};
    const Span *outs[] = {&gq, &gk, &gv, &gw, &ga, &ge, &gal, &g0, &sw};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span *s : ins)
            if (overlap(*outs[i], *s)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i]->name, s->name);
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(*outs[i], *outs[j]))
                return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i]->name, outs[j]->name);
    }
    ok();
    gdn::Bwd2Args p{};
    p.B = d->B; p.T = d->T; p.Hk = d->Hk; p.Hv = d->Hv; p.Dk = d->Dk; p.Dv = d->Dv;
    p.NC = (d->T + 63) / 64; p.scale = d->scale; p.f32 = d->dtype == GDN_F32;
    p.q = q; p.k = k; p.v = v; p.a = a; p.erase = erase; p.write = write; p.A_log = A_log;
    p.S0 = initial_state; p.dout = d_out; p.dST = d_final_state;
    p.dq = dq; p.dk = dk; p.dv = dv; p.da = da; p.derase = d_erase; p.dwrite = d_write;
    p.dA_log = dA_log; p.dS0 = d_initial_state;
    gdn::Bwd2Workspace ws{};
    if (T) gdn::bwd2_workspace_layout(d->B, d->T, d->Hv, d->Dk, d->Dv, workspace, &ws);
    const hipEvent_t *ev = (p.T > 0) ? (const hipEvent_t *)stage_events : nullptr;
    const hipError_t e = gdn::launch_bwd2(p, ws, (hipStream_t)stream, ev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn2_chunk_bwd(const gdn_dims *d, const void *q, const void *k, const void *v, const void *a,
                          const float *A_log, const void *erase, const void *write,
                          const float *initial_state, const void *d_out, const float *d_final_state,
                          float *dq, float *dk, float *dv, float *da, float *d_erase, float *d_write,
                          float *dA_log, float *d_initial_state, void *workspace, size_t workspace_bytes,
                          void *stream) {
    return gdn2_chunk_bwd_timed(d, q, k, v, a, A_log, erase, write, initial_state, d_out, d_final_state, dq,
                                dk, dv, da, d_erase, d_write, dA_log, d_initial_state, workspace,
                                workspace_bytes, stream, nullptr);
}

gdn_status gdn_recurrent_step(const gdn_dims *d, const void *q, const void *k, const void *v,
                              const float *a, const float *b, const float *A_log,
                              const float *dt_bias, float *state, void *out, void *stream) {
    gdn_status st = check_dims(d, false);
    if (st != GDN_OK) return st;
    const size_t B = d->B, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv, es = esize(d);
    const Span sq{"q", q, B * Hk * Dk * es}, sk{"k", k, B * Hk * Dk * es};
    const Span sv{"v", v, B * Hv * Dv * es};
    const Span sa{"a", a, B * Hv * 4}, sb{"b", b, B * Hv * 4};
    const Span sal{"A_log", A_log, Hv * 4}, sdt{"dt_bias", dt_bias, Hv * 4};
    const Span ss{"state", state, B * Hv * Dk * Dv * 4};
    const Span so{"out", out, B * Hv * Dv * es};
    for (const Span *s : {&sq, &sk, &sv, &ss, &so})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    for (const Span *s : {&sa, &sb, &sal, &sdt})
        if ((st = need(*s, 4)) != GDN_OK) return st;
    for (const Span *s : {&sq, &sk, &sv, &sa, &sb, &sal, &sdt, &ss})
        if (overlap(so, *s)) return fail(GDN_ERR_ALIAS, "out overlaps %s", s->name);
    for (const Span *s : {&sq, &sk, &sv, &sa, &sb, &sal, &sdt})
        if (overlap(ss, *s)) return fail(GDN_ERR_ALIAS, "state overlaps %s", s->name);
    ok();
    if (B == 0) return GDN_OK;
    gdn::DecodeArgs p;
    p.B = d->B; p.Hk = d->Hk; p.Hv = d->Hv; p.Dk = d->Dk; p.Dv = d->Dv;
    p.f32 = d->dtype == GDN_F32;
    p.gdn2 = false;
    p.scale = d->scale;
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.write = nullptr; p.A_log = A_log; p.dt_bias = dt_bias;
    p.state = state; p.out = out;
    const hipError_t e = gdn::launch_decode(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn2_recurrent_step(const gdn_dims *d, const void *q, const void *k, const void *v,
                               const void *a, const float *A_log, const void *erase, const void *write,
                               float *state, void *out, void *stream) {
    gdn_status st = check_dims(d, false);
    if (st != GDN_OK) return st;
    const size_t B = d->B, Hk = d->Hk, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv, es = esize(d);
    const Span sq{"q", q, B * Hk * Dk * es}, sk{"k", k, B * Hk * Dk * es};
    const Span sv{"v", v, B * Hv * Dv * es};
    const Span sa{"a", a, B * Hv * Dk * es}, se{"erase", erase, B * Hv * Dk * es};
    const Span swr{"write", write, B * Hv * Dv * es};
    const Span sal{"A_log", A_log, Hv * Dk * 4};
    const Span ss{"state", state, B * Hv * Dk * Dv * 4};
    const Span so{"out", out, B * Hv * Dv * es};
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &ss, &so})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    if ((st = need(sal, 4)) != GDN_OK) return st;
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &sal, &ss})
        if (overlap(so, *s)) return fail(GDN_ERR_ALIAS, "out overlaps %s", s->name);
    for (const Span *s : {&sq, &sk, &sv, &sa, &se, &swr, &sal})
        if (overlap(ss, *s)) return fail(GDN_ERR_ALIAS, "state overlaps %s", s->name);
    ok();
    if (B == 0) return GDN_OK;
    gdn::DecodeArgs p;
    p.B = d->B; p.Hk = d->Hk; p.Hv = d->Hv; p.Dk = d->Dk; p.Dv = d->Dv;
    p.f32 = d->dtype == GDN_F32;
    p.gdn2 = true;
    p.scale = d->scale;
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = erase; p.write = write; p.A_log = A_log; p.dt_bias = nullptr;
    p.state = state; p.out = out;
    const hipError_t e = gdn::launch_decode(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t d, int32_t dtype, const void *x, const void *z,
                             const float *weight, float eps, int32_t gate, void *out, void *stream) {
    if (rows < 0) return fail(GDN_ERR_SHAPE, "rows = %lld < 0", (long long)rows);
    if (rows > gdn::gated_rmsnorm_max_rows()) return fail(GDN_ERR_UNSUPPORTED, "rows = %lld: too many", (long long)rows);
    if (d != 64 && d != 128) return fail(GDN_ERR_UNSUPPORTED, "d = %d: supported 64, 128", d);
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "dtype = %d: supported GDN_F32, GDN_BF16", dtype);
    if (gate != GDN_GATE_SILU && gate != GDN_GATE_SIGMOID)
        return fail(GDN_ERR_UNSUPPORTED, "gate = %d: supported GDN_GATE_SILU, GDN_GATE_SIGMOID", gate);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(GDN_ERR_SHAPE, "eps must be finite and >= 0");
    const size_t es = dtype == GDN_F32 ? 4 : 2, bytes = (size_t)rows * d * es;
    const Span sx{"x", x, bytes}, sz{"z", z, bytes}, so{"out", out, bytes}, sw{"weight", weight, rows ? (size_t)d * 4 : 0};
    gdn_status st;
    for (const Span *s : {&sx, &sz, &so, &sw})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    if (overlap(so, sx) && out != x) return fail(GDN_ERR_ALIAS, "out partly overlaps x");
    for (const Span *s : {&sz, &sw})
        if (overlap(so, *s)) return fail(GDN_ERR_ALIAS, "out overlaps %s", s->name);
    ok();
    gdn::NormArgs p;
    p.rows = rows; p.d = d; p.f32 = dtype == GDN_F32; p.silu = gate == GDN_GATE_SILU; p.eps = eps;
    p.x = x; p.z = z; p.w = weight; p.out = out;
    const hipError_t e = gdn::launch_gated_rmsnorm(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_causal_conv1d(const gdn_dims *d, int32_t kernel_size, const void *x, const float *weight,
                             const float *bias, const void *conv_state, void *conv_state_out,
                             int32_t activation, void *q, void *k, void *v, void *stream) {
    gdn_status st = check_dims(d, false);
    if (st != GDN_OK) return st;
    if (d->T < 0) return fail(GDN_ERR_SHAPE, "T = %d < 0", d->T);
    if (kernel_size != 4) return fail(GDN_ERR_UNSUPPORTED, "kernel_size = %d: supported 4", kernel_size);
    if (activation != GDN_ACT_NONE && activation != GDN_ACT_SILU)
        return fail(GDN_ERR_UNSUPPORTED, "activation = %d: supported GDN_ACT_NONE, GDN_ACT_SILU", activation);
    if (d->B > 65535 || (long long)d->T > 65535LL * gdn::conv_tokens_per_block())
        return fail(GDN_ERR_UNSUPPORTED, "B = %d, T = %d: at most 65535 sequences and %lld tokens", d->B, d->T,
                    65535LL * gdn::conv_tokens_per_block());
    const size_t B = d->B, T = d->T, K = kernel_size, es = esize(d);
    const size_t qk = (size_t)d->Hk * d->Dk, vw = (size_t)d->Hv * d->Dv, C = 2 * qk + vw;
    const Span sx{"x", x, B * T * C * es}, sw{"weight", weight, C * K * 4}, sb{"bias", bias, bias ? C * 4 : 0};
    const Span ss{"conv_state", conv_state, conv_state ? B * (K - 1) * C * es : 0};
    const Span so{"conv_state_out", conv_state_out, conv_state_out ? B * (K - 1) * C * es : 0};
    const Span sq{"q", q, B * T * qk * es}, sk{"k", k, B * T * qk * es}, sv{"v", v, B * T * vw * es};
    for (const Span *s : {&sx, &sq, &sk, &sv, &ss, &so, &sb})
        if ((st = need(*s, 16)) != GDN_OK) return st;
    if (B && (st = need(sw, 16)) != GDN_OK) return st;
    const Span *outs[] = {&sq, &sk, &sv, &so};
    for (const Span *o : outs) {
        for (const Span *s : {&sx, &sw, &sb})
            if (overlap(*o, *s)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", o->name, s->name);
        for (const Span *o2 : outs)
            if (o2 != o && overlap(*o, *o2)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", o->name, o2->name);
    }
    for (const Span *o : {&sq, &sk, &sv})
        if (overlap(*o, ss)) return fail(GDN_ERR_ALIAS, "%s overlaps conv_state", o->name);
    if (overlap(so, ss) && conv_state_out != conv_state)
        return fail(GDN_ERR_ALIAS, "conv_state_out partly overlaps conv_state");
    ok();
    if (B == 0) return GDN_OK;
    gdn::ConvArgs p;
    p.B = d->B; p.T = d->T; p.C = (int)C; p.qk = (int)qk; p.K = kernel_size;
    p.f32 = d->dtype == GDN_F32; p.silu = activation == GDN_ACT_SILU;
    p.x = x; p.w = weight; p.bias = bias; p.state = conv_state; p.state_out = conv_state_out;
    p.q = q; p.k = k; p.v = v;
    const hipError_t e = gdn::launch_causal_conv1d(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_events_create(int n, void **events) {
    if (n < 0) return fail(GDN_ERR_SHAPE, "n = %d < 0", n);
    if (n && !events) return fail(GDN_ERR_NULL, "events is NULL");
    for (int i = 0; i < n; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) {
            for (int j = 0; j < i; ++j) (void)hipEventDestroy((hipEvent_t)events[j]);
            return fail(GDN_ERR_HIP, "hipEventCreate failed");
        }
        events[i] = (void *)e;
    }
    return ok();
}

gdn_status gdn_events_destroy(int n, void *const *events) {
    if (n && !events) return fail(GDN_ERR_NULL, "events is NULL");
    for (int i = 0; i < n; ++i)
        if (events[i]) (void)hipEventDestroy((hipEvent_t)events[i]);
    return ok();
}

gdn_status gdn_event_elapsed_ms(void *start, void *stop, float *ms) {
    if (!start || !stop || !ms) return fail(GDN_ERR_NULL, "NULL argument");
    const hipError_t e = hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)stop);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
