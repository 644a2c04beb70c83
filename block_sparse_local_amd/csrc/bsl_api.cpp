// bsl_api.cpp -- the C ABI declared in include/bsl.h: argument checks, device
// checks, dispatch to the kernel launchers.  No allocation on the device, no
// synchronisation, nothing thrown across the interface.
#include "bsl.h"

#include "bwd_launch.h"
#include "check.h"
#include "kmer_launch.h"
#include "launch.h"
#include "scratch.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

struct bsl_plan {
    bsl_desc desc;
    float scale;  // resolved
    int device;   // HIP ordinal the plan was made on
    int cu_count; // compute units of that device
};

namespace {

thread_local char g_last_error[512] = "";

bsl_status fail(bsl_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

bsl_status fail(bsl_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool overlaps(const void *a, size_t an, const void *b, size_t bn)
{
    const uint8_t *x = (const uint8_t *)a, *y = (const uint8_t *)b;
    return x < y + bn && y < x + an;
}

// A buffer the forward writes (o, lse, trace) or reads besides q, k, v (the
// lengths or offsets), with its size in bytes; ptr may be NULL (absent).
struct Span {
    const void *ptr;
    size_t bytes;
    const char *name;
};

// Every pair of spans in `w` (written) must be disjoint, and each must be
// disjoint from every span in `r` (read).  Absent (NULL) spans are skipped.
template <size_t NW, size_t NR>
bsl_status check_disjoint(const Span (&w)[NW], const Span (&r)[NR])
{
    for (size_t a = 0; a < NW; ++a) {
        if (!w[a].ptr)
            continue;
        for (size_t b = 0; b < NR; ++b)
            if (r[b].ptr && overlaps(w[a].ptr, w[a].bytes, r[b].ptr, r[b].bytes))
                return fail(BSL_E_INVALID, "%s overlaps %s", w[a].name, r[b].name);
        for (size_t b = a + 1; b < NW; ++b)
            if (w[b].ptr && overlaps(w[a].ptr, w[a].bytes, w[b].ptr, w[b].bytes))
                return fail(BSL_E_INVALID, "%s overlaps %s", w[a].name, w[b].name);
    }
    return BSL_OK;
}

// The block band the kernels sweep: R itself, or with a token window W the
// ceil(W / 32) blocks on either side that hold every key within W tokens.
int32_t band_radius(const bsl_desc &d)
{
    return d.window > 0 ? (d.window + d.block_size - 1) / d.block_size : d.radius;
}

bsl_status run(const bsl_plan *plan, int32_t batch, int32_t n, const void *q, const void *k,
               const void *v, void *o, const int32_t *seqlens, float *lse, int32_t *active,
               uint32_t *masks, void *stream, bool traced)
{
    if (!plan)
        return fail(BSL_E_INVALID, "plan is NULL");
    const bsl_desc &d = plan->desc;
    if (batch < 0 || n < 0)
        return fail(BSL_E_INVALID, "batch (%d) and n (%d) must be >= 0", batch, n);
    if (n % d.block_size != 0)
        return fail(BSL_E_INVALID, "n (%d) is not a multiple of the block size %d", n,
                    d.block_size);
    if (batch == 0 || n == 0)
        return BSL_OK;
    if (!q || !k || !v || !o)
        return fail(BSL_E_INVALID, "q, k, v and o must be non-NULL device pointers");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(BSL_E_INVALID, "q, k, v and o must be 16-byte aligned");
    if (traced && (!active || !masks))
        return fail(BSL_E_INVALID, "traced forward needs non-NULL active and masks");
    // element counts must fit comfortably in 64-bit offsets, grids in 31 bits
    const long double elems = (long double)batch * d.heads * (long double)n * d.head_dim;
    if (elems > 9.0e18L)
        return fail(BSL_E_INVALID, "tensor of %d x %d x %d x %d elements is too large", batch,
                    d.heads, n, d.head_dim);
    const long long nblk = n / d.block_size;
    if ((long long)batch * d.heads * nblk > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "batch * heads * n / 32 exceeds 2^31 - 1");
    if (lse && !aligned16(lse))
        return fail(BSL_E_INVALID, "lse must be 16-byte aligned");
    if (traced && (!aligned4(active) || !aligned4(masks)))
        return fail(BSL_E_INVALID, "active and masks must be 4-byte aligned");
    const int32_t radius = band_radius(d);
    // trace slots: batch * nblk * (2R + 1) words, 32 more per slot for the masks
    const long double slots = (long double)batch * (long double)nblk * (2.0L * radius + 1.0L);
    if (traced && slots * 128.0L > 9.0e18L)
        return fail(BSL_E_INVALID, "the trace of %d x %lld blocks x %d slots is too large", batch,
                    nblk, 2 * radius + 1);
    const size_t esz = d.dtype == BSL_BF16 ? 2 : 4;
    const size_t bytes = (size_t)elems * esz;
    const size_t rows = (size_t)batch * (size_t)d.heads * (size_t)n;
    const Span written[] = {{o, bytes, "o"},
                            {lse, rows * 4, "lse"},
                            {traced ? active : nullptr, (size_t)slots * 4, "active"},
                            {traced ? masks : nullptr, (size_t)slots * 128, "masks"}};
    const Span read[] = {{q, bytes, "q"}, {k, bytes, "k"}, {v, bytes, "v"},
                         {seqlens, (size_t)batch * 4, "seqlens"}};
    if (const bsl_status st = check_disjoint(written, read))
        return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(BSL_E_DEVICE, "hipGetDevice failed");
    if (dev != plan->device)
        return fail(BSL_E_INVALID, "current device %d is not the plan's device %d", dev,
                    plan->device);

    bsl::Launch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.seqlens = seqlens;
    a.cu_seqlens = nullptr;
    a.lse = lse;
    a.active = traced ? active : nullptr;
    a.masks = traced ? masks : nullptr;
    a.batch = batch;
    a.heads = d.heads;
    a.n = n;
    a.tokens = 0;
    a.head_dim = d.head_dim;
    a.radius = radius;
    a.window = d.window;
    a.causal = d.causal != 0;
    a.scale = plan->scale;
    a.stream = (hipStream_t)stream;
    const hipError_t e = d.dtype == BSL_BF16 ? bsl::launch_fwd_bf16(a) : bsl::launch_fwd_f32(a);
    if (e != hipSuccess)
        return fail(BSL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return BSL_OK;
}

bsl_status run_varlen(const bsl_plan *plan, int32_t batch, int32_t tokens, int32_t max_seqlen,
                      const void *q, const void *k, const void *v, void *o,
                      const int32_t *cu_seqlens, float *lse, void *stream)
{
    if (!plan)
        return fail(BSL_E_INVALID, "plan is NULL");
    const bsl_desc &d = plan->desc;
    if (batch < 0 || tokens < 0 || max_seqlen < 0)
        return fail(BSL_E_INVALID, "batch (%d), tokens (%d) and max_seqlen (%d) must be >= 0",
                    batch, tokens, max_seqlen);
    if (batch == 0 || tokens == 0 || max_seqlen == 0)
        return BSL_OK;
    if (!cu_seqlens)
        return fail(BSL_E_INVALID, "cu_seqlens must be a non-NULL device pointer");
    if (!q || !k || !v || !o)
        return fail(BSL_E_INVALID, "q, k, v and o must be non-NULL device pointers");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(BSL_E_INVALID, "q, k, v and o must be 16-byte aligned");
    const long double elems = (long double)tokens * d.heads * (long double)d.head_dim;
    if (elems > 9.0e18L)
        return fail(BSL_E_INVALID, "tensor of %d x %d x %d elements is too large", tokens,
                    d.heads, d.head_dim);
    const long long nblk = ((long long)max_seqlen + d.block_size - 1) / d.block_size;
    if ((long long)batch * d.heads * nblk > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "batch * heads * ceil(max_seqlen / 32) exceeds 2^31 - 1");
    if (lse && !aligned16(lse))
        return fail(BSL_E_INVALID, "lse must be 16-byte aligned");
    const size_t esz = d.dtype == BSL_BF16 ? 2 : 4;
    const size_t bytes = (size_t)elems * esz;
    const Span written[] = {{o, bytes, "o"}, {lse, (size_t)d.heads * (size_t)tokens * 4, "lse"}};
    const Span read[] = {{q, bytes, "q"}, {k, bytes, "k"}, {v, bytes, "v"},
                         {cu_seqlens, ((size_t)batch + 1) * 4, "cu_seqlens"}};
    if (const bsl_status st = check_disjoint(written, read))
        return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(BSL_E_DEVICE, "hipGetDevice failed");
    if (dev != plan->device)
        return fail(BSL_E_INVALID, "current device %d is not the plan's device %d", dev,
                    plan->device);

    bsl::Launch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.seqlens = nullptr;
    a.cu_seqlens = cu_seqlens;
    a.lse = lse;
    a.active = nullptr;
    a.masks = nullptr;
    a.batch = batch;
    a.heads = d.heads;
    a.n = max_seqlen;
    a.tokens = tokens;
    a.head_dim = d.head_dim;
    a.radius = band_radius(d);
    a.window = d.window;
    a.causal = d.causal != 0;
    a.scale = plan->scale;
    a.stream = (hipStream_t)stream;
    const hipError_t e = d.dtype == BSL_BF16 ? bsl::launch_fwd_bf16(a) : bsl::launch_fwd_f32(a);
    if (e != hipSuccess)
        return fail(BSL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return BSL_OK;
}

// Pointer, alignment, overlap and device checks shared by the two backward
// entry points: ins = {q, k, v, o, dout, lse}, outs = {dq, dk, dv, delta}; tb
// bytes per tensor, rb per row vector (lse, delta).  BSL_OK when all pass.
bsl_status check_bwd_buffers(const bsl_plan *plan, const void *const (&ins)[6],
                             void *const (&outs)[4], size_t tb, size_t rb, bool sizes_known)
{
    for (const void *x : ins)
        if (!x)
            return fail(BSL_E_INVALID, "q, k, v, o, dout and lse must be non-NULL device pointers");
    for (const void *x : outs)
        if (!x)
            return fail(BSL_E_INVALID, "dq, dk, dv and delta must be non-NULL device pointers");
    for (const void *x : ins)
        if (!aligned16(x))
            return fail(BSL_E_INVALID, "every tensor must be 16-byte aligned");
    for (const void *x : outs)
        if (!aligned16(x))
            return fail(BSL_E_INVALID, "every tensor must be 16-byte aligned");
    if (!sizes_known)
        return BSL_OK;
    const size_t in_bytes[] = {tb, tb, tb, tb, tb, rb};
    const size_t out_bytes[] = {tb, tb, tb, rb};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b]))
                return fail(BSL_E_INVALID, "dq, dk, dv and delta must not overlap any input");
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b]))
                return fail(BSL_E_INVALID, "dq, dk, dv and delta must not overlap each other");
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(BSL_E_DEVICE, "hipGetDevice failed");
    if (dev != plan->device)
        return fail(BSL_E_INVALID, "current device %d is not the plan's device %d", dev,
                    plan->device);
    return BSL_OK;
}

bsl_status run_backward(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                        const void *k, const void *v, const void *o, const void *dout,
                        const float *lse, const int32_t *seqlens, void *dq, void *dk, void *dv,
                        float *delta, void *stream)
{
    if (!plan)
        return fail(BSL_E_INVALID, "plan is NULL");
    const bsl_desc &d = plan->desc;
    if (batch < 0 || n < 0)
        return fail(BSL_E_INVALID, "batch (%d) and n (%d) must be >= 0", batch, n);
    if (n % d.block_size != 0)
        return fail(BSL_E_INVALID, "n (%d) is not a multiple of the block size %d", n,
                    d.block_size);
    if (batch == 0 || n == 0)
        return BSL_OK;
    const void *const ins[] = {q, k, v, o, dout, lse};
    void *const outs[] = {dq, dk, dv, delta};
    if (const bsl_status st = check_bwd_buffers(plan, ins, outs, 0, 0, false))
        return st;
    const long double elems = (long double)batch * d.heads * (long double)n * d.head_dim;
    if (elems > 9.0e18L)
        return fail(BSL_E_INVALID, "tensor of %d x %d x %d x %d elements is too large", batch,
                    d.heads, n, d.head_dim);
    const long long nblk = n / d.block_size;
    if ((long long)batch * d.heads * nblk > 0x7fffffffLL ||
        (long long)batch * d.heads * n > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "batch * heads * n exceeds 2^31 - 1");
    const size_t tb = (size_t)elems * (d.dtype == BSL_BF16 ? 2 : 4); // one tensor
    const size_t rb = (size_t)batch * d.heads * (size_t)n * 4;     // one float row vector
    if (const bsl_status st = check_bwd_buffers(plan, ins, outs, tb, rb, true))
        return st;
    {
        const Span written[] = {{dq, tb, "dq"}, {dk, tb, "dk"}, {dv, tb, "dv"},
                                {delta, rb, "delta"}};
        const Span read[] = {{seqlens, (size_t)batch * 4, "seqlens"}};
        if (const bsl_status st = check_disjoint(written, read))
            return st;
    }

    bsl::BwdLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.seqlens = seqlens;
    a.cu_seqlens = nullptr;
    a.tokens = 0;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.batch = batch;
    a.heads = d.heads;
    a.n = n;
    a.head_dim = d.head_dim;
    a.radius = band_radius(d);
    a.window = d.window;
    a.causal = d.causal != 0;
    a.scale = plan->scale;
    a.stream = (hipStream_t)stream;
    // bf16 at head_dim 64 and 128 on the matrix cores; the rest on the vector ALUs
    const hipError_t e = d.dtype == BSL_BF16 && d.head_dim != 32
                             ? bsl::launch_bwd_bf16(a)
                             : bsl::launch_bwd_valu(a, d.dtype == BSL_BF16);
    if (e != hipSuccess)
        return fail(BSL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return BSL_OK;
}

bsl_status run_backward_varlen(const bsl_plan *plan, int32_t batch, int32_t tokens,
                               int32_t max_seqlen, const void *q, const void *k, const void *v,
                               const void *o, const void *dout, const float *lse,
                               const int32_t *cu_seqlens, void *dq, void *dk, void *dv,
                               float *delta, void *stream)
{
    if (!plan)
        return fail(BSL_E_INVALID, "plan is NULL");
    const bsl_desc &d = plan->desc;
    if (batch < 0 || tokens < 0 || max_seqlen < 0)
        return fail(BSL_E_INVALID, "batch (%d), tokens (%d) and max_seqlen (%d) must be >= 0",
                    batch, tokens, max_seqlen);
    if (batch == 0 || tokens == 0 || max_seqlen == 0)
        return BSL_OK;
    if (!cu_seqlens)
        return fail(BSL_E_INVALID, "cu_seqlens must be a non-NULL device pointer");
    const void *const ins[] = {q, k, v, o, dout, lse};
    void *const outs[] = {dq, dk, dv, delta};
    if (const bsl_status st = check_bwd_buffers(plan, ins, outs, 0, 0, false))
        return st;
    const long double elems = (long double)tokens * d.heads * (long double)d.head_dim;
    if (elems > 9.0e18L)
        return fail(BSL_E_INVALID, "tensor of %d x %d x %d elements is too large", tokens,
                    d.heads, d.head_dim);
    const long long nblk = ((long long)max_seqlen + d.block_size - 1) / d.block_size;
    if ((long long)batch * d.heads * nblk > 0x7fffffffLL ||
        (long long)d.heads * tokens > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "batch * heads * ceil(max_seqlen / 32) or heads * tokens "
                                   "exceeds 2^31 - 1");
    const size_t tb = (size_t)elems * (d.dtype == BSL_BF16 ? 2 : 4); // one tensor
    const size_t rb = (size_t)d.heads * (size_t)tokens * 4;       // one float row vector
    if (const bsl_status st = check_bwd_buffers(plan, ins, outs, tb, rb, true))
        return st;
    {
        const Span written[] = {{dq, tb, "dq"}, {dk, tb, "dk"}, {dv, tb, "dv"},
                                {delta, rb, "delta"}};
        const Span read[] = {{cu_seqlens, ((size_t)batch + 1) * 4, "cu_seqlens"}};
        if (const bsl_status st = check_disjoint(written, read))
            return st;
    }

    bsl::BwdLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.seqlens = nullptr;
    a.cu_seqlens = cu_seqlens;
    a.tokens = tokens;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.batch = batch;
    a.heads = d.heads;
    a.n = max_seqlen;
    a.head_dim = d.head_dim;
    a.radius = band_radius(d);
    a.window = d.window;
    a.causal = d.causal != 0;
    a.scale = plan->scale;
    a.stream = (hipStream_t)stream;
    // bf16 at head_dim 64 and 128 on the matrix cores; the rest on the vector ALUs
    const hipError_t e = d.dtype == BSL_BF16 && d.head_dim != 32
                             ? bsl::launch_bwd_bf16(a)
                             : bsl::launch_bwd_valu(a, d.dtype == BSL_BF16);
    if (e != hipSuccess)
        return fail(BSL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return BSL_OK;
}

// Argument checks and launch shared by the two validators (mode 0: lengths,
// mode 1: offsets).
bsl_status check_common(int32_t batch, int32_t limit, const int32_t *v, int32_t *result,
                        void *stream, int mode)
{
    const char *what = mode == 0 ? "seqlens" : "cu_seqlens";
    if (batch < 0 || limit < 0)
        return fail(BSL_E_INVALID, "batch (%d) and the limit (%d) must be >= 0", batch, limit);
    if ((!v && (mode == 1 || batch > 0)) || !result)
        return fail(BSL_E_INVALID, "%s and result must be non-NULL device pointers", what);
    const size_t entries = (size_t)batch + (mode == 0 ? 0 : 1);
    if (v && overlaps(v, entries * 4, result, 8))
        return fail(BSL_E_INVALID, "result overlaps %s", what);
    const hipError_t e = bsl::launch_check(v, batch, limit, mode, result, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(BSL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return BSL_OK;
}

} // namespace

extern "C" {

bsl_status bsl_create(const bsl_desc *desc, bsl_plan **plan)
{
    if (!desc || !plan)
        return fail(BSL_E_INVALID, "desc and plan must be non-NULL");
    *plan = nullptr;
    const bsl_desc &d = *desc;
    if (d.heads < 1)
        return fail(BSL_E_INVALID, "heads must be >= 1 (got %d)", d.heads);
    if (d.radius < 0)
        return fail(BSL_E_INVALID, "radius must be >= 0 (got %d)", d.radius);
    if (d.causal != 0 && d.causal != 1)
        return fail(BSL_E_INVALID, "causal must be 0 or 1 (got %d)", d.causal);
    if (!std::isfinite(d.scale))
        return fail(BSL_E_INVALID, "scale must be finite");
    if (d.block_size != 32)
        return fail(BSL_E_UNSUPPORTED, "block_size must be 32 (got %d)", d.block_size);
    if (d.head_dim != 32 && d.head_dim != 64 && d.head_dim != 128)
        return fail(BSL_E_UNSUPPORTED, "head_dim must be 32, 64 or 128 (got %d)", d.head_dim);
    if (d.dtype != BSL_BF16 && d.dtype != BSL_F32)
        return fail(BSL_E_UNSUPPORTED, "unknown dtype %d", d.dtype);
    if (d.window < 0)
        return fail(BSL_E_INVALID, "window must be >= 0 (got %d)", d.window);
    if (d.radius > (1 << 24))
        return fail(BSL_E_UNSUPPORTED, "radius %d is too large", d.radius);
    if (d.window > (1 << 29))
        return fail(BSL_E_UNSUPPORTED, "window %d is too large", d.window);

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(BSL_E_DEVICE, "no HIP device");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(BSL_E_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(BSL_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                    prop.gcnArchName);

    // the fixed workspace of bsl_backward_noalloc: its address on this device,
    // looked up once per device while the device is current
    if (const hipError_t e = bsl::scratch_setup(dev); e != hipSuccess)
        return fail(BSL_E_DEVICE, "the fixed device workspace of device %d was not found: %s",
                    dev, hipGetErrorString(e));

    bsl_plan *p = new (std::nothrow) bsl_plan;
    if (!p)
        return fail(BSL_E_NOMEM, "out of host memory");
    p->desc = d;
    p->scale = d.scale > 0.0f ? d.scale : 1.0f / std::sqrt((float)d.head_dim);
    p->device = dev;
    p->cu_count = prop.multiProcessorCount;
    *plan = p;
    return BSL_OK;
}

bsl_status bsl_forward(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                       const void *k, const void *v, void *o, const int32_t *seqlens,
                       float *lse, void *stream)
{
    return run(plan, batch, n, q, k, v, o, seqlens, lse, nullptr, nullptr, stream, false);
}

bsl_status bsl_forward_traced(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                              const void *k, const void *v, void *o, const int32_t *seqlens,
                              float *lse, int32_t *active, uint32_t *masks, void *stream)
{
    return run(plan, batch, n, q, k, v, o, seqlens, lse, active, masks, stream, true);
}

bsl_status bsl_backward(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                        const void *k, const void *v, const void *o, const void *dout,
                        const float *lse, const int32_t *seqlens, void *dq, void *dk, void *dv,
                        float *delta, void *stream)
{
    return run_backward(plan, batch, n, q, k, v, o, dout, lse, seqlens, dq, dk, dv, delta, stream);
}

bsl_status bsl_backward_noalloc(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                                const void *k, const void *v, const void *o, const void *dout,
                                const float *lse, const int32_t *seqlens, void *dq, void *dk,
                                void *dv, void *stream)
{
    if (!plan)
        return fail(BSL_E_INVALID, "plan is NULL");
    if (batch > 0 && n > 0) {
        const long long rows = (long long)batch * plan->desc.heads * (long long)n;
        if (rows > (long long)bsl::SCRATCH_FLOATS)
            return fail(BSL_E_UNSUPPORTED,
                        "batch * heads * n = %lld rows; the fixed workspace of "
                        "bsl_backward_noalloc holds %zu rows (%zu MiB): use bsl_backward",
                        rows, bsl::SCRATCH_FLOATS, bsl::SCRATCH_FLOATS * 4 >> 20);
    }
    float *const ws = bsl::scratch_on(plan->device);
    if (!ws)
        return fail(BSL_E_DEVICE, "the fixed device workspace of device %d was not found",
                    plan->device);
    return run_backward(plan, batch, n, q, k, v, o, dout, lse, seqlens, dq, dk, dv, ws, stream);
}

bsl_status bsl_backward_varlen(const bsl_plan *plan, int32_t batch, int32_t tokens,
                               int32_t max_seqlen, const void *q, const void *k, const void *v,
                               const void *o, const void *dout, const float *lse,
                               const int32_t *cu_seqlens, void *dq, void *dk, void *dv,
                               float *delta, void *stream)
{
    return run_backward_varlen(plan, batch, tokens, max_seqlen, q, k, v, o, dout, lse, cu_seqlens,
                               dq, dk, dv, delta, stream);
}

bsl_status bsl_forward_varlen(const bsl_plan *plan, int32_t batch, int32_t tokens,
                              int32_t max_seqlen, const void *q, const void *k, const void *v,
                              void *o, const int32_t *cu_seqlens, float *lse, void *stream)
{
    return run_varlen(plan, batch, tokens, max_seqlen, q, k, v, o, cu_seqlens, lse, stream);
}

bsl_status bsl_varlen_offsets(int32_t batch, const int32_t *lengths, int32_t *cu_seqlens,
                              int32_t *max_seqlen, int32_t *ceiling)
{
    if (batch < 0)
        return fail(BSL_E_INVALID, "batch must be >= 0 (got %d)", batch);
    if (!cu_seqlens || !max_seqlen || !ceiling || (batch > 0 && !lengths))
        return fail(BSL_E_INVALID, "lengths, cu_seqlens, max_seqlen and ceiling must be non-NULL");
    long long sum = 0;
    int32_t mx = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (lengths[b] < 0)
            return fail(BSL_E_INVALID, "lengths[%d] = %d is negative", b, lengths[b]);
        sum += lengths[b];
        if (sum > 0x7fffffffLL)
            return fail(BSL_E_INVALID, "the lengths sum past 2^31 - 1");
        mx = lengths[b] > mx ? lengths[b] : mx;
    }
    const long long ceil32 = ((long long)mx + 31) / 32 * 32;
    if (ceil32 > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "the longest length rounds up past 2^31 - 1");
    cu_seqlens[0] = 0;
    for (int32_t b = 0; b < batch; ++b)
        cu_seqlens[b + 1] = cu_seqlens[b] + lengths[b];
    *max_seqlen = mx;
    *ceiling = (int32_t)ceil32;
    return BSL_OK;
}

bsl_status bsl_destroy(bsl_plan *plan)
{
    delete plan;
    return BSL_OK;
}

const char *bsl_status_string(bsl_status s)
{
    switch (s) {
    case BSL_OK: return "BSL_OK";
    case BSL_E_INVALID: return "BSL_E_INVALID: invalid argument";
    case BSL_E_UNSUPPORTED: return "BSL_E_UNSUPPORTED: not supported by this library or device";
    case BSL_E_DEVICE: return "BSL_E_DEVICE: HIP runtime error";
    case BSL_E_NOMEM: return "BSL_E_NOMEM: out of host memory";
    }
    return "unknown bsl_status";
}

const char *bsl_last_error(void) { return g_last_error; }

int32_t bsl_version(void) { return BSL_VERSION; }

} // extern "C"

extern "C" {

bsl_status bsl_kmer_tokenize(int32_t batch, const uint8_t *bases, int64_t nbytes,
                             const int64_t *starts, int32_t k, int32_t n_out, int32_t *ids,
                             int32_t *ntok, void *stream)
{
    if (batch < 0 || nbytes < 0 || n_out < 0)
        return fail(BSL_E_INVALID, "batch (%d), nbytes (%lld) and n_out (%d) must be >= 0", batch,
                    (long long)nbytes, n_out);
    if (k < 1 || k > 12)
        return fail(BSL_E_INVALID, "k must be in 1 .. 12 (got %d)", k);
    if (batch == 0)
        return BSL_OK;
    if (!starts || (n_out > 0 && !ids) || (nbytes > 0 && !bases))
        return fail(BSL_E_INVALID, "bases, starts and ids must be non-NULL device pointers");
    const long long tiles = bsl::kmer_tiles(n_out);
    if ((long long)batch * (tiles > 0 ? tiles : 1) > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "batch x tiles of the launch exceeds 2^31 - 1");
    const size_t id_bytes = (size_t)batch * (size_t)n_out * 4u;
    const size_t st_bytes = ((size_t)batch + 1u) * 8u;
    if (overlaps(ids, id_bytes, starts, st_bytes) ||
        (nbytes > 0 && overlaps(ids, id_bytes, bases, (size_t)nbytes)))
        return fail(BSL_E_INVALID, "ids overlaps bases or starts");
    if (ntok && (overlaps(ntok, (size_t)batch * 4u, starts, st_bytes) ||
                 (nbytes > 0 && overlaps(ntok, (size_t)batch * 4u, bases, (size_t)nbytes)) ||
                 overlaps(ntok, (size_t)batch * 4u, ids, id_bytes)))
        return fail(BSL_E_INVALID, "ntok overlaps bases, starts or ids");
    bsl::KmerLaunch a;
    a.bases = bases;
    a.nbytes = nbytes;
    a.starts = starts;
    a.ids = ids;
    a.ntok = ntok;
    a.batch = batch;
    a.k = k;
    a.n_out = n_out;
    a.stream = (hipStream_t)stream;
    if (n_out == 0) {
        if (!ntok)
            return BSL_OK;
        // only the counts: one workgroup per sequence, no windows
        a.n_out = 0;
    }
    const hipError_t e = bsl::launch_kmer(a);
    if (e != hipSuccess)
        return fail(BSL_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return BSL_OK;
}

bsl_status bsl_check_seqlens(int32_t batch, int32_t n, const int32_t *seqlens, int32_t *result,
                             void *stream)
{
    return check_common(batch, n, seqlens, result, stream, 0);
}

bsl_status bsl_check_cu_seqlens(int32_t batch, int32_t tokens, const int32_t *cu_seqlens,
                                int32_t *result, void *stream)
{
    return check_common(batch, tokens, cu_seqlens, result, stream, 1);
}

bsl_status bsl_kmer_ceiling(int32_t batch, const int64_t *starts, int32_t k, int32_t *n_out)
{
    if (batch < 0)
        return fail(BSL_E_INVALID, "batch must be >= 0 (got %d)", batch);
    if (k < 1 || k > 12)
        return fail(BSL_E_INVALID, "k must be in 1 .. 12 (got %d)", k);
    if (!starts || !n_out)
        return fail(BSL_E_INVALID, "starts and n_out must be non-NULL");
    if (starts[0] < 0)
        return fail(BSL_E_INVALID, "starts[0] = %lld is negative", (long long)starts[0]);
    long long mx = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (starts[b + 1] < starts[b])
            return fail(BSL_E_INVALID, "starts decreases at %d", b);
        const long long w = (long long)(starts[b + 1] - starts[b]) - k + 1;
        mx = w > mx ? w : mx;
    }
    const long long ceil32 = (mx + 31) / 32 * 32;
    if (ceil32 > 0x7fffffffLL)
        return fail(BSL_E_INVALID, "the longest window count rounds up past 2^31 - 1");
    *n_out = (int32_t)ceil32;
    return BSL_OK;
}

} // extern "C"
