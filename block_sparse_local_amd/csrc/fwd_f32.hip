// fwd_f32.hip -- banded block-sparse attention forward, fp32 in/out, gfx950.
//
// Same operation as fwd_bf16.hip (NucleoByte project page, section 3: the band
// |i - j| <= R over blocks of 32, S = Q K^T / sqrt(d_k), the running maximum /
// denominator / output across the active key blocks, O / l at the end), with
// every product and sum in fp32 on the vector ALUs: no reduced-precision matrix
// instruction touches the data.  It serves fp32 callers and small problems; the
// bf16 kernel is the fast path.
//
// One workgroup of 256 threads per (batch, head, query block).  Thread t owns
// query row t / 8 and the head dimensions e * 8 + t % 8 of it; the eight threads
// of a row reduce their partial dot products with three xor shuffles.  Each
// active K/V block is staged in LDS, and the row state (m, l, O slice) is updated
// once per block, as the page's recurrence is written.  With a token window W
// (section 2, item 3, read as |t - s| <= W) the band is the ceil(W/32) blocks on
// either side and the window joins the per-key mask.
#include "launch.h"

#include <math.h>

namespace bsl {
namespace {

constexpr int BLK = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Params {
    const float *q, *k, *v;
    float *o;
    const int32_t *seqlens; // padded layout: lengths (or nullptr)
    const int32_t *cu;      // packed layout: sequence start offsets, batch + 1 of them
    float *lse;
    int32_t *active;
    uint32_t *masks;
    // n: padded buffer length, or the longest sequence the grid covers (packed)
    int32_t heads, n, nblk, radius, total;
    int32_t tokens; // packed layout: rows in the buffer
    int32_t window; // 0: the block band; >= 1: keys within this many tokens
    float c;        // scale * log2(e)
};

// Padded layout [batch][heads][n][D]: rows D apart.  Packed layout
// [tokens][heads][D]: sequence b's rows of head h start at (cu[b] heads + h) D,
// heads D apart, lse [heads][tokens]; offsets are clamped into the buffer.
template <int D, bool CAUSAL, bool TRACE, bool VARLEN>
__global__ void __launch_bounds__(256) fwd_f32_kernel(Params p)
{
    static_assert(!(TRACE && VARLEN), "the trace describes the padded layout");
    constexpr int E = D / 8; // dims per thread
    const size_t RS = VARLEN ? (size_t)p.heads * D : (size_t)D;
    __shared__ float kl[BLK][D + 1];
    __shared__ float vl[BLK][D + 1];

    const int tid = threadIdx.x;
    const int r = tid >> 3, sub = tid & 7;
    const int g = (int)blockIdx.x;
    const int i = g % p.nblk;
    const int bh = g / p.nblk;
    const int b = bh / p.heads, h = bh % p.heads;
    int len;
    size_t base, lse_base;
    if (VARLEN) {
        int s0 = p.cu[b], s1 = p.cu[b + 1];
        s0 = s0 < 0 ? 0 : (s0 > p.tokens ? p.tokens : s0);
        s1 = s1 < s0 ? s0 : (s1 > p.tokens ? p.tokens : s1);
        len = s1 - s0 > p.n ? p.n : s1 - s0;
        base = ((size_t)s0 * (size_t)p.heads + (size_t)h) * D;
        lse_base = (size_t)h * (size_t)p.tokens + (size_t)s0;
    } else {
        len = p.seqlens ? p.seqlens[b] : p.n;
        len = len < 0 ? 0 : (len > p.n ? p.n : len);
        base = (size_t)bh * (size_t)p.n * D;
        lse_base = (size_t)bh * (size_t)p.n;
    }
    const int nb = (len + BLK - 1) / BLK;
    // packed layout: blocks past the sequence hold the next sequence's rows
    if (VARLEN && i >= nb)
        return;
    const int R = p.radius, W = 2 * R + 1;
    const int t = i * BLK + r;
    const bool tvalid = t < len;
    const bool trace_here = TRACE && h == 0;
    const size_t trace_row = ((size_t)b * p.nblk + (size_t)i) * (size_t)W;

    int lo = 1, hi = 0;
    if (i < nb) {
        lo = i - R < 0 ? 0 : i - R;
        hi = i + R > nb - 1 ? nb - 1 : i + R;
        if (CAUSAL && hi > i)
            hi = i;
    }

    float qv[E], ov[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = tvalid ? p.q[base + (size_t)t * RS + e * 8 + sub] : 0.0f;
        ov[e] = 0.0f;
    }
    // running maximum: finite, so that a block whose keys all lie outside the
    // row's token window leaves alpha = exp2(0) and weights exp2(-inf) = 0
    // instead of NaN; the first real score gives alpha = exp2(-1e30 - m) = 0
    float m = -1.0e30f, l = 0.0f;

    for (int j = lo; j <= hi; ++j) {
        __syncthreads();
        for (int x = tid; x < BLK * D; x += 256) {
            const int kr = x / D, kc = x % D;
            const int s = j * BLK + kr;
            // packed layout: rows past the end repeat the last row (masked)
            const int sr = VARLEN ? min(s, len - 1) : s;
            kl[kr][kc] = p.k[base + (size_t)sr * RS + kc];
            const float vv = p.v[base + (size_t)sr * RS + kc];
            vl[kr][kc] = s < len ? vv : 0.0f; // padded keys: zero V, never NaN
        }
        __syncthreads();

        float sc[BLK];
        float bmax = -INFINITY;
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < BLK; ++c) {
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                part = fmaf(qv[e], kl[c][e * 8 + sub], part);
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
            part += __shfl_xor(part, 4);
            const int s = j * BLK + c;
            const int dist = t > s ? t - s : s - t;
            const bool keep = s < len && (!CAUSAL || s <= t) && (p.window <= 0 || dist <= p.window);
            sc[c] = keep ? part * p.c : -INFINITY;
            word |= (keep ? 1u : 0u) << c;
            bmax = fmaxf(bmax, sc[c]);
        }
        if (trace_here) {
            const size_t slot = trace_row + (size_t)(j - lo);
            if (sub == 0)
                p.masks[slot * BLK + r] = tvalid ? word : 0u;
            if (tid == 0)
                p.active[slot] = j;
        }
        const float mn = fmaxf(m, bmax);
        const float alpha = __builtin_amdgcn_exp2f(m - mn); // 0 at the first kept key
        float add = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            ov[e] *= alpha;
#pragma unroll
        for (int c = 0; c < BLK; ++c) {
            const float w = __builtin_amdgcn_exp2f(sc[c] - mn);
            add += w;
#pragma unroll
            for (int e = 0; e < E; ++e)
                ov[e] = fmaf(w, vl[c][e * 8 + sub], ov[e]);
        }
        l = l * alpha + add;
        m = mn;
    }

    if (VARLEN && !tvalid)
        return; // the next sequence's row
    const float inv = tvalid ? 1.0f / l : 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        p.o[base + (size_t)t * RS + e * 8 + sub] = tvalid ? ov[e] * inv : 0.0f;
    if (p.lse && sub == 0)
        p.lse[lse_base + (size_t)t] =
            tvalid ? (m + __builtin_amdgcn_logf(l)) * LN2 : -INFINITY;
    if (trace_here) {
        const int used = hi >= lo ? hi - lo + 1 : 0;
        for (int s = used + tid; s < W; s += 256)
            p.active[trace_row + s] = -1;
        for (int s = used; s < W; ++s)
            if (sub == 0)
                p.masks[(trace_row + s) * BLK + r] = 0u;
    }
}

template <int D, bool CAUSAL, bool TRACE, bool VARLEN>
hipError_t launch_t(const Launch &a, const Params &p)
{
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, TRACE, VARLEN>), dim3(p.total), dim3(256), 0,
                       a.stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Launch &a, const Params &p)
{
    if (a.cu_seqlens)
        return a.causal ? launch_t<D, true, false, true>(a, p) : launch_t<D, false, false, true>(a, p);
    const bool tr = a.active != nullptr;
    if (a.causal)
        return tr ? launch_t<D, true, true, false>(a, p) : launch_t<D, true, false, false>(a, p);
    return tr ? launch_t<D, false, true, false>(a, p) : launch_t<D, false, false, false>(a, p);
}

} // namespace

hipError_t launch_fwd_f32(const Launch &a)
{
    Params p;
    p.q = (const float *)a.q;
    p.k = (const float *)a.k;
    p.v = (const float *)a.v;
    p.o = (float *)a.o;
    p.seqlens = a.seqlens;
    p.cu = a.cu_seqlens;
    p.lse = a.lse;
    p.active = a.active;
    p.masks = a.masks;
    p.heads = a.heads;
    p.n = a.n;
    p.tokens = a.tokens;
    p.nblk = (a.n + BLK - 1) / BLK;
    p.radius = a.radius;
    p.window = a.window;
    p.total = a.batch * a.heads * p.nblk;
    p.c = a.scale * LOG2E;
    switch (a.head_dim) {
    case 32: return launch_d<32>(a, p);
    case 64: return launch_d<64>(a, p);
    case 128: return launch_d<128>(a, p);
    default: return hipErrorInvalidValue;
    }
}

} // namespace bsl
