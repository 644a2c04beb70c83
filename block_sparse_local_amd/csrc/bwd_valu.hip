// bwd_valu.hip -- backward pass of the banded block-sparse attention on the
// vector ALUs, gfx950.
//
// The gradients bwd_bf16.hip computes (NucleoByte project page, section 3,
// "Custom Backpropagation": D_t = sum_c dO_tc O_tc, dS_ts = P_ts (dO_t . V_s -
// D_t), then dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q), with every
// product and sum in fp32 on the vector ALUs, as fwd_f32.hip does for the
// forward: the path for fp32 plans at every head size and for bf16 plans at
// head_dim 32 (inputs widened to fp32, gradients rounded once to bf16), not
// the fast one.  P is
// recomputed from the scores and the forward's lse; the band, padding, causal
// and token-window rules are the forward's.
//
// Two kernels of 256 threads, each thread owning one row of a 32-row block and
// the head dimensions e * 8 + t % 8 of it (eight threads per row reduce their
// partial dot products with three xor shuffles):
//  * dq: one workgroup per (batch, head, query block): D of its rows (written
//    for dkv), then over the key blocks of its band (K and V staged in LDS)
//    dQ += scale dS K;
//  * dkv: one workgroup per (batch, head, key block): over the query blocks
//    whose band holds it (Q, dO, lse and D staged in LDS) dV += P^T dO and
//    dK += scale dS^T Q.
// Rows past a sequence's end are zero in LDS, so NaN padding cannot meet a
// zero probability.
#include "bwd_launch.h"

#include <math.h>

namespace bsl {
namespace {

constexpr int BLK = 32;
constexpr float LOG2E = 1.4426950408889634f;

// Elements are float or bf16 bits (uint16_t); arithmetic is fp32 either way.
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x)
{
    return __builtin_bit_cast(float, (uint32_t)x << 16);
}
__device__ __forceinline__ void put(float *p, float x) { *p = x; }
__device__ __forceinline__ void put(uint16_t *p, float x)
{
    *p = __builtin_bit_cast(uint16_t, (__bf16)x); // round to nearest even
}

template <typename T>
struct FParams {
    const T *q, *k, *v, *o, *dout;
    const float *lse;
    const int32_t *seqlens; // padded layout: lengths (or nullptr)
    const int32_t *cu;      // packed layout: sequence start offsets, batch + 1 of them
    T *dq, *dk, *dv;
    float *delta;
    int32_t heads, n, nblk, radius, total, tokens, window;
    float c;     // scale * log2(e)
    float scale;
};

// Where sequence b's rows of head h live (see the bf16 kernels): padded
// [batch][heads][n][D] with lse / delta [batch][heads][n]; packed
// [tokens][heads][D] with lse / delta [heads][tokens], offsets clamped.
template <int D, bool VARLEN>
struct FSeq {
    size_t base, lbase, rs;
    int len;
    template <typename T>
    __device__ __forceinline__ FSeq(const FParams<T> &p, int b, int h)
    {
        if (VARLEN) {
            int s0 = p.cu[b], s1 = p.cu[b + 1];
            s0 = s0 < 0 ? 0 : (s0 > p.tokens ? p.tokens : s0);
            s1 = s1 < s0 ? s0 : (s1 > p.tokens ? p.tokens : s1);
            len = s1 - s0 > p.n ? p.n : s1 - s0;
            base = ((size_t)s0 * (size_t)p.heads + (size_t)h) * D;
            lbase = (size_t)h * (size_t)p.tokens + (size_t)s0;
            rs = (size_t)p.heads * D;
        } else {
            len = p.seqlens ? p.seqlens[b] : p.n;
            len = len < 0 ? 0 : (len > p.n ? p.n : len);
            base = ((size_t)b * p.heads + h) * (size_t)p.n * D;
            lbase = ((size_t)b * p.heads + h) * (size_t)p.n;
            rs = D;
        }
    }
};

__device__ __forceinline__ float row_sum8(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x;
}

__device__ __forceinline__ bool kept(int t, int s, int len, bool causal, int window)
{
    const int dist = t > s ? t - s : s - t;
    return t < len && s < len && (!causal || s <= t) && (window <= 0 || dist <= window);
}

// ------------------------------------------------------------------- dq
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) dq_valu_kernel(FParams<T> p)
{
    constexpr int E = D / 8;
    __shared__ float kl[BLK][D + 1];
    __shared__ float vl[BLK][D + 1];

    const int tid = threadIdx.x, r = tid >> 3, sub = tid & 7;
    const int g = (int)blockIdx.x;
    const int i = g % p.nblk, bh = g / p.nblk, b = bh / p.heads, h = bh % p.heads;
    const FSeq<D, VARLEN> sq(p, b, h);
    const int len = sq.len, nb = (len + BLK - 1) / BLK, R = p.radius;
    if (VARLEN && i >= nb)
        return; // the next sequence's rows
    const int t = i * BLK + r;
    const bool tvalid = t < len;
    const size_t row = sq.base + (size_t)t * sq.rs;

    float qv[E], gv[E], acc[E];
    float dpart = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = tvalid ? widen(p.q[row + e * 8 + sub]) : 0.0f;
        gv[e] = tvalid ? widen(p.dout[row + e * 8 + sub]) : 0.0f;
        const float ov = tvalid ? widen(p.o[row + e * 8 + sub]) : 0.0f;
        dpart = fmaf(gv[e], ov, dpart);
        acc[e] = 0.0f;
    }
    const float Dt = row_sum8(dpart);
    if (sub == 0 && (tvalid || !VARLEN))
        p.delta[sq.lbase + t] = Dt;
    const float lse2 = tvalid ? p.lse[sq.lbase + t] * LOG2E : 0.0f;

    int lo = 1, hi = 0;
    if (i < nb) {
        lo = i - R < 0 ? 0 : i - R;
        hi = i + R > nb - 1 ? nb - 1 : i + R;
        if (CAUSAL && hi > i)
            hi = i;
    }
    for (int j = lo; j <= hi; ++j) {
        __syncthreads();
        for (int x = tid; x < BLK * D; x += 256) {
            const int kr = x / D, kc = x % D;
            const int s = j * BLK + kr;
            const bool ok = s < len;
            const size_t src = sq.base + (size_t)(ok ? s : 0) * sq.rs + kc;
            kl[kr][kc] = ok ? widen(p.k[src]) : 0.0f;
            vl[kr][kc] = ok ? widen(p.v[src]) : 0.0f;
        }
        __syncthreads();
        for (int c = 0; c < BLK; ++c) {
            float sp = 0.0f, dpp = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sp = fmaf(qv[e], kl[c][e * 8 + sub], sp);
                dpp = fmaf(gv[e], vl[c][e * 8 + sub], dpp);
            }
            const float s_tc = row_sum8(sp), dp = row_sum8(dpp);
            const int s = j * BLK + c;
            const float pr = kept(t, s, len, CAUSAL, p.window)
                                 ? __builtin_amdgcn_exp2f(fmaf(s_tc, p.c, -lse2))
                                 : 0.0f;
            const float ds = pr * (dp - Dt);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] = fmaf(ds, kl[c][e * 8 + sub], acc[e]);
        }
    }
    if (VARLEN && !tvalid)
        return;
#pragma unroll
    for (int e = 0; e < E; ++e)
        put(&p.dq[row + e * 8 + sub], tvalid ? acc[e] * p.scale : 0.0f);
}

// ------------------------------------------------------------------ dkv
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) dkv_valu_kernel(FParams<T> p)
{
    constexpr int E = D / 8;
    __shared__ float ql[BLK][D + 1];
    __shared__ float gl[BLK][D + 1];
    __shared__ float ll[BLK], dl[BLK];

    const int tid = threadIdx.x, r = tid >> 3, sub = tid & 7;
    const int g = (int)blockIdx.x;
    const int j = g % p.nblk, bh = g / p.nblk, b = bh / p.heads, h = bh % p.heads;
    const FSeq<D, VARLEN> sq(p, b, h);
    const int len = sq.len, nb = (len + BLK - 1) / BLK, R = p.radius;
    if (VARLEN && j >= nb)
        return;
    const int s = j * BLK + r;
    const bool svalid = s < len;
    const size_t row = sq.base + (size_t)s * sq.rs;

    float kv[E], vv[E], dk[E], dv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kv[e] = svalid ? widen(p.k[row + e * 8 + sub]) : 0.0f;
        vv[e] = svalid ? widen(p.v[row + e * 8 + sub]) : 0.0f;
        dk[e] = 0.0f;
        dv[e] = 0.0f;
    }
    // query blocks whose band holds key block j (causal: those at or after it)
    int lo = 1, hi = 0;
    if (j < nb) {
        lo = j - R < 0 ? 0 : j - R;
        hi = j + R > nb - 1 ? nb - 1 : j + R;
        if (CAUSAL && lo < j)
            lo = j;
    }
    for (int i = lo; i <= hi; ++i) {
        __syncthreads();
        for (int x = tid; x < BLK * D; x += 256) {
            const int qr = x / D, qc = x % D;
            const int t = i * BLK + qr;
            const bool ok = t < len;
            const size_t src = sq.base + (size_t)(ok ? t : 0) * sq.rs + qc;
            ql[qr][qc] = ok ? widen(p.q[src]) : 0.0f;
            gl[qr][qc] = ok ? widen(p.dout[src]) : 0.0f;
        }
        if (tid < BLK) {
            const int t = i * BLK + tid;
            const bool ok = t < len;
            ll[tid] = ok ? p.lse[sq.lbase + t] * LOG2E : 0.0f;
            dl[tid] = ok ? p.delta[sq.lbase + t] : 0.0f;
        }
        __syncthreads();
        for (int c = 0; c < BLK; ++c) {
            float sp = 0.0f, dpp = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sp = fmaf(ql[c][e * 8 + sub], kv[e], sp);
                dpp = fmaf(gl[c][e * 8 + sub], vv[e], dpp);
            }
            const float s_cs = row_sum8(sp), dp = row_sum8(dpp);
            const int t = i * BLK + c;
            const float pr = kept(t, s, len, CAUSAL, p.window)
                                 ? __builtin_amdgcn_exp2f(fmaf(s_cs, p.c, -ll[c]))
                                 : 0.0f;
            const float ds = pr * (dp - dl[c]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dv[e] = fmaf(pr, gl[c][e * 8 + sub], dv[e]);
                dk[e] = fmaf(ds, ql[c][e * 8 + sub], dk[e]);
            }
        }
    }
    if (VARLEN && !svalid)
        return;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        put(&p.dk[row + e * 8 + sub], svalid ? dk[e] * p.scale : 0.0f);
        put(&p.dv[row + e * 8 + sub], svalid ? dv[e] : 0.0f);
    }
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_v(const BwdLaunch &a, const FParams<T> &p)
{
    // dq also writes D, which dkv reads
    hipLaunchKernelGGL((dq_valu_kernel<T, D, CAUSAL, VARLEN>), dim3(p.total), dim3(256), 0,
                       a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((dkv_valu_kernel<T, D, CAUSAL, VARLEN>), dim3(p.total), dim3(256), 0,
                       a.stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const BwdLaunch &a, const FParams<T> &p)
{
    if (a.cu_seqlens)
        return a.causal ? launch_v<T, D, true, true>(a, p) : launch_v<T, D, false, true>(a, p);
    return a.causal ? launch_v<T, D, true, false>(a, p) : launch_v<T, D, false, false>(a, p);
}

template <typename T>
hipError_t launch_typed(const BwdLaunch &a)
{
    FParams<T> p;
    p.q = (const T *)a.q;
    p.k = (const T *)a.k;
    p.v = (const T *)a.v;
    p.o = (const T *)a.o;
    p.dout = (const T *)a.dout;
    p.lse = a.lse;
    p.seqlens = a.seqlens;
    p.cu = a.cu_seqlens;
    p.dq = (T *)a.dq;
    p.dk = (T *)a.dk;
    p.dv = (T *)a.dv;
    p.delta = a.delta;
    p.heads = a.heads;
    p.n = a.n;
    p.tokens = a.tokens;
    p.nblk = (a.n + BLK - 1) / BLK;
    p.radius = a.radius;
    p.window = a.window;
    p.total = a.batch * a.heads * p.nblk;
    p.c = a.scale * LOG2E;
    p.scale = a.scale;
    switch (a.head_dim) {
    case 32: return launch_d<T, 32>(a, p);
    case 64: return launch_d<T, 64>(a, p);
    case 128: return launch_d<T, 128>(a, p);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_bwd_valu(const BwdLaunch &a, bool bf16)
{
    return bf16 ? launch_typed<uint16_t>(a) : launch_typed<float>(a);
}

} // namespace bsl
