// abi_host_test.cpp -- drives the C ABI of include/bsl.h on the host, against
// the fake device of fake_device.cpp, to check that every argument error is
// caught before any launch (and that good calls reach the right launcher with
// the right description).  Built with the address and undefined-behaviour
// sanitizers by tests/test_host_sanitize.py; prints one line per check and
// exits non-zero on the first failure.
//
// TEST INFRASTRUCTURE.  The "device" buffers are carved from one host arena:
// the ABI layer only compares and offsets pointers, it never dereferences them.
#include "bsl.h"
#include "fake_device.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

int g_checks = 0;

#define EXPECT(cond)                                                                              \
    do {                                                                                          \
        ++g_checks;                                                                               \
        if (!(cond)) {                                                                            \
            std::fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__,      \
                         #cond, bsl_last_error());                                                \
            std::exit(1);                                                                         \
        }                                                                                         \
    } while (0)

// A rejected call returns BSL_E_INVALID and launches nothing.
#define EXPECT_REJECTED(call)                                                                     \
    do {                                                                                          \
        const int before = fake::state().launches();                                             \
        const bsl_status st_ = (call);                                                            \
        EXPECT(st_ == BSL_E_INVALID);                                                             \
        EXPECT(fake::state().launches() == before);                                               \
        EXPECT(std::strlen(bsl_last_error()) > 0);                                                \
    } while (0)

struct Arena {
    unsigned char *base;
    size_t used = 0, size;
    explicit Arena(size_t n) : size(n) { base = (unsigned char *)std::aligned_alloc(256, n); }
    ~Arena() { std::free(base); }
    // a fresh, 256-byte aligned, disjoint piece
    template <class T>
    T *take(size_t bytes)
    {
        used = (used + 255) / 256 * 256;
        EXPECT(used + bytes <= size);
        T *p = (T *)(base + used);
        used += bytes;
        return p;
    }
};

bsl_plan *make_plan(int head_dim, int heads, int radius, int causal, int dtype, int window = 0)
{
    bsl_desc d{};
    d.head_dim = head_dim;
    d.heads = heads;
    d.block_size = 32;
    d.radius = radius;
    d.causal = causal;
    d.dtype = dtype;
    d.window = window;
    bsl_plan *p = nullptr;
    EXPECT(bsl_create(&d, &p) == BSL_OK && p != nullptr);
    return p;
}

void test_create()
{
    bsl_desc d{};
    d.head_dim = 64;
    d.heads = 1;
    d.block_size = 32;
    d.radius = 1;
    bsl_plan *p = nullptr;
    fake::state().arch = "gfx942:sramecc+:xnack-";
    EXPECT(bsl_create(&d, &p) == BSL_E_UNSUPPORTED && p == nullptr);
    fake::state().arch = "gfx950:sramecc+:xnack-";
    d.head_dim = 96;
    EXPECT(bsl_create(&d, &p) == BSL_E_UNSUPPORTED && p == nullptr);
    d.head_dim = 64;
    d.window = -3;
    EXPECT(bsl_create(&d, &p) == BSL_E_INVALID && p == nullptr);
    d.window = 0;
    EXPECT(bsl_create(&d, &p) == BSL_OK && p != nullptr);
    EXPECT(bsl_destroy(p) == BSL_OK);
    EXPECT(bsl_destroy(nullptr) == BSL_OK);
    std::printf("create: device and descriptor checks\n");
}

void test_forward()
{
    const int batch = 2, heads = 2, n = 128, dd = 64, R = 1;
    bsl_plan *p = make_plan(dd, heads, R, 0, BSL_BF16);
    const size_t tb = (size_t)batch * heads * n * dd * 2, rb = (size_t)batch * heads * n * 4;
    const size_t slots = (size_t)batch * (n / 32) * (2 * R + 1);
    Arena ar(16 * tb);
    void *q = ar.take<void>(tb), *k = ar.take<void>(tb), *v = ar.take<void>(tb);
    void *o = ar.take<void>(tb);
    float *lse = ar.take<float>(rb);
    int32_t *sl = ar.take<int32_t>(batch * 4);
    int32_t *act = ar.take<int32_t>(slots * 4);
    uint32_t *msk = ar.take<uint32_t>(slots * 128);

    const int before = fake::state().fwd_bf16;
    EXPECT(bsl_forward(p, batch, n, q, k, v, o, sl, lse, nullptr) == BSL_OK);
    EXPECT(fake::state().fwd_bf16 == before + 1);
    const bsl::Launch &a = fake::state().last_fwd;
    EXPECT(a.q == q && a.k == k && a.v == v && a.o == o && a.lse == lse && a.seqlens == sl);
    EXPECT(a.batch == batch && a.heads == heads && a.n == n && a.head_dim == dd);
    EXPECT(a.radius == R && a.window == 0 && !a.causal && a.active == nullptr);
    EXPECT(a.scale > 0.124f && a.scale < 0.126f); // 1 / sqrt(64)
    EXPECT(bsl_forward(p, batch, n, q, k, v, o, nullptr, nullptr, nullptr) == BSL_OK);
    // no-ops
    const int n0 = fake::state().launches();
    EXPECT(bsl_forward(p, 0, n, q, k, v, o, sl, lse, nullptr) == BSL_OK);
    EXPECT(bsl_forward(p, batch, 0, q, k, v, o, sl, lse, nullptr) == BSL_OK);
    EXPECT(fake::state().launches() == n0);

    EXPECT_REJECTED(bsl_forward(nullptr, batch, n, q, k, v, o, sl, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, -1, n, q, k, v, o, sl, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, 40, q, k, v, o, sl, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, nullptr, k, v, o, sl, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, (char *)q + 2, k, v, o, sl, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, (char *)o + 8, sl, lse, nullptr));
    // o overlapping an input
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, (char *)v + tb / 2, sl, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, q, sl, lse, nullptr));
    // lse: misaligned, overlapping an input, overlapping o
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, o, sl, lse + 1, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, o, sl, (float *)k, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, o, sl, (float *)((char *)o + tb - 16),
                                nullptr));
    // seqlens inside a buffer the call writes
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, o, (int32_t *)o, lse, nullptr));
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, o, (int32_t *)lse, lse, nullptr));
    // the plan belongs to device 0
    fake::state().current_device = 1;
    EXPECT_REJECTED(bsl_forward(p, batch, n, q, k, v, o, sl, lse, nullptr));
    fake::state().current_device = 0;
    // a failing launch is a device error
    fake::state().launch_result = hipErrorInvalidValue;
    EXPECT(bsl_forward(p, batch, n, q, k, v, o, sl, lse, nullptr) == BSL_E_DEVICE);
    EXPECT(std::strstr(bsl_last_error(), "fake launch failure") != nullptr);
    fake::state().launch_result = hipSuccess;

    // traced
    EXPECT(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, act, msk, nullptr) == BSL_OK);
    EXPECT(fake::state().last_fwd.active == act && fake::state().last_fwd.masks == msk);
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, nullptr, msk, nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, act, nullptr, nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse,
                                       (int32_t *)((char *)act + 2), msk, nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, act,
                                       (uint32_t *)((char *)msk + 1), nullptr));
    // trace buffers overlapping each other, o, lse, an input or the lengths
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, act,
                                       (uint32_t *)(act + 4), nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, (int32_t *)o, msk,
                                       nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, act, (uint32_t *)lse,
                                       nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, act, (uint32_t *)q,
                                       nullptr));
    EXPECT_REJECTED(bsl_forward_traced(p, batch, n, q, k, v, o, sl, lse, sl, msk, nullptr));
    bsl_destroy(p);

    // fp32 plans go to the vector-ALU kernel; a token window sets the band
    p = make_plan(32, 1, 0, 1, BSL_F32, 40);
    EXPECT(bsl_forward(p, 1, 64, q, k, v, o, nullptr, nullptr, nullptr) == BSL_OK);
    EXPECT(fake::state().fwd_f32 == 1 && fake::state().last_fwd.radius == 2 &&
           fake::state().last_fwd.window == 40 && fake::state().last_fwd.causal);
    bsl_destroy(p);
    std::printf("forward: alignment, overlap, trace buffers, device, launch failure\n");
}

void test_forward_varlen()
{
    const int heads = 2, dd = 128, tokens = 300, batch = 3;
    bsl_plan *p = make_plan(dd, heads, 2, 0, BSL_BF16);
    const size_t tb = (size_t)tokens * heads * dd * 2, rb = (size_t)heads * tokens * 4;
    Arena ar(8 * tb);
    void *q = ar.take<void>(tb), *k = ar.take<void>(tb), *v = ar.take<void>(tb);
    void *o = ar.take<void>(tb);
    float *lse = ar.take<float>(rb);
    int32_t *cu = ar.take<int32_t>((batch + 1) * 4);
    EXPECT(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, cu, lse, nullptr) == BSL_OK);
    const bsl::Launch &a = fake::state().last_fwd;
    EXPECT(a.cu_seqlens == cu && a.tokens == tokens && a.n == 200 && a.seqlens == nullptr);
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, nullptr, lse, nullptr));
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, -1, q, k, v, o, cu, lse, nullptr));
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, cu, lse + 2, nullptr));
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, cu, (float *)v, nullptr));
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, cu, (float *)o, nullptr));
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, (int32_t *)lse, lse,
                                       nullptr));
    EXPECT_REJECTED(bsl_forward_varlen(p, batch, tokens, 200, q, k, v, o, (int32_t *)o, nullptr,
                                       nullptr));
    const int n0 = fake::state().launches();
    EXPECT(bsl_forward_varlen(p, batch, 0, 200, q, k, v, o, cu, lse, nullptr) == BSL_OK);
    EXPECT(fake::state().launches() == n0);
    bsl_destroy(p);
    std::printf("forward_varlen: offsets, lse alignment and overlap\n");
}

void test_backward()
{
    const int batch = 1, heads = 2, n = 96, dd = 64;
    bsl_plan *p = make_plan(dd, heads, 1, 0, BSL_BF16);
    const size_t tb = (size_t)batch * heads * n * dd * 2, rb = (size_t)batch * heads * n * 4;
    Arena ar(16 * tb);
    void *q = ar.take<void>(tb), *k = ar.take<void>(tb), *v = ar.take<void>(tb);
    void *o = ar.take<void>(tb), *g = ar.take<void>(tb);
    void *dq = ar.take<void>(tb), *dk = ar.take<void>(tb), *dv = ar.take<void>(tb);
    float *lse = ar.take<float>(rb), *delta = ar.take<float>(rb);
    int32_t *sl = ar.take<int32_t>(batch * 4);
    EXPECT(bsl_backward(p, batch, n, q, k, v, o, g, lse, sl, dq, dk, dv, delta, nullptr) ==
           BSL_OK);
    EXPECT(fake::state().bwd_bf16 == 1 && fake::state().last_bwd.delta == delta);
    EXPECT_REJECTED(bsl_backward(p, batch, n, q, k, v, o, g, lse, sl, dq, dk, dv, lse, nullptr));
    EXPECT_REJECTED(bsl_backward(p, batch, n, q, k, v, o, g, lse, sl, dq, dq, dv, delta, nullptr));
    EXPECT_REJECTED(bsl_backward(p, batch, n, q, k, v, o, g, lse, sl, (char *)dq + 4, dk, dv, delta,
                                 nullptr));
    EXPECT_REJECTED(bsl_backward(p, batch, n, q, k, v, o, g, lse, (int32_t *)dk, dq, dk, dv, delta,
                                 nullptr));
    EXPECT_REJECTED(bsl_backward(p, batch, n, q, k, v, o, g, nullptr, sl, dq, dk, dv, delta,
                                 nullptr));
    bsl_destroy(p);
    // bf16 at head_dim 32 takes the vector-ALU backward with bf16 rounding
    p = make_plan(32, 1, 1, 0, BSL_BF16);
    EXPECT(bsl_backward(p, 1, 64, q, k, v, o, g, lse, nullptr, dq, dk, dv, delta, nullptr) ==
           BSL_OK);
    EXPECT(fake::state().bwd_valu == 1 && fake::state().last_bwd_valu_bf16);
    bsl_destroy(p);

    // no-alloc variant: the library's fixed workspace stands in for delta
    const int lookups = fake::state().scratch_lookups;
    bsl_plan *p2 = make_plan(64, heads, 1, 0, BSL_BF16);
    EXPECT(fake::state().scratch_lookups == lookups); // once per device, not per plan
    const int nb0 = fake::state().bwd_bf16;
    EXPECT(bsl_backward_noalloc(p2, batch, n, q, k, v, o, g, lse, sl, dq, dk, dv, nullptr) ==
           BSL_OK);
    EXPECT(fake::state().bwd_bf16 == nb0 + 1 &&
           fake::state().last_bwd.delta == fake::state().scratch);
    EXPECT_REJECTED(bsl_backward_noalloc(p2, batch, n, q, k, v, o, g, lse, sl, dq, dq, dv,
                                         nullptr));
    EXPECT_REJECTED(bsl_backward_noalloc(nullptr, batch, n, q, k, v, o, g, lse, sl, dq, dk, dv,
                                         nullptr));
    {
        // 8 Mi rows is the limit: 2 x 2 x 2^21 rows fits, one more block does not
        const int before = fake::state().launches();
        EXPECT(bsl_backward_noalloc(p2, 2, 2 << 20, q, k, v, o, g, lse, nullptr, dq, dk, dv,
                                    nullptr) != BSL_E_UNSUPPORTED);
        EXPECT(bsl_backward_noalloc(p2, 2, (2 << 20) + 32, q, k, v, o, g, lse, nullptr, dq, dk,
                                    dv, nullptr) == BSL_E_UNSUPPORTED);
        EXPECT(std::strstr(bsl_last_error(), "fixed workspace") != nullptr);
        EXPECT(fake::state().launches() <= before + 1);
    }
    bsl_destroy(p2);

    // packed layout
    const int tokens = 90;
    p = make_plan(128, 1, 1, 1, BSL_BF16);
    int32_t *cu = ar.take<int32_t>(3 * 4);
    EXPECT(bsl_backward_varlen(p, 2, tokens, 60, q, k, v, o, g, lse, cu, dq, dk, dv, delta,
                               nullptr) == BSL_OK);
    EXPECT(fake::state().last_bwd.cu_seqlens == cu && fake::state().last_bwd.tokens == tokens);
    EXPECT_REJECTED(bsl_backward_varlen(p, 2, tokens, 60, q, k, v, o, g, lse, (int32_t *)delta,
                                        dq, dk, dv, delta, nullptr));
    EXPECT_REJECTED(bsl_backward_varlen(p, 2, tokens, 60, q, k, v, o, g, lse, nullptr, dq, dk, dv,
                                        delta, nullptr));
    bsl_destroy(p);
    std::printf("backward: dispatch, alignment, overlap with inputs and lengths\n");
}

void test_host_helpers()
{
    int32_t lens[4] = {5, 0, 70, 32}, cu[5], mx = -1, ceil = -1;
    EXPECT(bsl_varlen_offsets(4, lens, cu, &mx, &ceil) == BSL_OK);
    EXPECT(cu[0] == 0 && cu[4] == 107 && mx == 70 && ceil == 96);
    lens[1] = -2;
    cu[0] = -7;
    EXPECT(bsl_varlen_offsets(4, lens, cu, &mx, &ceil) == BSL_E_INVALID && cu[0] == -7);
    int64_t starts[3] = {0, 100, 2100};
    int32_t n_out = -1;
    EXPECT(bsl_kmer_ceiling(2, starts, 6, &n_out) == BSL_OK && n_out == 2016);
    starts[1] = 3000;
    EXPECT(bsl_kmer_ceiling(2, starts, 6, &n_out) == BSL_E_INVALID);
    Arena ar(1 << 16);
    uint8_t *bases = ar.take<uint8_t>(1000);
    int64_t *st = ar.take<int64_t>(3 * 8);
    int32_t *ids = ar.take<int32_t>(2 * 64 * 4), *nt = ar.take<int32_t>(2 * 4);
    EXPECT(bsl_kmer_tokenize(2, bases, 1000, st, 6, 64, ids, nt, nullptr) == BSL_OK);
    EXPECT(fake::state().kmer == 1 && fake::state().last_kmer.n_out == 64);
    EXPECT_REJECTED(bsl_kmer_tokenize(2, bases, 1000, st, 6, 64, (int32_t *)bases, nt, nullptr));
    EXPECT_REJECTED(bsl_kmer_tokenize(2, bases, 1000, st, 13, 64, ids, nt, nullptr));
    int32_t *res = ar.take<int32_t>(8);
    EXPECT(bsl_check_seqlens(2, 64, nt, res, nullptr) == BSL_OK && fake::state().check == 1);
    EXPECT_REJECTED(bsl_check_seqlens(2, 64, nt, nt, nullptr));
    EXPECT(std::strcmp(bsl_status_string(BSL_E_DEVICE), "BSL_E_DEVICE: HIP runtime error") == 0);
    EXPECT(bsl_version() == BSL_VERSION);
    std::printf("host helpers: collator, k-mer ceiling, tokenizer and validator arguments\n");
}

} // namespace

int main()
{
    static float workspace[64];
    fake::state().scratch = workspace;
    test_create();
    EXPECT(fake::state().scratch_lookups == 1); // looked up by the first bsl_create
    test_forward();
    test_forward_varlen();
    test_backward();
    test_host_helpers();
    std::printf("abi_host_test: %d checks passed\n", g_checks);
    return 0;
}
