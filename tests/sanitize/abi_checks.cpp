// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitizers.py).
// Every call here is rejected by argument validation before any HIP call,
// so no GPU is needed; fake device addresses are never dereferenced.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tessera_attn.h"
#include "tessera_attn_bwd.h"
#include "tessera_paged.h"
#include "tessera_rmsnorm.h"

static int failures = 0;

static void expect(const char *what, long long got, long long want) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
        ++failures;
    }
}

static void *addr(int i) { return (void *)((uintptr_t)i << 44); }

int main() {
    void *q = addr(1), *k = addr(2), *v = addr(3), *o = addr(4);
    float *l = (float *)addr(5);
    const float nan = NAN, inf = INFINITY;

    // forward, bf16 and fp32
    expect("fwd null", tessera_attn_fwd(nullptr, k, v, o, l, 1, 4, 2, 64, 64, 1, 0.125f, nullptr),
           TESSERA_ERR_NULL);
    expect("fwd shape", tessera_attn_fwd(q, k, v, o, l, 1, 3, 2, 64, 64, 1, 0.125f, nullptr),
           TESSERA_ERR_SHAPE);
    expect("fwd D", tessera_attn_fwd(q, k, v, o, l, 1, 4, 2, 64, 48, 1, 0.125f, nullptr),
           TESSERA_ERR_UNSUPPORTED);
    expect("fwd causal", tessera_attn_fwd(q, k, v, o, l, 1, 4, 2, 64, 64, 2, 0.125f, nullptr),
           TESSERA_ERR_CAUSAL);
    expect("fwd scale", tessera_attn_fwd(q, k, v, o, l, 1, 4, 2, 64, 64, 1, nan, nullptr),
           TESSERA_ERR_SCALE);
    expect("fwd align", tessera_attn_fwd((char *)q + 8, k, v, o, l, 1, 4, 2, 64, 64, 1, 0.125f,
                                         nullptr),
           TESSERA_ERR_ALIGN);
    expect("fwd alias", tessera_attn_fwd(q, k, v, q, l, 1, 4, 2, 64, 64, 1, 0.125f, nullptr),
           TESSERA_ERR_ALIAS);
    expect("fwd too large", tessera_attn_fwd(q, k, v, o, l, 1 << 16, 1 << 15, 1 << 15, 1, 64, 1,
                                             0.125f, nullptr),
           TESSERA_ERR_TOO_LARGE);
    expect("f32 inf", tessera_attn_fwd_f32((float *)q, (float *)k, (float *)v, (float *)o, l, 1, 4,
                                           2, 64, 32, 1, inf, nullptr),
           TESSERA_ERR_SCALE);
    expect("kv shape", tessera_attn_fwd_kv(q, k, v, o, l, 1, 4, 2, 65, 64, 64, 1, 0.125f, nullptr),
           TESSERA_ERR_SHAPE);

    // tile configurations
    tessera_attn_tile_config c = {4, 32, 1, 0};
    expect("config null", tessera_attn_fwd_with_config(q, k, v, o, l, 1, 4, 2, 64, 64, 64, 1,
                                                       0.125f, nullptr, nullptr),
           TESSERA_ERR_NULL);
    tessera_attn_tile_config bad[] = {{3, 32, 1, 0}, {4, 48, 1, 0}, {4, 32, 3, 0}, {4, 32, 1, 2},
                                      {4, 64, 2, 0}, {4, 32, 2, 1}};
    for (const tessera_attn_tile_config &b : bad)
        expect("config not allowed", tessera_attn_fwd_with_config(q, k, v, o, l, 1, 4, 1, 64, 64,
                                                                  64, 1, 0.125f, &b, nullptr),
               TESSERA_ERR_UNSUPPORTED);
    tessera_attn_tile_config d128 = {1, 64, 1, 0};
    expect("config rows at D=128", tessera_attn_fwd_with_config(q, k, v, o, l, 1, 4, 4, 64, 64,
                                                                128, 1, 0.125f, &d128, nullptr),
           TESSERA_ERR_UNSUPPORTED);
    expect("config query", tessera_attn_fwd_tile_config(1, 32, 8, 16384, 16384, 128, 1, &c),
           TESSERA_OK);
    expect("config pick in range", c.heads_per_workgroup >= 1 && c.heads_per_workgroup <= 4, 1);
    expect("config query D", tessera_attn_fwd_tile_config(1, 4, 2, 8, 8, 96, 1, &c),
           TESSERA_ERR_UNSUPPORTED);
    expect("config query null", tessera_attn_fwd_tile_config(1, 4, 2, 8, 8, 64, 1, nullptr),
           TESSERA_ERR_NULL);

    // backward
    void *dq = addr(10), *dk = addr(11), *dv = addr(12), *dout = addr(9);
    float *dl = (float *)addr(13);
    expect("bwd alias", tessera_attn_bwd(q, k, v, o, dout, l, q, dk, dv, dl, 1, 4, 2, 64, 64, 1,
                                         0.125f, nullptr),
           TESSERA_ERR_ALIAS);
    expect("bwd D", tessera_attn_bwd(q, k, v, o, dout, l, dq, dk, dv, dl, 1, 4, 2, 64, 80, 1,
                                     0.125f, nullptr),
           TESSERA_ERR_UNSUPPORTED);

    // RMSNorm
    expect("rmsnorm eps", tessera_rmsnorm_fwd(q, k, o, 4, 64, -1.f, nullptr), TESSERA_ERR_EPS);
    expect("rmsnorm n", tessera_rmsnorm_fwd(q, k, o, 4, 12, 1e-6f, nullptr),
           TESSERA_ERR_UNSUPPORTED);
    expect("rmsnorm large", tessera_rmsnorm_fwd(q, k, o, 1ll << 60, 64, 1e-6f, nullptr),
           TESSERA_ERR_TOO_LARGE);

    // paged decode, with and without a workspace
    const int *bt = (const int *)addr(16), *cl = (const int *)addr(17);
    void *ws = addr(18);
    expect("paged workspace", tessera_paged_decode(q, k, v, bt, cl, o, l, 2, 8, 2, 2, 64, 64, 16,
                                                   100, 1, 0.125f, nullptr, 0, nullptr),
           TESSERA_ERR_WORKSPACE);
    expect("paged alias", tessera_paged_decode(q, k, v, bt, cl, o, l, 2, 8, 2, 2, 64, 64, 16, 100,
                                               1, 0.125f, (void *)cl, 1 << 20, nullptr),
           TESSERA_ERR_ALIAS);
    expect("paged bs", tessera_paged_decode_noalloc(q, k, v, bt, cl, o, l, 2, 8, 2, 2, 64, 64, 8,
                                                    100, 1, 0.125f, nullptr),
           TESSERA_ERR_UNSUPPORTED);
    // 32 query rows per KV head in 8 x 256 slots: 34 MB of workspace > 32 MiB
    expect("paged scratch", tessera_paged_decode_noalloc(q, k, v, bt, cl, o, l, 64, 256, 8, 1, 128,
                                                         64, 16, 4096, 1, 0.125f, nullptr),
           TESSERA_ERR_SCRATCH);
    expect("paged sizes", tessera_paged_decode_workspace(64, 32, 8, 1, 128, 16, 1024) > 0, 1);
    expect("paged sizes bad", tessera_paged_decode_workspace(1, 8, 3, 1, 32, 16, 100),
           -TESSERA_ERR_SHAPE);
    expect("scratch limit", tessera_paged_decode_scratch_limit(), 32ll << 20);

    // status text
    for (int s = -2; s < 20; ++s)
        if (!tessera_attn_status_string(s) || !strlen(tessera_attn_status_string(s)))
            expect("status string", 0, 1);
    expect("no launch error", strlen(tessera_attn_last_error()), 0);

    if (failures) return 1;
    printf("abi checks: ok\n");
    return 0;
}
