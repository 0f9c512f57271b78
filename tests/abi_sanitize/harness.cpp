// Host-side drive of the C ABI's validation and planning under ASan/UBSan
// (built by tests/test_abi_sanitize.py).  Every call here either is host-only
// (capacity, scratch size, plan, workspace) or fails validation before any
// device work, so it runs without a GPU.  Exit status 0 and no sanitizer
// report means no out-of-bounds access and no undefined behaviour (signed
// overflow, bad shifts, misaligned loads) on these paths.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>

#include "moe.h"

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull) + off); }

static moe_forward_args base_args() {
    moe_forward_args a;
    std::memset(&a, 0, sizeof(a));
    a.T = 16; a.E = 128; a.H = 4096; a.I = 1536; a.topk = 8; a.wdtype = MOE_WDTYPE_BF16;
    a.x = a.w13 = a.w2 = a.out = fake();
    a.topk_ids = static_cast<const int32_t*>(fake());
    a.topk_weights = static_cast<const float*>(fake());
    return a;
}

static void check_plan(const moe_forward_args& a) {
    moe_plan_info p;
    const int st = moe_plan(&a, &p);
    const int64_t ws = moe_forward_workspace(&a);
    if (st != MOE_OK) {
        CHECK(st < 0 && ws == st);
        return;
    }
    CHECK(ws == p.workspace_bytes);
    CHECK(p.block_m > 0 && p.capacity == int64_t(a.T) * a.topk + int64_t(a.E) * (p.block_m - 1));
    CHECK(p.num_blocks == (p.capacity + p.block_m - 1) / p.block_m);
    const int64_t offs[] = {p.off_sorted_ids, p.off_expert_ids, p.off_num_post_padded, p.off_xq,
                            p.off_xs, p.off_inter, p.off_inter_scale, p.off_y};
    int64_t prev = -1;
    for (int64_t o : offs) {
        if (o < 0) continue;
        // with T = 0 the per-token regions are empty and may share an offset
        if (a.T > 0) CHECK(o % 256 == 0 && o > prev && o < p.workspace_bytes);
        else CHECK(o % 256 == 0 && o >= prev && o <= p.workspace_bytes);
        prev = o;
    }
    // y: bf16 for fp8 and MXFP8 weights, fp32 for bf16 weights
    CHECK(p.off_y + int64_t(a.T) * a.topk * a.H * (a.wdtype == MOE_WDTYPE_BF16 ? 4 : 2) <= p.workspace_bytes);
    // a too-small workspace is rejected before any launch
    if (a.T > 0) {
        const int st2 = moe_forward(&a, fake(), p.workspace_bytes - 1, nullptr);
        CHECK(st2 == MOE_ERR_WORKSPACE || st2 == MOE_ERR_INVALID_ARG);
    }
    // moe_forward_noalloc rejects what does not fit its array before touching the device
    if (p.workspace_bytes > MOE_NOALLOC_MAX_BYTES) CHECK(moe_forward_noalloc(&a, nullptr) == MOE_ERR_WORKSPACE);
}

int main() {
    // status strings and version
    for (int s = -20; s <= 20; ++s) CHECK(moe_status_string(s) != nullptr);
    CHECK((moe_version() >> 16) == 1);

    // capacity and alignment scratch over edges, overflow included
    const int32_t big = std::numeric_limits<int32_t>::max(), small = std::numeric_limits<int32_t>::min();
    const int32_t vals[] = {small, -1, 0, 1, 2, 7, 16, 63, 64, 65, 255, 256, 1023, 1024, 1025, 4096, 1 << 20, big};
    for (int32_t T : vals)
        for (int32_t k : vals)
            for (int32_t E : vals) {
                (void)moe_align_scratch_bytes(T, k, E);
                for (int32_t B : {small, -1, 0, 1, 16, 64, 256, 1024, 1025, big}) {
                    const int64_t c = moe_align_capacity(T, k, E, B);
                    if (c >= 0) CHECK(c == int64_t(T) * k + int64_t(E) * (B - 1));
                }
            }

    // planner over a deterministic random sweep (extremes included)
    std::mt19937_64 rng(12345);
    auto pick = [&](std::initializer_list<int32_t> l) {
        auto it = l.begin();
        std::advance(it, rng() % l.size());
        return *it;
    };
    const float fvals[] = {-1.0f, 0.0f, 0.5f, std::numeric_limits<float>::infinity(), std::nanf("")};
    for (int it = 0; it < 200000; ++it) {
        moe_forward_args a = base_args();
        a.T = pick({small, -5, 0, 1, 3, 16, 64, 1000, 4096, 8192, 1 << 20, 1 << 26, big});
        a.E = pick({small, -1, 0, 1, 5, 8, 128, 256, 1024, 1025, big});
        a.H = pick({small, -64, 0, 64, 128, 192, 256, 4096, 7168, 1 << 16, 1 << 30, big});
        a.I = pick({small, -128, 0, 64, 128, 256, 384, 1536, 2048, 1 << 20, big});
        a.topk = pick({small, -1, 0, 1, 2, 8, 64, 65, big});
        a.wdtype = pick({-1, 0, 1, 2, 3});
        a.path = pick({-1, 0, 1, 2, 3});
        a.block_m = pick({small, -16, 0, 1, 16, 32, 64, 100, 256, 512, big});
        a.flags = int32_t(rng() & 7);
        a.clamp_limit = fvals[rng() % 5];
        if (rng() % 2) a.w13_scale = a.w2_scale = fake();
        check_plan(a);
    }

    // every entry point: invalid arguments are reported, nothing is launched
    {
        moe_forward_args a = base_args();
        CHECK(moe_forward(nullptr, fake(), 1 << 30, nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_plan(&a, nullptr) == MOE_ERR_INVALID_ARG);
        a.x = nullptr;
        CHECK(moe_forward(&a, fake(), int64_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
        a = base_args();
        a.out = fake(2);
        CHECK(moe_forward(&a, fake(), int64_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
        a = base_args();
        CHECK(moe_forward(&a, fake(8), int64_t(1) << 40, nullptr) == MOE_ERR_WORKSPACE);   // misaligned workspace
        CHECK(moe_forward_profiled(&a, fake(), int64_t(1) << 40, nullptr, nullptr, 0) == MOE_ERR_INVALID_ARG);
        a.wdtype = MOE_WDTYPE_FP8_E4M3;
        CHECK(moe_forward(&a, fake(), int64_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);   // no scales
        a = base_args();
        a.flags = MOE_FLAG_MX_PACKED_SCALES;
        CHECK(moe_forward(&a, fake(), int64_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
        a = base_args();
        uint32_t* sync = static_cast<uint32_t*>(fake());
        CHECK(moe_decode_layer(&a, nullptr, 1, nullptr, nullptr, nullptr, fake(), int64_t(1) << 40, nullptr) ==
              MOE_ERR_INVALID_ARG);
        CHECK(moe_decode_layer(&a, static_cast<const float*>(fake()), 1, nullptr, nullptr, sync, fake(),
                               int64_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
        a.T = 4096;
        CHECK(moe_decode_layer(&a, nullptr, 1, nullptr, nullptr, sync, fake(), int64_t(1) << 40, nullptr) ==
              MOE_ERR_UNSUPPORTED);
        CHECK(moe_route(nullptr, 4, 8, 2, 1, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_route(static_cast<const float*>(fake()), 4, 8, 9, 1, static_cast<int32_t*>(fake()),
                        static_cast<float*>(fake()), nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_route(static_cast<const float*>(fake()), small, 8, 2, 1, nullptr, nullptr, nullptr) ==
              MOE_ERR_INVALID_ARG);
        CHECK(moe_align(nullptr, 4, 2, 8, 16, nullptr, nullptr, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
        int32_t* p = static_cast<int32_t*>(fake());
        CHECK(moe_align(p, 4, 2, 8, 0, p, p, p, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_align_ws(p, 4096, 8, 128, 64, p, p, p, nullptr, nullptr, 0, nullptr) == MOE_ERR_WORKSPACE);
        CHECK(moe_quant_act(fake(), 4, 100, static_cast<uint8_t*>(fake()), static_cast<float*>(fake()),
                            nullptr) == MOE_ERR_UNSUPPORTED);
        CHECK(moe_quant_act(fake(), small, 128, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_quant_act_mx(fake(2), 4, 64, static_cast<uint8_t*>(fake()), static_cast<uint8_t*>(fake()),
                               nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_pack_mx_scales(static_cast<const uint8_t*>(fake()), 2, 48, 128, static_cast<uint8_t*>(fake()),
                                 nullptr) == MOE_ERR_INVALID_ARG);   // overlap
        CHECK(moe_pack_mx_scales(nullptr, 2, 47, 128, nullptr, nullptr) == MOE_ERR_UNSUPPORTED);
        CHECK(moe_pack_mx_scales(nullptr, big, big, big, nullptr, nullptr) != MOE_OK);
    }
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi sanitize harness: ok\n");
    return 0;
}
