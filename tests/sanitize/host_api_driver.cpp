// Exercises the library's host-side code -- descriptor and argument
// validation, workspace sizing and the path / chunk choice of the C ABI
// (api.cpp, sizing.cpp) and the block-format packer (pack_blocks.cpp) --
// under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU. The
// kernel launchers are replaced by stubs that count calls: every call made
// here returns before a launch (invalid arguments, or T == 0). Packer
// destinations are heap blocks of exactly moe_qb_packed_bytes(), so a write
// past them is reported. Returns nonzero on a failed check.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "internal.h"
#include "moe.h"

static int launches = 0;

namespace moe {
int launch_decode_route(const moe_layer_desc *, const float *, int, int32_t *, float *, float *, void *, hipStream_t)
{
    ++launches;
    return MOE_EUNSUPPORTED;
}
int launch_decode_forward(const moe_layer_desc *, const float *, int, float *, const int32_t *, const float *,
                          const float *, int32_t *, float *, float *, void *, hipStream_t)
{
    ++launches;
    return MOE_EUNSUPPORTED;
}
int launch_prefill_route(const moe_layer_desc *, const float *, int, int32_t *, float *, float *, void *, hipStream_t)
{
    ++launches;
    return MOE_EUNSUPPORTED;
}
int launch_prefill_forward(const moe_layer_desc *, const float *, int, float *, const int32_t *, const float *,
                           const float *, int32_t *, float *, float *, void *, hipStream_t)
{
    ++launches;
    return MOE_EUNSUPPORTED;
}
int launch_qb_unpack(int, const void *, int64_t, int64_t, float *, hipStream_t)
{
    ++launches;
    return MOE_EUNSUPPORTED;
}
int launch_sort_by_expert(const int32_t *, int, int, int, int32_t *, int32_t *, int32_t *, void *, hipStream_t,
                          int32_t *, int, int, int4 *)
{
    ++launches;
    return MOE_EUNSUPPORTED;
}
}  // namespace moe

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }   // never dereferenced

static moe_layer_desc base_desc(int et)
{
    moe_layer_desc d;
    std::memset(&d, 0, sizeof d);
    d.hidden = 2048;
    d.n_experts = 512;
    d.top_k = 10;
    d.inter = 512;
    d.shared_inter = 512;
    d.renormalize = 1;
    d.router_t = MOE_BF16;
    d.expert_t = et;
    d.shared_t = MOE_BF16;
    d.router_w = fake(0x10000);
    d.shared_gate_w = fake(0x10100);
    d.exp_gate = fake(0x20000);
    d.exp_up = fake(0x30000);
    d.exp_down = fake(0x40000);
    d.sh_gate = fake(0x50000);
    d.sh_up = fake(0x60000);
    d.sh_down = fake(0x70000);
    d.norm_eps = 1e-6f;
    return d;
}

static int fwd(const moe_layer_desc *d, int T, const float *x, float *y, void *ws, size_t wsb)
{
    return moe_forward(d, x, T, y, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, ws, wsb, nullptr);
}

static void test_validation()
{
    const float *x = static_cast<const float *>(fake(0x80000));
    float *y = static_cast<float *>(fake(0x90000));
    void *ws = fake(0xA0000);
    for (int et = MOE_F32; et <= MOE_Q4B32; ++et) {
        moe_layer_desc d = base_desc(et);
        const size_t need = moe_workspace_bytes(&d, 1);
        CHECK(need > 0);
        CHECK(fwd(&d, 0, x, y, ws, need) == MOE_OK);
        CHECK(fwd(&d, -1, x, y, ws, need) == MOE_EINVAL);
        CHECK(fwd(&d, 1, nullptr, y, ws, need) == MOE_EINVAL);
        CHECK(fwd(&d, 1, x, y, ws, need - 1) == MOE_EWORKSPACE);
        CHECK(fwd(&d, 1, static_cast<const float *>(fake(0x80004)), y, ws, need) == MOE_EALIGN);
        // every field out of range, one at a time
        moe_layer_desc b;
        const int bad_ints[][2] = {{0, 0}, {0, 2050}, {3, 500}, {2, 0}, {2, 513}, {2, 17}, {5, 2}};
        for (const auto &bi : bad_ints) {
            b = d;
            int *field = bi[0] == 0 ? &b.hidden : bi[0] == 2 ? &b.top_k : bi[0] == 3 ? &b.inter : &b.renormalize;
            *field = bi[1];
            CHECK(moe_workspace_bytes(&b, 1) == 0);
            CHECK(fwd(&b, 1, x, y, ws, 1u << 30) != MOE_OK);
        }
        b = d;
        b.expert_t = 5;
        CHECK(fwd(&b, 1, x, y, ws, 1u << 30) == MOE_EINVAL);
        b = d;
        b.bias_mode = 2;
        CHECK(fwd(&b, 1, x, y, ws, 1u << 30) == MOE_EINVAL);
        b = d;
        b.norm_w = static_cast<const float *>(fake(0xB0000));
        b.norm_eps = -1.0f;
        CHECK(fwd(&b, 1, x, y, ws, 1u << 30) == MOE_EINVAL);
        b.norm_eps = NAN;
        CHECK(fwd(&b, 1, x, y, ws, 1u << 30) == MOE_EINVAL);
        b = d;
        b.exp_up = fake(0x30008);
        CHECK(fwd(&b, 1, x, y, ws, 1u << 30) == MOE_EALIGN);
        b = d;
        b.n_experts = 2048;
        CHECK(fwd(&b, 1, x, y, ws, 1u << 30) == MOE_EUNSUPPORTED);
        CHECK(moe_route(&d, x, 1, nullptr, nullptr, nullptr, ws, need, nullptr) == MOE_EINVAL);
    }
    CHECK(launches == 0);
}

static void test_sizing()
{
    // every call size up to the largest T, at the default and the largest shapes
    const int Ts[] = {1, 2, 3, 4, 5, 8, 12, 13, 16, 100, 2048, 8192, 65536, 1 << 20, INT_MAX};
    for (int et = MOE_F32; et <= MOE_Q4B32; ++et) {
        for (int big = 0; big < 2; ++big) {
            moe_layer_desc d = base_desc(et);
            if (big) {
                d.hidden = 8192;
                d.inter = 4096;
                d.shared_inter = 4096;
                d.n_experts = 1024;
                d.top_k = 16;
                d.norm_w = static_cast<const float *>(fake(0xB0000));
            }
            size_t prev = 0;
            for (int T : Ts) {
                const size_t n = moe_workspace_bytes(&d, T);
                CHECK(n > 0 && n <= (static_cast<size_t>(3) << 29));
                if (T > 16)
                    CHECK(n >= prev || T > 65536);   // chunked beyond the bound
                prev = n;
            }
        }
    }
    CHECK(moe_sort_workspace_bytes(INT_MAX, 16, 1024) > 0);
    CHECK(moe_sort_workspace_bytes(-1, 4, 8) == 0 || moe_sort_workspace_bytes(-1, 4, 8) > 0);
    CHECK(moe_sort_by_expert(nullptr, 4, 2, 8, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == MOE_EINVAL);
    CHECK(moe_qb_unpack(3, fake(0x1000), 4, 48, static_cast<float *>(fake(0x2000)), nullptr) == MOE_EINVAL);
    CHECK(moe_qb_unpack(5, fake(0x1000), 4, 64, static_cast<float *>(fake(0x2000)), nullptr) == MOE_EINVAL);
    CHECK(moe_qb_unpack(4, fake(0x1008), 4, 64, static_cast<float *>(fake(0x2000)), nullptr) == MOE_EALIGN);
    CHECK(launches == 0);
}

static void test_packer()
{
    uint64_t s = 12345;
    auto rnd = [&]() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return static_cast<float>(static_cast<int64_t>(s >> 11) - (int64_t(1) << 52)) * 0x1.0p-52f;
    };
    const int shapes[][2] = {{1, 32}, {3, 96}, {7, 2048}, {64, 512}};
    for (int bits = 2; bits <= 4; ++bits) {
        for (const auto &sh : shapes) {
            const int rows = sh[0], cols = sh[1];
            std::vector<float> w(static_cast<size_t>(rows) * cols);
            for (auto &v : w)
                v = rnd() * 0.05f;
            w[0] = 0.99999f;
            if (cols >= 64)
                for (int j = 32; j < 64; ++j)
                    w[j] = 0.0123f;
            const size_t n = moe_qb_packed_bytes(bits, rows, cols);
            CHECK(n % 256 == 0 && n >= static_cast<size_t>(rows) * cols * (bits + 1) / 8);
            uint8_t *dst = static_cast<uint8_t *>(std::malloc(n));   // exactly the documented size
            CHECK(moe_qb_pack(bits, w.data(), rows, cols, dst, n) == MOE_OK);
            CHECK(moe_qb_pack(bits, w.data(), rows, cols, dst, n - 1) == MOE_EWORKSPACE);
            w[5] = NAN;
            CHECK(moe_qb_pack(bits, w.data(), rows, cols, dst, n) == MOE_ENONFINITE);
            w[5] = 1e30f;
            CHECK(moe_qb_pack(bits, w.data(), rows, cols, dst, n) == MOE_ENONFINITE);
            std::free(dst);
        }
        CHECK(moe_qb_packed_bytes(bits, 1, 48) == 0 && moe_qb_packed_bytes(bits, 0, 64) == 0);
        CHECK(moe_qb_packed_bytes(bits, INT64_C(1) << 20, INT64_C(1) << 20) > 0);
    }
    std::vector<float> w(64, 0.0f);
    CHECK(moe_qb_pack(1, w.data(), 2, 32, fake(0x1000), 1 << 20) == MOE_EINVAL);
    CHECK(moe_qb_pack(5, w.data(), 2, 32, fake(0x1000), 1 << 20) == MOE_EINVAL);
    CHECK(moe_qb_pack(2, nullptr, 2, 32, fake(0x1000), 1 << 20) == MOE_EINVAL);
    CHECK(moe_q2_packed_bytes(4, 64) == moe_qb_packed_bytes(2, 4, 64));
}

int main()
{
    CHECK(moe_abi_version() == MOE_ABI_VERSION);
    for (int c = 1; c >= -7; --c)
        CHECK(moe_strerror(c) != nullptr);
    test_validation();
    test_sizing();
    test_packer();
    if (failures)
        std::fprintf(stderr, "%d checks failed\n", failures);
    else
        std::printf("host api driver: all checks passed\n");
    return failures ? 1 : 0;
}
