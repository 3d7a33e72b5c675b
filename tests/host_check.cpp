// Driver for the host code of the library (packer, scale check, shape
// contract, tile table and its override file) built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  It exercises
// every host entry point, including the error paths, and prints "host ok".
// Usage: host_check [expect_tilefile_status]
#include <cmath>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <string>
#include <vector>

#include "nvfp4_w4a16.h"
#include "../verify_nvfp4_w4a16_amd/csrc/host/tiles.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

static void pack_cases() {
    std::mt19937 gen(7);
    std::normal_distribution<float> nd(0.0f, 0.02f);
    const int64_t shapes[][2] = {{1, 16}, {3, 32}, {17, 256}, {1536, 2048}, {5, 4096}};
    for (auto& s : shapes) {
        const int64_t n = s[0], k = s[1];
        std::vector<float> w(size_t(n * k));
        for (auto& v : w) v = nd(gen);
        w[0] = 0.0f;
        if (n * k > 40) w[17] = 1e-40f;                     // fp32 subnormal
        std::vector<uint8_t> p(size_t(n * k / 2)), sc(size_t(n * k / 16));
        float t = 0.0f;
        CHECK(nvfp4_pack(w.data(), n, k, p.data(), sc.data(), &t) == NVFP4_OK);
        CHECK(t > 0.0f && std::isfinite(t));
        CHECK(nvfp4_check_scales(sc.data(), n, k) == NVFP4_OK);
    }
    // zero matrix, huge values, errors
    std::vector<float> z(64 * 32, 0.0f);
    std::vector<uint8_t> p(64 * 16), sc(64 * 2);
    float t = 0.0f;
    CHECK(nvfp4_pack(z.data(), 64, 32, p.data(), sc.data(), &t) == NVFP4_OK && t == 1.0f);
    z[5] = 3e38f;
    CHECK(nvfp4_pack(z.data(), 64, 32, p.data(), sc.data(), &t) == NVFP4_OK);
    z[9] = std::numeric_limits<float>::quiet_NaN();
    CHECK(nvfp4_pack(z.data(), 64, 32, p.data(), sc.data(), &t) == NVFP4_ERR_NONFINITE);
    z[9] = std::numeric_limits<float>::infinity();
    CHECK(nvfp4_pack(z.data(), 64, 32, p.data(), sc.data(), &t) == NVFP4_ERR_NONFINITE);
    CHECK(nvfp4_pack(nullptr, 64, 32, p.data(), sc.data(), &t) == NVFP4_ERR_NULL);
    CHECK(nvfp4_pack(z.data(), 0, 32, p.data(), sc.data(), &t) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_pack(z.data(), 4, 24, p.data(), sc.data(), &t) == NVFP4_ERR_SHAPE);
    // FP8 block-scaled packer
    {
        std::vector<float> w8(256 * 384);
        for (auto& v : w8) v = nd(gen);
        std::vector<uint8_t> c8(w8.size());
        std::vector<float> s8(2 * 3);
        CHECK(fp8_w8a16_pack(w8.data(), 256, 384, c8.data(), s8.data()) == NVFP4_OK);
        CHECK(fp8_w8a16_pack(w8.data(), 100, 384, c8.data(), s8.data()) == NVFP4_ERR_SHAPE);
        CHECK(fp8_w8a16_pack(nullptr, 256, 384, c8.data(), s8.data()) == NVFP4_ERR_NULL);
        w8[77] = std::numeric_limits<float>::infinity();
        CHECK(fp8_w8a16_pack(w8.data(), 256, 384, c8.data(), s8.data()) == NVFP4_ERR_NONFINITE);
        CHECK(fp8_w8a16_shape_ok(32, 128, 128) == NVFP4_OK && fp8_w8a16_shape_ok(1, 128, 64) == NVFP4_ERR_SHAPE);
    }
    // scale check
    std::vector<uint8_t> s2(32, 0x38);
    CHECK(nvfp4_check_scales(s2.data(), 2, 256) == NVFP4_OK);
    s2[31] = 0x7F;
    CHECK(nvfp4_check_scales(s2.data(), 2, 256) == NVFP4_ERR_BADSCALE);
    s2[31] = 0x80;
    CHECK(nvfp4_check_scales(s2.data(), 2, 256) == NVFP4_ERR_BADSCALE);
    CHECK(nvfp4_check_scales(nullptr, 2, 256) == NVFP4_ERR_NULL);
    CHECK(nvfp4_check_scales(s2.data(), 2, 8) == NVFP4_ERR_SHAPE);
}

static void contract_cases() {
    CHECK(nvfp4_linear_shape_ok(0, 1, 256) == NVFP4_OK);
    CHECK(nvfp4_linear_shape_ok(32, int64_t(1) << 28, int64_t(1) << 20) == NVFP4_OK);
    CHECK(nvfp4_linear_shape_ok(33, 1, 256) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_linear_shape_ok(-1, 1, 256) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_linear_shape_ok(1, 0, 256) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_linear_shape_ok(1, (int64_t(1) << 28) + 1, 256) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_linear_shape_ok(1, 1, 128) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_linear_shape_ok(1, 1, 384) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_linear_shape_ok(1, 1, (int64_t(1) << 20) + 256) == NVFP4_ERR_SHAPE);
    CHECK(nvfp4_gemm_shape_ok(4096, 8192, 4096) == NVFP4_OK && nvfp4_gemm_shape_ok(65535 * 128 + 1, 1, 256) != 0);
    CHECK(nvfp4_gemm_shape_ok(1, 1, 100) == NVFP4_ERR_SHAPE && nvfp4_gemm_shape_ok(-1, 1, 256) == NVFP4_ERR_SHAPE);
    CHECK(fp8_w8a16_gemm_shape_ok(0, 128, 128) == NVFP4_OK && fp8_w8a16_gemm_shape_ok(65535 * 128, 128, 128) == NVFP4_OK);
    CHECK(fp8_w8a16_gemm_shape_ok(65535 * 128 + 1, 128, 128) == NVFP4_ERR_SHAPE);
    CHECK(fp8_w8a16_gemm_shape_ok(64, 100, 128) == NVFP4_ERR_SHAPE && fp8_w8a16_gemm_shape_ok(64, 128, 64) == NVFP4_ERR_SHAPE);
    CHECK(fp8_w8a16_gemm_shape_ok(int64_t(1) << 22, int64_t(1) << 19, 128) == NVFP4_ERR_SHAPE);   // M * N above 2^40
    for (int st = 1; st >= -40; --st) CHECK(nvfp4_strerror(st) != nullptr);
}

static void tile_cases() {
    for (int64_t k = 256; k <= (int64_t(1) << 20); k *= 2)
        for (int64_t n : {int64_t(1), int64_t(17), int64_t(4096), int64_t(151552), int64_t(1) << 28}) {
            nvfp4::Tile t = nvfp4::tile_for(n, k);
            CHECK(nvfp4::tile_valid(t, n, k));
            CHECK(!nvfp4::tile_text(n, k, t).empty());
        }
    nvfp4::Tile bad;
    bad.cols = 48;
    CHECK(!nvfp4::tile_valid(bad, 4096, 4096));
    bad = nvfp4::Tile();
    bad.split = 3;
    CHECK(!nvfp4::tile_valid(bad, 4096, 4096));
    bad = nvfp4::Tile();
    bad.waves = 8;
    bad.unroll = 4;
    CHECK(!nvfp4::tile_valid(bad, 4096, 1536));
    CHECK(nvfp4::default_split(128, 8) == 2 || nvfp4::default_split(128, 8) >= 1);
}

int main(int argc, char** argv) {
    // the grouped launch's record as the Python binding lays it out
    CHECK(sizeof(nvfp4_group_t) == 40 && offsetof(nvfp4_group_t, w_packed) == 8 &&
          offsetof(nvfp4_group_t, scales_e4m3) == 16 && offsetof(nvfp4_group_t, y) == 24 &&
          offsetof(nvfp4_group_t, tensor_scale) == 32 && offsetof(nvfp4_group_t, m) == 36);
    pack_cases();
    contract_cases();
    tile_cases();
    // the override file named by NVFP4_TILES (if any): its status is expected
    // to be argv[1]; an accepted file's entries are what tile_for returns
    const int want = argc > 1 ? std::atoi(argv[1]) : NVFP4_OK;
    const int st = nvfp4::load_tile_override();
    CHECK(st == want);
    CHECK(nvfp4::load_tile_override() == st);          // the same status every call
    if (st == NVFP4_OK && std::getenv("NVFP4_TILES")) {
        nvfp4::Tile t = nvfp4::tile_for(4096, 4096);
        CHECK(t.cols == 32 && t.waves == 4 && t.unroll == 2 && t.split == 2 && t.mwaves == 6);
    }
    std::printf("host ok\n");
    return 0;
}
