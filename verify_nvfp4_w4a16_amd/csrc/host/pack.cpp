// Host quantiser fp32 -> NVFP4 and the pure host checks of the C ABI.
//
// Stored format ("Module ops", metrale_model_layers::layers::ops:
// nvfp4_mmq_repack and quantize_bf16_to_nvfp4): packed e2m1 [N, K/2] with the
// low nibble holding the even k, one e4m3 scale per 16 consecutive k [N, K/16],
// plus one fp32 per-tensor scale (dequant_nvfp4_to_bf16's "scale2").
//
// The quantisation rule is spelled out in include/nvfp4_w4a16.h.  Every step is
// IEEE binary64 in a fixed order (built with -ffp-contract=off), so the result
// is a pure function of the input; rows are spread over threads only after the
// global maximum is known, and each row is written by exactly one thread.
#include "nvfp4_w4a16.h"

#include <sched.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr double kE2m1Max = 6.0;
constexpr double kE4m3Max = 448.0;
constexpr int kGroup = 16;

// Value of a non-negative e4m3 code (0x00..0x7E): 4 exponent bits with bias 7,
// 3 mantissa bits; exponent field 0 is subnormal with quantum 2^-9.
double e4m3_decode(uint8_t code) {
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 0) return std::ldexp(double(m), -9);
    return std::ldexp(double(8 + m), e - 10);
}

// Nearest e4m3 code to u >= 0 (finite), ties to the even code, saturating at
// 448 (0x7E).  Inside one binade the representable values are r * q for an
// integer r and a power-of-two quantum q, and the code increases by one per
// step of q across the whole range, so rounding u / q to the nearest even
// integer is the same as choosing the even code on a tie.
uint8_t e4m3_encode(double u) {
    if (!(u < kE4m3Max)) return 0x7E;
    if (u == 0.0) return 0;
    int exp2;
    std::frexp(u, &exp2);                 // u = f * 2^exp2, f in [0.5, 1)
    int unbiased = exp2 - 1;              // u = 1.xxx * 2^unbiased
    double quantum = unbiased < -6 ? std::ldexp(1.0, -9) : std::ldexp(1.0, unbiased - 3);
    double r = std::nearbyint(u / quantum);   // default rounding: ties to even
    double v = r * quantum;
    if (v >= kE4m3Max) return 0x7E;
    if (v < std::ldexp(1.0, -6)) return static_cast<uint8_t>(r);   // subnormal codes 0..7
    std::frexp(v, &exp2);
    int e = exp2 - 1;                                              // -6..8
    int mant = static_cast<int>(std::ldexp(v, -e) * 8.0) - 8;      // 0..7
    return static_cast<uint8_t>(((e + 7) << 3) | mant);
}

// Nearest e2m1 magnitude code (0..7 for 0, .5, 1, 1.5, 2, 3, 4, 6) to a >= 0,
// ties to the even code, saturating at 6.  The thresholds are the midpoints
// between neighbouring magnitudes; ">" or ">=" puts a tie on the even side.
// Counting the thresholds passed keeps the loop free of branches.
inline uint8_t e2m1_encode_magnitude(double a) {
    return static_cast<uint8_t>((a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) +
                                (a > 2.5) + (a >= 3.5) + (a > 5.0));
}

void pack_rows(const float* w, int64_t k, int64_t row0, int64_t row1, double t,
               uint8_t* w_packed, uint8_t* scales) {
    const int64_t groups = k / kGroup;
    uint8_t codes[kGroup];
    for (int64_t n = row0; n < row1; ++n) {
        const float* row = w + n * k;
        for (int64_t g = 0; g < groups; ++g) {
            const float* grp = row + g * kGroup;
            double amax = 0.0;
            for (int i = 0; i < kGroup; ++i) amax = std::max(amax, std::fabs(double(grp[i])));
            double u = (amax / kE2m1Max) / t;
            uint8_t s = e4m3_encode(u);
            double big_s = e4m3_decode(s) * t;
            for (int i = 0; i < kGroup; ++i) {
                if (big_s == 0.0) { codes[i] = 0; continue; }
                double v = double(grp[i]) / big_s;
                uint8_t mag = e2m1_encode_magnitude(std::fabs(v));
                codes[i] = static_cast<uint8_t>(mag | ((v < 0.0 && mag != 0) ? 8 : 0));
            }
            scales[n * groups + g] = s;
            uint8_t* out = w_packed + n * (k / 2) + g * (kGroup / 2);
            for (int j = 0; j < kGroup / 2; ++j)
                out[j] = static_cast<uint8_t>(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
}

// Threads the packer may use: the CPUs this process may run on, at most 16.
int cpu_budget() {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0) return std::max(1, std::min(16, CPU_COUNT(&set)));
    return std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
}

template <class F>
void run_parallel(int workers, F&& f) {
    if (workers == 1) { f(0); return; }
    std::vector<std::thread> pool;
    pool.reserve(workers);
    for (int i = 0; i < workers; ++i) pool.emplace_back(f, i);
    for (auto& th : pool) th.join();
}

int worker_count(int64_t rows, int64_t k) {
    int hw = cpu_budget();
    int64_t by_work = (rows * k) / (1 << 20) + 1;     // at least ~1M weights per thread
    int64_t t = std::min<int64_t>(hw, by_work);
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(t, rows)));
}

}  // namespace

extern "C" int nvfp4_pack(const float* w, int64_t n, int64_t k, uint8_t* w_packed,
                          uint8_t* scales_e4m3, float* tensor_scale) {
    if (!w || !w_packed || !scales_e4m3 || !tensor_scale) return NVFP4_ERR_NULL;
    if (n < 1 || k < kGroup || k % kGroup) return NVFP4_ERR_SHAPE;
    int workers = worker_count(n, k);
    // Q1: the largest magnitude (a maximum is exact in any order) and the
    // finiteness check, over row ranges in parallel.
    std::vector<double> part_max(workers, 0.0);
    std::vector<int> part_bad(workers, 0);
    const int64_t per = (n + workers - 1) / workers;
    auto scan = [&](int i) {
        int64_t r0 = i * per, r1 = std::min(n, r0 + per);
        double m = 0.0;
        int bad = 0;
        for (int64_t j = r0 * k; j < r1 * k; ++j) {
            double a = std::fabs(double(w[j]));
            bad |= !std::isfinite(a);
            m = std::max(m, a);
        }
        part_max[i] = m;
        part_bad[i] = bad;
    };
    run_parallel(workers, scan);
    double amax = 0.0;
    for (int i = 0; i < workers; ++i) {
        if (part_bad[i]) return NVFP4_ERR_NONFINITE;
        amax = std::max(amax, part_max[i]);
    }
    float t32 = static_cast<float>(amax / (kE2m1Max * kE4m3Max));
    if (amax == 0.0 || t32 == 0.0f) t32 = 1.0f;
    const double t = double(t32);

    // Q2..Q6 row by row; each row is written by exactly one thread.
    run_parallel(workers, [&](int i) {
        int64_t r0 = i * per, r1 = std::min(n, r0 + per);
        if (r0 < r1) pack_rows(w, k, r0, r1, t, w_packed, scales_e4m3);
    });
    *tensor_scale = t32;
    return NVFP4_OK;
}

extern "C" int fp8_w8a16_pack(const float* w, int64_t n, int64_t k, uint8_t* w_e4m3, float* block_scales) {
    constexpr int64_t kB = 128;
    if (!w || !w_e4m3 || !block_scales) return NVFP4_ERR_NULL;
    if (n < kB || k < kB || n % kB || k % kB) return NVFP4_ERR_SHAPE;
    for (int64_t i = 0; i < n * k; ++i)
        if (!std::isfinite(w[i])) return NVFP4_ERR_NONFINITE;
    const int64_t kb = k / kB;
    const int workers = worker_count(n / kB, kB * k);
    const int64_t rows_per = (n / kB + workers - 1) / workers;     // 128-row block rows per thread
    run_parallel(workers, [&](int t) {
        for (int64_t br = t * rows_per; br < std::min(n / kB, (t + 1) * rows_per); ++br)
            for (int64_t bc = 0; bc < kb; ++bc) {
                double amax = 0.0;
                for (int64_t r = 0; r < kB; ++r)
                    for (int64_t c = 0; c < kB; ++c)
                        amax = std::max(amax, std::fabs(double(w[(br * kB + r) * k + bc * kB + c])));
                float s = static_cast<float>(amax / kE4m3Max);
                if (amax == 0.0 || s == 0.0f) s = 1.0f;
                block_scales[br * kb + bc] = s;
                for (int64_t r = 0; r < kB; ++r)
                    for (int64_t c = 0; c < kB; ++c) {
                        const int64_t i = (br * kB + r) * k + bc * kB + c;
                        const double v = double(w[i]) / double(s);
                        const uint8_t mag = e4m3_encode(std::fabs(v));
                        w_e4m3[i] = static_cast<uint8_t>(mag | ((v < 0.0 && mag != 0) ? 0x80 : 0));
                    }
            }
    });
    return NVFP4_OK;
}

extern "C" int nvfp4_check_scales(const uint8_t* scales_e4m3, int64_t n, int64_t k) {
    if (!scales_e4m3) return NVFP4_ERR_NULL;
    if (n < 1 || k < kGroup || k % kGroup) return NVFP4_ERR_SHAPE;
    const int64_t total = n * (k / kGroup);
    for (int64_t i = 0; i < total; ++i) {
        uint8_t b = scales_e4m3[i];
        if ((b & 0x80) || b == 0x7F) return NVFP4_ERR_BADSCALE;
    }
    return NVFP4_OK;
}

extern "C" int nvfp4_linear_shape_ok(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || m > NVFP4_MAX_M) return NVFP4_ERR_SHAPE;
    if (n < 1 || n > (int64_t(1) << 28)) return NVFP4_ERR_SHAPE;
    if (k < NVFP4_K_MULTIPLE || k > (int64_t(1) << 20) || k % NVFP4_K_MULTIPLE) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

extern "C" int nvfp4_gemm_shape_ok(int64_t m, int64_t n, int64_t k) {
    // rows: at most 65535 workgroup rows (the grid's y limit) of 128
    if (m < 0 || m > int64_t(65535) * 128) return NVFP4_ERR_SHAPE;
    if (n < 1 || n > (int64_t(1) << 28)) return NVFP4_ERR_SHAPE;
    if (k < NVFP4_K_MULTIPLE || k > (int64_t(1) << 20) || k % NVFP4_K_MULTIPLE) return NVFP4_ERR_SHAPE;
    if (m * n > (int64_t(1) << 40)) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

extern "C" int fp8_w8a16_shape_ok(int64_t m, int64_t n, int64_t k) {
    constexpr int64_t kB = 128;
    if (m < 0 || m > NVFP4_MAX_M) return NVFP4_ERR_SHAPE;
    if (n < kB || n > (int64_t(1) << 28) || n % kB) return NVFP4_ERR_SHAPE;
    if (k < kB || k > (int64_t(1) << 20) || k % kB) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

extern "C" int fp8_w8a16_gemm_shape_ok(int64_t m, int64_t n, int64_t k) {
    constexpr int64_t kB = 128;
    // rows: at most 65535 workgroup rows (the grid's y limit) of 128
    if (m < 0 || m > int64_t(65535) * 128) return NVFP4_ERR_SHAPE;
    if (n < kB || n > (int64_t(1) << 28) || n % kB) return NVFP4_ERR_SHAPE;
    if (k < kB || k > (int64_t(1) << 20) || k % kB) return NVFP4_ERR_SHAPE;
    if (m * n > (int64_t(1) << 40)) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

extern "C" const char* nvfp4_strerror(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_NULL: return "a required pointer is NULL";
        case NVFP4_ERR_SHAPE: return "shape outside the contract (0<=M<=32, N>=1, K%256==0 for nvfp4_linear; K%16==0 for packing)";
        case NVFP4_ERR_ALIGN: return "pointer misaligned (x, w_packed, scales: 16 bytes; y: element size)";
        case NVFP4_ERR_DTYPE: return "y_dtype must be NVFP4_OUT_BF16 or NVFP4_OUT_F32";
        case NVFP4_ERR_NONFINITE: return "weight matrix holds NaN or infinity";
        case NVFP4_ERR_BADSCALE: return "a scale byte is negative or NaN";
        case NVFP4_ERR_HIP: return "HIP runtime error";
        case NVFP4_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
        case NVFP4_ERR_TILEFILE: return "NVFP4_TILES override file unreadable or invalid";
        case NVFP4_ERR_BUFFER: return "text buffer too small";
        case NVFP4_ERR_TILE: return "launch tile does not fit the shape";
        case NVFP4_ERR_SCRATCH: return "the call needs more exchange memory than the fixed scratch of nvfp4_linear_noalloc holds";
        case NVFP4_ERR_LIBRARY: return "the GEMM library (hipBLASLt) reported an error";
        default: return "unknown status";
    }
}
