// Device helpers shared by the NVFP4 kernels for gfx950: operand types, the
// exact e2m1 x e4m3 -> bf16 decode into the B operand of
// v_mfma_f32_16x16x32_bf16, and the loads and conversions around it.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockK = 128;    // k covered by one 16-byte weight load per lane (4 MFMAs)
constexpr int kMaxLdsBytes = 160 * 1024;

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Two e2m1 codes of byte `sel` of `w` times the group scale, as a bf16 pair.
template <int sel>
__device__ __forceinline__ bf16x2 decode_pair(uint32_t w, float scale) {
    f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, sel);
    f32x2 p = {v[0] * scale, v[1] * scale};
    return __builtin_convertvector(p, bf16x2);
}

// 8 consecutive k (one dword of packed nibbles) as the B operand.
__device__ __forceinline__ bf16x8 decode8(uint32_t w, float scale) {
    bf16x2 a = decode_pair<0>(w, scale);
    bf16x2 b = decode_pair<1>(w, scale);
    bf16x2 c = decode_pair<2>(w, scale);
    bf16x2 d = decode_pair<3>(w, scale);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight e4m3 codes (two dwords) as a bf16 B operand, exactly (e4m3 has 4
// significant bits).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// fp32 <-> its bits through memcpy: with this compiler, bit-casting a vector
// element (v[j]) yields element 0 for every j.
__device__ __forceinline__ uint32_t f32_bits(float f) {
    uint32_t u;
    __builtin_memcpy(&u, &f, sizeof u);
    return u;
}

__device__ __forceinline__ float bits_f32(uint32_t u) {
    float f;
    __builtin_memcpy(&f, &u, sizeof f);
    return f;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    bf16x2 p = __builtin_convertvector(f32x2{f, 0.0f}, bf16x2);
    uint16_t out;
    __builtin_memcpy(&out, &p, sizeof out);
    return out;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bits_f32(uint32_t(b) << 16); }

// silu(g) * u in fp32 (one division and the library exponential), rounded
// once to bf16: the activation of "Module ops" w4a16_gemv_silu_input.  One
// definition for every kernel that forms it, so they agree bit for bit.
__device__ __forceinline__ uint16_t silu_mul(uint16_t g, uint16_t u) {
    const float gf = bf16_to_f32(g);
    const float s = gf / (1.0f + expf(-gf));
    return f32_to_bf16_rne(s * bf16_to_f32(u));
}

__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    // Weights are read exactly once: a non-temporal load keeps them from
    // displacing the activations in the caches.
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint64_t load8_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
}

// For the many-row GEMMs, whose x and weights come in by direct-to-LDS loads.
// Waits until at most N vector memory operations of this wavefront are
// outstanding (direct-to-LDS loads included) and keeps LDS reads below it.
template <int N>
__device__ __forceinline__ void gemm_wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that waits for this wavefront's LDS operations only
// (__syncthreads would also drain the weight loads in flight).
__device__ __forceinline__ void gemm_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace
