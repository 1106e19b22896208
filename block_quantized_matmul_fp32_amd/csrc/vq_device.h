// vq_device.h -- device helpers shared by the gfx950 kernels of this library.
//
// Wave64 lane exchange, binary16 conversion through the hardware converter
// (round to nearest even), signed dot4 (v_dot4_i32_i8), LDS reads at 2-byte
// alignment, and the one Q8_K / Q8_1 activation quantizer body used by both
// the standalone quantizer and the GEMV prologue, so the two produce the same
// bytes by construction (vllm.cpp PR #2890, commit "Lever-C norm-quant
// epilogue": one shared quant-block body for fused and standalone paths).
#pragma once

// Binary32 expressions are evaluated as written (no multiply-add contraction).
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqk {

constexpr int kQK = 256;    // super-block of Q4_K, Q6_K, Q8_K
constexpr int kQK8 = 32;    // block of Q8_0, Q8_1
constexpr int kQ4KBytes = 144;
constexpr int kQ6KBytes = 210;
constexpr int kQ80Bytes = 34;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_i(int v, int src) { return __shfl(v, src, 64); }
__device__ __forceinline__ float shfl_f(float v, int src) { return __shfl(v, src, 64); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    _Float16 v = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, v);
}

__device__ __forceinline__ int sdot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// 16 bytes at a 2-byte aligned LDS address, as four dwords, using only
// 4-byte aligned reads.
__device__ __forceinline__ void lds_read16_a2(const uint8_t* p, uint32_t out[4]) {
    uintptr_t a = (uintptr_t)p;
    const uint32_t* q = (const uint32_t*)(a & ~(uintptr_t)3);
    uint32_t sh = (uint32_t)(a & 3);
    uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
    if (sh == 0) {
        out[0] = w0; out[1] = w1; out[2] = w2; out[3] = w3;
    } else {
        uint32_t w4 = q[4];
        out[0] = __builtin_amdgcn_alignbyte(w1, w0, sh);
        out[1] = __builtin_amdgcn_alignbyte(w2, w1, sh);
        out[2] = __builtin_amdgcn_alignbyte(w3, w2, sh);
        out[3] = __builtin_amdgcn_alignbyte(w4, w3, sh);
    }
}

// ---------------------------------------------------------------------------
// Q8_K quantizer body (vllm.cpp PR #2890, commit "QuantizeQ8KKWarpCoop", and
// commit "gamma predicate + amax-seed fix").  One wave quantizes one
// super-block of 256 values; lane l holds values 4l..4l+3.
//   - each lane scans its 4 values ascending with a strict compare from
//     amax = 0 (first occurrence, a NaN never wins);
//   - the wave reduction keeps the larger magnitude and, on a tie, the lower
//     element index, which equals the sequential first occurrence;
//   - iscale = -127/mx (IEEE division), q = min(127, rint(iscale*x)), d =
//     1/iscale; amax == 0 gives the zero block;
//   - bsum_j (16 values = lanes 4j..4j+3) is left on every lane of the quad.
// ---------------------------------------------------------------------------
struct Q8KLane {
    uint32_t q4;   // the lane's 4 quants, little-endian bytes
    float d;       // super-block scale (wave-uniform)
    int bsum;      // sum of the 16 quants of this lane's quad
};

__device__ __forceinline__ Q8KLane q8k_quant_lane(float4 v, int lane) {
    float amax = 0.0f, mx = 0.0f;
    int idx = 0x7FFFFFFF;
    const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float ax = fabsf(xs[i]);
        if (ax > amax) { amax = ax; mx = xs[i]; idx = 4 * lane + i; }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float oa = shfl_xor_f(amax, o);
        float om = shfl_xor_f(mx, o);
        int oi = shfl_xor_i(idx, o);
        bool take = (oa > amax) || (oa == amax && oi < idx);
        if (take) { amax = oa; mx = om; idx = oi; }
    }
    Q8KLane r;
    if (amax == 0.0f) {
        r.q4 = 0u;
        r.d = 0.0f;
        r.bsum = 0;
        return r;
    }
    const float iscale = -127.0f / mx;
    uint32_t packed = 0;
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float t = iscale * xs[i];
        int q = (int)__builtin_rintf(t);
        q = q > 127 ? 127 : q;
        s += q;
        packed |= ((uint32_t)(q & 0xFF)) << (8 * i);
    }
    s += shfl_xor_i(s, 1);
    s += shfl_xor_i(s, 2);
    r.q4 = packed;
    r.d = 1.0f / iscale;
    r.bsum = s;
    return r;
}

// ---------------------------------------------------------------------------
// Q8_1 quantizer body (strix-llama.cpp PR #18, commits "mul_mat_vec_q_fq" and
// "mul_mat_vec_q_fq generic").  Eight lanes hold one 32-block (lane l holds
// values 4l..4l+3 of the wave's 256).  amax over the block; d = amax/127;
// q = roundf(x/d) (0 when amax == 0); s = binary32 butterfly sum: element i
// first meets i^16 (lane ^4), then i^8 (lane ^2), i^4 (lane ^1), i^2 and i^1
// (inside the lane).  Returns the 4 quants, d (binary32) and s (binary32).
// ---------------------------------------------------------------------------
struct Q81Lane {
    uint32_t q4;
    float d;
    float s;
};

__device__ __forceinline__ Q81Lane q81_quant_lane(float4 v) {
    const float xs[4] = {v.x, v.y, v.z, v.w};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float ax = fabsf(xs[i]);
        if (ax > amax) amax = ax;
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
        float oa = shfl_xor_f(amax, o);
        if (oa > amax) amax = oa;
    }
    const float d = amax / 127.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int q = 0;
        if (amax != 0.0f) q = (int)roundf(xs[i] / d);
        packed |= ((uint32_t)(q & 0xFF)) << (8 * i);
    }
    float b0 = xs[0], b1 = xs[1], b2 = xs[2], b3 = xs[3];
    b0 = b0 + shfl_xor_f(b0, 4); b1 = b1 + shfl_xor_f(b1, 4);
    b2 = b2 + shfl_xor_f(b2, 4); b3 = b3 + shfl_xor_f(b3, 4);
    b0 = b0 + shfl_xor_f(b0, 2); b1 = b1 + shfl_xor_f(b1, 2);
    b2 = b2 + shfl_xor_f(b2, 2); b3 = b3 + shfl_xor_f(b3, 2);
    b0 = b0 + shfl_xor_f(b0, 1); b1 = b1 + shfl_xor_f(b1, 1);
    b2 = b2 + shfl_xor_f(b2, 1); b3 = b3 + shfl_xor_f(b3, 1);
    float t0 = b0 + b2;
    float t1 = b1 + b3;
    Q81Lane r;
    r.q4 = packed;
    r.d = d;
    r.s = t0 + t1;
    return r;
}

// Planar activation layout (see include/vq.h).
__host__ __device__ __forceinline__ size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace vqk
