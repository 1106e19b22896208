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
constexpr int kQ5KBytes = 176;
constexpr int kQ80Bytes = 34;

__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_i(int v, int src) { return __shfl(v, src, 64); }

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

// ---------------------------------------------------------------------------
// Lane exchange through DPP (VALU, no LDS round trip).  Control codes:
//   0xB1 quad_perm [1,0,3,2] (lane ^ 1)     0x4E quad_perm [2,3,0,1] (lane ^ 2)
//   0x141 row_half_mirror (lane i <-> 7-i in each 8)   0x140 row_mirror (16)
//   0x10n row_shl:n (lane i reads lane i+n inside its row of 16)
// bound_ctrl zero-fills lanes whose source is outside the row.
// ---------------------------------------------------------------------------
template <int C>
__device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, C, 0xF, 0xF, true);
}
template <int C>
__device__ __forceinline__ float dppf(float v) {
    return __builtin_bit_cast(float, dppi<C>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// ---------------------------------------------------------------------------
// Q8_K quantizer body (vllm.cpp PR #2890, commit "QuantizeQ8KKWarpCoop", and
// commit "gamma predicate + amax-seed fix").  One wave quantizes one
// super-block of 256 values; lane l holds values 4l..4l+3.
//   - amax: each lane scans its 4 values with a strict compare from 0 (a NaN
//     never wins), then the wave maximum;
//   - mx is the value at the lowest index whose magnitude equals amax (lowest
//     lane by ballot, then lowest component), which is exactly the first
//     occurrence an ascending strict-compare scan keeps;
//   - iscale = -127/mx (IEEE division), q = min(127, rint(iscale*x)), d =
//     1/iscale; amax == 0 (all zero or all NaN) gives the zero block;
//   - bsum_j (16 values = lanes 4j..4j+3) is left on every lane of the quad.
// ---------------------------------------------------------------------------
struct Q8KLane {
    uint32_t q4;   // the lane's 4 quants, little-endian bytes
    float d;       // super-block scale (wave-uniform)
    int bsum;      // sum of the 16 quants of this lane's quad
};

// N independent super-blocks per wave, processed in lockstep so that their
// dependency chains (reductions, divisions) overlap.
template <int N>
__device__ __forceinline__ void q8k_quant_lanes(const float4 (&v)[N], Q8KLane (&out)[N]) {
    float a[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float xs[4] = {v[n].x, v[n].y, v[n].z, v[n].w};
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ax = fabsf(xs[i]);
            if (ax > m) m = ax;
        }
        a[n] = m;
    }
#pragma unroll
    for (int n = 0; n < N; ++n) a[n] = fmaxf(a[n], dppf<0xB1>(a[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) a[n] = fmaxf(a[n], dppf<0x4E>(a[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) a[n] = fmaxf(a[n], dppf<0x141>(a[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) a[n] = fmaxf(a[n], dppf<0x140>(a[n]));
    float amax[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        amax[n] = fmaxf(fmaxf(readlane_f(a[n], 0), readlane_f(a[n], 16)),
                        fmaxf(readlane_f(a[n], 32), readlane_f(a[n], 48)));
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float xs[4] = {v[n].x, v[n].y, v[n].z, v[n].w};
        // first occurrence of the largest magnitude: the lowest lane holding one,
        // and inside that lane the lowest component
        const bool hit = fabsf(xs[0]) == amax[n] || fabsf(xs[1]) == amax[n] ||
                         fabsf(xs[2]) == amax[n] || fabsf(xs[3]) == amax[n];
        const unsigned long long mask = __ballot(hit);
        const float sel = fabsf(xs[0]) == amax[n] ? xs[0]
                        : (fabsf(xs[1]) == amax[n] ? xs[1] : (fabsf(xs[2]) == amax[n] ? xs[2] : xs[3]));
        const int first = mask ? __builtin_ctzll(mask) : 0;
        const float mx = readlane_f(sel, first);
        if (amax[n] == 0.0f) {
            out[n].q4 = 0u;
            out[n].d = 0.0f;
            out[n].bsum = 0;
            continue;
        }
        const float iscale = -127.0f / mx;
        uint32_t packed = 0;
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float t = iscale * xs[i];
            int q = (int)__builtin_rintf(t);
            q = q > 127 ? 127 : q;
            sum += q;
            packed |= ((uint32_t)(q & 0xFF)) << (8 * i);
        }
        sum += dppi<0xB1>(sum);
        sum += dppi<0x4E>(sum);
        out[n].q4 = packed;
        out[n].d = 1.0f / iscale;
        out[n].bsum = sum;
    }
}

__device__ __forceinline__ Q8KLane q8k_quant_lane(float4 v, int lane) {
    (void)lane;
    const float4 vv[1] = {v};
    Q8KLane r[1];
    q8k_quant_lanes<1>(vv, r);
    return r[0];
}

// ---------------------------------------------------------------------------
// Q8_1 quantizer body (strix-llama.cpp PR #18, commits "mul_mat_vec_q_fq" and
// "mul_mat_vec_q_fq generic").  Eight lanes hold one 32-block (lane l holds
// values 4l..4l+3 of the wave's 256).  amax over the block; d = amax/127;
// q = roundf(x/d) (0 when amax == 0); s = binary32 butterfly sum: element i
// first meets i^16 (lane +4), then i^8 (lane +2), i^4 (lane +1), i^2 and i^1
// (inside the lane).  s is exact on the first lane of each group of 8 (the
// other lanes' s is not the block sum).
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
        const float ax = fabsf(xs[i]);
        if (ax > amax) amax = ax;
    }
    amax = fmaxf(amax, dppf<0xB1>(amax));
    amax = fmaxf(amax, dppf<0x4E>(amax));
    amax = fmaxf(amax, dppf<0x141>(amax));
    const float d = amax / 127.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int q = 0;
        if (amax != 0.0f) q = (int)roundf(xs[i] / d);
        packed |= ((uint32_t)(q & 0xFF)) << (8 * i);
    }
    float b0 = xs[0], b1 = xs[1], b2 = xs[2], b3 = xs[3];
    b0 = b0 + dppf<0x104>(b0); b1 = b1 + dppf<0x104>(b1);
    b2 = b2 + dppf<0x104>(b2); b3 = b3 + dppf<0x104>(b3);
    b0 = b0 + dppf<0x102>(b0); b1 = b1 + dppf<0x102>(b1);
    b2 = b2 + dppf<0x102>(b2); b3 = b3 + dppf<0x102>(b3);
    b0 = b0 + dppf<0x101>(b0); b1 = b1 + dppf<0x101>(b1);
    b2 = b2 + dppf<0x101>(b2); b3 = b3 + dppf<0x101>(b3);
    const float t0 = b0 + b2;
    const float t1 = b1 + b3;
    Q81Lane r;
    r.q4 = packed;
    r.d = d;
    r.s = t0 + t1;
    return r;
}

// Planar activation layout (see include/vq.h).
__host__ __device__ __forceinline__ size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace vqk
