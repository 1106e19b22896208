// produce.hip -- producers that emit their consumer's activation blocks in
// the same launch: RMSNorm -> Q8_K / Q8_1 and silu(gate) * up -> Q8_K / Q8_1
// (vllm.cpp PR #2890, commits "Norm epilogue" and "SiLU-mul quant": the
// producer writes its normal output and the quantized blocks, and the
// consumer skips the standalone quantizer launch and its re-read).
//
// One workgroup per row, one wave per 256-value step (lane l holds values
// 4l..4l+3 of the step), at most 16 waves.  The quantizer is the shared body
// of vq_device.h applied to the binary32 values this kernel stores, so the
// bytes equal those of the standalone quantizer run on the stored output.
#include "vq_device.h"
#include "vq_internal.h"

#pragma clang fp contract(off)

namespace vqk {

constexpr int kProdWaves = 16;
constexpr int64_t kSplitRows = 16;  // RMSNorm rows split over workgroups up to this many rows

__device__ __forceinline__ float4 load4(const float* p, bool vec) {
    return vec ? *(const float4*)p : make_float4(p[0], p[1], p[2], p[3]);
}

__device__ __forceinline__ void store4(float* p, float4 v, bool vec) {
    if (vec) {
        *(float4*)p = v;
    } else {
        p[0] = v.x; p[1] = v.y; p[2] = v.z; p[3] = v.w;
    }
}

// The quantizer epilogue of one 256-value step s (values v, lane l holds
// 4l..4l+3): Y (optional) and the step's Q8_K super-block or eight Q8_1 blocks.
template <int ACT>
__device__ __forceinline__ void emit_step(float4 v, int s, int lane, int64_t m, int K, float* Y, int64_t ldy,
                                          const ActQ8K& o8k, const ActQ81& o81, bool vec) {
    const int e = s * kQK + 4 * lane;
    const bool valid = e < K;
    if (Y != nullptr && valid) store4(Y + m * ldy + e, v, vec);
    if (ACT == 0) {
        const Q8KLane q = q8k_quant_lane(v, lane);
        const int64_t nsb = K / kQK;
        *(uint32_t*)(o8k.qs + m * K + e) = q.q4;
        if (lane == 0) o8k.d[m * nsb + s] = q.d;
        if ((lane & 3) == 0) o8k.bsums[(m * nsb + s) * 16 + (lane >> 2)] = (int16_t)q.bsum;
    } else {
        const Q81Lane q = q81_quant_lane(v);  // every lane takes part in the exchanges
        if (valid) {
            const int64_t nb = K / kQK8;
            *(uint32_t*)(o81.qs + m * K + e) = q.q4;
            if ((lane & 7) == 0) {
                o81.d[m * nb + e / kQK8] = (uint16_t)float_to_half_bits(q.d);
                o81.s[m * nb + e / kQK8] = (uint16_t)float_to_half_bits(q.s);
            }
        }
    }
}

__device__ __forceinline__ float4 silu_mul4(float4 g, float4 u) {
    return make_float4((g.x / (1.0f + expf(-g.x))) * u.x, (g.y / (1.0f + expf(-g.y))) * u.y,
                       (g.z / (1.0f + expf(-g.z))) * u.z, (g.w / (1.0f + expf(-g.w))) * u.w);
}

__device__ __forceinline__ float4 norm4(float4 x, float r, float4 g) {
    return make_float4((x.x * r) * g.x, (x.y * r) * g.y, (x.z * r) * g.z, (x.w * r) * g.w);
}

__device__ __forceinline__ float sumsq4(float ss, float4 v) {
    ss = ss + v.x * v.x;
    ss = ss + v.y * v.y;
    ss = ss + v.z * v.z;
    return ss + v.w * v.w;
}

// RMSNorm, y = (x * r) * gamma with r = 1 / sqrt(sum(x^2) / K + eps); one
// workgroup per row (A = X with row stride lda, B = gamma shared by the
// rows).  ACT 0: Q8_K output, ACT 1: Q8_1.  Wave w takes steps w, w + nw, ...
// (at most IT, about two).  Rows of up to 8 steps per wave keep x and gamma
// in registers between the sum and the output; longer rows read each step
// again where it is used (the second read hits the cache).
template <int ACT, int IT>
__global__ __launch_bounds__(1024) void rmsnorm_quant_kernel(const float* __restrict__ A,
                                                             const float* __restrict__ B, int64_t lda,
                                                             int K, float eps, float* __restrict__ Y,
                                                             int64_t ldy, ActQ8K o8k, ActQ81 o81, int vec) {
    constexpr bool kHold = IT <= 8;
    __shared__ float red[kProdWaves];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int64_t m = blockIdx.x;
    const int steps = (K + kQK - 1) / kQK;
    const bool vx = vec != 0;
    const float* a = A + m * lda;
    const float* b = B;

    float4 v[kHold ? IT : 1], gv[kHold ? IT : 1];
    float ss = 0.0f;
    if (kHold) {
        // x and gamma both requested up front: one memory latency per row
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int s = wave + nw * i;
            const int e = s * kQK + 4 * lane;
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            gv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s < steps && e < K) {
                v[i] = load4(a + e, vx);
                gv[i] = load4(b + e, vx);
            }
        }
#pragma unroll
        for (int i = 0; i < IT; ++i) ss = sumsq4(ss, v[i]);
    } else {
        for (int s = wave; s < steps; s += nw) {
            const int e = s * kQK + 4 * lane;
            if (e < K) ss = sumsq4(ss, load4(a + e, vx));
        }
    }
    // wave sum: quad, 8-lane and 16-lane exchanges (both partners of an
    // exchange form the same sum), then the four rows in order
    ss = ss + dppf<0xB1>(ss);
    ss = ss + dppf<0x4E>(ss);
    ss = ss + dppf<0x141>(ss);
    ss = ss + dppf<0x140>(ss);
    ss = ((readlane_f(ss, 0) + readlane_f(ss, 16)) + readlane_f(ss, 32)) + readlane_f(ss, 48);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < nw; ++w) tot = tot + red[w];
    const float r = 1.0f / sqrtf(tot / (float)K + eps);

    if (kHold && ACT == 0) {
        // the wave's super-blocks quantized in lockstep (their reductions overlap)
        float4 y[kHold ? IT : 1];
        Q8KLane q[kHold ? IT : 1];
#pragma unroll
        for (int i = 0; i < IT; ++i) y[i] = norm4(v[i], r, gv[i]);
        q8k_quant_lanes<kHold ? IT : 1>(y, q);
        const int64_t nsb = K / kQK;
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int s = wave + nw * i;
            if (s >= steps) break;  // wave-uniform
            const int e = s * kQK + 4 * lane;
            if (Y != nullptr) store4(Y + m * ldy + e, y[i], vx);
            *(uint32_t*)(o8k.qs + m * K + e) = q[i].q4;
            if (lane == 0) o8k.d[m * nsb + s] = q[i].d;
            if ((lane & 3) == 0) o8k.bsums[(m * nsb + s) * 16 + (lane >> 2)] = (int16_t)q[i].bsum;
        }
    } else if (kHold) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int s = wave + nw * i;
            if (s >= steps) break;  // wave-uniform
            const int e = s * kQK + 4 * lane;
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < K) y = norm4(v[i], r, gv[i]);
            emit_step<ACT>(y, s, lane, m, K, Y, ldy, o8k, o81, vx);
        }
    } else {
        for (int s = wave; s < steps; s += nw) {
            const int e = s * kQK + 4 * lane;
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < K) y = norm4(load4(a + e, vx), r, load4(b + e, vx));
            emit_step<ACT>(y, s, lane, m, K, Y, ldy, o8k, o81, vx);
        }
    }
}

// SiLU-mul, y = (g / (1 + exp(-g))) * u (G, U with row stride ldx): no row
// reduction, so one wave per 256-value step and four steps per workgroup
// (workgroup b: row b / groups, step group b % groups), like the standalone
// quantizer.
template <int ACT>
__global__ __launch_bounds__(256) void silu_mul_quant_kernel(const float* __restrict__ G,
                                                             const float* __restrict__ U, int64_t ldx, int K,
                                                             int groups, float* __restrict__ Y, int64_t ldy,
                                                             ActQ8K o8k, ActQ81 o81, int vec) {
    const int lane = threadIdx.x & 63;
    const int64_t m = blockIdx.x / groups;
    const int s = (int)(blockIdx.x - m * groups) * 4 + (threadIdx.x >> 6);
    if (s * kQK >= K) return;  // wave-uniform
    const bool vx = vec != 0;
    const int e = s * kQK + 4 * lane;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e < K) y = silu_mul4(load4(G + m * ldx + e, vx), load4(U + m * ldx + e, vx));
    emit_step<ACT>(y, s, lane, m, K, Y, ldy, o8k, o81, vx);
}

// RMSNorm of a few rows (decode): a row is split over `groups` workgroups of
// four waves, each wave emitting one step.  Every workgroup forms the row's
// sum of squares itself, over the whole row in the same partition and order
// (wave w sums steps w, w + 4, ...), so all of them derive the same r; the
// row is read from the cache after the first.
template <int ACT>
__global__ __launch_bounds__(256) void rmsnorm_quant_split_kernel(const float* __restrict__ A,
                                                                  const float* __restrict__ B, int64_t lda,
                                                                  int K, int groups, float eps,
                                                                  float* __restrict__ Y, int64_t ldy, ActQ8K o8k,
                                                                  ActQ81 o81, int vec) {
    __shared__ float red[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m = blockIdx.x / groups;
    const int so = (int)(blockIdx.x - m * groups) * 4 + wave;  // the step this wave emits
    const int steps = (K + kQK - 1) / kQK;
    const bool vx = vec != 0;
    const float* a = A + m * lda;
    const int eo = so * kQK + 4 * lane;
    float4 xo = make_float4(0.f, 0.f, 0.f, 0.f), go = xo;
    if (so < steps && eo < K) {
        xo = load4(a + eo, vx);
        go = load4(B + eo, vx);
    }
    // at most 16 steps per wave (rows of at most 64 steps): all loads in flight at once
    float4 xs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int s = wave + 4 * i;
        const int e = s * kQK + 4 * lane;
        xs[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (s < steps && e < K) xs[i] = load4(a + e, vx);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = sumsq4(ss, xs[i]);
    ss = ss + dppf<0xB1>(ss);
    ss = ss + dppf<0x4E>(ss);
    ss = ss + dppf<0x141>(ss);
    ss = ss + dppf<0x140>(ss);
    ss = ((readlane_f(ss, 0) + readlane_f(ss, 16)) + readlane_f(ss, 32)) + readlane_f(ss, 48);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float r = 1.0f / sqrtf(tot / (float)K + eps);
    if (so >= steps) return;  // wave-uniform, after the barrier
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    if (eo < K) y = norm4(xo, r, go);
    emit_step<ACT>(y, so, lane, m, K, Y, ldy, o8k, o81, vx);
}

template <int ACT>
static hipError_t launch_rmsnorm_t(int it, int nw, const float* A, const float* B, int64_t lda, int64_t M,
                                   int K, float eps, float* Y, int64_t ldy, ActQ8K o8k, ActQ81 o81, int vec,
                                   hipStream_t st) {
    const dim3 grid((unsigned)M), block((unsigned)(64 * nw));
    switch (it) {
        case 1: rmsnorm_quant_kernel<ACT, 1><<<grid, block, 0, st>>>(A, B, lda, K, eps, Y, ldy, o8k, o81, vec); break;
        case 2: rmsnorm_quant_kernel<ACT, 2><<<grid, block, 0, st>>>(A, B, lda, K, eps, Y, ldy, o8k, o81, vec); break;
        case 4: rmsnorm_quant_kernel<ACT, 4><<<grid, block, 0, st>>>(A, B, lda, K, eps, Y, ldy, o8k, o81, vec); break;
        case 8: rmsnorm_quant_kernel<ACT, 8><<<grid, block, 0, st>>>(A, B, lda, K, eps, Y, ldy, o8k, o81, vec); break;
        case 16: rmsnorm_quant_kernel<ACT, 16><<<grid, block, 0, st>>>(A, B, lda, K, eps, Y, ldy, o8k, o81, vec); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_produce_quant(int kind, int act, const float* A, const float* B, int64_t lda, int64_t M,
                                int64_t K, float eps, float* Y, int64_t ldy, ActQ8K o8k, ActQ81 o81,
                                hipStream_t st) {
    if (M == 0) return hipSuccess;
    const int steps = (int)((K + kQK - 1) / kQK);
    const int vec = ((((uintptr_t)A) | ((uintptr_t)B) | ((uintptr_t)Y)) & 15) == 0 && (lda & 3) == 0 &&
                    (Y == nullptr || (ldy & 3) == 0);
    if (kind == 0 && M <= kSplitRows && steps <= 64) {
        const int groups = (steps + 3) / 4;
        const dim3 grid((unsigned)(M * groups));
        if (act == 0)
            rmsnorm_quant_split_kernel<0><<<grid, 256, 0, st>>>(A, B, lda, (int)K, groups, eps, Y, ldy, o8k, o81, vec);
        else
            rmsnorm_quant_split_kernel<1><<<grid, 256, 0, st>>>(A, B, lda, (int)K, groups, eps, Y, ldy, o8k, o81, vec);
        return hipGetLastError();
    }
    if (kind == 0) {
        // about two steps per wave (measured 6 % faster than four at [2048, 9728],
        // even at [2048, 2560]; one step per wave no faster)
        int nw = (steps + 1) / 2;
        nw = nw < kProdWaves ? nw : kProdWaves;
        const int need = (steps + nw - 1) / nw;
        int it = 1;
        while (it < need) it <<= 1;
        if (it > 16) it = 16;  // rows past 16 x 8 steps take the re-reading path at any length
        if (act == 0) return launch_rmsnorm_t<0>(it, nw, A, B, lda, M, (int)K, eps, Y, ldy, o8k, o81, vec, st);
        return launch_rmsnorm_t<1>(it, nw, A, B, lda, M, (int)K, eps, Y, ldy, o8k, o81, vec, st);
    }
    const int groups = (steps + 3) / 4;
    if (M * groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(M * groups));
    if (act == 0)
        silu_mul_quant_kernel<0><<<grid, 256, 0, st>>>(A, B, lda, (int)K, groups, Y, ldy, o8k, o81, vec);
    else
        silu_mul_quant_kernel<1><<<grid, 256, 0, st>>>(A, B, lda, (int)K, groups, Y, ldy, o8k, o81, vec);
    return hipGetLastError();
}

}  // namespace vqk
