// quant.hip -- activation quantizers (Q8_K, Q8_1) and weight encoders
// (Q4_K, Q5_K, Q6_K, Q8_0) for gfx950.
//
// Activation quantizers: HBM-bound elementwise passes (read 4 B, write about
// 1.14 B per value); one wave per Q8_K super-block, eight lanes per Q8_1
// block, fully coalesced dword/dwordx4 traffic.  The quantizer arithmetic is
// the shared body in vq_device.h.
//
// Weight encoders are data preparation (the matmuls only read block bytes):
// the plainest min/max scale fit of each format, all in binary32 with no FMA
// contraction, d and dmin rounded to binary16 before the sub-block scales are
// fitted against them.
#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

// ---------------------------------------------------------------------------
// Q8_K: one wave per super-block.
// ---------------------------------------------------------------------------
template <bool kVec>
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float* __restrict__ X, int64_t M,
                                                           int64_t K, int64_t ldx, ActQ8K out) {
    const int lane = threadIdx.x & 63;
    const int64_t nb = K / kQK;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= M * nb) return;
    const int64_t m = blk / nb, b = blk % nb;
    const float* src = X + m * ldx + b * kQK + 4 * lane;
    float4 v;
    if (kVec) {
        v = *(const float4*)src;
    } else {
        v = make_float4(src[0], src[1], src[2], src[3]);
    }
    Q8KLane r = q8k_quant_lane(v, lane);
    *(uint32_t*)(out.qs + m * K + b * kQK + 4 * lane) = r.q4;
    if (lane == 0) out.d[m * nb + b] = r.d;
    if ((lane & 3) == 0) out.bsums[(m * nb + b) * 16 + (lane >> 2)] = (int16_t)r.bsum;
}

hipError_t launch_quantize_q8k(const float* X, int64_t M, int64_t K, int64_t ldx, ActQ8K out,
                               hipStream_t st) {
    const int64_t blocks = M * (K / kQK);
    if (blocks == 0) return hipSuccess;
    dim3 grid((unsigned)((blocks + 3) / 4));
    bool vec = (((uintptr_t)X) & 15) == 0 && (ldx & 3) == 0;
    if (vec)
        quantize_q8k_kernel<true><<<grid, 256, 0, st>>>(X, M, K, ldx, out);
    else
        quantize_q8k_kernel<false><<<grid, 256, 0, st>>>(X, M, K, ldx, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q8_1: eight lanes per 32-block, eight blocks per wave.
// ---------------------------------------------------------------------------
template <bool kVec>
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float* __restrict__ X, int64_t M,
                                                            int64_t K, int64_t ldx, ActQ81 out) {
    const int lane = threadIdx.x & 63;
    const int64_t nb = K / kQK8;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t blk = wave * 8 + (lane >> 3);
    const bool valid = blk < M * nb;
    const int64_t bb = valid ? blk : 0;
    const int64_t m = bb / nb, b = bb % nb;
    const float* src = X + m * ldx + b * kQK8 + 4 * (lane & 7);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
        if (kVec) v = *(const float4*)src;
        else v = make_float4(src[0], src[1], src[2], src[3]);
    }
    Q81Lane r = q81_quant_lane(v);  // all lanes take part in the exchanges
    if (!valid) return;
    *(uint32_t*)(out.qs + m * K + b * kQK8 + 4 * (lane & 7)) = r.q4;
    if ((lane & 7) == 0) {
        out.d[m * nb + b] = (uint16_t)float_to_half_bits(r.d);
        out.s[m * nb + b] = (uint16_t)float_to_half_bits(r.s);
    }
}

hipError_t launch_quantize_q8_1(const float* X, int64_t M, int64_t K, int64_t ldx, ActQ81 out,
                                hipStream_t st) {
    const int64_t blocks = M * (K / kQK8);
    if (blocks == 0) return hipSuccess;
    const int64_t waves = (blocks + 7) / 8;
    dim3 grid((unsigned)((waves + 3) / 4));
    bool vec = (((uintptr_t)X) & 15) == 0 && (ldx & 3) == 0;
    if (vec)
        quantize_q8_1_kernel<true><<<grid, 256, 0, st>>>(X, M, K, ldx, out);
    else
        quantize_q8_1_kernel<false><<<grid, 256, 0, st>>>(X, M, K, ldx, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight encoders.
// ---------------------------------------------------------------------------

// Max that keeps the value of the lower lane on ties, reduced over lane
// distances o0 <= o < o1: the same value as a sequential scan that starts
// from the first element and replaces only on a strictly larger value.
__device__ __forceinline__ float ordered_max(float v, int lane, int o0, int o1) {
    for (int o = o0; o < o1; o <<= 1) {
        float other = shfl_xor_f(v, o);
        bool i_am_lower = (lane & o) == 0;
        if (i_am_lower) v = (other > v) ? other : v;
        else v = (v > other) ? v : other;
    }
    return v;
}

__device__ __forceinline__ int clamp_rint(float x, int lo, int hi) {
    int q = (int)__builtin_rintf(x);
    return q < lo ? lo : (q > hi ? hi : q);
}

// Q4_K (QMAX 15) and Q5_K (QMAX 31): one wave per super-block; lane l holds
// values 4l..4l+3 (sub-block l/8).  Q5_K is the Q4_K block with the nibbles
// moved 32 bytes up and a plane of fifth bits in between.
template <int QMAX>
__global__ __launch_bounds__(256) void encode_q4k_kernel(const float* __restrict__ W, int64_t N,
                                                         int64_t K, uint8_t* __restrict__ out) {
    constexpr int kBytes = (QMAX == 15) ? kQ4KBytes : kQ5KBytes;
    constexpr int kQsOff = (QMAX == 15) ? 16 : 48;
    const int lane = threadIdx.x & 63;
    const int64_t nb = K / kQK;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= N * nb) return;
    const int64_t n = blk / nb, b = blk % nb;
    const float4 v = *(const float4*)(W + n * K + b * kQK + 4 * lane);
    const float w[4] = {v.x, v.y, v.z, v.w};
    // sub-block minimum (only values below +0 count) and ordered maximum
    float mn = fminf(fminf(w[0], w[1]), fminf(w[2], w[3]));
    for (int o = 1; o < 8; o <<= 1) mn = fminf(mn, shfl_xor_f(mn, o));
    const float lo = (mn < 0.0f) ? mn : 0.0f;
    float hi = w[0];
    for (int i = 1; i < 4; ++i) hi = (w[i] > hi) ? w[i] : hi;
    hi = ordered_max(hi, lane, 1, 8);
    const float span = hi - lo;
    const float s = span / (float)QMAX;
    const float o_ = -lo;
    const float maxs = ordered_max(s, lane, 8, 64);
    const float maxo = ordered_max(o_, lane, 8, 64);
    const uint32_t d16 = float_to_half_bits(maxs / 63.0f);
    const uint32_t dmin16 = float_to_half_bits(maxo / 63.0f);
    const float d = half_bits_to_float(d16), dmin = half_bits_to_float(dmin16);
    const int sc = (d != 0.0f) ? clamp_rint(s / d, 0, 63) : 0;
    const int mm = (dmin != 0.0f) ? clamp_rint(o_ / dmin, 0, 63) : 0;
    const float off = dmin * (float)mm;
    const float div = d * (float)sc;
    uint32_t q4 = 0;
    for (int i = 0; i < 4; ++i) {
        int q = 0;
        if (div != 0.0f) {
            float num = w[i] + off;
            q = clamp_rint(num / div, 0, QMAX);
        }
        q4 |= (uint32_t)q << (8 * i);
    }
    uint8_t* blkp = out + (n * nb + b) * kBytes;
    // nibbles: byte 32c + l holds element 64c+l (low) and 64c+32+l (high);
    // element 64c+32+l lives 8 lanes above element 64c+l.
    const uint32_t hi4 = (uint32_t)shfl_xor_i((int)q4, 8);
    if (((lane >> 3) & 1) == 0) {
        const int c = lane >> 4, u = lane & 7;
        *(uint32_t*)(blkp + kQsOff + 32 * c + 4 * u) = (q4 & 0x0F0F0F0Fu) | ((hi4 & 0x0F0F0F0Fu) << 4);
    }
    if (QMAX == 31) {
        // fifth bits: bit j of byte 16 + l is bit 4 of element 32j + l; lane
        // 8j + u holds elements 32j + 4u .. 32j + 4u + 3, i.e. bit j of bytes
        // 16 + 4u .. 16 + 4u + 3; the eight lanes u, u + 8, ... are OR-ed.
        uint32_t hb = ((q4 >> 4) & 0x01010101u) << (lane >> 3);
        hb |= (uint32_t)shfl_xor_i((int)hb, 8);
        hb |= (uint32_t)shfl_xor_i((int)hb, 16);
        hb |= (uint32_t)shfl_xor_i((int)hb, 32);
        if (lane < 8) *(uint32_t*)(blkp + 16 + 4 * lane) = hb;
    }
    // header: d, dmin, 12 bytes of 6-bit scales and mins
    int scj[8], mj[8];
    for (int j = 0; j < 8; ++j) {
        scj[j] = shfl_i(sc, 8 * j);
        mj[j] = shfl_i(mm, 8 * j);
    }
    if (lane == 0) {
        uint8_t sb[12];
        for (int j = 0; j < 12; ++j) sb[j] = 0;
        for (int j = 0; j < 8; ++j) {
            sb[j] = (uint8_t)((scj[j] & 63) | ((mj[j] & 3) << 6));
            sb[8 + (j >> 1)] |= (uint8_t)(((mj[j] >> 2) & 15) << (4 * (j & 1)));
        }
        uint32_t h0 = d16 | (dmin16 << 16);
        uint32_t h1 = sb[0] | (sb[1] << 8) | (sb[2] << 16) | ((uint32_t)sb[3] << 24);
        uint32_t h2 = sb[4] | (sb[5] << 8) | (sb[6] << 16) | ((uint32_t)sb[7] << 24);
        uint32_t h3 = sb[8] | (sb[9] << 8) | (sb[10] << 16) | ((uint32_t)sb[11] << 24);
        *(uint4*)blkp = make_uint4(h0, h1, h2, h3);
    }
}

// Q6_K: one wave per super-block; lane l holds values 4l..4l+3 (sub-block l/4).
// The 210-byte blocks are only 2-byte aligned, so every store is 16-bit.
__global__ __launch_bounds__(256) void encode_q6k_kernel(const float* __restrict__ W, int64_t N,
                                                         int64_t K, uint8_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t nb = K / kQK;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= N * nb) return;
    const int64_t n = blk / nb, b = blk % nb;
    const float4 v = *(const float4*)(W + n * K + b * kQK + 4 * lane);
    const float w[4] = {v.x, v.y, v.z, v.w};
    float amax = 0.0f;
    for (int i = 0; i < 4; ++i) {
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    for (int o = 1; o < 4; o <<= 1) {
        float t = shfl_xor_f(amax, o);
        if (t > amax) amax = t;
    }
    const float s = amax / 31.0f;
    const float maxs = ordered_max(s, lane, 4, 64);
    const uint32_t d16 = float_to_half_bits(maxs / 127.0f);
    const float d = half_bits_to_float(d16);
    const int sc = (d != 0.0f) ? clamp_rint(s / d, 0, 127) : 0;
    const float div = d * (float)sc;
    int q[4];
    for (int i = 0; i < 4; ++i) {
        int t = 0;
        if (div != 0.0f) t = clamp_rint(w[i] / div, -32, 31);
        q[i] = t + 32;
    }
    const uint32_t q4 = q[0] | (q[1] << 8) | (q[2] << 16) | ((uint32_t)q[3] << 24);
    const uint32_t p8 = (uint32_t)shfl_xor_i((int)q4, 8);
    const uint32_t p16 = (uint32_t)shfl_xor_i((int)q4, 16);
    const uint32_t p24 = (uint32_t)shfl_xor_i((int)q4, 24);
    uint8_t* blkp = out + (n * nb + b) * kQ6KBytes;
    const int h = lane >> 5, u = lane & 31;
    uint16_t* p16s = (uint16_t*)blkp;  // 2-byte aligned block
    if (u < 16) {
        // ql byte 64h + r: low nibble = element r, high = element r+64 (16 lanes up)
        const uint32_t ql = (q4 & 0x0F0F0F0Fu) | ((p16 & 0x0F0F0F0Fu) << 4);
        const int off = 64 * h + 4 * u;
        p16s[off / 2] = (uint16_t)(ql & 0xFFFF);
        p16s[off / 2 + 1] = (uint16_t)(ql >> 16);
    }
    if (u < 8) {
        // qh byte 32h + r: bit pairs of elements r, r+32, r+64, r+96
        const uint32_t qh = ((q4 >> 4) & 0x03030303u) | (((p8 >> 4) & 0x03030303u) << 2) |
                            (((p16 >> 4) & 0x03030303u) << 4) | (((p24 >> 4) & 0x03030303u) << 6);
        const int off = 128 + 32 * h + 4 * u;
        p16s[off / 2] = (uint16_t)(qh & 0xFFFF);
        p16s[off / 2 + 1] = (uint16_t)(qh >> 16);
    }
    int scj[16];
    for (int j = 0; j < 16; ++j) scj[j] = shfl_i(sc, 4 * j);
    if (lane == 0) {
        for (int j = 0; j < 8; ++j)
            p16s[96 + j] = (uint16_t)((scj[2 * j] & 0xFF) | ((scj[2 * j + 1] & 0xFF) << 8));
        p16s[104] = (uint16_t)d16;
    }
}

// Q8_0: eight lanes per 32-block.
__global__ __launch_bounds__(256) void encode_q8_0_kernel(const float* __restrict__ W, int64_t N,
                                                          int64_t K, uint8_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t nb = K / kQK8;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t blk = wave * 8 + (lane >> 3);
    const bool valid = blk < N * nb;
    const int64_t bb = valid ? blk : 0;
    const int64_t n = bb / nb, b = bb % nb;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *(const float4*)(W + n * K + b * kQK8 + 4 * (lane & 7));
    const float w[4] = {v.x, v.y, v.z, v.w};
    float amax = 0.0f;
    for (int i = 0; i < 4; ++i) {
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    for (int o = 1; o < 8; o <<= 1) {
        float t = shfl_xor_f(amax, o);
        if (t > amax) amax = t;
    }
    if (!valid) return;
    const float d = amax / 127.0f;
    uint32_t q4 = 0;
    for (int i = 0; i < 4; ++i) {
        int q = 0;
        if (amax != 0.0f) {
            q = (int)roundf(w[i] / d);
            q = q < -127 ? -127 : (q > 127 ? 127 : q);
        }
        q4 |= (uint32_t)(q & 0xFF) << (8 * i);
    }
    uint16_t* p = (uint16_t*)(out + (n * nb + b) * kQ80Bytes);
    const int u = lane & 7;
    p[1 + 2 * u] = (uint16_t)(q4 & 0xFFFF);
    p[2 + 2 * u] = (uint16_t)(q4 >> 16);
    if (u == 0) p[0] = (uint16_t)float_to_half_bits(d);
}

hipError_t launch_quantize_weights(int wtype, const float* W, int64_t N, int64_t K, uint8_t* out,
                                   hipStream_t st) {
    if (wtype == 0 || wtype == 1 || wtype == 5) {
        const int64_t blocks = N * (K / kQK);
        if (blocks == 0) return hipSuccess;
        dim3 grid((unsigned)((blocks + 3) / 4));
        if (wtype == 0)
            encode_q4k_kernel<15><<<grid, 256, 0, st>>>(W, N, K, out);
        else if (wtype == 5)
            encode_q4k_kernel<31><<<grid, 256, 0, st>>>(W, N, K, out);
        else
            encode_q6k_kernel<<<grid, 256, 0, st>>>(W, N, K, out);
    } else {
        const int64_t blocks = N * (K / kQK8);
        if (blocks == 0) return hipSuccess;
        const int64_t waves = (blocks + 7) / 8;
        dim3 grid((unsigned)((waves + 3) / 4));
        encode_q8_0_kernel<<<grid, 256, 0, st>>>(W, N, K, out);
    }
    return hipGetLastError();
}

}  // namespace vqk
