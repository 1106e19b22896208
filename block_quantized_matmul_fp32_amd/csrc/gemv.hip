// gemv.hip -- decode GEMV (M = 1) for Q4_K / Q6_K weights x Q8_K and Q8_0
// weights x Q8_1, with the activation quantizer fused into the prologue.
//
// Pages: vllm.cpp PR #2890, commit "T4a VT_GEMV_MMVQ" (the K-quant decode
// GEMV folds the activation quantizer into its prologue, bit-exact against
// the CPU oracle); strix-llama.cpp PR #18, commit "mul_mat_vec_q_fq" (a
// block quantizes the activation once into shared memory, with weight loads
// issued before the quantization and its barrier) and commit "batch-one MMVQ
// on one wave" (a fixed fp32 reduction order keeps decode deterministic).
//
// MI355X design.  The GEMV is HBM-bound: ~14-20 MB of weights, 1.8-2.6 us at
// 8 TB/s, i.e. about one DRAM round trip's worth of bytes per CU.  So:
//  * one 1024-thread workgroup per CU owns a contiguous run of rows; its
//    weight bytes form one contiguous slab that is fetched with aligned
//    16-byte loads, every load of the workgroup issued before anything is
//    consumed (all bytes in flight at once);
//  * while those loads are in flight the 16 waves quantize x into LDS with the
//    shared quantizer body (one wave per Q8_K super-block);
//  * the slab is parked in LDS (Q6_K and Q8_0 blocks are only 2-byte aligned;
//    LDS reads at that alignment are rebuilt with v_alignbyte);
//  * eight lanes own one (row, super-block): exact int32 sub-block sums with
//    v_dot4_i32_i8, an exact int reduction over the eight lanes, then the
//    block's binary32 combine; blocks of a row are summed in ascending order,
//    so y is bit-identical to the fixed-order definition.
#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

constexpr int kGemvThreads = 1024;
constexpr int kGemvChunks = 8;  // 16-byte chunks per thread: slab <= 128 KiB
constexpr size_t kMaxLds = 160 * 1024;

template <int WT>
struct WFmt;
template <>
struct WFmt<0> { static constexpr int kBlk = kQ4KBytes; static constexpr int kVals = kQK; };
template <>
struct WFmt<1> { static constexpr int kBlk = kQ6KBytes; static constexpr int kVals = kQK; };
template <>
struct WFmt<2> { static constexpr int kBlk = kQ80Bytes; static constexpr int kVals = kQK8; };

struct GemvLayout {
    int act_qs, act_d, act_bs, partial, slab, total;
};

__host__ __device__ inline int align16i(int x) { return (x + 15) & ~15; }

// LDS layout of the GEMV workgroup; identical on host and device.
__host__ __device__ inline GemvLayout gemv_layout(int wt, int K, int rows, int rb) {
    GemvLayout L;
    const int nbw = (wt == 2) ? K / kQK8 : K / kQK;
    L.act_qs = 0;
    L.act_d = align16i(K);
    const int nd = (wt == 2) ? K / kQK8 : K / kQK;
    L.act_bs = L.act_d + align16i(nd * 4);
    const int nbs = (wt == 2) ? 0 : K / 16;
    L.partial = L.act_bs + align16i(nbs * 2);
    L.slab = L.partial + align16i(rows * nbw * 4);
    L.total = L.slab + rows * rb + 48;
    return L;
}

template <int WT>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint8_t* __restrict__ W, int N, int K, int64_t wbytes, const float* __restrict__ x,
    float* __restrict__ y, uint8_t* __restrict__ xq_out, int rows_per_wg, int x_vec) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int BB = WFmt<WT>::kBlk;
    constexpr int QV = WFmt<WT>::kVals;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb = K / QV;
    const int rb = nb * BB;
    const int n0 = blockIdx.x * rows_per_wg;
    const int rows = min(rows_per_wg, N - n0);
    const GemvLayout L = gemv_layout(WT, K, rows_per_wg, rb);

    // 1. Issue every weight load of this workgroup (aligned 16-byte chunks of
    //    the contiguous row slab; the buffer's last partial chunk bytewise).
    const int64_t s0 = (int64_t)n0 * rb, s1 = (int64_t)(n0 + rows) * rb;
    const int64_t c0 = s0 >> 4, c1 = (s1 + 15) >> 4;
    const int64_t full = wbytes >> 4;
    uint4 buf[kGemvChunks];
#pragma unroll
    for (int i = 0; i < kGemvChunks; ++i) {
        const int64_t c = c0 + tid + (int64_t)i * kGemvThreads;
        buf[i] = make_uint4(0, 0, 0, 0);
        if (c < c1) {
            if (c < full) {
                buf[i] = *(const uint4*)(W + 16 * c);
            } else {
                uint32_t wv[4] = {0, 0, 0, 0};
                for (int bi = 0; bi < 16; ++bi) {
                    const int64_t a = 16 * c + bi;
                    if (a < wbytes) wv[bi >> 2] |= (uint32_t)W[a] << (8 * (bi & 3));
                }
                buf[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
    }

    // 2. Quantize x into LDS while the weight loads are in flight.
    int8_t* act_qs = (int8_t*)(smem + L.act_qs);
    float* act_d = (float*)(smem + L.act_d);
    int16_t* act_bs = (int16_t*)(smem + L.act_bs);
    const bool dump = (xq_out != nullptr) && blockIdx.x == 0;
    if (WT != 2) {
        const int nsb = K / kQK;
        int8_t* gq = (int8_t*)xq_out;
        float* gd = (float*)(xq_out + align256((size_t)K));
        int16_t* gb = (int16_t*)(xq_out + align256((size_t)K) + align256((size_t)nsb * 4));
        for (int sb = wave; sb < nsb; sb += kGemvThreads / 64) {
            const float* src = x + sb * kQK + 4 * lane;
            float4 v = x_vec ? *(const float4*)src : make_float4(src[0], src[1], src[2], src[3]);
            Q8KLane r = q8k_quant_lane(v, lane);
            *(uint32_t*)(act_qs + sb * kQK + 4 * lane) = r.q4;
            if (lane == 0) act_d[sb] = r.d;
            if ((lane & 3) == 0) act_bs[sb * 16 + (lane >> 2)] = (int16_t)r.bsum;
            if (dump) {
                *(uint32_t*)(gq + sb * kQK + 4 * lane) = r.q4;
                if (lane == 0) gd[sb] = r.d;
                if ((lane & 3) == 0) gb[sb * 16 + (lane >> 2)] = (int16_t)r.bsum;
            }
        }
    } else {
        const int nblk = K / kQK8;
        int8_t* gq = (int8_t*)xq_out;
        uint16_t* gd = (uint16_t*)(xq_out + align256((size_t)K));
        uint16_t* gs = (uint16_t*)(xq_out + align256((size_t)K) + align256((size_t)nblk * 2));
        const int steps = (K + kQK - 1) / kQK;
        for (int st = wave; st < steps; st += kGemvThreads / 64) {
            const int e = st * kQK + 4 * lane;
            const bool valid = e < K;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) {
                const float* src = x + e;
                v = x_vec ? *(const float4*)src : make_float4(src[0], src[1], src[2], src[3]);
            }
            Q81Lane r = q81_quant_lane(v);
            if (valid) {
                const int blk = e / kQK8;
                *(uint32_t*)(act_qs + e) = r.q4;
                const uint32_t d16 = float_to_half_bits(r.d);
                if ((lane & 7) == 0) act_d[blk] = half_bits_to_float(d16);
                if (dump) {
                    *(uint32_t*)(gq + e) = r.q4;
                    if ((lane & 7) == 0) {
                        gd[blk] = (uint16_t)d16;
                        gs[blk] = (uint16_t)float_to_half_bits(r.s);
                    }
                }
            }
        }
    }

    // 3. Park the weight slab in LDS.
    uint8_t* slab = smem + L.slab;
#pragma unroll
    for (int i = 0; i < kGemvChunks; ++i) {
        const int64_t c = c0 + tid + (int64_t)i * kGemvThreads;
        if (c < c1) *(uint4*)(slab + 16 * (c - c0)) = buf[i];
    }
    __syncthreads();

    // 4. Per (row, block) partials.
    float* partial = (float*)(smem + L.partial);
    const int soff = (int)(s0 - 16 * c0);
    const int ntask = rows * nb;
    if (WT == 0) {
        const int g = tid & 7;
        const int c = g >> 1, l0 = (g & 1) * 16;
        for (int t = tid >> 3; t < ntask; t += kGemvThreads / 8) {
            const int r = t / nb, blk = t - r * nb;
            const uint8_t* bp = slab + soff + r * rb + blk * BB;
            const uint4 hdr = *(const uint4*)bp;
            const uint4 qv = *(const uint4*)(bp + 16 + 16 * g);
            const int8_t* ab = act_qs + blk * kQK + 64 * c + l0;
            const uint4 alo = *(const uint4*)ab;
            const uint4 ahi = *(const uint4*)(ab + 32);
            const uint32_t sword = (c < 2) ? hdr.y : hdr.z;
            const uint32_t s_lo = (sword >> (16 * (c & 1))) & 0xFF;
            const uint32_t s_hi = (sword >> (16 * (c & 1) + 8)) & 0xFF;
            const uint32_t mb = (hdr.w >> (8 * c)) & 0xFF;
            const int sc0 = s_lo & 63, sc1 = s_hi & 63;
            const int m0 = (int)((s_lo >> 6) | ((mb & 15) << 2));
            const int m1 = (int)((s_hi >> 6) | ((mb >> 4) << 2));
            int plo = 0, phi = 0;
            plo = sdot4((int)(qv.x & 0x0F0F0F0Fu), (int)alo.x, plo);
            plo = sdot4((int)(qv.y & 0x0F0F0F0Fu), (int)alo.y, plo);
            plo = sdot4((int)(qv.z & 0x0F0F0F0Fu), (int)alo.z, plo);
            plo = sdot4((int)(qv.w & 0x0F0F0F0Fu), (int)alo.w, plo);
            phi = sdot4((int)((qv.x >> 4) & 0x0F0F0F0Fu), (int)ahi.x, phi);
            phi = sdot4((int)((qv.y >> 4) & 0x0F0F0F0Fu), (int)ahi.y, phi);
            phi = sdot4((int)((qv.z >> 4) & 0x0F0F0F0Fu), (int)ahi.z, phi);
            phi = sdot4((int)((qv.w >> 4) & 0x0F0F0F0Fu), (int)ahi.w, phi);
            int S = sc0 * plo + sc1 * phi;
            int Mn = 0;
            if ((g & 1) == 0) {
                const int16_t* bs = act_bs + blk * 16 + 4 * c;
                Mn = m0 * ((int)bs[0] + (int)bs[1]) + m1 * ((int)bs[2] + (int)bs[3]);
            }
            S += shfl_xor_i(S, 1); Mn += shfl_xor_i(Mn, 1);
            S += shfl_xor_i(S, 2); Mn += shfl_xor_i(Mn, 2);
            S += shfl_xor_i(S, 4); Mn += shfl_xor_i(Mn, 4);
            if (g == 0) {
                const float d = half_bits_to_float(hdr.x & 0xFFFF);
                const float dmin = half_bits_to_float(hdr.x >> 16);
                const float t1 = d * (float)S;
                const float t2 = dmin * (float)Mn;
                const float t3 = t1 - t2;
                partial[r * nb + blk] = act_d[blk] * t3;
            }
        }
    } else if (WT == 1) {
        const int g = tid & 7;
        const int h = g >> 2, k = g & 3;
        const int sha = 2 * (k >> 1), shb = 2 * (2 + (k >> 1));
        for (int t = tid >> 3; t < ntask; t += kGemvThreads / 8) {
            const int r = t / nb, blk = t - r * nb;
            const uint8_t* bp = slab + soff + r * rb + blk * BB;
            uint32_t ql[4], qh[4];
            lds_read16_a2(bp + 64 * h + 16 * k, ql);
            lds_read16_a2(bp + 128 + 32 * h + 16 * (k & 1), qh);
            const int sca = (int)(int8_t)bp[192 + 8 * h + k];
            const int scb = (int)(int8_t)bp[192 + 8 * h + 4 + k];
            const int8_t* ab = act_qs + blk * kQK + 128 * h + 16 * k;
            const uint4 alo = *(const uint4*)ab;
            const uint4 ahi = *(const uint4*)(ab + 64);
            const uint32_t al[4] = {alo.x, alo.y, alo.z, alo.w};
            const uint32_t ah[4] = {ahi.x, ahi.y, ahi.z, ahi.w};
            int ia = 0, ib = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t qa = (ql[i] & 0x0F0F0F0Fu) | (((qh[i] >> sha) & 0x03030303u) << 4);
                const uint32_t qb = ((ql[i] >> 4) & 0x0F0F0F0Fu) | (((qh[i] >> shb) & 0x03030303u) << 4);
                ia = sdot4((int)qa, (int)al[i], ia);
                ib = sdot4((int)qb, (int)ah[i], ib);
            }
            const int16_t* bs = act_bs + blk * 16 + 8 * h + k;
            ia -= 32 * (int)bs[0];
            ib -= 32 * (int)bs[4];
            int S = sca * ia + scb * ib;
            S += shfl_xor_i(S, 1);
            S += shfl_xor_i(S, 2);
            S += shfl_xor_i(S, 4);
            if (g == 0) {
                const float d = half_bits_to_float(*(const uint16_t*)(bp + 208));
                const float t1 = d * (float)S;
                partial[r * nb + blk] = act_d[blk] * t1;
            }
        }
    } else {
        for (int t = tid; t < ntask; t += kGemvThreads) {
            const int r = t / nb, blk = t - r * nb;
            const uint8_t* bp = slab + soff + r * rb + blk * BB;
            uint32_t q0[4], q1[4];
            lds_read16_a2(bp + 2, q0);
            lds_read16_a2(bp + 18, q1);
            const uint4 a0 = *(const uint4*)(act_qs + blk * kQK8);
            const uint4 a1 = *(const uint4*)(act_qs + blk * kQK8 + 16);
            int I = 0;
            I = sdot4((int)q0[0], (int)a0.x, I);
            I = sdot4((int)q0[1], (int)a0.y, I);
            I = sdot4((int)q0[2], (int)a0.z, I);
            I = sdot4((int)q0[3], (int)a0.w, I);
            I = sdot4((int)q1[0], (int)a1.x, I);
            I = sdot4((int)q1[1], (int)a1.y, I);
            I = sdot4((int)q1[2], (int)a1.z, I);
            I = sdot4((int)q1[3], (int)a1.w, I);
            const float dw = half_bits_to_float(*(const uint16_t*)bp);
            const float s = dw * act_d[blk];
            partial[r * nb + blk] = s * (float)I;
        }
    }
    __syncthreads();

    // 5. Rows: blocks summed in ascending order from 0.
    for (int r = tid; r < rows; r += kGemvThreads) {
        float acc = 0.0f;
        const float* p = partial + r * nb;
        for (int b = 0; b < nb; ++b) acc = acc + p[b];
        y[n0 + r] = acc;
    }
}

static int g_num_cus = 0;

static int num_cus() {
    if (g_num_cus == 0) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        g_num_cus = v;
    }
    return g_num_cus;
}

static int block_bytes_of(int wt) { return wt == 0 ? kQ4KBytes : (wt == 1 ? kQ6KBytes : kQ80Bytes); }
static int block_vals_of(int wt) { return wt == 2 ? kQK8 : kQK; }

// Rows per workgroup: about one workgroup per CU, fewer rows when the slab
// would not fit the per-thread chunk budget or LDS.
static int gemv_rows_per_wg(int wt, int64_t N, int64_t K) {
    const int rb = (int)(K / block_vals_of(wt)) * block_bytes_of(wt);
    int rows = (int)((N + num_cus() - 1) / num_cus());
    if (rows < 1) rows = 1;
    const int max_slab = kGemvChunks * kGemvThreads * 16 - 48;
    while (rows > 1 && (rows * rb > max_slab ||
                        (size_t)gemv_layout(wt, (int)K, rows, rb).total > kMaxLds))
        --rows;
    return rows;
}

size_t gemv_lds_bytes(int wtype, int64_t N, int64_t K) {
    const int rb = (int)(K / block_vals_of(wtype)) * block_bytes_of(wtype);
    const int rows = gemv_rows_per_wg(wtype, N, K);
    if ((int64_t)rb > (int64_t)kGemvChunks * kGemvThreads * 16 - 48) return (size_t)-1;
    return (size_t)gemv_layout(wtype, (int)K, rows, rb).total;
}

template <int WT>
static hipError_t launch_gemv_t(const uint8_t* W, int64_t N, int64_t K, const float* x, float* y,
                                uint8_t* xq_out, hipStream_t st) {
    static bool attr_set = false;
    const int rb = (int)(K / WFmt<WT>::kVals) * WFmt<WT>::kBlk;
    const int rows = gemv_rows_per_wg(WT, N, K);
    const int lds = gemv_layout(WT, (int)K, rows, rb).total;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemv_kernel<WT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int grid = (int)((N + rows - 1) / rows);
    const int x_vec = (((uintptr_t)x) & 15) == 0;
    gemv_kernel<WT><<<grid, kGemvThreads, lds, st>>>(W, (int)N, (int)K, (int64_t)N * rb, x, y,
                                                     xq_out, rows, x_vec);
    return hipGetLastError();
}

hipError_t launch_gemv(int wtype, const uint8_t* W, int64_t N, int64_t K, const float* x, float* y,
                       uint8_t* xq_out, hipStream_t st) {
    if (N == 0) return hipSuccess;
    if (wtype == 0) return launch_gemv_t<0>(W, N, K, x, y, xq_out, st);
    if (wtype == 1) return launch_gemv_t<1>(W, N, K, x, y, xq_out, st);
    return launch_gemv_t<2>(W, N, K, x, y, xq_out, st);
}

}  // namespace vqk
