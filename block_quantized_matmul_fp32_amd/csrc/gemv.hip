// gemv.hip -- decode GEMV (M = 1) for Q4_K / Q6_K weights x Q8_K and Q8_0
// weights x Q8_1, with the activation quantizer fused into the prologue.
//
// Pages: vllm.cpp PR #2890, commit "T4a VT_GEMV_MMVQ" (the K-quant decode
// GEMV folds the activation quantizer into its prologue, bit-exact against
// the CPU oracle); strix-llama.cpp PR #18, commit "mul_mat_vec_q_fq" (a
// block quantizes the activation once into shared memory, with weight loads
// issued before the quantization and its barrier), commit "warp reduce via
// DPP" (lane exchange without LDS round trips) and the overview commit that
// keeps batch-one MMVQ in a fixed fp32 reduction order (deterministic decode).
//
// MI355X design.  The GEMV streams 9-20 MB of weights: a few microseconds of
// HBM time, so everything else has to hide under the stream.  A CU's share of
// the stream is ~17 KB/us and a wave that issues weight loads stalls in issue
// until earlier misses return, so the waves of a workgroup take two roles:
//  * One workgroup per CU owns a contiguous run of rows; its (row, block)
//    tasks split into a first part and a last part of at most one full pass
//    per SIMD.
//  * Loader waves (one per SIMD) copy the workgroup's whole weight slice
//    straight into LDS with global_load_lds_dwordx4 (no registers, no parking
//    step), first part then last part, a fixed number of 1 KiB instructions
//    per wave per part so that a vmcnt wait can tell the parts apart.
//  * Quantizer waves issue no weight load: they load x, quantize it into LDS
//    with the shared quantizer body (DPP reductions), then -- once the first
//    part has landed -- compute it while the last part streams in; the
//    loader waves compute the last part after it lands, so only that one pass
//    follows the end of the stream.
//  * Two lanes own one (row, super-block) -- one lane per Q8_0 block: exact
//    int32 sub-block sums with v_dot4_i32_i8, a DPP exchange of the halves,
//    then the block's binary32 combine into an LDS partial.
//  * After the last barrier, one lane per row adds the row's partials in
//    ascending block order from 0, so y is bit-identical to the fixed-order
//    definition.
#include <atomic>

#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

constexpr int kGemvThreads = 1024;              // most threads per workgroup
constexpr int kGemvWaves = kGemvThreads / 64;   // most waves per workgroup
constexpr int kNonTemporal = 2;     // cache-policy operand of the weight DMA: nt
constexpr int kGroupMB = 4;         // rows per group when a small batch runs in several groups
constexpr int kXPre = 8;            // x rounds (256 values each) loaded up front per quantizer wave
constexpr int kMaxHalfInstr = 31;   // 1 KiB load instructions per loader wave per half (vmcnt <= 63)
constexpr size_t kMaxLds = 160 * 1024;
constexpr size_t kStaticLds = 64;   // the kernel's static LDS (the loaders' counter), rounded up
// LDS bytes per quantized super-block of x: 256 + 16, so the 16 tasks of a
// wave round (consecutive super-blocks) start on 16 different bank groups.
constexpr int kActStride = kQK + 16;

template <int WT>
struct WFmt;
template <>
struct WFmt<0> { static constexpr int kBlk = kQ4KBytes; static constexpr int kVals = kQK; };
template <>
struct WFmt<1> { static constexpr int kBlk = kQ6KBytes; static constexpr int kVals = kQK; };
template <>
struct WFmt<2> { static constexpr int kBlk = kQ80Bytes; static constexpr int kVals = kQK8; };
template <>
struct WFmt<3> { static constexpr int kBlk = kQ5KBytes; static constexpr int kVals = kQK; };

struct GemvLayout {
    int act_qs, act_row, act_d, act_bs, partial, wslice, slice_bytes, total;
};

__host__ __device__ inline int align16i(int x) { return (x + 15) & ~15; }

// LDS layout of the GEMV workgroup for mb activation rows; identical on host
// and device.  Per activation row: the quantized bytes (act_row bytes), the
// block scales (K/QK floats) and the Q8_K sub-block sums (K/16 int16) or the
// Q8_1 packed d | s words (K/32).  The weight slice region holds the slice's
// 16-byte chunks, 1 KiB past the slice for the last instruction's lanes
// beyond it, 1 KiB for padding instructions, and over-read slack.
__host__ __device__ inline GemvLayout gemv_layout(int wt, int K, int rows, int slice_bytes, int mb) {
    GemvLayout L;
    const int nbw = (wt == 2) ? K / kQK8 : K / kQK;
    L.act_qs = 0;
    L.act_row = (wt == 2) ? align16i(K) : (K / kQK) * kActStride;
    L.act_d = mb * L.act_row;
    L.act_bs = L.act_d + align16i(mb * nbw * 4);
    const int nbs_bytes = (wt == 2) ? (K / kQK8) * 4 : (K / 16) * 2;
    L.partial = L.act_bs + align16i(mb * nbs_bytes);
    L.wslice = L.partial + align16i(mb * rows * ((nbw + 3) & ~3) * 4);
    L.slice_bytes = slice_bytes;
    L.total = L.wslice + slice_bytes;
    return L;
}

// Byte span (relative to the workgroup's first row) of tasks [t0, t1).
__host__ __device__ inline void task_span(int t0, int t1, int nb, int rb, int bb, int* b0, int* b1) {
    if (t1 <= t0) { *b0 = 0; *b1 = 0; return; }
    const int r0 = t0 / nb, k0 = t0 - r0 * nb;
    const int r1 = (t1 - 1) / nb, k1 = (t1 - 1) - r1 * nb;
    *b0 = r0 * rb + k0 * bb;
    *b1 = r1 * rb + (k1 + 1) * bb;
}

// Barrier for LDS data only: wait for this wave's LDS operations, then
// s_barrier (no wait on outstanding global loads, unlike __syncthreads).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// 32 bytes at a 2-byte aligned LDS address (9 aligned dword reads).
__device__ __forceinline__ void lds_read32_a2(const uint8_t* p, uint32_t out[8]) {
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
    const uint32_t* q = (const uint32_t*)(p - sh);
    uint32_t w[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = q[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63].
__device__ __forceinline__ void wait_vmcnt(int n) {
#define VQ_VMW(k) case k: __builtin_amdgcn_s_waitcnt((((k) & 15) | (((k) >> 4) << 14)) | 0x0F70); break;
    switch (n) {
        VQ_VMW(0) VQ_VMW(1) VQ_VMW(2) VQ_VMW(3) VQ_VMW(4) VQ_VMW(5) VQ_VMW(6) VQ_VMW(7)
        VQ_VMW(8) VQ_VMW(9) VQ_VMW(10) VQ_VMW(11) VQ_VMW(12) VQ_VMW(13) VQ_VMW(14) VQ_VMW(15)
        VQ_VMW(16) VQ_VMW(17) VQ_VMW(18) VQ_VMW(19) VQ_VMW(20) VQ_VMW(21) VQ_VMW(22) VQ_VMW(23)
        VQ_VMW(24) VQ_VMW(25) VQ_VMW(26) VQ_VMW(27) VQ_VMW(28) VQ_VMW(29) VQ_VMW(30) VQ_VMW(31)
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;  // vmcnt(0)
    }
#undef VQ_VMW
}

typedef __attribute__((address_space(3))) void lds_void;

// MB activation rows (1: the decode GEMV; 2, 4, 8: small batches).  With
// xq_in == nullptr the quantizer waves quantize x (MB == 1); otherwise they
// copy M rows of a planar pre-quantized activation buffer into LDS.
template <int WT, int MB>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint8_t* __restrict__ W, int N, int K, int64_t wbytes, const float* __restrict__ x,
    float* __restrict__ y, uint8_t* __restrict__ xq_out, int rows_per_wg, int slice_bytes, int x_vec,
    int nq, int h1_tasks, int kh0, int kh1, const uint8_t* __restrict__ xq_in, int M, int64_t ldy,
    int64_t xq_d_off, int64_t xq_aux_off, int wait_polls, unsigned int* __restrict__ err_word) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_loaders_done;  // loader waves whose second part has landed
    __shared__ int s_bad;           // a loader wave's wait gave up: this workgroup's rows are NaN
    constexpr int BB = WFmt<WT>::kBlk;
    constexpr int QV = WFmt<WT>::kVals;
    constexpr int LPT = (WT == 2) ? 1 : 2;    // lanes per task
    constexpr int GPW = 64 / LPT;             // tasks per wave pass
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control
    const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
    const int G = nq;                         // quantizer waves (first half); the rest load
    const int GL = nw - nq;                   // loader waves (second half)
    const int nthr = 64 * nw;
    const int nb = K / QV;
    const int rb = nb * BB;
    const int n0 = blockIdx.x * rows_per_wg;
    const int rows = min(rows_per_wg, N - n0);
    const GemvLayout L = gemv_layout(WT, K, rows_per_wg, slice_bytes, MB);
    int8_t* act_qs = (int8_t*)(smem + L.act_qs);
    float* act_d = (float*)(smem + L.act_d);
    int16_t* act_bs = (int16_t*)(smem + L.act_bs);
    uint32_t* act_ds = (uint32_t*)(smem + L.act_bs);  // Q8_1: binary16 d | s << 16 per block
    float* partial = (float*)(smem + L.partial);
    uint8_t* wsl = smem + L.wslice;
    uint8_t* dummy = wsl + slice_bytes - 1024 - 64;   // target of padding instructions

    // Slice geometry: chunks [cb, ce) of 16 bytes hold the rows' bytes; the
    // first part of the tasks (computed by the quantizer waves while the rest
    // streams in) ends inside chunk cm - 1.
    const int ntask = rows * nb;
    const int th = ntask - min(ntask, h1_tasks);
    const int64_t s0 = (int64_t)n0 * rb;
    const int64_t cb = s0 >> 4;
    const int64_t ce = (s0 + (int64_t)rows * rb + 15) >> 4;
    int hb0, hb1;
    task_span(0, th, nb, rb, BB, &hb0, &hb1);
    const int64_t cm = (th > 0) ? ((s0 + hb1 + 15) >> 4) : cb;
    const int64_t full = wbytes >> 4;          // complete chunks of the buffer
    const int rbase = (int)(s0 - 16 * cb);     // LDS byte of slice byte o: wsl + rbase + o
    const bool loader = wave >= G;

    // Activation rows [row0, row0 + n) of a planar pre-quantized buffer into
    // the LDS rows 0..n-1 (threads t0, t0 + stride, ...).
    auto copy_rows = [&](int row0, int n, int t0, int stride) {
        const int nbw = (WT == 2) ? K / kQK8 : K / kQK;
        const int cpr = K / 16;  // 16-byte chunks per row
        for (int i = t0; i < n * cpr; i += stride) {
            const int m = i / cpr, c = i - m * cpr;
            const uint4 v = *(const uint4*)(xq_in + (int64_t)(row0 + m) * K + 16 * c);
            const int dst = (WT == 2) ? 16 * c : (c >> 4) * kActStride + 16 * (c & 15);
            *(uint4*)(act_qs + m * L.act_row + dst) = v;
        }
        if (WT == 2) {
            const uint16_t* dsrc = (const uint16_t*)(xq_in + xq_d_off) + (int64_t)row0 * nbw;
            for (int i = t0; i < n * nbw; i += stride) act_d[i] = half_bits_to_float(dsrc[i]);
        } else {
            const float* dsrc = (const float*)(xq_in + xq_d_off) + (int64_t)row0 * nbw;
            for (int i = t0; i < n * nbw; i += stride) act_d[i] = dsrc[i];
            const int16_t* bsrc = (const int16_t*)(xq_in + xq_aux_off) + (int64_t)row0 * (K / 16);
            for (int i = t0; i < n * (K / 16); i += stride) act_bs[i] = bsrc[i];
        }
    };
    // rows of activations in LDS (the current group of at most MB rows)
    int Mg = M < MB ? M : MB;

    if (loader) {
        // ---- loaders: both parts into LDS, kh0 / kh1 instructions each
        const int lw = wave - G;
        auto issue_half = [&](int64_t hs, int64_t he, int kh) {
            const int64_t ninstr = (he - hs + 63) >> 6;
            for (int i = 0; i < kh; ++i) {
                const int64_t j = lw + (int64_t)GL * i;
                const uint8_t* src;
                uint8_t* dst;
                if (j < ninstr) {
                    const int64_t base = hs + 64 * j;
                    int64_t c = base + lane;
                    c = c < ce ? c : ce - 1;           // lanes past the slice repeat its last chunk
                    c = c < full ? c : full - 1;       // a partial last chunk is patched below
                    src = W + 16 * c;
                    dst = wsl + 16 * (base - cb);      // lane l lands at dst + 16 l
                } else {
                    int64_t c = cb + lane;
                    c = c < ce ? c : ce - 1;
                    c = c < full ? c : full - 1;
                    src = W + 16 * c;
                    dst = dummy;
                }
                // non-temporal: each weight byte is read once, so it should not
                // displace x or other data in the caches (measured 3% faster)
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)dst, 16, 0, kNonTemporal);
            }
        };
        issue_half(cb, cm, kh0);
        issue_half(cm, ce, kh1);
        wait_vmcnt(kh1);  // the first part has landed
    } else if (xq_in != nullptr) {
        // ---- quantizer waves, pre-quantized input: the first group of rows into LDS
        copy_rows(0, Mg, tid, 64 * G);
    } else {
        // ---- quantizer waves: x loads, then the shared quantizer into LDS
        const int xsteps = (K + kQK - 1) / kQK;  // 256 values per wave step
        float4 xv[kXPre];
#pragma unroll
        for (int r = 0; r < kXPre; ++r) {
            const int e = min((wave + G * r) * kQK + 4 * lane, K - 4);
            const float* src = x + e;
            xv[r] = x_vec ? *(const float4*)src : make_float4(src[0], src[1], src[2], src[3]);
        }
    if (WT != 2) {
        const int nsb = K / kQK;
#pragma unroll
        for (int r = 0; r < kXPre; ++r) {
            const int sb = wave + G * r;
            if (sb < nsb) {
                const Q8KLane q = q8k_quant_lane(xv[r], lane);
                *(uint32_t*)(act_qs + sb * kActStride + 4 * lane) = q.q4;
                if (lane == 0) act_d[sb] = q.d;
                if ((lane & 3) == 0) act_bs[sb * 16 + (lane >> 2)] = (int16_t)q.bsum;
            }
        }
        for (int sb = wave + G * kXPre; sb < nsb; sb += G) {
            const float* src = x + sb * kQK + 4 * lane;
            const Q8KLane q1 = q8k_quant_lane(x_vec ? *(const float4*)src
                                                    : make_float4(src[0], src[1], src[2], src[3]), lane);
            *(uint32_t*)(act_qs + sb * kActStride + 4 * lane) = q1.q4;
            if (lane == 0) act_d[sb] = q1.d;
            if ((lane & 3) == 0) act_bs[sb * 16 + (lane >> 2)] = (int16_t)q1.bsum;
        }
    } else {
        auto quant_step = [&](int stp, float4 v) {
            const int e = stp * kQK + 4 * lane;
            const bool valid = e < K;
            const Q81Lane q = q81_quant_lane(v);
            if (valid) {
                const int blk = e / kQK8;
                *(uint32_t*)(act_qs + e) = q.q4;
                const uint32_t d16 = float_to_half_bits(q.d);
                if ((lane & 7) == 0) {
                    act_d[blk] = half_bits_to_float(d16);
                    act_ds[blk] = d16 | (float_to_half_bits(q.s) << 16);
                }
            }
        };
#pragma unroll
        for (int r = 0; r < kXPre; ++r)
            if (wave + G * r < xsteps) quant_step(wave + G * r, xv[r]);
        for (int stp = wave + G * kXPre; stp < xsteps; stp += G) {
            const int e = stp * kQK + 4 * lane;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < K) {
                const float* src = x + e;
                v = x_vec ? *(const float4*)src : make_float4(src[0], src[1], src[2], src[3]);
            }
            quant_step(stp, v);
        }
    }
    }
    if (tid == 0) {  // wave 0 is a quantizer wave; visible after the barrier
        s_loaders_done = 0;
        s_bad = 0;
    }
    lds_barrier();  // quantized x and the first half of the slice visible to every wave

    const int grp = lane / LPT, sub = lane % LPT;
    // One (row, block) task for each of the MB activation rows: the weight
    // bytes are read and unpacked once and reused for every row.
    const int nbw_ = (WT == 2) ? K / kQK8 : K / kQK;
    const int nbp = (nb + 3) & ~3;  // partial row stride: 16-byte aligned rows
    auto compute_task = [&](int r, int blk) {
        const uint8_t* bp = wsl + rbase + __mul24(r, rb) + __mul24(blk, BB);
        if (WT == 0 || WT == 3) {
            // lane half hf: sub-blocks 4hf..4hf+3 = qs bytes [64hf, 64hf+64);
            // Q5_K: the nibbles start at byte 48 and bit j of byte 16 + l
            // adds bit 4 to element 32j + l.
            constexpr int kQsOff = (WT == 3) ? 48 : 16;
            const int hf = sub;
            const uint4 hdr = *(const uint4*)bp;
            uint32_t lo[16], hi[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = *(const uint4*)(bp + kQsOff + 64 * hf + 16 * i);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lo[4 * i + k] = w4[k] & 0x0F0F0F0Fu;
                    hi[4 * i + k] = (w4[k] >> 4) & 0x0F0F0F0Fu;
                }
            }
            if (WT == 3) {
                // qs piece i holds bytes l = 16 (i & 1) + 4k + byte of chunk
                // c = 2hf + (i >> 1): low nibbles are sub-block 2c, high 2c + 1
                const uint4 h0 = *(const uint4*)(bp + 16);
                const uint4 h1 = *(const uint4*)(bp + 32);
                const uint32_t qh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 2 * hf + (i >> 1);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t hw = qh[4 * (i & 1) + k];
                        lo[4 * i + k] |= ((hw >> (2 * c)) & 0x01010101u) << 4;
                        hi[4 * i + k] |= ((hw >> (2 * c + 1)) & 0x01010101u) << 4;
                    }
                }
            }
            const uint32_t sw = hf ? hdr.z : hdr.y;             // scales bytes 4hf..4hf+3
            const uint32_t mw = hdr.w >> (16 * hf);             // min high nibbles, 2 bytes
            const float d = half_bits_to_float(hdr.x & 0xFFFF);
            const float dmin = half_bits_to_float(hdr.x >> 16);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if (m >= Mg) break;
                const int8_t* ab = act_qs + m * L.act_row + __mul24(blk, kActStride) + 128 * hf;
                uint32_t av[32];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4 v = *(const uint4*)(ab + 16 * i);
                    av[4 * i] = v.x; av[4 * i + 1] = v.y; av[4 * i + 2] = v.z; av[4 * i + 3] = v.w;
                }
                int P[4] = {0, 0, 0, 0};  // sub-blocks 4hf + j
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        P[2 * c] = sdot4((int)lo[8 * c + i], (int)av[16 * c + i], P[2 * c]);
                        P[2 * c + 1] = sdot4((int)hi[8 * c + i], (int)av[16 * c + 8 + i], P[2 * c + 1]);
                    }
                const uint4 bsv = *(const uint4*)(act_bs + m * (K / 16) + blk * 16 + 8 * hf);
                const uint32_t bw[4] = {bsv.x, bsv.y, bsv.z, bsv.w};
                int S = 0, Mn = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t sj = (sw >> (8 * j)) & 0xFF;
                    const uint32_t mh = (mw >> (4 * j)) & 15;
                    const int mm = (int)((sj >> 6) | (mh << 2));
                    const int bs32 = (int)(int16_t)(bw[j] & 0xFFFF) + (int)(int16_t)(bw[j] >> 16);
                    S += __mul24((int)(sj & 63), P[j]);
                    Mn += __mul24(mm, bs32);
                }
                S += dppi<0xB1>(S);
                Mn += dppi<0xB1>(Mn);
                if (hf == 0) {
                    const float t1f = d * (float)S;
                    const float t2f = dmin * (float)Mn;
                    const float t3f = t1f - t2f;
                    partial[(m * rows_per_wg + r) * nbp + blk] = act_d[m * nbw_ + blk] * t3f;
                }
            }
        } else if (WT == 1) {
            // lane half h: values 128h..128h+127 (sub-blocks 8h..8h+7)
            const int h = sub;
            uint32_t ql[16], qh[8];
            lds_read32_a2(bp + 64 * h, ql);
            lds_read32_a2(bp + 64 * h + 32, ql + 8);
            lds_read32_a2(bp + 128 + 32 * h, qh);
            const uint16_t* scp = (const uint16_t*)(bp + 192 + 8 * h);
            const uint32_t scw[4] = {scp[0], scp[1], scp[2], scp[3]};
            uint32_t qa[16], qb[16];  // 6-bit quants of sub-blocks 8h + k (qa) and 8h + 4 + k (qb)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t l = ql[4 * k + i];
                    const uint32_t hq = qh[4 * (k & 1) + i];
                    const int sa = 2 * (k >> 1), sb = 2 * (2 + (k >> 1));
                    qa[4 * k + i] = (l & 0x0F0F0F0Fu) | (((hq >> sa) & 0x03030303u) << 4);
                    qb[4 * k + i] = ((l >> 4) & 0x0F0F0F0Fu) | (((hq >> sb) & 0x03030303u) << 4);
                }
            const float d = half_bits_to_float(*(const uint16_t*)(bp + 208));
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if (m >= Mg) break;
                const int8_t* ab = act_qs + m * L.act_row + __mul24(blk, kActStride) + 128 * h;
                uint32_t av[32];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4 v = *(const uint4*)(ab + 16 * i);
                    av[4 * i] = v.x; av[4 * i + 1] = v.y; av[4 * i + 2] = v.z; av[4 * i + 3] = v.w;
                }
                int I[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // sub-blocks 8h + j
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        I[k] = sdot4((int)qa[4 * k + i], (int)av[4 * k + i], I[k]);
                        I[4 + k] = sdot4((int)qb[4 * k + i], (int)av[16 + 4 * k + i], I[4 + k]);
                    }
                const uint4 bsv = *(const uint4*)(act_bs + m * (K / 16) + blk * 16 + 8 * h);
                const uint32_t bw[4] = {bsv.x, bsv.y, bsv.z, bsv.w};
                int S = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int bsj = (int)(int16_t)((bw[j >> 1] >> (16 * (j & 1))) & 0xFFFF);
                    const int scj = (int)(int8_t)((scw[j >> 1] >> (8 * (j & 1))) & 0xFF);
                    S += __mul24(scj, I[j] - 32 * bsj);
                }
                S += dppi<0xB1>(S);
                if (h == 0) {
                    const float t1f = d * (float)S;
                    partial[(m * rows_per_wg + r) * nbp + blk] = act_d[m * nbw_ + blk] * t1f;
                }
            }
        } else {
            uint32_t qw[8];
            lds_read32_a2(bp + 2, qw);
            const float dw = half_bits_to_float(*(const uint16_t*)bp);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if (m >= Mg) break;
                const int8_t* ab = act_qs + m * L.act_row + blk * kQK8;
                const uint4 a0 = *(const uint4*)ab;
                const uint4 a1 = *(const uint4*)(ab + 16);
                const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                int I = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) I = sdot4((int)qw[i], (int)av[i], I);
                const float sc = dw * act_d[m * nbw_ + blk];
                partial[(m * rows_per_wg + r) * nbp + blk] = sc * (float)I;
            }
        }
    };

    // Tasks [t0, t1), one pass per GPW tasks.
    auto compute_range = [&](int t0, int t1) {
        for (int base = t0; base < t1; base += GPW) {
            const int t = base + grp;
            if (t < t1) {
                const int r = t / nb;
                compute_task(r, t - r * nb);
            }
        }
    };

    if (loader) {
        wait_vmcnt(0);  // the second half has landed
        // A partial last chunk of the buffer (loaded as its predecessor above)
        // is patched byte by byte by the lane whose chunk it is.
        if (full < ce && (wbytes & 15) != 0) {
            const int lw = wave - G;
            const int64_t ninstr = (ce - cm + 63) >> 6;
            const int64_t j = (full - cm) >> 6;   // instruction of the partial chunk
            if (full >= cm && j < ninstr && (j % GL) == lw && lane == (int)((full - cm) & 63)) {
                uint8_t* d = wsl + 16 * (full - cb);
                for (int bi = 0; bi < 16; ++bi) {
                    const int64_t a = 16 * full + bi;
                    d[bi] = (a < wbytes) ? W[a] : (uint8_t)0;
                }
            }
        }
        // The loaders alone meet here (the quantizer waves may still be on the
        // first part): each signals that its loads (and any patch) are in LDS,
        // then waits for the others, whose chunks its tasks read.  Bounded
        // (wait_polls polls), so the wave always moves on; if it gives up, the
        // workgroup's rows are written as NaN and the device error word gets
        // bit 1, which vq_device_status reports.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the patch bytes are written
        if (lane == 0) atomicAdd(&s_loaders_done, 1);
        bool ok = false;
        for (int spin = 0; spin < wait_polls; ++spin) {
            const int done = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(&s_loaders_done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (done >= GL) {
                ok = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!ok && lane == 0) {
            s_bad = 1;
            __hip_atomic_fetch_or(err_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- 5. rows: blocks summed in ascending order from 0.  The partials
    // are read 16 at a time with independent float4 loads before the adds,
    // so a row costs a few LDS round trips, not one per block.
    auto sum_rows = [&](int row0) {
    const bool bad = s_bad != 0;  // set before the barrier that precedes every call
    for (int idx = tid; idx < MB * rows; idx += nthr) {
        const int m = idx / rows, r = idx - m * rows;
        if (m >= Mg) break;
        const float* p = partial + (m * rows_per_wg + r) * nbp;
        float acc = 0.0f;
        int b = 0;
        for (; b + 16 <= nb; b += 16) {
            const float4 u0 = *(const float4*)(p + b);
            const float4 u1 = *(const float4*)(p + b + 4);
            const float4 u2 = *(const float4*)(p + b + 8);
            const float4 u3 = *(const float4*)(p + b + 12);
            acc = acc + u0.x; acc = acc + u0.y; acc = acc + u0.z; acc = acc + u0.w;
            acc = acc + u1.x; acc = acc + u1.y; acc = acc + u1.z; acc = acc + u1.w;
            acc = acc + u2.x; acc = acc + u2.y; acc = acc + u2.z; acc = acc + u2.w;
            acc = acc + u3.x; acc = acc + u3.y; acc = acc + u3.z; acc = acc + u3.w;
        }
        if (b < nb) {
            // fewer than 16 left: the float4s that hold them (inside the padded row)
            float t[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
                if (b + 4 * q < nb) u = *(const float4*)(p + b + 4 * q);
                t[4 * q] = u.x; t[4 * q + 1] = u.y; t[4 * q + 2] = u.z; t[4 * q + 3] = u.w;
            }
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (b + j < nb) acc = acc + t[j];
        }
        y[(row0 + m) * ldy + n0 + r] = bad ? __builtin_nanf("") : acc;
    }
    };

    // The first group of rows: the quantizer waves compute the first part of
    // the tasks while the rest streams in, the loaders the last part.  Further
    // groups of MB rows (small batches above 8 rows, built with MB = 4 only):
    // the slice stays in LDS, every wave copies the group's rows, then takes
    // an equal share of all tasks.  One compute call site for all groups.
    for (int row0 = 0;;) {
        int t0, t1;
        if (row0 == 0) {
            if (!loader) {
                t0 = (int)((int64_t)th * wave / G);
                t1 = (int)((int64_t)th * (wave + 1) / G);
            } else {
                const int lw = wave - G;
                t0 = th + (int)((int64_t)(ntask - th) * lw / GL);
                t1 = th + (int)((int64_t)(ntask - th) * (lw + 1) / GL);
            }
        } else {
            t0 = (int)((int64_t)ntask * wave / nw);
            t1 = (int)((int64_t)ntask * (wave + 1) / nw);
        }
        // The loaders' pass over the last part ends the launch: they get the
        // SIMDs' issue priority over the quantizer waves' first-part pass
        // (Q6_K decode 8.51-8.60 -> 8.42-8.44 us; Q8_0's one-block tasks
        // measured 1 % slower with it, so they keep the default).
        const bool pr = (WT != 2) && (row0 == 0) && loader;
        if (pr) __builtin_amdgcn_s_setprio(2);
        compute_range(t0, t1);
        if (pr) __builtin_amdgcn_s_setprio(0);
        lds_barrier();  // every partial of the group written
        sum_rows(row0);
        row0 += MB;
        if (MB != kGroupMB || row0 >= M) break;
        Mg = (M - row0) < MB ? (M - row0) : MB;
        __syncthreads();  // the previous group's rows and partials are no longer read
        copy_rows(row0, Mg, tid, nthr);
        __syncthreads();
    }

    // ---- 6. the fused quantizer's bytes, for callers that want them
    if (xq_out != nullptr && blockIdx.x == 0) {
        const size_t od = align256((size_t)K);
        const int stride = (WT == 2) ? kQK : kActStride;
        for (int i = tid; i < K / 4; i += nthr)
            ((uint32_t*)xq_out)[i] = *(const uint32_t*)(act_qs + (i / 64) * stride + 4 * (i % 64));
        if (WT != 2) {
            const int nsb = K / kQK;
            float* gd = (float*)(xq_out + od);
            int16_t* gb = (int16_t*)(xq_out + od + align256((size_t)nsb * 4));
            for (int i = tid; i < nsb; i += nthr) gd[i] = act_d[i];
            for (int i = tid; i < K / 16; i += nthr) gb[i] = act_bs[i];
        } else {
            const int nblk = K / kQK8;
            uint16_t* gd = (uint16_t*)(xq_out + od);
            uint16_t* gs = (uint16_t*)(xq_out + od + align256((size_t)nblk * 2));
            for (int i = tid; i < nblk; i += nthr) {
                gd[i] = (uint16_t)(act_ds[i] & 0xFFFF);
                gs[i] = (uint16_t)(act_ds[i] >> 16);
            }
        }
    }
}

// Compute units of the current device, cached per device (the plans size
// the grid to one workgroup per CU).
static std::atomic<int> g_num_cus[kMaxDevices];

int num_cus() {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = g_num_cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        g_num_cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

static int block_bytes_of(int wt) {
    return wt == 0 ? kQ4KBytes : (wt == 1 ? kQ6KBytes : (wt == 3 ? kQ5KBytes : kQ80Bytes));
}
// Kernel template index of a library weight type (Q5_K = 5 is index 3).
static int wt_of(int wtype) { return wtype == 5 ? 3 : wtype; }
static int block_vals_of(int wt) { return wt == 2 ? kQK8 : kQK; }

struct GemvPlan {
    int rows;          // rows per workgroup
    int nq, nl;        // quantizer waves (first part of the tasks), loader waves (the rest)
    int h1;            // tasks of the second part
    int kh0, kh1;      // load instructions per loader wave for each part
    int slice_bytes;   // LDS bytes of the weight slice region
    int lds;           // dynamic LDS bytes
    bool ok;
};

// About one workgroup per CU.  The loader waves compute the last part of the
// tasks after the whole slice has landed, so that part is kept to one pass of
// at most one wave per SIMD (4 x 32 tasks, or a third of the tasks); the
// quantizer waves take the rest in one pass each while it streams in.  Fewer
// rows when the slice would not fit LDS, the waves would exceed 16, or the
// loaders would need more instructions than a vmcnt wait can count.
static GemvPlan gemv_plan(int wt, int64_t N, int64_t K, int mb) {
    GemvPlan p;
    const int bb = block_bytes_of(wt);
    const int nb = (int)(K / block_vals_of(wt));
    const int rb = nb * bb;
    const int gpw = (wt == 2) ? 64 : 32;  // tasks per wave pass
    int rows = (int)((N + num_cus() - 1) / num_cus());
    if (rows < 1) rows = 1;
    for (;;) {
        const int ntask = rows * nb;
        int h1 = ntask / 3;
        h1 = h1 < 4 * gpw ? h1 : 4 * gpw;
        h1 = h1 < 1 ? (ntask < 1 ? 0 : 1) : h1;
        const int th = ntask - h1;
        int nl = (h1 + gpw - 1) / gpw;
        nl = nl < 1 ? 1 : nl;
        int nq = (th + gpw - 1) / gpw;
        nq = nq < 1 ? 1 : nq;
        int hb0, hb1;
        task_span(0, th, nb, rb, bb, &hb0, &hb1);
        const int64_t slice = (int64_t)rows * rb;
        const int64_t c_h0 = (th > 0) ? (hb1 + 15) / 16 + 1 : 0;
        const int64_t c_h1 = (slice - hb1 + 15) / 16 + 2;
        const int kh0 = (int)(((c_h0 + 63) / 64 + nl - 1) / nl);
        const int kh1 = (int)(((c_h1 + 63) / 64 + nl - 1) / nl);
        const int64_t sbytes = 16 * ((slice + 15) / 16 + 2) + 1024 + 1024 + 64;
        const bool small = sbytes < (int64_t)kMaxLds;
        const GemvLayout L = gemv_layout(wt, (int)K, rows, small ? (int)sbytes : 0, mb);
        const bool fits = small && nq + nl <= kGemvWaves && kh0 + kh1 <= 63 && kh1 <= kMaxHalfInstr &&
                          (size_t)L.total + kStaticLds <= kMaxLds;
        if (fits || rows == 1) {
            p.rows = rows;
            p.nq = nq;
            p.nl = nl;
            p.h1 = h1;
            p.kh0 = kh0 < 1 ? 1 : kh0;
            p.kh1 = kh1 < 1 ? 1 : kh1;
            p.slice_bytes = (int)sbytes;
            p.lds = L.total;
            p.ok = fits;
            return p;
        }
        --rows;
    }
}

size_t gemv_lds_bytes(int wtype, int64_t N, int64_t K, int mb) {
    const GemvPlan p = gemv_plan(wt_of(wtype), N, K, mb);
    return p.ok ? (size_t)p.lds : (size_t)-1;
}

// Rows per group for M activation rows: 1, 2, 4 or 8 in one group; above 8
// rows (or when the 8-row plan would need a second round of workgroups),
// groups of 4.
static int mb_for(int wt, int64_t N, int64_t K, int64_t M) {
    if (M <= 1) return 1;
    if (M <= 2) return 2;
    if (M <= 4) return 4;
    if (M <= 8) {
        const GemvPlan p = gemv_plan(wt, N, K, 8);
        if (p.ok && (N + p.rows - 1) / p.rows <= num_cus()) return 8;
    }
    return kGroupMB;
}

template <int WT, int MB>
static hipError_t launch_gemv_t(const uint8_t* W, int64_t N, int64_t K, const float* x, float* y, int64_t ldy,
                                uint8_t* xq_out, const uint8_t* xq_in, int64_t M, int64_t d_off, int64_t aux_off,
                                hipStream_t st) {
    // the dynamic-LDS limit is raised once per device for this kernel
    static std::atomic<uint64_t> attr_set{0};
    const GemvPlan p = gemv_plan(WT, N, K, MB);
    if (!p.ok) return hipErrorInvalidValue;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = 1ull << ((dev >= 0 && dev < kMaxDevices) ? dev : 0);
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
        hipError_t e = hipFuncSetAttribute((const void*)gemv_kernel<WT, MB>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxLds - kStaticLds));
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_release);
    }
    const int rb = (int)(K / WFmt<WT>::kVals) * WFmt<WT>::kBlk;
    const int grid = (int)((N + p.rows - 1) / p.rows);
    const int x_vec = (x != nullptr && (((uintptr_t)x) & 15) == 0) ? 1 : 0;
    gemv_kernel<WT, MB><<<grid, 64 * (p.nq + p.nl), p.lds, st>>>(
        W, (int)N, (int)K, (int64_t)N * rb, x, y, xq_out, p.rows, p.slice_bytes, x_vec, p.nq, p.h1, p.kh0, p.kh1,
        xq_in, (int)M, ldy, d_off, aux_off, g_dbg.wait_polls, g_dbg.err_word);
    return hipGetLastError();
}

// Streaming floor of a decode GEMV launch: the GEMV's grid and workgroup
// size, each workgroup reading its rows' weight bytes [b0, b1) once and
// nothing else -- 16-byte loads of the aligned interior, eight in flight per
// lane, single bytes for the unaligned ends -- folded into one word that is
// stored only if it equals a value the caller never sees (so the loads are
// kept and nothing is written).
__global__ __launch_bounds__(1024) void stream_probe_kernel(const uint8_t* __restrict__ W, int64_t total,
                                                            int64_t slice, uint32_t* __restrict__ sink) {
    const int64_t b0 = (int64_t)blockIdx.x * slice;
    const int64_t b1 = min(total, b0 + slice);
    const int64_t a0 = (b0 + 15) & ~(int64_t)15, a1 = b1 & ~(int64_t)15;
    const int nt = blockDim.x;
    uint32_t acc = 0;
    if (a0 < a1) {
        constexpr int kU = 8;
        const int64_t step = (int64_t)16 * nt;
        for (int64_t off = a0 + 16 * (int64_t)threadIdx.x; off < a1; off += kU * step) {
            uint4 v[kU];
#pragma unroll
            for (int k = 0; k < kU; ++k) {
                const int64_t o = off + k * step;
                v[k] = (o < a1) ? *(const uint4*)(W + o) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < kU; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
        }
        const int64_t head = a0 - b0, tail = b1 - a1;
        if (threadIdx.x < head) acc ^= W[b0 + threadIdx.x];
        if (threadIdx.x < tail) acc ^= W[a1 + threadIdx.x];
    } else {
        for (int64_t o = b0 + threadIdx.x; o < b1; o += nt) acc ^= W[o];
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

hipError_t launch_stream_probe(int wtype, const uint8_t* W, int64_t N, int64_t K, uint32_t* sink, int64_t* grid_out,
                               hipStream_t st) {
    const int wt = wt_of(wtype);
    const GemvPlan p = gemv_plan(wt, N, K, 1);
    if (!p.ok) return hipErrorInvalidValue;
    const int64_t rb = (K / block_vals_of(wt)) * block_bytes_of(wt);
    const int64_t grid = (N + p.rows - 1) / p.rows;
    if (grid_out) *grid_out = grid;
    if (N == 0) return hipSuccess;
    stream_probe_kernel<<<(unsigned)grid, 64 * (p.nq + p.nl), 0, st>>>(W, N * rb, (int64_t)p.rows * rb, sink);
    return hipGetLastError();
}

hipError_t launch_gemv(int wtype, const uint8_t* W, int64_t N, int64_t K, const float* x, float* y,
                       uint8_t* xq_out, hipStream_t st) {
    if (N == 0) return hipSuccess;
    if (wtype == 0) return launch_gemv_t<0, 1>(W, N, K, x, y, N, xq_out, nullptr, 1, 0, 0, st);
    if (wtype == 1) return launch_gemv_t<1, 1>(W, N, K, x, y, N, xq_out, nullptr, 1, 0, 0, st);
    if (wtype == 5) return launch_gemv_t<3, 1>(W, N, K, x, y, N, xq_out, nullptr, 1, 0, 0, st);
    return launch_gemv_t<2, 1>(W, N, K, x, y, N, xq_out, nullptr, 1, 0, 0, st);
}

template <int WT>
static hipError_t launch_skinny_t(const uint8_t* W, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                                  int64_t d_off, int64_t aux_off, float* Y, int64_t ldy, hipStream_t st) {
    switch (mb_for(WT, N, K, M)) {
        case 1: return launch_gemv_t<WT, 1>(W, N, K, nullptr, Y, ldy, nullptr, xq, M, d_off, aux_off, st);
        case 2: return launch_gemv_t<WT, 2>(W, N, K, nullptr, Y, ldy, nullptr, xq, M, d_off, aux_off, st);
        case 4: return launch_gemv_t<WT, 4>(W, N, K, nullptr, Y, ldy, nullptr, xq, M, d_off, aux_off, st);
        default: return launch_gemv_t<WT, 8>(W, N, K, nullptr, Y, ldy, nullptr, xq, M, d_off, aux_off, st);
    }
}

bool gemm_skinny_ok(int wtype, int64_t N, int64_t K, int64_t M, int64_t max_m) {
    return M >= 1 && M <= max_m && M <= kSkinnyMaxM && N > 0 &&
           gemv_lds_bytes(wtype, N, K, mb_for(wt_of(wtype), N, K, M)) <= kMaxLds;
}

hipError_t launch_gemm_skinny(int wtype, const uint8_t* W, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                              int64_t d_off, int64_t aux_off, float* Y, int64_t ldy, hipStream_t st) {
    if (wtype == 0) return launch_skinny_t<0>(W, N, K, xq, M, d_off, aux_off, Y, ldy, st);
    if (wtype == 1) return launch_skinny_t<1>(W, N, K, xq, M, d_off, aux_off, Y, ldy, st);
    if (wtype == 5) return launch_skinny_t<3>(W, N, K, xq, M, d_off, aux_off, Y, ldy, st);
    return launch_skinny_t<2>(W, N, K, xq, M, d_off, aux_off, Y, ldy, st);
}

}  // namespace vqk
