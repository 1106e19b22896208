// gemv.hip -- decode GEMV (M = 1) for Q4_K / Q6_K weights x Q8_K and Q8_0
// weights x Q8_1, with the activation quantizer fused into the prologue.
//
// Pages: vllm.cpp PR #2890, commit "T4a VT_GEMV_MMVQ" (the K-quant decode
// GEMV folds the activation quantizer into its prologue, bit-exact against
// the CPU oracle); strix-llama.cpp PR #18, commit "mul_mat_vec_q_fq" (a
// block quantizes the activation once into shared memory, with weight loads
// issued before the quantization and its barrier), commit "warp reduce via
// DPP" (lane exchange without LDS round trips) and commit "batch-one MMVQ on
// one wave" (a fixed fp32 reduction order keeps decode deterministic).
//
// MI355X design.  The GEMV streams 9-20 MB of weights: a few microseconds of
// HBM time, so everything else has to hide under the loads.
//  * One 1024-thread workgroup per CU owns a contiguous run of rows.  Its
//    (row, block) tasks are split into 16 contiguous ranges, one per wave; a
//    wave's bytes are one contiguous span, fetched with aligned 16-byte
//    loads into registers.
//  * Order of issue: first the few x loads (L2 hits), then every weight load
//    of the wave, so the quantizer only waits for x while the weights stream.
//  * The 16 waves quantize x into LDS with the shared quantizer body (DPP
//    reductions); one barrier publishes it.
//  * Each wave then parks its own weight span in a private LDS region (the
//    Q6_K / Q8_0 blocks are only 2-byte aligned; LDS reads at that alignment
//    are rebuilt with v_alignbyte) and computes as soon as its own bytes are
//    in: no workgroup barrier between a wave's loads and its compute.
//  * Eight lanes own one (row, super-block) -- one lane per Q8_0 block: exact
//    int32 sub-block sums with v_dot4_i32_i8, an exact DPP reduction over the
//    eight lanes, then the block's binary32 combine into an LDS partial.
//  * After one more barrier, one lane per row adds the row's partials in
//    ascending block order from 0, so y is bit-identical to the fixed-order
//    definition.
#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

constexpr int kGemvThreads = 1024;              // most threads per workgroup
constexpr int kGemvWaves = kGemvThreads / 64;   // most waves per workgroup
constexpr int kLMax = 8;            // 16-byte chunks per lane: a wave span <= 8 KiB
constexpr int kXPre = 4;            // x rounds loaded before the weights
constexpr int kStepLoads = kLMax;   // loads parked before computing (one step: measured fastest)
constexpr size_t kMaxLds = 160 * 1024;
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

struct GemvLayout {
    int act_qs, act_d, act_bs, partial, regions, region_bytes, total;
};

__host__ __device__ inline int align16i(int x) { return (x + 15) & ~15; }

// LDS layout of the GEMV workgroup; identical on host and device.
__host__ __device__ inline GemvLayout gemv_layout(int wt, int K, int rows, int region_bytes, int nwaves) {
    GemvLayout L;
    const int nbw = (wt == 2) ? K / kQK8 : K / kQK;
    L.act_qs = 0;
    L.act_d = (wt == 2) ? align16i(K) : (K / kQK) * kActStride;
    L.act_bs = L.act_d + align16i(nbw * 4);
    const int nbs_bytes = (wt == 2) ? (K / kQK8) * 4 : (K / 16) * 2;
    L.partial = L.act_bs + align16i(nbs_bytes);
    L.regions = L.partial + align16i(rows * nbw * 4);
    L.region_bytes = region_bytes;
    L.total = L.regions + nwaves * region_bytes;
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

// Number of whole tasks (row-major (row, block) order) inside the first E
// bytes of the workgroup's rows.
__device__ __forceinline__ int tasks_within(int E, int nb, int rb, int bb) {
    const int r = E / rb;
    const int k = (E - r * rb) / bb;
    return r * nb + (k < nb ? k : nb);
}

template <int WT>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint8_t* __restrict__ W, int N, int K, int64_t wbytes, const float* __restrict__ x,
    float* __restrict__ y, uint8_t* __restrict__ xq_out, int rows_per_wg, int region_bytes, int x_vec) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int BB = WFmt<WT>::kBlk;
    constexpr int QV = WFmt<WT>::kVals;
    constexpr int LPT = (WT == 2) ? 1 : 2;    // lanes per task
    constexpr int GPW = 64 / LPT;             // tasks per wave round
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
    const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
    const int nthr = 64 * nw;
    const int nb = K / QV;
    const int rb = nb * BB;
    const int n0 = blockIdx.x * rows_per_wg;
    const int rows = min(rows_per_wg, N - n0);
    const GemvLayout L = gemv_layout(WT, K, rows_per_wg, region_bytes, nw);
    int8_t* act_qs = (int8_t*)(smem + L.act_qs);
    float* act_d = (float*)(smem + L.act_d);
    int16_t* act_bs = (int16_t*)(smem + L.act_bs);
    uint32_t* act_ds = (uint32_t*)(smem + L.act_bs);  // Q8_1: binary16 d | s << 16 per block
    float* partial = (float*)(smem + L.partial);
    uint8_t* region = smem + L.regions + wave * region_bytes;

    // ---- 1. x loads.  Loads are unconditional (addresses clamped into the
    // buffers) so the code stays straight-line and each wait counts only the
    // loads it needs.  The vector L1 returns data in order, so every wave's x
    // loads are queued before any weight load of the workgroup: a bare
    // s_barrier (no memory wait) separates the two.
    const int xsteps = (K + kQK - 1) / kQK;  // 256 values per wave step
    float4 xv[kXPre];
#pragma unroll
    for (int r = 0; r < kXPre; ++r) {
        const int e = min((wave + nw * r) * kQK + 4 * lane, K - 4);
        const float* src = x + e;
        xv[r] = x_vec ? *(const float4*)src : make_float4(src[0], src[1], src[2], src[3]);
    }
    __builtin_amdgcn_s_barrier();

    // ---- 2. every weight load of this wave's span
    const int ntask = rows * nb;
    const int t0 = (int)((int64_t)ntask * wave / nw);
    const int t1 = (int)((int64_t)ntask * (wave + 1) / nw);
    int sb0, sb1;
    task_span(t0, t1, nb, rb, BB, &sb0, &sb1);
    const int64_t s0 = (int64_t)n0 * rb;
    const int64_t wc0 = (s0 + sb0) >> 4;
    const int64_t wc1 = (t1 > t0) ? ((s0 + sb1 + 15) >> 4) : wc0;
    const int64_t full = wbytes >> 4;
    uint4 buf[kLMax];
#pragma unroll
    for (int i = 0; i < kLMax; ++i) {
        // past the span: the wave's last chunk again (one cache line, no new traffic)
        const int64_t c = max(min(wc0 + lane + 64 * i, min(wc1, full) - 1), (int64_t)0);
        buf[i] = *(const uint4*)(W + 16 * c);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. quantize x into LDS
    if (WT != 2) {
        const int nsb = K / kQK;
#pragma unroll
        for (int r = 0; r < kXPre; ++r) {
            const int sb = wave + nw * r;
            if (sb < nsb) {
                const Q8KLane q = q8k_quant_lane(xv[r], lane);
                *(uint32_t*)(act_qs + sb * kActStride + 4 * lane) = q.q4;
                if (lane == 0) act_d[sb] = q.d;
                if ((lane & 3) == 0) act_bs[sb * 16 + (lane >> 2)] = (int16_t)q.bsum;
            }
        }
        for (int sb = wave + nw * kXPre; sb < nsb; sb += nw) {
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
            if (wave + nw * r < xsteps) quant_step(wave + nw * r, xv[r]);
        for (int stp = wave + nw * kXPre; stp < xsteps; stp += nw) {
            const int e = stp * kQK + 4 * lane;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < K) {
                const float* src = x + e;
                v = x_vec ? *(const float4*)src : make_float4(src[0], src[1], src[2], src[3]);
            }
            quant_step(stp, v);
        }
    }
    lds_barrier();  // quantized x visible to every wave; weights keep streaming

    // ---- 4. park this wave's bytes in its region and compute its tasks
    const int rbase = (int)(s0 - 16 * wc0);  // LDS byte of task byte o: region + rbase + o
    const int grp = lane / LPT, sub = lane % LPT;
    int next = t0;
    int tr = (t0 + grp) / nb, tb = (t0 + grp) - ((t0 + grp) / nb) * nb;  // this lane's task (row, block)
    auto advance = [&](int adv) {
        next += adv;
        tb += adv;
        while (tb >= nb) { tb -= nb; ++tr; }
    };
    auto compute_task = [&](int r, int blk) {
        const uint8_t* bp = region + rbase + __mul24(r, rb) + __mul24(blk, BB);
        if (WT == 0) {
            // lane half hf: sub-blocks 4hf..4hf+3 = qs bytes [64hf, 64hf+64)
            const int hf = sub;
            const uint4 hdr = *(const uint4*)bp;
            uint32_t qw[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = *(const uint4*)(bp + 16 + 64 * hf + 16 * i);
                qw[4 * i] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
            }
            const int8_t* ab = act_qs + __mul24(blk, kActStride) + 128 * hf;
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
                    const uint32_t w = qw[8 * c + i];
                    P[2 * c] = sdot4((int)(w & 0x0F0F0F0Fu), (int)av[16 * c + i], P[2 * c]);
                    P[2 * c + 1] = sdot4((int)((w >> 4) & 0x0F0F0F0Fu), (int)av[16 * c + 8 + i], P[2 * c + 1]);
                }
            const uint32_t sw = hf ? hdr.z : hdr.y;             // scales bytes 4hf..4hf+3
            const uint32_t mw = hdr.w >> (16 * hf);             // min high nibbles, 2 bytes
            const uint4 bsv = *(const uint4*)(act_bs + blk * 16 + 8 * hf);
            const uint32_t bw[4] = {bsv.x, bsv.y, bsv.z, bsv.w};
            int S = 0, Mn = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sj = (sw >> (8 * j)) & 0xFF;
                const uint32_t mh = (mw >> (4 * j)) & 15;
                const int m = (int)((sj >> 6) | (mh << 2));
                const int bs32 = (int)(int16_t)(bw[j] & 0xFFFF) + (int)(int16_t)(bw[j] >> 16);
                S += __mul24((int)(sj & 63), P[j]);
                Mn += __mul24(m, bs32);
            }
            S += dppi<0xB1>(S);
            Mn += dppi<0xB1>(Mn);
            if (hf == 0) {
                const float d = half_bits_to_float(hdr.x & 0xFFFF);
                const float dmin = half_bits_to_float(hdr.x >> 16);
                const float t1f = d * (float)S;
                const float t2f = dmin * (float)Mn;
                const float t3f = t1f - t2f;
                partial[__mul24(r, nb) + blk] = act_d[blk] * t3f;
            }
        } else if (WT == 1) {
            // lane half h: values 128h..128h+127 (sub-blocks 8h..8h+7)
            const int h = sub;
            uint32_t ql[16], qh[8];
            lds_read32_a2(bp + 64 * h, ql);
            lds_read32_a2(bp + 64 * h + 32, ql + 8);
            lds_read32_a2(bp + 128 + 32 * h, qh);
            const uint16_t* scp = (const uint16_t*)(bp + 192 + 8 * h);
            const uint32_t sc01 = scp[0], sc23 = scp[1], sc45 = scp[2], sc67 = scp[3];
            const int8_t* ab = act_qs + __mul24(blk, kActStride) + 128 * h;
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
                    const uint32_t l = ql[4 * k + i];
                    const uint32_t hq = qh[4 * (k & 1) + i];
                    const int sa = 2 * (k >> 1), sb = 2 * (2 + (k >> 1));
                    const uint32_t qa = (l & 0x0F0F0F0Fu) | (((hq >> sa) & 0x03030303u) << 4);
                    const uint32_t qb = ((l >> 4) & 0x0F0F0F0Fu) | (((hq >> sb) & 0x03030303u) << 4);
                    I[k] = sdot4((int)qa, (int)av[4 * k + i], I[k]);
                    I[4 + k] = sdot4((int)qb, (int)av[16 + 4 * k + i], I[4 + k]);
                }
            const uint4 bsv = *(const uint4*)(act_bs + blk * 16 + 8 * h);
            const uint32_t bw[4] = {bsv.x, bsv.y, bsv.z, bsv.w};
            const uint32_t scw[4] = {sc01, sc23, sc45, sc67};
            int S = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int bsj = (int)(int16_t)((bw[j >> 1] >> (16 * (j & 1))) & 0xFFFF);
                const int scj = (int)(int8_t)((scw[j >> 1] >> (8 * (j & 1))) & 0xFF);
                S += __mul24(scj, I[j] - 32 * bsj);
            }
            S += dppi<0xB1>(S);
            if (h == 0) {
                const float d = half_bits_to_float(*(const uint16_t*)(bp + 208));
                const float t1f = d * (float)S;
                partial[__mul24(r, nb) + blk] = act_d[blk] * t1f;
            }
        } else {
            uint32_t qw[8];
            lds_read32_a2(bp + 2, qw);
            const uint4 a0 = *(const uint4*)(act_qs + blk * kQK8);
            const uint4 a1 = *(const uint4*)(act_qs + blk * kQK8 + 16);
            const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            int I = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) I = sdot4((int)qw[i], (int)av[i], I);
            const float dw = half_bits_to_float(*(const uint16_t*)bp);
            const float sc = dw * act_d[blk];
            partial[__mul24(r, nb) + blk] = sc * (float)I;
        }
    };

#pragma unroll
    for (int st = 0; st < kLMax / kStepLoads; ++st) {
#pragma unroll
        for (int j = 0; j < kStepLoads; ++j) {
            const int i = kStepLoads * st + j;
            const int64_t c = wc0 + lane + 64 * i;
            if (c < wc1) {
                uint4 v = buf[i];
                if (c >= full) {  // the buffer's last partial chunk (last wave of the grid only)
                    uint32_t wv[4] = {0, 0, 0, 0};
                    for (int bi = 0; bi < 16; ++bi) {
                        const int64_t a = 16 * c + bi;
                        if (a < wbytes) wv[bi >> 2] |= (uint32_t)W[a] << (8 * (bi & 3));
                    }
                    v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                }
                *(uint4*)(region + 16 * (int)(c - wc0)) = v;
            }
        }
        // LDS operations of one wave complete in order: the parked bytes are
        // visible to this wave's later reads without a barrier.
        const int E = (int)(16 * (wc0 + 64 * kStepLoads * (st + 1)) - s0);
        const int ready = min(t1, tasks_within(E, nb, rb, BB));
        while (next < ready) {
            const int cnt = min(GPW, ready - next);
            if (grp < cnt) compute_task(tr, tb);
            advance(cnt);
        }
    }
    lds_barrier();

    // ---- 5. rows: blocks summed in ascending order from 0
    for (int r = tid; r < rows; r += nthr) {
        const float* p = partial + r * nb;
        float acc = 0.0f;
        int b = 0;
        if ((nb & 3) == 0) {
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
        }
        for (; b < nb; ++b) acc = acc + p[b];
        y[n0 + r] = acc;
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

struct GemvPlan {
    int rows;          // rows per workgroup
    int waves;         // waves per workgroup
    int region_bytes;  // LDS bytes per wave region
    int lds;           // dynamic LDS bytes
    bool ok;
};

// Largest per-wave span (bytes, incl. 16-byte alignment slack) for a given
// rows-per-workgroup and wave count, by walking the task split the kernel uses.
static int max_wave_span(int rows, int nb, int rb, int bb, int nw) {
    const int ntask = rows * nb;
    int best = 0;
    for (int w = 0; w < nw; ++w) {
        const int t0 = (int)((int64_t)ntask * w / nw);
        const int t1 = (int)((int64_t)ntask * (w + 1) / nw);
        int b0, b1;
        task_span(t0, t1, nb, rb, bb, &b0, &b1);
        best = b1 - b0 > best ? b1 - b0 : best;
    }
    return best;
}

// About one workgroup per CU, with just enough waves that each wave computes
// its tasks in one pass (a pass costs the same instructions however many of
// its lanes hold a task); more waves only when a wave's span would not fit
// its chunk budget, fewer rows when the workgroup would not fit LDS.
static GemvPlan gemv_plan(int wt, int64_t N, int64_t K) {
    GemvPlan p;
    const int bb = block_bytes_of(wt);
    const int nb = (int)(K / block_vals_of(wt));
    const int rb = nb * bb;
    const int gpw = (wt == 2) ? 64 : 32;  // tasks per wave pass (64 lanes / lanes per task)
    int rows = (int)((N + num_cus() - 1) / num_cus());
    if (rows < 1) rows = 1;
    for (;;) {
        const int ntask = rows * nb;
        int nw = (ntask + gpw - 1) / gpw;
        nw = nw < 1 ? 1 : (nw > kGemvWaves ? kGemvWaves : nw);
        int span = max_wave_span(rows, nb, rb, bb, nw);
        while (nw < kGemvWaves && span + 32 > kLMax * 64 * 16) span = max_wave_span(rows, nb, rb, bb, ++nw);
        const int region = align16i(span + 32) + 32;  // alignment slack + over-read slack
        const GemvLayout L = gemv_layout(wt, (int)K, rows, region, nw);
        const bool fits = span + 32 <= kLMax * 64 * 16 && (size_t)L.total <= kMaxLds;
        if (fits || rows == 1) {
            p.rows = rows;
            p.waves = nw;
            p.region_bytes = region;
            p.lds = L.total;
            p.ok = fits;
            return p;
        }
        --rows;
    }
}

size_t gemv_lds_bytes(int wtype, int64_t N, int64_t K) {
    const GemvPlan p = gemv_plan(wtype, N, K);
    return p.ok ? (size_t)p.lds : (size_t)-1;
}

template <int WT>
static hipError_t launch_gemv_t(const uint8_t* W, int64_t N, int64_t K, const float* x, float* y,
                                uint8_t* xq_out, hipStream_t st) {
    static bool attr_set = false;
    const GemvPlan p = gemv_plan(WT, N, K);
    if (!p.ok) return hipErrorInvalidValue;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemv_kernel<WT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int rb = (int)(K / WFmt<WT>::kVals) * WFmt<WT>::kBlk;
    const int grid = (int)((N + p.rows - 1) / p.rows);
    const int x_vec = (((uintptr_t)x) & 15) == 0;
    gemv_kernel<WT><<<grid, 64 * p.waves, p.lds, st>>>(W, (int)N, (int)K, (int64_t)N * rb, x, y, xq_out,
                                                        p.rows, p.region_bytes, x_vec);
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
