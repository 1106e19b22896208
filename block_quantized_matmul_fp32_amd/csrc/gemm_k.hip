// gemm_k.hip -- prefill GEMM Y = X * W^T on int8 MFMA for gfx950 with K-quant
// weights (Q4_K, Q5_K, Q6_K) and Q8_K activations, and its routed-expert
// (MUL_MAT_ID) variant.
//
// Pages: vllm.cpp PR #3035 "scope a cooperative activation share for the WMMA
// kernels" (one activation tile per block, loaded once and shared by all of
// its waves, instead of a private copy per warp); strix-llama.cpp PR #18
// "Optimize ROCM Prefill and Decode", commits "MMQ register prefetch" (the
// next 256-wide K step is already in flight while the current one is
// consumed), "routed-compact" (MUL_MAT_ID tiles sized from the rows each
// expert receives) and the overview's determinism note (results of a call do
// not depend on timing).
//
// gfx950 design:
//  * Y tile = activations (MFMA A, rows m) x weights (MFMA B, columns n) on
//    v_mfma_i32_32x32x32_i8.  A lane's output column is its own weight row,
//    so the weight scales d, dmin are per-lane scalars in the epilogue.
//  * A workgroup is four waves over a 128-row weight tile: wave w owns
//    weight rows 32w..32w+31, lane (n, h) half h of each 32-wide K chunk's
//    sub-block piece.  Every wave runs all MT 32-row activation tiles
//    (BM = 32 MT activation rows per workgroup).
//  * Per 256-wide K step: the activation tile (int8 Q8_K bytes, XOR-swizzled
//    rows) and its scales are copied HBM -> LDS by the LDS-DMA path
//    (global_load_lds) into one of two distinct buffers, and each lane's raw
//    weight block bytes are loaded straight into its registers by buffer
//    loads, both one step ahead; one barrier per step.
//  * The per-sub-block integer scales are folded into two int8 weight
//    operands ("planes"), unpacked once per step and reused by all MT tiles,
//    so a super-block is two int32 MFMA accumulations per tile:
//      Q4_K: sc (6 bit) = 8 hi + lo; planes q lo, q hi (<= 105); S = 8 R1 + R0.
//      Q5_K: planes of the centred q - 16 times the two 3-bit scale digits;
//            S = 8 R1 + R0 + 16 sum_j sc_j bsum32_j, the last term on a
//            second binary16 MFMA.
//      Q6_K: P = sc (q - 32) in 16-bit lanes, planes P mod 256 (as int8)
//            and (P + 128) >> 8 in [-16, 16]; S = 256 R1 + R0.
//    The integer sums are exact.  The Q4_K/Q5_K min term
//    Mn = sum_j m_j (bsum_2j + bsum_2j+1) runs on one
//    v_mfma_f32_32x32x16_f16 per tile (m_j <= 63 and |bsum| <= 2032 are exact
//    in binary16, the products and the sum of 16 are exact in binary32).
//  * Epilogue per output and super-block: y += da (d S - dmin Mn) in
//    binary32 with fused multiply-adds; the fp32 order is the kernel's own
//    and fixed, so two runs are bitwise equal.
//  * Split K (deterministic): a grid with too few tiles to fill the chip
//    splits the super-block range into S parts; each part writes its fp32
//    partial tile to the workspace, and the part that arrives last (a
//    per-tile counter) adds the S partials in part order 0..S-1 and stores Y.
//    The sum order is fixed whichever part arrives last; the counter is
//    reset to zero by that part.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <type_traits>

#include "vq_device.h"
#include "vq_internal.h"

namespace vqk {
namespace kq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBN = 128;  // weight rows per workgroup (four waves of 32)
constexpr int kKS = 256;  // K per step (one super-block)

// The four bytes of v times f, when every byte product lies in [0, 255]: one
// packed 16-bit multiply (the low byte of a 16-bit lane cannot carry into the
// high byte, and the high byte's product stays below 2^16).
__device__ __forceinline__ uint32_t bytes_mul_u(uint32_t v, uint32_t f2) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(us2, v) * __builtin_bit_cast(us2, f2));
}

// Q6_K plane bytes ((q - 32) * dg) mod 256 for four 6-bit quants q (bytes of
// v), dg in [-3, 4]: in each 16-bit lane L = qa + 256 qb,
//   L * dg + (128 - 32 dg) * 257 = ((qa-32) dg + 128) + 256 ((qb-32) dg + 128)
// with both brackets in [0, 252], so no carry crosses a byte and the modular
// 16-bit arithmetic is exact; xor 0x80 then removes the +128 bias of each
// byte (as a signed byte).  mul2 = dg in both halves, add2 = (128 - 32 dg) * 257
// in both halves.
__device__ __forceinline__ uint32_t q6_plane(uint32_t v, uint32_t mul2, uint32_t add2) {
    const us2 r = __builtin_bit_cast(us2, v) * __builtin_bit_cast(us2, mul2) + __builtin_bit_cast(us2, add2);
    return __builtin_bit_cast(uint32_t, r) ^ 0x80808080u;
}

__device__ __forceinline__ uint32_t pair16(uint32_t x) { return (x & 0xFFFFu) * 0x10001u; }

// Raw buffer loads of weight bytes: a buffer resource over [base, base +
// bytes) (bytes < 2^32; reads outside it return zeros instead of faulting),
// a 32-bit per-lane offset and a uniform (SGPR) offset.  The loads need not
// be 16-byte aligned: the 2-byte aligned Q6_K fields are read with one
// dwordx4 each.
typedef __amdgpu_buffer_rsrc_t WRsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ WRsrc make_wrsrc(const uint8_t* base, int64_t bytes) {
    const int64_t n = bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(uint32_t)n, kRsrcWord3);
}
__device__ __forceinline__ u4v bload16(WRsrc r, uint32_t off, uint32_t soff) {
    return __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ uint2 bload8(WRsrc r, uint32_t off, uint32_t soff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ uint32_t bload2(WRsrc r, uint32_t off, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, (int)soff, 0);
}

// Buffer loads of 16 or 4 bytes per lane straight into LDS (lane i's bytes
// at lds + 16 i or lds + 4 i), at byte offset voff + soff of the resource;
// reads past the resource's range return zeros.  Device pass only (the host
// pass of this single-source file sees kernel bodies but compiles none of
// them).
__device__ __forceinline__ void bload16_lds(WRsrc r, lds_void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, (int)voff, (int)soff, 0, 0);
#else
    (void)r;
    (void)lds;
    (void)voff;
    (void)soff;
#endif
}
__device__ __forceinline__ void bload4_lds(WRsrc r, lds_void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, (int)voff, (int)soff, 0, 0);
#else
    (void)r;
    (void)lds;
    (void)voff;
    (void)soff;
#endif
}

// Orders a computation after `dep`: x passes through an empty asm that also
// reads dep, so nothing that depends on x can be scheduled before dep is
// complete.  The asm exists in the device pass only (the host pass of this
// single-source file sees kernel bodies but compiles none of them).
template <typename D>
__device__ __forceinline__ void order_after(int& x, const D& dep) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x) : "v"(dep));
#else
    (void)x;
    (void)dep;
#endif
}

// Row indirection of the routed-expert variant.
struct GroupArgs {
    const int32_t* tiles;   // [ntiles][4]: expert, first list slot, rows, 0
    const int32_t* ntiles;  // device count of valid tiles
    const int32_t* list;    // pair indices grouped per expert
    int top_k;
    int per_row;            // 1: pair p reads activation row p; 0: row p / top_k
    int64_t expert_stride;  // bytes of one expert's [N][K/256] blocks
};

struct Args {
    const uint8_t* W;       // weight blocks (expert 0 for the grouped variant)
    int N, K;
    const int8_t* aqs;      // planar Q8_K activation: qs [rows][K]
    const float* ad;        // d [rows][K/256]
    const int16_t* abs;     // bsums [rows][K/16]
    int M;                  // activation rows (dense)
    float* Y;
    int64_t ldy;
    float* part;            // split-K partial tiles, [tile][split][threads][MT*16]
    int* cnt;               // split-K arrival counters, [tile]
    int splits;             // S
    int nblk_n;             // weight-row blocks
    int nblk_m;             // activation-row blocks (dense) or routed tiles (grouped)
};

// 8 x 16-bit from the two 16-bit halves of each dword of four dwords:
// v_perm byte selectors.
constexpr uint32_t kSelEven = 0x0C020C00u;  // bytes 0, 2 -> low bytes of the two 16-bit lanes
constexpr uint32_t kSelOdd = 0x0C030C01u;   // bytes 1, 3
constexpr uint32_t kSelPack = 0x06020400u;    // low bytes of (even lanes, odd lanes) -> 4 bytes in order
constexpr uint32_t kSelPackHi = 0x07030501u;  // high bytes of (even lanes, odd lanes) -> 4 bytes in order

// Plane bytes of one 16-value piece (four dwords of quants, one per 4 values)
// for the two planes of each weight type, and the per-lane constants of a
// step.  Lane (n, h) of a wave holds weight row n and half h of each
// super-block; its chunk c (0..7) is values 128h + 16c .. 128h + 16c + 15.
//   Q4_K: q in [0,15] (4-bit), sub-block (32 values) 4h + c/2 with 6-bit sc =
//         8 hi + lo; planes q*lo and q*hi (<= 105); S = 8 R1 + R0.
//   Q5_K: q in [0,31]; centred q' = q - 16 in [-16,15]; planes q'*lo and
//         q'*hi (|.| <= 112, built as biased 16-bit products); S' = 8 R1 + R0
//         and S = S' + 16 sum_j sc_j bsum32_j, the second term on an exact
//         binary16 MFMA.
//   Q6_K: q in [0,63], sub-block (16 values) 8h + c with int8 sc; the
//         product P = sc (q - 32) in [-4096, 4064] is split P = 256 hi + lo
//         with lo = P mod 256 read as int8 and hi = (P + 128) >> 8 in
//         [-16, 16] (the high byte of P + 128, formed in the same 16-bit
//         multiply-add); S = 256 R1 + R0.
template <int WT>
struct Unpack;

// Weights in registers: W is the workgroup's first row of this step's blocks
// (a uniform pointer), `off` the lane's 32-bit byte offset of its row.
template <>
struct Unpack<0> {
    static constexpr int RAW = 5;  // 16-byte pieces per lane and step
    static constexpr int SH = 3;   // S = (R1 << SH) + R0
    static __device__ __forceinline__ void load(WRsrc W, uint32_t off, uint32_t soff, int h, u4v (&raw)[8]) {
        raw[0] = bload16(W, off, soff);
#pragma unroll
        for (int k = 0; k < 4; ++k) raw[1 + k] = bload16(W, off + 16 + 64 * h + 16 * k, soff);
    }
    static __device__ __forceinline__ void unpack(const u4v (&raw)[8], int h, v4i (&pl)[8][2], float& d, float& dmin,
                                                  h8& mco, h8& sco) {
        const u4v hd = raw[0];
        d = half_bits_to_float(hd.x & 0xFFFF);
        dmin = half_bits_to_float(hd.x >> 16);
        const uint32_t scw = h ? hd.z : hd.y;
        const uint32_t mhw = hd.w >> (16 * h);
        uint32_t flo[4], fhi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b = (scw >> (8 * j)) & 0xFF;
            const uint32_t sc = b & 63;
            const uint32_t mm = (b >> 6) | (((mhw >> (4 * j)) & 15) << 2);
            flo[j] = (sc & 7) * 0x10001u;
            fhi[j] = (sc >> 3) * 0x10001u;
            const _Float16 mf = (_Float16)(float)mm;
            mco[2 * j] = mf;
            mco[2 * j + 1] = mf;
        }
        (void)sco;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // nibble bytes 32(c/4) + 16(c%2) of the lane's 64, nibble (c/2)%2; sub-block c/2
            const u4v nb = raw[1 + 2 * (c >> 2) + (c & 1)];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t v = ((c >> 1) & 1) ? ((nb[k] >> 4) & 0x0F0F0F0Fu) : (nb[k] & 0x0F0F0F0Fu);
                pl[c][0][k] = (int)bytes_mul_u(v, flo[c >> 1]);
                pl[c][1][k] = (int)bytes_mul_u(v, fhi[c >> 1]);
            }
        }
    }
};

template <>
struct Unpack<3> {
    static constexpr int RAW = 7;
    static constexpr int SH = 3;
    static __device__ __forceinline__ void load(WRsrc W, uint32_t off, uint32_t soff, int h, u4v (&raw)[8]) {
        raw[0] = bload16(W, off, soff);
        raw[1] = bload16(W, off + 16, soff);
        raw[2] = bload16(W, off + 32, soff);
#pragma unroll
        for (int k = 0; k < 4; ++k) raw[3 + k] = bload16(W, off + 48 + 64 * h + 16 * k, soff);
    }
    static __device__ __forceinline__ void unpack(const u4v (&raw)[8], int h, v4i (&pl)[8][2], float& d, float& dmin,
                                                  h8& mco, h8& sco) {
        const u4v hd = raw[0];
        d = half_bits_to_float(hd.x & 0xFFFF);
        dmin = half_bits_to_float(hd.x >> 16);
        const uint32_t scw = h ? hd.z : hd.y;
        const uint32_t mhw = hd.w >> (16 * h);
        uint32_t mlo[4], mhi[4], alo[4], ahi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b = (scw >> (8 * j)) & 0xFF;
            const uint32_t sc = b & 63;
            const uint32_t mm = (b >> 6) | (((mhw >> (4 * j)) & 15) << 2);
            const uint32_t lo = sc & 7, hi = sc >> 3;
            mlo[j] = lo * 0x10001u;
            mhi[j] = hi * 0x10001u;
            // (q - 16) dg + 128 = q dg + (128 - 16 dg) in [16, 233] for dg in [0, 7]
            alo[j] = (128u - 16u * lo) * 0x01010101u;
            ahi[j] = (128u - 16u * hi) * 0x01010101u;
            const _Float16 mf = (_Float16)(float)mm;
            mco[2 * j] = mf;
            mco[2 * j + 1] = mf;
            const _Float16 sf = (_Float16)(float)(16 * sc);
            sco[2 * j] = sf;
            sco[2 * j + 1] = sf;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u4v nb = raw[3 + 2 * (c >> 2) + (c & 1)];
            const u4v qh = raw[1 + (c & 1)];
            const int bit = 4 * h + (c >> 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t v = ((c >> 1) & 1) ? ((nb[k] >> 4) & 0x0F0F0F0Fu) : (nb[k] & 0x0F0F0F0Fu);
                v |= ((qh[k] >> bit) & 0x01010101u) << 4;
                pl[c][0][k] = (int)q6_plane(v, mlo[c >> 1], alo[c >> 1]);
                pl[c][1][k] = (int)q6_plane(v, mhi[c >> 1], ahi[c >> 1]);
            }
        }
    }
};

template <>
struct Unpack<1> {
    static constexpr int RAW = 8;  // ql 4, qh 2, sc and d in one
    static constexpr int SH = 8;
    static __device__ __forceinline__ void load(WRsrc W, uint32_t off, uint32_t soff, int h, u4v (&raw)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) raw[k] = bload16(W, off + 64 * h + 16 * k, soff);
        raw[4] = bload16(W, off + 128 + 32 * h, soff);
        raw[5] = bload16(W, off + 144 + 32 * h, soff);
        const uint2 sc = bload8(W, off + 192 + 8 * h, soff);
        raw[6] = (u4v){sc.x, sc.y, bload2(W, off + 208, soff), 0u};
    }
    static __device__ __forceinline__ void unpack(const u4v (&raw)[8], int h, v4i (&pl)[8][2], float& d, float& dmin,
                                                  h8& mco, h8& sco) {
        (void)h;
        (void)mco;
        (void)sco;
        d = half_bits_to_float(raw[6].z & 0xFFFF);
        dmin = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // ql bytes 16(c%4) of the lane's 64, nibble c/4; qh bytes 16(c%2) of its 32, pair c/2
            const int sc = (int)(int8_t)((((c < 4) ? raw[6].x : raw[6].y) >> (8 * (c & 3))) & 0xFF);
            const uint32_t f = pair16((uint32_t)sc);
            const uint32_t a = pair16((uint32_t)(128 - 32 * sc));
            const u4v ql = raw[c & 3];
            const u4v qh = raw[4 + (c & 1)];
            const int pr = c >> 1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = (c >> 2) ? ((ql[k] >> 4) & 0x0F0F0F0Fu) : (ql[k] & 0x0F0F0F0Fu);
                const uint32_t hs = (pr == 3) ? (qh[k] >> 2) : (qh[k] << (4 - 2 * pr));
                const uint32_t q6 = (hs & 0x30303030u) | lo;
                const uint32_t ev = __builtin_amdgcn_perm(0u, q6, kSelEven);
                const uint32_t od = __builtin_amdgcn_perm(0u, q6, kSelOdd);
                // P + 128 = sc q - 32 sc + 128 in 16-bit lanes (exact: it
                // lies in [-3968, 4192]); its low byte xor 0x80 is P mod 256,
                // its high byte (P + 128) >> 8
                const uint32_t pe = __builtin_bit_cast(
                    uint32_t, __builtin_bit_cast(us2, ev) * __builtin_bit_cast(us2, f) + __builtin_bit_cast(us2, a));
                const uint32_t po = __builtin_bit_cast(
                    uint32_t, __builtin_bit_cast(us2, od) * __builtin_bit_cast(us2, f) + __builtin_bit_cast(us2, a));
                pl[c][0][k] = (int)(__builtin_amdgcn_perm(po, pe, kSelPack) ^ 0x80808080u);
                pl[c][1][k] = (int)__builtin_amdgcn_perm(po, pe, kSelPackHi);
            }
        }
    }
};

template <int WT>
struct KQ2 {
    static constexpr bool kMin = (WT == 0 || WT == 3);  // Q4_K, Q5_K: the min term
    static constexpr bool kSc = (WT == 3);              // Q5_K: the centring term
    static constexpr int BB = (WT == 0) ? 144 : ((WT == 1) ? 210 : 176);
};

// Workgroup of four waves; wave w owns weight rows 32w..32w+31 of the
// 128-row tile (their raw blocks go straight into its lanes' registers) and
// all MT 32-row activation tiles (BM = 32 MT rows, one activation tile in LDS
// shared by the four waves).  Per step: unpack the planes of the whole
// super-block once, then each activation tile in turn: 16 MFMAs (two planes
// x eight 32-wide chunks), the binary16 min/centring MFMAs and the epilogue.
// kMode: 0 dense; 1 routed rows with 32-bit activation offsets (rows * K
// below 2^31, checked by the host); 2 routed rows with 64-bit offsets.
// Two workgroups per CU.
template <int WT, int MT, int kMode>
__global__ __launch_bounds__(256, 2) void gemm_kq2_kernel(Args a, GroupArgs ga) {
    constexpr bool kGrouped = kMode != 0;
    using U = Unpack<WT>;
    using T = KQ2<WT>;
    constexpr int NT = 256;
    constexpr int BM = 32 * MT;
    constexpr int NAI = BM / 4;         // activation DMA instructions per step (4 rows each)
    constexpr int AIPW = (NAI + 3) / 4; // per wave
    constexpr int NDI = (BM + 63) / 64; // d DMA instructions per step
    constexpr bool kMin = T::kMin;
    constexpr bool kB16 = T::kMin;      // binary16 bsums needed
    constexpr int BSI = kB16 ? BM * 2 : 0;

    __shared__ __attribute__((aligned(16))) int8_t sA0[BM * kKS];
    __shared__ __attribute__((aligned(16))) int8_t sA1[BM * kKS];
    // the d DMA writes 64 floats per instruction: NDI * 64 >= BM (96-row tiles: 128)
    __shared__ __attribute__((aligned(16))) float sD0[64 * NDI];
    __shared__ __attribute__((aligned(16))) float sD1[64 * NDI];
    __shared__ __attribute__((aligned(16))) _Float16 sB0[kB16 ? BM * 16 : 8];
    __shared__ __attribute__((aligned(16))) _Float16 sB1[kB16 ? BM * 16 : 8];
    __shared__ int sRow[BM];
    // byte offset of each bsum-loading thread's piece (32-bit offsets): read
    // from LDS every step instead of held in a register across the loop
    __shared__ uint32_t sBo[(kB16 && kMode != 2) ? 256 : 1];
    __shared__ int sOut[BM];
    __shared__ int sLast;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    // activation byte offsets: 32-bit while the host keeps rows * K below
    // 2^31 (one launch of the dense GEMM, most routed calls), else 64-bit
    using AOff = typename std::conditional<kMode == 2, uint64_t, uint32_t>::type;

    // One output unit: weight-row block nb, activation-row block (or routed
    // tile) mb, K part sp.
    auto run_unit = [&](const int nb, const int mb, const int sp) __attribute__((always_inline)) {
    const int n0 = nb * kBN;
    const int nsteps_all = a.K / kKS;
    const int s_begin = (int)(((int64_t)nsteps_all * sp) / a.splits);
    const int s_end = (int)(((int64_t)nsteps_all * (sp + 1)) / a.splits);
    const int nst = s_end - s_begin;

    const uint8_t* W = a.W;
    int rows_here;  // valid activation rows of this tile (uniform)
    if (kGrouped) {
        const int tix = mb;
        const int e = ga.tiles[4 * tix + 0];
        const int first = ga.tiles[4 * tix + 1];
        const int rows = ga.tiles[4 * tix + 2];
        rows_here = rows;
        W = a.W + (int64_t)e * ga.expert_stride;
        for (int r = tid; r < BM; r += NT) {
            if (r < rows) {
                const int p = ga.list[first + r];
                sRow[r] = ga.per_row ? p : p / ga.top_k;
                sOut[r] = p;
            } else {
                sRow[r] = -1;
                sOut[r] = -1;
            }
        }
    } else {
        const int m0 = mb * BM;
        rows_here = min(BM, a.M - m0);
        for (int r = tid; r < BM; r += NT) {
            const int m = m0 + r;
            sRow[r] = (m < a.M) ? m : -1;
            sOut[r] = (m < a.M) ? m : -1;
        }
    }
    rows_here = __builtin_amdgcn_readfirstlane(rows_here);
    // 32-row activation tiles that hold a valid row (the rest are skipped:
    // their MFMAs and epilogue would only compute padding)
    const int mt_live = (rows_here + 31) / 32;
    __syncthreads();
    if constexpr (kB16 && kMode != 2) {
        // written and later read by the same thread
        if (tid < BSI) {
            int ar = sRow[tid >> 1];
            ar = ar >= 0 ? ar : 0;
            sBo[tid] = (uint32_t)ar * (uint32_t)(a.K / 8) + 16u * (uint32_t)(tid & 1);
        }
    }

    const int nbk = a.K / kKS;
    const int64_t rowbytes = (int64_t)nbk * T::BB;
    // weight rows of this workgroup: lane offset from the first row (< 2^31:
    // 128 rows of one expert)
    const int wn = min(n0 + 32 * wave + l32, a.N - 1);
    const uint8_t* Wg = W + (int64_t)n0 * rowbytes;
    const uint32_t woff = (uint32_t)((int64_t)(wn - n0) * rowbytes);
    const WRsrc wrs = make_wrsrc(Wg, (int64_t)(a.N - n0) * rowbytes);
    // activation DMA: instruction gi = wave + 4 j covers tile rows 4 gi .. 4 gi + 3;
    // lane -> row 4 gi + lane/16, physical chunk lane%16 holding logical chunk
    // (lane%16) ^ (row & 15); 32-bit offsets from the activation base (the host
    // keeps rows * K below 2^31)
    // Routed tiles gather their rows (an offset per instruction); the dense
    // tile's rows are consecutive, so its instruction j is the first one
    // plus 16 j rows: one offset register, and buffer loads whose range ends
    // at the launch's last row (rows past it read zeros, never stored).
    constexpr int kAOffs = (kMode == 0) ? 1 : AIPW;
    AOff aoff[kAOffs];
    if constexpr (kMode == 0) {
        const int r = 4 * wave + (lane >> 4);
        aoff[0] = (uint32_t)(mb * BM + r) * (uint32_t)a.K + 16u * (uint32_t)((lane & 15) ^ (r & 15));
    } else {
#pragma unroll
        for (int j = 0; j < AIPW; ++j) {
            const int gi = wave + 4 * j;
            const int r = 4 * gi + (lane >> 4);
            int ar = (gi < NAI) ? sRow[r] : -1;
            ar = ar >= 0 ? ar : 0;  // rows past the tile read row 0 (never stored)
            aoff[j] = (AOff)ar * (AOff)a.K + (AOff)(16u * (uint32_t)((lane & 15) ^ (r & 15)));
        }
    }
    AOff doff = 0;
    if constexpr (kMode == 2) {
        const int r = 64 * wave + lane;
        int ar = (r < BM) ? sRow[r] : -1;
        ar = ar >= 0 ? ar : 0;
        doff = (AOff)ar * (AOff)nbk;
    }
    AOff boff = 0;
    if (kB16 && kMode == 2) {
        const int r = tid >> 1;
        int ar = (tid < BSI) ? sRow[r] : -1;
        ar = ar >= 0 ? ar : 0;
        boff = (AOff)ar * (AOff)(a.K / 16) + (AOff)(8u * (uint32_t)(tid & 1));
    }

    u4v raw[8];
    uint4 rb = make_uint4(0, 0, 0, 0);
    // the bsums and the scales d of the launch's activation rows (< 2^32
    // bytes while the offsets are 32-bit)
    const WRsrc brs = make_wrsrc((const uint8_t*)a.abs, (int64_t)a.M * (a.K / 16) * 2);
    const WRsrc drs = make_wrsrc((const uint8_t*)a.ad, (int64_t)a.M * nbk * 4);
    const WRsrc ars = make_wrsrc((const uint8_t*)a.aqs, (int64_t)a.M * a.K);
    // Copies of step s: activations and their scales by LDS-DMA into buffer
    // B, bsums and the weight blocks into registers.
    auto issue_act = [&](int s, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        int8_t* sAb = buf ? sA1 : sA0;
        float* sDb = buf ? sD1 : sD0;
#pragma unroll
        for (int j = 0; j < AIPW; ++j) {
            const int gi = wave + 4 * j;
            if constexpr (kMode == 0) {
                if (gi < NAI)
                    // the row part in the lane offset, which the range
                    // check covers; the step offset (< K) in the uniform one
                    bload16_lds(ars, (lds_void*)(sAb + 4 * gi * kKS), aoff[0] + (uint32_t)(16 * j) * (uint32_t)a.K,
                                (uint32_t)s * kKS);
            } else {
                const int8_t* ab = a.aqs + (int64_t)s * kKS;
                if (gi < NAI)
                    __builtin_amdgcn_global_load_lds((const void*)(ab + aoff[j]), (lds_void*)(sAb + 4 * gi * kKS), 16,
                                                     0, 0);
            }
        }
        if (wave < NDI) {
            if constexpr (kMode == 2) {
                __builtin_amdgcn_global_load_lds((const void*)(a.ad + s + doff), (lds_void*)(sDb + 64 * wave), 4, 0,
                                                 0);
            } else {
                // 32-bit offsets: a buffer load into LDS, its row from LDS each
                // step (an address kept across the loop is spilled, and its
                // reload's wait would also wait for the copies just issued)
                const int r = 64 * wave + lane;
                int ar = (r < BM) ? sRow[r] : -1;
                ar = ar >= 0 ? ar : 0;
                bload4_lds(drs, (lds_void*)(sDb + 64 * wave), (uint32_t)ar * (uint32_t)nbk * 4u, (uint32_t)s * 4u);
            }
        }
        if (kB16 && tid < BSI) {
            // 32-bit offsets: a buffer load with a uniform resource
            if constexpr (kMode == 2) {
                rb = *(const uint4*)(a.abs + (int64_t)s * 16 + boff);
            } else {
                // the offset from LDS each step (an offset kept across the
                // loop is spilled, and its reload's wait would also wait for
                // the activation copies just issued)
                rb = __builtin_bit_cast(uint4, bload16(brs, sBo[tid], (uint32_t)s * 32u));
            }
        }
    };
    auto issue_w = [&](int s) __attribute__((always_inline)) {
        U::load(wrs, woff, (uint32_t)(s * T::BB), h, raw);
    };
    auto store_bs = [&](auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        if (kB16 && tid < BSI) {
            _Float16* sBb = buf ? sB1 : sB0;
            const uint32_t ww[4] = {rb.x, rb.y, rb.z, rb.w};
            h8 hv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[2 * i] = (_Float16)(float)(int16_t)(ww[i] & 0xFFFF);
                hv[2 * i + 1] = (_Float16)(float)(int16_t)(ww[i] >> 16);
            }
            *(h8*)(sBb + 8 * tid) = hv;
        }
    };

    v16f y[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) y[t][i] = 0.0f;

    int abase[MT];
    int ax7[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int mrow = 32 * t + l32;
        const int sw = mrow & 15;
        abase[t] = mrow * kKS + 16 * ((8 * h) ^ (sw & 8));
        ax7[t] = sw & 7;
    }

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto step = [&](int i, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        using Bn = std::integral_constant<int, buf ^ 1>;
        // this thread's copies of step i have landed (weights, bsums, DMA)
        __builtin_amdgcn_s_waitcnt(0);
        store_bs(bufc);
        v4i pl[8][2];
        float dw, dmn;
        h8 mco, sco;
        U::unpack(raw, h, pl, dw, dmn, mco, sco);
        __syncthreads();  // everyone's step-i copies are in LDS; step i-1 reads are done
        if (i + 1 < nst) {
            issue_act(s_begin + i + 1, Bn{});
            issue_w(s_begin + i + 1);
        }
        const int8_t* abuf = buf ? sA1 : sA0;
        const _Float16* sBc = buf ? sB1 : sB0;
        const float* sDc = buf ? sD1 : sD0;
        // Activation fragments are read one chunk ahead of their MFMAs.
        v4i av = *(const v4i*)(abuf + abase[0] + 16 * (0 ^ ax7[0]));
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t > 0 && t >= mt_live) break;  // uniform: only padding rows left
            v16i R0 = {}, R1 = {};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                v4i avn = av;
                if (c < 7) avn = *(const v4i*)(abuf + abase[t] + 16 * ((c + 1) ^ ax7[t]));
                R0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, pl[c][0], R0, 0, 0, 0);
                R1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, pl[c][1], R1, 0, 0, 0);
                av = avn;
            }
            const int tb = 32 * t;
            v16f sf;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sf[r] = (float)(int)(((uint32_t)R1[r] << U::SH) + (uint32_t)R0[r]);
            v16f mn = {};
            if (kMin) {
                const h8 bsv = *(const h8*)(sBc + 16 * (tb + l32) + 8 * h);
                if (T::kSc) sf = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsv, sco, sf, 0, 0, 0);
                mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsv, mco, (v16f){}, 0, 0, 0);
            }
            const float* dp = sDc + tb + 4 * h;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float4 da4 = *(const float4*)(dp + 8 * kk);
                const float da[4] = {da4.x, da4.y, da4.z, da4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = 4 * kk + q;
                    float u = dw * sf[r];
                    if (kMin) u = __builtin_fmaf(-dmn, mn[r], u);
                    y[t][r] = __builtin_fmaf(da[q], u, y[t][r]);
                }
            }
            // The next tile's first fragment is read after this epilogue (its
            // address is ordered after all of this tile's outputs), so the
            // compiler keeps one tile's accumulators live, not several.
            if (t + 1 < MT) {
                int nxt = abase[t + 1] + 16 * (0 ^ ax7[t + 1]);
                order_after(nxt, y[t]);
                av = *(const v4i*)(abuf + nxt);
            }
        }
    };

    if (nst > 0) {
        issue_act(s_begin, B0{});
        issue_w(s_begin);
    }
    for (int i = 0; i < nst; i += 2) {
        step(i, B0{});
        if (i + 1 < nst) step(i + 1, B1{});
    }

    // ---- output: lane holds column n0 + 32 wave + l32, rows 32 t + 8 kk + 4 h + q
    const int n = n0 + 32 * wave + l32;
    if (a.splits == 1) {
        if (n < a.N) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int orow = sOut[32 * t + 8 * (r >> 2) + 4 * h + (r & 3)];
                    if (orow >= 0) a.Y[(int64_t)orow * a.ldy + n] = y[t][r];
                }
            }
        }
        return;
    }
    // split K: this part's partial tile, then the arrival count.  The partial
    // stores and loads are device-scope atomics (written through to the
    // memory side, coherent across the XCDs' L2 caches), so no cache-wide
    // write-back fence is needed: every thread waits for its own stores to
    // complete before the barrier that precedes the arrival count.
    const int tile = mb * a.nblk_n + nb;
    float* pbase = a.part + ((int64_t)tile * a.splits) * (NT * MT * 16);
    {
        float* mine = pbase + (int64_t)sp * (NT * MT * 16);
        // only the 32-row tiles that hold a valid row: the others are never
        // read back (a small M leaves most of a 128-row tile as padding)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t > 0 && t >= mt_live) break;  // uniform
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __hip_atomic_store(mine + (t * 16 + r) * NT + tid, y[t][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.cnt + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sLast = (old == a.splits - 1);
    }
    __syncthreads();
    if (!sLast) return;
    // last arrival: the parts in order 0..S-1 (its own from registers)
    float acc[MT][16];
    int z = 0;
    if (mt_live == 1) {
        // one live 32-row tile (small M): the loads of four parts at a time
        // are in flight together, then added in part order
        for (; z + 4 <= a.splits; z += 4) {
            float v[4][16];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float* pz = pbase + (int64_t)(z + k) * (NT * MT * 16);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    v[k][r] = (z + k == sp) ? y[0][r]
                                            : __hip_atomic_load(pz + r * NT + tid, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[0][r] = (z + k == 0) ? v[k][r] : acc[0][r] + v[k][r];
        }
    }
    for (; z < a.splits; ++z) {
        const float* pz = pbase + (int64_t)z * (NT * MT * 16);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t > 0 && t >= mt_live) break;  // uniform: tiles of padding rows were not stored
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float v = (z == sp) ? y[t][r]
                                          : __hip_atomic_load(pz + (t * 16 + r) * NT + tid, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT);
                acc[t][r] = (z == 0) ? v : acc[t][r] + v;
            }
        }
    }
    if (tid == 0) __hip_atomic_store(a.cnt + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n < a.N) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t > 0 && t >= mt_live) break;  // uniform: only padding rows left
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int orow = sOut[32 * t + 8 * (r >> 2) + 4 * h + (r & 3)];
                if (orow >= 0) a.Y[(int64_t)orow * a.ldy + n] = acc[t][r];
            }
        }
    }
    };  // run_unit

    if constexpr (kGrouped) {
        // Routed tiles: the grid is sized to the chip, not to the worst-case
        // tile count; each workgroup takes units blockIdx.x, + gridDim.x, ...
        // (column block fastest) up to the routing's device tile count.
        const int units = __builtin_amdgcn_readfirstlane(*ga.ntiles) * a.nblk_n;
        for (int u = blockIdx.x; u < units; u += gridDim.x) {
            run_unit(u % a.nblk_n, u / a.nblk_n, 0);
            __syncthreads();  // the unit's LDS reads are done before the next unit's writes
        }
    } else {
        // Dense: one unit per workgroup, consecutive units on one XCD
        // (workgroups are dealt to the eight XCDs round-robin); the K parts
        // of a tile are consecutive, so their partial tiles are written and
        // read in one XCD's L2 within a short time.  Tiles run in groups of
        // kGroupN weight-row blocks, activation-row block by block, so the
        // workgroups resident on one XCD at a time share a few weight and a
        // few activation blocks instead of each reading its own weight block.
        const int nwg = a.nblk_n * a.nblk_m * a.splits;
        int g = blockIdx.x;
        if ((nwg & 7) == 0) g = (g & 7) * (nwg >> 3) + (g >> 3);
        const int rest = g / a.splits;
        constexpr int kGroupN = 8;
        const int per_group = kGroupN * a.nblk_m;
        const int grp = rest / per_group;
        const int first_nb = grp * kGroupN;
        const int gn = min(kGroupN, a.nblk_n - first_nb);
        const int within = rest - grp * per_group;
        run_unit(first_nb + within % gn, within / gn, g % a.splits);
    }
}

}  // namespace kq
}  // namespace vqk

namespace vqk {

// ---------------------------------------------------------------------------
// Host side of the K-quant GEMM: split-K plan and launch.
// ---------------------------------------------------------------------------
namespace {

constexpr int kDenseMT = 4;                                   // 128 x 128 tiles
constexpr int kDenseBM = 32 * kDenseMT;
constexpr int kDenseNT = 256;
constexpr int kPartThreads = 256;
constexpr int64_t kPartTileBytes = (int64_t)kPartThreads * kDenseMT * 16 * 4;  // one partial tile
constexpr int kMaxSplits = 8;

}  // namespace

// Workgroups resident per CU (four waves of up to 256 registers, 66-75 KB LDS each).
constexpr int kResident = 2;
// Split-K workspace layout, the same for every shape: arrival counters in
// the first kCntBytes (one int per tile), then the partial tiles.  A fixed
// counter region matters because callers reuse one workspace across calls:
// a region sized per call would let one call's partial tiles lie where a
// later call with more tiles keeps its counters, which must be zero.
constexpr int64_t kCntBytes = 65536;
constexpr int64_t kMaxSplitTiles = kCntBytes / 4;
// Largest split-K workspace the plan asks for (with at least two parts it
// keeps the tile count within the counter region).
constexpr int64_t kMaxPlanWsBytes = (int64_t)1 << 30;
static_assert(kMaxPlanWsBytes / (2 * kPartTileBytes) <= kMaxSplitTiles, "the counters of a split grid fit");

// Splits of the K range for a dense K-quant GEMM (1 = no split), from
// measured times at the prefill shapes.  Partial tiles are 64 KiB each,
// written and read back once, and cost about as much as the compute they
// redistribute once the grid fills the chip (Q4_K at M = 2048: 141 us
// unsplit, 431 us in eight parts), so only short grids split:
//  * at most one tile per CU: the largest S that keeps one workgroup per CU
//    (Q6_K at M = 512, 80 tiles: S = 3, 156 -> 63 us), or the largest that
//    keeps two per CU when that at least doubles S and leaves every part
//    three steps or more (Q6_K at M = 512: S = 6, 63 -> 60 us; Q4_K at
//    M = 200, 152 tiles: S = 3, 35.5 -> 31.3 us; Q5_K at M = 512, 256 tiles:
//    S = 2, 46 -> 44 us).  Smaller gains in S, or shorter parts, measured
//    slower (Q6_K at M = 200, 40 tiles: 6 -> 8 parts 46 -> 53 us; Q4_K at
//    M = 64, 76 tiles: 3 -> 6 parts 17.5 -> 20.7 us);
//  * up to two tiles per CU with a long K (at least 16 steps): two or three
//    parts, whichever leaves the last round of workgroups (two per CU)
//    fuller, ties to two (Q6_K at M = 2048, 320 tiles: three parts fill 1.875
//    rounds, two 1.25; measured 214 / 192 / 181 / 195 us for 1 / 2 / 3 / 4
//    parts);
//  * else none.
// The workspace it needs is capped at kMaxPlanWsBytes.
int gemm_kq_splits(int wtype, int64_t M, int64_t N, int64_t K) {
    (void)wtype;
    const int64_t cus = num_cus();
    const int64_t tiles = ((N + kq::kBN - 1) / kq::kBN) * ((M + kDenseBM - 1) / kDenseBM);
    const int64_t nsteps = K / 256;
    if (tiles <= 0 || nsteps <= 1) return 1;
    int s = 1;
    if (tiles <= cus) {
        const int64_t cap = std::min<int64_t>(kMaxSplits, nsteps);
        const int64_t s1 = std::max<int64_t>(1, std::min<int64_t>(cap, cus / tiles));
        const int64_t s2 = std::max<int64_t>(1, std::min<int64_t>(cap, kResident * cus / tiles));
        s = (int)((s2 >= 2 * s1 && nsteps >= 3 * s2) ? s2 : s1);
    }
    else if (tiles <= kResident * cus && nsteps >= 16) {
        // fill of the last round: (units / slots) / ceil(units / slots), compared exactly
        const int64_t slots = kResident * cus;
        const int64_t u2 = 2 * tiles, u3 = 3 * tiles;
        const int64_t r2 = (u2 + slots - 1) / slots, r3 = (u3 + slots - 1) / slots;
        s = (u3 * r2 > u2 * r3 && nsteps >= 24) ? 3 : 2;
    }
    while (s > 1 && tiles * s * kPartTileBytes > kMaxPlanWsBytes) --s;
    if (tiles > kMaxSplitTiles) s = 1;
    return s;
}

size_t gemm_kq_ws_bytes(int wtype, int64_t M, int64_t N, int64_t K) {
    const int s = gemm_kq_splits(wtype, M, N, K);
    if (s <= 1) return 0;
    const int64_t tiles = ((N + kq::kBN - 1) / kq::kBN) * ((M + kDenseBM - 1) / kDenseBM);
    return (size_t)kCntBytes + (size_t)(tiles * s) * (size_t)kPartTileBytes;
}

template <int WT>
static hipError_t launch_kq_dense(const uint8_t* W, int64_t N, int64_t K, const void* aqs, const void* ad,
                                  const void* aux, int64_t M, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                  hipStream_t st) {
    kq::Args a = {};
    a.W = W;
    a.N = (int)N;
    a.K = (int)K;
    a.aqs = (const int8_t*)aqs;
    a.ad = (const float*)ad;
    a.abs = (const int16_t*)aux;
    a.M = (int)M;
    a.Y = Y;
    a.ldy = ldy;
    a.nblk_n = (int)((N + kq::kBN - 1) / kq::kBN);
    a.nblk_m = (int)((M + kDenseBM - 1) / kDenseBM);
    const int64_t tiles = (int64_t)a.nblk_n * a.nblk_m;
    int s = gemm_kq_splits(WT == 3 ? 5 : WT, M, N, K);
    // a smaller workspace than the plan asks for: the largest split it holds
    while (s > 1 && (!ws || tiles > kMaxSplitTiles ||
                     (size_t)kCntBytes + (size_t)(tiles * s) * (size_t)kPartTileBytes > ws_bytes))
        --s;
    a.splits = s;
    if (s > 1) {
        a.cnt = (int*)ws;
        a.part = (float*)((uint8_t*)ws + kCntBytes);
    }
    const int64_t nwg = tiles * s;
    if (nwg > INT32_MAX) return hipErrorInvalidValue;
    kq::GroupArgs ga = {};
    kq::gemm_kq2_kernel<WT, kDenseMT, 0><<<dim3((unsigned)nwg), kDenseNT, 0, st>>>(a, ga);
    return hipGetLastError();
}

// Activation rows per launch: the kernel addresses one launch's activation
// bytes with 32-bit offsets, so at most 2^31 bytes (floor(2^31 / K) rows,
// whole tiles), further capped by the calling thread's test override.
int64_t gemm_kq_rows_max(int64_t K) {
    int64_t rows = ((int64_t(1) << 31) / K) / kDenseBM * kDenseBM;
    const int64_t rb = gemm_row_block();
    if (rb > 0) rows = std::min(rows, rb);
    return rows;
}

// Workspace for the whole call: the larger of its full row block and its tail.
size_t gemm_kq_call_ws_bytes(int wtype, int64_t M, int64_t N, int64_t K) {
    const int64_t rows = gemm_kq_rows_max(K);
    const int64_t full = std::min(M, rows), tail = M % rows;
    size_t b = gemm_kq_ws_bytes(wtype, full, N, K);
    if (tail > 0) b = std::max(b, gemm_kq_ws_bytes(wtype, tail, N, K));
    return b;
}

// Dense K-quant GEMM (wtype 0 = Q4_K, 1 = Q6_K, 5 = Q5_K), one launch per row
// block; the planar activation planes (qs [M][K], d [M][K/256], bsums
// [M][K/16]) are sliced by row with the same strides.
hipError_t launch_gemm_kq(int wtype, const uint8_t* W, int64_t N, int64_t K, const void* aqs, const void* ad,
                          const void* aux, int64_t M, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                          hipStream_t st) {
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t rows = gemm_kq_rows_max(K);
    if (rows < 1) return hipErrorInvalidValue;
    for (int64_t m0 = 0; m0 < M; m0 += rows) {
        const int64_t mc = std::min(rows, M - m0);
        const int8_t* q = (const int8_t*)aqs + m0 * K;
        const float* d = (const float*)ad + m0 * (K / 256);
        const int16_t* b = (const int16_t*)aux + m0 * (K / 16);
        float* y = Y + m0 * ldy;
        hipError_t e;
        if (wtype == 0) e = launch_kq_dense<0>(W, N, K, q, d, b, mc, y, ldy, ws, ws_bytes, st);
        else if (wtype == 1) e = launch_kq_dense<1>(W, N, K, q, d, b, mc, y, ldy, ws, ws_bytes, st);
        else e = launch_kq_dense<3>(W, N, K, q, d, b, mc, y, ldy, ws, ws_bytes, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Routed tile height of a grouped call (the routed-compact "J rule" of
// strix-llama.cpp PR #18, restated for 32-row MFMA tiles): tiles are sized
// from the rows each expert receives, not from the total pair count.  The
// weights dominate the grouped call's traffic, so the height is the smallest
// multiple of 32 that holds the mean rows per expert r = T top_k / E plus
// three standard deviations of a uniform routing (sqrt r): nearly every
// expert is then one tile and its weights are read once.  r = 16 -> 32
// rows, 32 -> 64, 64 and more -> 96.  The height stops at 96: the 128-row
// routed kernel (its gathered-row offsets on top of the dense kernel's
// registers) spills, and two or three 96-row tiles per expert measured
// 5-10 % faster (warm, 96 to 256 rows per expert: 4,096 tokens 206 -> 196 us,
// 8,192 tokens 349 -> 317 us).
// Q8_0 keeps its GEMM's 96-row tiles.  A call whose activation rows take
// 2^31 bytes or more runs the 64-bit-offset kernel, capped at 64-row tiles.
int grouped_tile_rows(int wtype, int64_t E, int64_t T, int64_t top_k, int64_t K, int per_row) {
    if (wtype == 2) return kGroupTileRows;
    if (E <= 0 || T <= 0) return kGroupMinTileRows;
    const double r = (double)T * (double)top_k / (double)E;
    const int mt = (int)std::ceil((r + 3.0 * std::sqrt(r)) / 32.0);
    int rows = 32 * std::min(3, std::max(1, mt));
    const int64_t arows = per_row ? T * top_k : T;
    if (arows * K >= ((int64_t)1 << 31)) rows = std::min(rows, 64);
    return rows;
}

template <int WT, int MT, int kMode>
static hipError_t launch_kq_grouped_t(const uint8_t* W, int64_t E, int64_t N, int64_t K, const void* aqs,
                                      const void* ad, const void* aux, int64_t T, int64_t top_k, int per_row,
                                      const RouteWs& ws, float* Y, hipStream_t st) {
    const int64_t nbk = K / 256;
    kq::Args a = {};
    a.W = W;
    a.N = (int)N;
    a.K = (int)K;
    a.aqs = (const int8_t*)aqs;
    a.ad = (const float*)ad;
    a.abs = (const int16_t*)aux;
    a.M = (int)(per_row ? T * top_k : T);
    a.Y = Y;
    a.ldy = N;
    a.splits = 1;
    a.nblk_n = (int)((N + kq::kBN - 1) / kq::kBN);
    // the tile table holds at most ceil(pairs / rows) + E tiles
    const int64_t max_tiles = (T * top_k + 32 * MT - 1) / (32 * MT) + E;
    a.nblk_m = (int)max_tiles;
    kq::GroupArgs ga = {};
    ga.tiles = ws.tiles;
    ga.ntiles = ws.ntiles;
    ga.list = ws.list;
    ga.top_k = (int)top_k;
    ga.per_row = per_row;
    ga.expert_stride = N * nbk * kq::KQ2<WT>::BB;
    const int64_t units = max_tiles * a.nblk_n;
    const int64_t grid = std::min<int64_t>(units, (int64_t)num_cus() * kResident);
    if (grid <= 0) return hipSuccess;
    kq::gemm_kq2_kernel<WT, MT, kMode><<<dim3((unsigned)grid), kDenseNT, 0, st>>>(a, ga);
    return hipGetLastError();
}

template <int WT>
static hipError_t launch_kq_grouped_w(int tile_rows, const uint8_t* W, int64_t E, int64_t N, int64_t K,
                                      const void* aqs, const void* ad, const void* aux, int64_t T, int64_t top_k,
                                      int per_row, const RouteWs& ws, float* Y, hipStream_t st) {
    const int64_t arows = per_row ? T * top_k : T;
    if (arows * K >= ((int64_t)1 << 31)) {
        // 64-bit activation offsets (more registers): at most 64-row tiles
        if (tile_rows == 32)
            return launch_kq_grouped_t<WT, 1, 2>(W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
        if (tile_rows == 64)
            return launch_kq_grouped_t<WT, 2, 2>(W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
        return hipErrorInvalidValue;  // grouped_tile_rows never gives more here
    }
    switch (tile_rows) {
        case 32: return launch_kq_grouped_t<WT, 1, 1>(W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
        case 64: return launch_kq_grouped_t<WT, 2, 1>(W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
        case 96: return launch_kq_grouped_t<WT, 3, 1>(W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_kq_grouped(int wtype, const uint8_t* W, int64_t E, int64_t N, int64_t K, const void* aqs,
                                  const void* ad, const void* aux, int64_t T, int64_t top_k, int per_row,
                                  int tile_rows, RouteWs ws, float* Y, hipStream_t st) {
    if (T == 0 || N == 0) return hipSuccess;
    if (wtype == 0)
        return launch_kq_grouped_w<0>(tile_rows, W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
    if (wtype == 1)
        return launch_kq_grouped_w<1>(tile_rows, W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
    return launch_kq_grouped_w<3>(tile_rows, W, E, N, K, aqs, ad, aux, T, top_k, per_row, ws, Y, st);
}

// The int8 MFMA ceiling: every lane of every wave keeps eight independent
// v_mfma_i32_32x32x32_i8 accumulator chains busy on register operands for
// `iters` rounds and does nothing else, two workgroups of four waves per CU
// (two waves per SIMD), so its rate is what the matrix cores sustain at the
// clocks this part runs under load.  The accumulators are folded into one
// word that is stored only if it equals `key` (in practice never), so the
// MFMAs are kept and nothing is written.
constexpr int kMfmaProbeChains = 8;
constexpr int kMfmaProbeThreads = 256;
constexpr int kMfmaProbeWgsPerCu = 2;
__global__ __launch_bounds__(kMfmaProbeThreads, kMfmaProbeWgsPerCu) void mfma_probe_kernel(int64_t iters,
                                                                                       uint32_t key,
                                                                                       uint32_t* sink) {
    const int t = (int)threadIdx.x;
    const kq::v4i a = {t * 0x01010101, t ^ 0x5A5A5A5A, ~t, t * 3};
    const kq::v4i b = {t + 1, t * 7, t ^ 0x33333333, t << 3};
    kq::v16i acc[kMfmaProbeChains];
#pragma unroll
    for (int c = 0; c < kMfmaProbeChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = c;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kMfmaProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < kMfmaProbeChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) x ^= (uint32_t)acc[c][r];
    if (x == key) sink[0] = x;
}

hipError_t launch_mfma_probe(int64_t iters, uint32_t* sink, int64_t* ops_out, hipStream_t st) {
    const int64_t grid = (int64_t)num_cus() * kMfmaProbeWgsPerCu;
    const int64_t waves = grid * (kMfmaProbeThreads / 64);
    if (ops_out) *ops_out = waves * iters * kMfmaProbeChains * (2 * 32 * 32 * 32);
    mfma_probe_kernel<<<(unsigned)grid, kMfmaProbeThreads, 0, st>>>(iters, 0x9E3779B9u, sink);
    return hipGetLastError();
}

}  // namespace vqk
