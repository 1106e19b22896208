// gemm.hip -- the Q8_0 x Q8_1 prefill GEMM Y = X * W^T on int8 MFMA for
// gfx950, and its routed-expert (MUL_MAT_ID) variant.  (The K-quant weight
// types run on gemm_k.hip; this kernel template keeps their plane unpacking,
// which only Q8_0's single plane instantiates.)
//
// Pages: vllm.cpp PR #3035 "scope a cooperative activation share for the WMMA
// kernels" (each warp re-reading the same activation rows is the diagnosed
// redundancy; one cooperatively loaded tile per block shared by all warps is
// the fix), strix-llama.cpp PR #18 commits "MMQ register prefetch" (stage the
// next 256-wide K iteration in registers while the current one is consumed)
// and "routed-compact" (MUL_MAT_ID tiles sized to the rows of each expert).
//
// MI355X design (not the pages' RDNA WMMA tiles):
//  * A 2 x WM grid of waves (8 or 16 for the prefill GEMM, 4 for the grouped
//    one); each wave owns 32 weight rows x 16 TM activation rows as 16x16
//    MFMA tiles; the workgroup tile is 64 x BM (BM = 16 TM WM).
//  * Per 256-wide K step the workgroup stages ONE activation tile (int8 Q8_K
//    or Q8_1 bytes plus scales) in LDS, shared by all its waves, and ONE
//    unpacked weight tile, also shared; the next step's global bytes are
//    already in flight in registers while the current step computes.
//  * The per-sub-block integer scales are folded into the int8 MFMA operand
//    so that a whole super-block is one int32 accumulation with no per-
//    sub-block ALU work:
//      Q4_K: sc (6 bit) = 8*sc_hi + sc_lo; planes q*sc_lo and q*sc_hi (each
//            <= 105) -> S = 8*P_hi + P_lo.  The min term Mn = sum_j m_j*bs32_j
//            runs on two 16x16x32 MFMAs with bs32 = 64*h + l.
//      Q6_K: sc (int8) = 64*d2 + 8*d1 + d0 with digits in [-3,4]; planes
//            (q-32)*d_i fit int8 -> S = 64*P2 + 8*P1 + P0.
//      Q5_K: q up to 31, so sc = 16*d2 + 4*d1 + d0 with digits in [0,3];
//            planes q*d_i <= 93 -> S = 16*P2 + 4*P1 + P0; mins as Q4_K.
//      Q8_0: one 16x16x32 MFMA per 32-block, combined per block.
//    The integer sums are exact, and the binary32 combine of each block and
//    the ascending-block accumulation follow the fixed-order definition, so Y
//    is bit-identical to it.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short ss2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));  // native vector: plain loads and stores

constexpr int kBN = 64;   // weight rows per workgroup
constexpr int kKS = 256;  // K per step
constexpr int kLD = 272;  // LDS row stride of the int8 tiles (256 + 16 against bank conflicts)

// 16 bytes from a 2-byte aligned global address using 4-byte aligned loads;
// never reads at or beyond `end`.
__device__ __forceinline__ void gload16_a2(const uint8_t* p, const uint8_t* end, uint32_t out[4]) {
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
    const uint32_t* q = (const uint32_t*)(p - sh);
    uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
    if (sh == 0) {
        out[0] = w0; out[1] = w1; out[2] = w2; out[3] = w3;
        return;
    }
    uint32_t w4;
    if ((const uint8_t*)(q + 5) <= end) w4 = q[4];
    else w4 = (uint32_t)(*(const uint16_t*)(q + 4));
    out[0] = __builtin_amdgcn_alignbyte(w1, w0, sh);
    out[1] = __builtin_amdgcn_alignbyte(w2, w1, sh);
    out[2] = __builtin_amdgcn_alignbyte(w3, w2, sh);
    out[3] = __builtin_amdgcn_alignbyte(w4, w3, sh);
}

// Multiply the four bytes of v by f when every byte's product lies in
// [0, 255] (Q4_K / Q5_K quants times a scale digit): each 16-bit lane holds
// two bytes, the low byte's product cannot carry into the high byte, and the
// high byte's product times 256 stays below 2^16, so one packed 16-bit
// multiply is exact.
__device__ __forceinline__ uint32_t bytes_mul_u(uint32_t v, int f) {
    const us2 fe = (us2){(unsigned short)f, (unsigned short)f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(us2, v) * fe);
}

// Q6_K plane bytes ((q - 32) * d) mod 256 for 6-bit quants q, given as their
// even bytes (ev = q & 0x00FF00FF) and odd bytes (od = q & 0xFF00FF00).  The
// even products sit in the low byte of each 16-bit lane (carries land in the
// high byte, masked off); the odd products sit in the high byte and their low
// byte stays zero.  The offset -32 * d is added in the same multiply-add.
__device__ __forceinline__ uint32_t q6_plane_bytes(uint32_t ev, uint32_t od, int d) {
    const unsigned short f = (unsigned short)d;
    const unsigned short c = (unsigned short)(-32 * d);
    const unsigned short c8 = (unsigned short)(c << 8);
    const us2 e = __builtin_bit_cast(us2, ev) * (us2){f, f} + (us2){c, c};
    const us2 o = __builtin_bit_cast(us2, od) * (us2){f, f} + (us2){c8, c8};
    return (__builtin_bit_cast(uint32_t, e) & 0x00FF00FFu) | __builtin_bit_cast(uint32_t, o);
}

template <int WT>
struct GemmCfg;
template <>
struct GemmCfg<0> { static constexpr int P = 2; static constexpr int BB = kQ4KBytes; };
template <>
struct GemmCfg<1> { static constexpr int P = 3; static constexpr int BB = kQ6KBytes; };
template <>
struct GemmCfg<2> { static constexpr int P = 1; static constexpr int BB = kQ80Bytes; };
template <>
struct GemmCfg<3> { static constexpr int P = 3; static constexpr int BB = kQ5KBytes; };

// Row indirection of the grouped (MUL_MAT_ID) variant.
struct GroupArgs {
    const int32_t* tiles;   // [ntiles][4]: expert, first list slot, rows, 0
    const int32_t* ntiles;  // device count of valid tiles
    const int32_t* list;    // pair indices grouped per expert
    int top_k;
    int per_row;            // 1: pair p reads activation row p (per-row arm); 0: row p / top_k
    int64_t expert_stride;  // bytes of one expert's [N][K/QK] blocks
    int tile_base;          // routed tile of blockIdx.y = 0 (launches of at most kMaxGridY tiles)
};

// Most workgroup rows (gridDim.y) per launch; larger grids run as several
// launches.
constexpr int64_t kMaxGridY = 32768;

// Workgroup of 2 x WM waves (128 * WM threads) computing a 64 x (16 * TM * WM)
// output tile; each wave owns 32 weight rows x 16 * TM activation rows
// (2 x TM MFMA tiles of 16 x 16).  A weight row's step (one super-block, or eight
// Q8_0 blocks) is unpacked by 2 * WM threads (by the first 512 threads, eight
// per row, when there are more), each taking an equal share of its eight
// 16-byte pieces, so the unpack cost per output falls as the tile grows.
template <int WT, int WM, int TM, bool kGrouped>
__global__ __launch_bounds__(128 * WM, 2) void gemm_kernel(const uint8_t* __restrict__ Wbase, int N, int K,
                                                           int64_t wbytes, const int8_t* __restrict__ aqs,
                                                           const void* __restrict__ ad,
                                                           const int16_t* __restrict__ abs_, int M,
                                                           float* __restrict__ Y, int64_t ldy,
                                                           GroupArgs ga) {
    constexpr int P = GemmCfg<WT>::P;
    constexpr int BB = GemmCfg<WT>::BB;
    constexpr bool kMin = (WT == 0 || WT == 3);  // Q4_K, Q5_K: scales and mins
    constexpr int kShift = (WT == 3) ? 2 : 3;     // digit base of the scale planes (4 or 8)
    constexpr int NT = 128 * WM;           // threads
    constexpr int BM = 16 * TM * WM;       // activation rows per workgroup
    constexpr int ACH = BM * 16 / NT;      // 16-byte activation chunks per thread per step
    constexpr int NU = (NT >= 512) ? 512 : ((NT >= 256) ? 256 : NT);  // threads that load and unpack weights
    constexpr int UPR = NU / kBN;          // threads per weight row
    constexpr int PPT = 8 / UPR;           // 16-byte pieces per thread
    static_assert(UPR * PPT == 8, "a weight row's eight 16-byte pieces are split evenly");
    static_assert((BM * 16) % NT == 0, "activation chunks are split evenly");
    __shared__ __attribute__((aligned(16))) int8_t sA[BM * kLD];
    __shared__ __attribute__((aligned(16))) int8_t sW[P * kBN * kLD];
    // Scales, double-buffered by step parity (a late wave combines step s - 1
    // while step s is current).
    __shared__ __attribute__((aligned(16))) float sDa2[2][(WT == 2) ? BM * 8 : BM];
    __shared__ __attribute__((aligned(16))) float sDw2[2][(WT == 2) ? kBN * 8 : 2 * kBN];
    __shared__ __attribute__((aligned(16))) int8_t sMw2[2][kMin ? kBN * 8 : 16];
    __shared__ __attribute__((aligned(16))) int8_t sHl2[2][kMin ? BM * 16 : 16];
    __shared__ int sRow[BM];    // activation row of each tile row (-1: none)
    __shared__ int sOut[BM];    // output row of each tile row (-1: none)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int r16 = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * kBN;

    const uint8_t* W = Wbase;
    int rows_here;  // valid activation rows of this tile
    if (kGrouped) {
        const int tix = ga.tile_base + (int)blockIdx.y;
        if (tix >= *ga.ntiles) return;
        const int e = ga.tiles[4 * tix + 0];
        const int first = ga.tiles[4 * tix + 1];
        rows_here = ga.tiles[4 * tix + 2];
        W = Wbase + (int64_t)e * ga.expert_stride;
        if (tid < BM) {
            if (tid < rows_here) {
                const int p = ga.list[first + tid];
                sRow[tid] = ga.per_row ? p : p / ga.top_k;
                sOut[tid] = p;
            } else {
                sRow[tid] = -1;
                sOut[tid] = -1;
            }
        }
    } else {
        const int m0 = blockIdx.y * BM;
        rows_here = min(BM, M - m0);
        if (tid < BM) {
            const int m = m0 + tid;
            sRow[tid] = (m < M) ? m : -1;
            sOut[tid] = (m < M) ? m : -1;
        }
    }
    rows_here = __builtin_amdgcn_readfirstlane(rows_here);
    __syncthreads();

    const int nbw = (WT == 2) ? K / kQK8 : K / kQK;
    const int64_t rb = (int64_t)nbw * BB;
    const uint8_t* wend = Wbase + wbytes;
    const int nsteps = (K + kKS - 1) / kKS;

    // Activation chunks of this thread: row (tid >> 4) + (NT / 16) * i, bytes
    // 16 * (tid & 15) of each step.  Rows past the tile read activation row 0
    // (their outputs are never stored).  The prefill launch keeps the
    // activation bytes of one launch below 2^31, so their offsets from aqs are
    // 32-bit (one VGPR per chunk, no 64-bit address arithmetic per load); the
    // grouped variant gathers rows from the whole activation matrix.
    typedef typename std::conditional<kGrouped, int64_t, uint32_t>::type AOff;
    const int acol = 16 * (tid & 15);
    AOff aoff[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int ar = sRow[(tid >> 4) + (NT / 16) * i];
        aoff[i] = (AOff)(ar >= 0 ? ar : 0) * (AOff)K + (AOff)acol;
    }
    const int my_ar = (tid < BM) ? sRow[tid] : -1;  // scale row of threads < BM

    // Weight unpack role (threads below NU, whole waves): row wr, pieces
    // [PPT * wu, PPT * wu + PPT).
    const bool wthr = (NT <= NU) || tid < NU;
    const int wr = tid / UPR, wu = tid % UPR;
    const bool wvalid = (n0 + wr) < N;
    const uint8_t* wrow_p = W + (int64_t)(wvalid ? n0 + wr : 0) * rb;

    // Register-staged global data of one step.
    u4v regA[ACH];
    constexpr int SCW = (PPT + 1) / 2;     // Q6_K: words of per-piece scale byte pairs
    uint32_t regW[(WT == 0) ? 4 + 4 * PPT : ((WT == 3) ? 4 + 8 * PPT : ((WT == 1) ? 8 * PPT + SCW + 1 : 9 * PPT))];
    float regDa;
    uint4 regBs[2];

    // part < 0: every load of step s; part 0..3: a quarter of the activation
    // chunks, plus the scales (part 0) or the weights (part 1), so that the
    // next step's loads can be spread between the current step's MFMAs.
    auto load_step = [&](int s, int part) __attribute__((always_inline)) {
        const int kk = s * kKS;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            if (part >= 0 && (i * 4 / ACH) != part) continue;
            // Branch-free: a row past the tile reads row 0 (its outputs are
            // never stored, and every output depends on its own row only);
            // Q8_0 columns past K read inside the row and are never used.
            AOff off = (AOff)kk;
            if (WT == 2 && kk + acol >= K) off = (AOff)(K - 16 - acol);
            regA[i] = *(const u4v*)(aqs + (aoff[i] + off));
        }
        if (part > 1) return;
        if (part <= 0 && tid < BM) {
            const int ar = my_ar >= 0 ? my_ar : 0;
            if (WT == 2) {
                const uint16_t* dp = (const uint16_t*)ad + (int64_t)ar * nbw;
                uint32_t h[8];
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const int blk = s * 8 + b;
                    h[b] = (blk < nbw) ? dp[blk] : 0u;
                }
                regBs[0] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                      h[6] | (h[7] << 16));
            } else {
                regDa = ((const float*)ad)[(int64_t)ar * nbw + s];
                if (kMin) {
                    const uint4* bp = (const uint4*)(abs_ + ((int64_t)ar * nbw + s) * 16);
                    regBs[0] = bp[0];
                    regBs[1] = bp[1];
                }
            }
        }
        if (part == 0 || !wthr) return;
        if (WT == 0 || WT == 3) {
            // Q5_K: the nibbles at byte 48, and for piece pc the 16 fifth-bit
            // bytes 16 + 16 (pc % 2) .. that cover its values
            const uint8_t* bp = wrow_p + (int64_t)s * BB;
            const uint4 h = *(const uint4*)bp;
            regW[0] = h.x; regW[1] = h.y; regW[2] = h.z; regW[3] = h.w;
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int pc = PPT * wu + j;
                const uint4 q = *(const uint4*)(bp + ((WT == 3) ? 48 : 16) + 16 * pc);
                regW[4 + 4 * j] = q.x; regW[5 + 4 * j] = q.y; regW[6 + 4 * j] = q.z; regW[7 + 4 * j] = q.w;
                if (WT == 3) {
                    const uint4 hq = *(const uint4*)(bp + 16 + 16 * (pc & 1));
                    regW[4 + 4 * PPT + 4 * j] = hq.x; regW[5 + 4 * PPT + 4 * j] = hq.y;
                    regW[6 + 4 * PPT + 4 * j] = hq.z; regW[7 + 4 * PPT + 4 * j] = hq.w;
                }
            }
        } else if (WT == 1) {
            const uint8_t* bp = wrow_p + (int64_t)s * kQ6KBytes;
            uint32_t scw[SCW];
#pragma unroll
            for (int k = 0; k < SCW; ++k) scw[k] = 0;
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int pc = PPT * wu + j, h = pc >> 2, v = pc & 3;
                gload16_a2(bp + 64 * h + 16 * v, wend, regW + 8 * j);                  // ql
                gload16_a2(bp + 128 + 32 * h + 16 * (v & 1), wend, regW + 8 * j + 4);  // qh
                const uint32_t sa = bp[192 + 8 * h + v], sb = bp[196 + 8 * h + v];
                scw[j >> 1] |= (sa | (sb << 8)) << (16 * (j & 1));
            }
#pragma unroll
            for (int k = 0; k < SCW; ++k) regW[8 * PPT + k] = scw[k];
            regW[8 * PPT + SCW] = *(const uint16_t*)(bp + 208);
        } else {
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int blk = s * 8 + PPT * wu + j;
                if (blk < nbw) {
                    const uint8_t* bp = wrow_p + (int64_t)blk * kQ80Bytes;
                    gload16_a2(bp + 2, wend, regW + 9 * j);
                    gload16_a2(bp + 18, wend, regW + 9 * j + 4);
                    regW[9 * j + 8] = *(const uint16_t*)bp;
                } else {
#pragma unroll
                    for (int i = 0; i < 9; ++i) regW[9 * j + i] = 0;
                }
            }
        }
    };

    auto store_step = [&](int ss) __attribute__((always_inline)) {
        float* sDa = sDa2[ss & 1];
        float* sDw = sDw2[ss & 1];
        int8_t* sMw = sMw2[ss & 1];
        int8_t* sHl = sHl2[ss & 1];
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            *(u4v*)(sA + ((tid >> 4) + (NT / 16) * i) * kLD + acol) = regA[i];
        if (tid < BM) {
            if (WT == 2) {
                const uint32_t hw[4] = {regBs[0].x, regBs[0].y, regBs[0].z, regBs[0].w};
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    sDa[tid * 8 + b] = half_bits_to_float((hw[b >> 1] >> (16 * (b & 1))) & 0xFFFF);
            } else {
                sDa[tid] = regDa;
                if (kMin) {
                    // bs32_j = bsums[2j] + bsums[2j+1] = 64 * h + l, 0 <= l < 64 (int8
                    // operands).  Two sums per word in 16-bit halves (|bs32| < 2^15),
                    // then the low byte of each half.
                    const uint32_t bw[8] = {regBs[0].x, regBs[0].y, regBs[0].z, regBs[0].w,
                                            regBs[1].x, regBs[1].y, regBs[1].z, regBs[1].w};
                    uint32_t hp[4], lp[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t ev = __builtin_amdgcn_perm(bw[2 * k + 1], bw[2 * k], 0x05040100u);
                        const uint32_t od = __builtin_amdgcn_perm(bw[2 * k + 1], bw[2 * k], 0x07060302u);
                        const us2 sum = __builtin_bit_cast(us2, ev) + __builtin_bit_cast(us2, od);
                        hp[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(ss2, sum) >> (ss2){6, 6});
                        lp[k] = __builtin_bit_cast(uint32_t, sum) & 0x003F003Fu;
                    }
                    *(uint4*)(sHl + tid * 16) = make_uint4(
                        __builtin_amdgcn_perm(hp[1], hp[0], 0x06040200u), __builtin_amdgcn_perm(hp[3], hp[2], 0x06040200u),
                        __builtin_amdgcn_perm(lp[1], lp[0], 0x06040200u), __builtin_amdgcn_perm(lp[3], lp[2], 0x06040200u));
                }
            }
        }
        if (!wthr) return;
        int8_t* wdst = sW + wr * kLD;
        if (WT == 0 || WT == 3) {
            // piece pc = 16 qs bytes at 16 * pc: low nibbles are values
            // 64c + 16hf + i (sub-block 2c), high nibbles 64c + 32 + 16hf + i
            // (sub-block 2c + 1), c = pc / 2, hf = pc % 2.  Q4_K: plane 0
            // holds q * (sc & 7), plane 1 q * (sc >> 3).  Q5_K (q up to 31,
            // bits 2c and 2c + 1 of the fifth-bit bytes 16hf + i): planes of
            // the base-4 digits of sc, q * digit <= 93.
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int pc = PPT * wu + j, c = pc >> 1, hf = pc & 1;
                const uint32_t sw = (c < 2) ? regW[1] : regW[2];
                const int sh = 16 * (c & 1);
                const int scl = (int)((sw >> sh) & 63), sch = (int)((sw >> (sh + 8)) & 63);
                int fl[P], fh[P];
                if (WT == 0) {
                    fl[0] = scl & 7; fl[1] = scl >> 3;
                    fh[0] = sch & 7; fh[1] = sch >> 3;
                } else {
                    fl[0] = scl & 3; fl[1] = (scl >> 2) & 3; fl[P - 1] = scl >> 4;
                    fh[0] = sch & 3; fh[1] = (sch >> 2) & 3; fh[P - 1] = sch >> 4;
                }
                uint32_t ql[4], qh[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t q = regW[4 + 4 * j + i];
                    ql[i] = q & 0x0F0F0F0Fu;
                    qh[i] = (q >> 4) & 0x0F0F0F0Fu;
                    if (WT == 3) {
                        const uint32_t hw = regW[4 + 4 * PPT + 4 * j + i];
                        ql[i] |= ((hw >> (2 * c)) & 0x01010101u) << 4;
                        qh[i] |= ((hw >> (2 * c + 1)) & 0x01010101u) << 4;
                    }
                }
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lo[i] = bytes_mul_u(ql[i], fl[p]);
                        hi[i] = bytes_mul_u(qh[i], fh[p]);
                    }
                    int8_t* dst = wdst + p * kBN * kLD + 64 * c + 16 * hf;
                    *(uint4*)dst = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                    *(uint4*)(dst + 32) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                }
            }
            // d and dmin from two lanes of the row; the eight 6-bit mins
            // m_j = (scales[j] >> 6) | (nibble j % 2 of scales[8 + j / 2]) << 2
            // spread over the row's lanes, PPT each.
            if (wu == 0) sDw[wr] = half_bits_to_float(regW[0] & 0xFFFF);
            if (wu == 1 % UPR) sDw[kBN + wr] = half_bits_to_float(regW[0] >> 16);
#pragma unroll
            for (int jj = 0; jj < PPT; ++jj) {
                const int j = PPT * wu + jj;
                const uint32_t sj = ((j < 4 ? regW[1] : regW[2]) >> (8 * (j & 3))) & 0xFF;
                const uint32_t nb_ = (regW[3] >> (4 * j)) & 15;
                sMw[wr * 8 + j] = (int8_t)((sj >> 6) | (nb_ << 2));
            }
        } else if (WT == 1) {
            // piece pc = (h, v): ql bytes 64h + 16v.. hold values 128h + 16v + i
            // (low nibbles, sub-block 8h + v) and 128h + 64 + 16v + i (high,
            // sub-block 8h + 4 + v); their top bits are pairs v/2 and 2 + v/2
            // of qh bytes 32h + 16(v % 2) + i.  Planes: the base-8 digits
            // (each in [-3, 4]) of the int8 scale times (q - 32).
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int pc = PPT * wu + j, h = pc >> 2, v = pc & 3;
                const int sa = 2 * (v >> 1);
                const uint32_t scp = (regW[8 * PPT + (j >> 1)] >> (16 * (j & 1))) & 0xFFFF;
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    const int sc = (int)(int8_t)((scp >> (8 * part)) & 0xFF);
                    const int d0 = ((sc + 3) & 7) - 3;
                    const int t1 = (sc - d0) >> 3;
                    const int d1 = ((t1 + 3) & 7) - 3;
                    const int d2 = (t1 - d1) >> 3;
                    uint32_t ev[4], od[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t ql = regW[8 * j + i];
                        const uint32_t qh = regW[8 * j + 4 + i];
                        const uint32_t q6 = part ? (((ql >> 4) & 0x0F0F0F0Fu) | ((qh >> sa) & 0x30303030u))
                                                 : ((ql & 0x0F0F0F0Fu) | ((qh << (4 - sa)) & 0x30303030u));
                        ev[i] = q6 & 0x00FF00FFu;
                        od[i] = q6 & 0xFF00FF00u;
                    }
                    const int dg[3] = {d0, d1, d2};
#pragma unroll
                    for (int p = 0; p < 3; ++p) {
                        int8_t* dst = wdst + p * kBN * kLD + 128 * h + 64 * part + 16 * v;
                        *(uint4*)dst = make_uint4(q6_plane_bytes(ev[0], od[0], dg[p]), q6_plane_bytes(ev[1], od[1], dg[p]),
                                                  q6_plane_bytes(ev[2], od[2], dg[p]), q6_plane_bytes(ev[3], od[3], dg[p]));
                    }
                }
            }
            if (wu == 0) sDw[wr] = half_bits_to_float(regW[8 * PPT + SCW] & 0xFFFF);
        } else {
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const int b = PPT * wu + j;
                int8_t* dst = wdst + 32 * b;
                *(uint4*)dst = make_uint4(regW[9 * j + 0], regW[9 * j + 1], regW[9 * j + 2], regW[9 * j + 3]);
                *(uint4*)(dst + 16) =
                    make_uint4(regW[9 * j + 4], regW[9 * j + 5], regW[9 * j + 6], regW[9 * j + 7]);
                sDw[wr * 8 + b] = half_bits_to_float(regW[9 * j + 8] & 0xFFFF);
            }
        }
    };

    float acc[2][TM][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

    const int wn0 = 32 * wn, wm0 = 16 * TM * wm;
    const bool late = (WM >= 4) && ((wave >> 2) & 1);
    const bool active = wm0 < rows_here;  // the wave has valid activation rows
    v4i R[2][TM];  // integer sums S of the current super-block

    // Binary32 combine of step ss (its scales are in buffer ss & 1).
    auto epilogue = [&](int ss) __attribute__((always_inline)) {
        const float* sDa = sDa2[ss & 1];
        const float* sDw = sDw2[ss & 1];
        v4i mn[2][TM];
        if (kMin) {
            const int8_t* sMw = sMw2[ss & 1];
            const int8_t* sHl = sHl2[ss & 1];
            long am[2][2], bm[TM];
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const long mv = *(const long*)(sMw + (wn0 + 16 * tn + r16) * 8);
                am[tn][0] = (g == 0) ? mv : 0;
                am[tn][1] = (g == 1) ? mv : 0;
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int8_t* hp = sHl + (wm0 + 16 * tm + r16) * 16;
                bm[tm] = (g == 0) ? *(const long*)hp : ((g == 1) ? *(const long*)(hp + 8) : 0);
            }
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    v4i z = {0, 0, 0, 0};
                    const v4i dh = __builtin_amdgcn_mfma_i32_16x16x32_i8(am[tn][0], bm[tm], z, 0, 0, 0);
                    const v4i dl = __builtin_amdgcn_mfma_i32_16x16x32_i8(am[tn][1], bm[tm], z, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) mn[tn][tm][i] = (dh[i] << 6) + dl[i];
                }
        }
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
            const int nb4 = wn0 + 16 * tn + 4 * g;
            const float4 dv = *(const float4*)(sDw + nb4);
            const float dd[4] = {dv.x, dv.y, dv.z, dv.w};
            float dm[4] = {0.f, 0.f, 0.f, 0.f};
            if (kMin) {
                const float4 dmv = *(const float4*)(sDw + kBN + nb4);
                dm[0] = dmv.x; dm[1] = dmv.y; dm[2] = dmv.z; dm[3] = dmv.w;
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const float da = sDa[wm0 + 16 * tm + r16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float t1 = dd[i] * (float)R[tn][tm][i];
                    if (kMin) {
                        const float t2 = dm[i] * (float)mn[tn][tm][i];
                        const float t3 = t1 - t2;
                        const float c = da * t3;
                        acc[tn][tm][i] = acc[tn][tm][i] + c;
                    } else {
                        const float c = da * t1;
                        acc[tn][tm][i] = acc[tn][tm][i] + c;
                    }
                }
            }
        }
    };

    load_step(0, -1);
    for (int s = 0; s < nsteps; ++s) {
        __syncthreads();
        store_step(s);
        __syncthreads();
        const bool more = s + 1 < nsteps;
        if (WT == 2 && more) load_step(s + 1, -1);

        if (WT == 2) {
            const float* sDa = sDa2[s & 1];
            const float* sDw = sDw2[s & 1];
            const int nval = min(8, nbw - 8 * s);
            for (int b = 0; b < nval; ++b) {
                long av[2], bv[TM];
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    av[tn] = *(const long*)(sW + (wn0 + 16 * tn + r16) * kLD + 32 * b + 8 * g);
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    bv[tm] = *(const long*)(sA + (wm0 + 16 * tm + r16) * kLD + 32 * b + 8 * g);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    float dwv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) dwv[i] = sDw[(wn0 + 16 * tn + 4 * g + i) * 8 + b];
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm) {
                        v4i z = {0, 0, 0, 0};
                        const v4i I = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[tn], bv[tm], z, 0, 0, 0);
                        const float da = sDa[(wm0 + 16 * tm + r16) * 8 + b];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float sc = dwv[i] * da;
                            const float c = sc * (float)I[i];
                            acc[tn][tm][i] = acc[tn][tm][i] + c;
                        }
                    }
                }
            }
        } else {
            // Late waves combine the previous step before this step's MFMAs,
            // early waves after them: each SIMD holds one of each, so one
            // wave's epilogue VALU runs while the other's MFMAs run.
            if (!active) {
                // no valid activation rows for this wave: only its share of the loads
                if (more) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) load_step(s + 1, t);
                }
                continue;
            }
            if (late && s > 0) epilogue(s - 1);
            v4i bv[4][TM];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    bv[t][tm] = *(const v4i*)(sA + (wm0 + 16 * tm + r16) * kLD + 64 * t + 16 * g);
            // One accumulator per tile through the digit planes, high digit
            // first: R = (((P2 << 3) + P1) << 3) + P0 (Q6_K), (P1 << 3) + P0
            // (Q4_K) or (((P2 << 2) + P1) << 2) + P0 (Q5_K) = S, exact in int32.
#pragma unroll
            for (int p = P - 1; p >= 0; --p) {
                if (p < P - 1) {
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm) R[tn][tm] = R[tn][tm] << kShift;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v4i av[2];
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn)
                        av[tn] = *(const v4i*)(sW + (p * kBN + wn0 + 16 * tn + r16) * kLD + 64 * t + 16 * g);
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm)
                            R[tn][tm] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                av[tn], bv[t][tm], (p == P - 1 && t == 0) ? (v4i){0, 0, 0, 0} : R[tn][tm], 0, 0, 0);
                    if (p == P - 1 && more) load_step(s + 1, t);
                }
            }
            if (!late) epilogue(s);
        }
    }
    if (WT != 2 && active && late && nsteps > 0) epilogue(nsteps - 1);

    // Store: lane holds rows n = 4g + i of a 16x16 tile, column m = r16.
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
        const int n = n0 + wn0 + 16 * tn + 4 * g;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int orow = sOut[wm0 + 16 * tm + r16];
            if (orow < 0) continue;
            float* yp = Y + (int64_t)orow * ldy + n;
            if (n + 3 < N && ((((uintptr_t)yp) & 15) == 0)) {
                *(float4*)yp = make_float4(acc[tn][tm][0], acc[tn][tm][1], acc[tn][tm][2], acc[tn][tm][3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n + i < N) yp[i] = acc[tn][tm][i];
            }
        }
    }
}

// Per calling thread, so a test's override never reaches another thread's calls.
static thread_local int64_t g_row_block = 0;

void set_gemm_row_block(int64_t rows) { g_row_block = rows; }
int64_t gemm_row_block() { return g_row_block; }

template <int WT, int WM, int TM>
static hipError_t launch_gemm_cfg(const uint8_t* W, int64_t N, int64_t K, const void* aqs, const void* ad,
                                  const void* aux, int64_t M, float* Y, int64_t ldy, hipStream_t st) {
    constexpr int BM = 16 * TM * WM;
    const int nbw = (WT == 2) ? (int)(K / kQK8) : (int)(K / kQK);
    const int64_t wbytes = N * (int64_t)nbw * GemmCfg<WT>::BB;
    // Row blocks of at most 2^31 activation bytes per launch (the kernel's
    // 32-bit activation offsets); one launch for every practical shape.
    int64_t rows_max = ((int64_t(1) << 31) / K) / BM * BM;
    if (rows_max < BM) return hipErrorInvalidValue;
    rows_max = std::min(rows_max, kMaxGridY * BM);
    const int64_t rb = g_row_block;
    if (rb > 0) rows_max = std::min(rows_max, rb);
    // bytes per activation row in the planar planes: per block a binary32 d
    // and sixteen int16 sums (Q8_K), or a binary16 d and a binary16 s (Q8_1)
    const int64_t d_row = (WT == 2) ? (int64_t)nbw * 2 : (int64_t)nbw * 4;
    const int64_t aux_row = (WT == 2) ? (int64_t)nbw * 2 : (int64_t)nbw * 32;
    GroupArgs ga = {};
    for (int64_t m0 = 0; m0 < M; m0 += rows_max) {
        const int64_t mc = std::min(rows_max, M - m0);
        dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((mc + BM - 1) / BM));
        gemm_kernel<WT, WM, TM, false><<<grid, 128 * WM, 0, st>>>(
            W, (int)N, (int)K, wbytes, (const int8_t*)aqs + m0 * K, (const uint8_t*)ad + m0 * d_row,
            aux ? (const int16_t*)((const uint8_t*)aux + m0 * aux_row) : nullptr, (int)mc, Y + m0 * ldy, ldy, ga);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Q8_0 x Q8_1 takes 64 x 128 tiles (its per-block epilogue dominates; the
// other tile heights measured slower at every workload shape).
hipError_t launch_gemm(int wtype, const uint8_t* W, int64_t N, int64_t K, const void* act_qs,
                       const void* act_d, const void* act_aux, int64_t M, float* Y, int64_t ldy,
                       hipStream_t st) {
    // the K-quant weight types run on the K-quant GEMM (gemm_k.hip)
    if (wtype != 2) return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    return launch_gemm_cfg<2, 4, 2>(W, N, K, act_qs, act_d, act_aux, M, Y, ldy, st);
}

// Grouped launch: one 64 x kGroupTileRows tile per (weight-row block, routed
// tile) on four waves; a routed tile holds up to kGroupTileRows rows of one
// expert, and waves whose rows are all past the tile's rows skip their MFMAs.
constexpr int kGroupBM = kGroupTileRows;
static_assert(kGroupBM % 32 == 0, "two rows of waves, each wave 16 * (kGroupBM / 32) activation rows");

template <int WT>
static hipError_t launch_gemm_grouped_t(const uint8_t* W, int64_t E, int64_t N, int64_t K, const void* aqs,
                                        const void* ad, const void* aux, int64_t T, int64_t top_k, int per_row,
                                        RouteWs ws, float* Y, hipStream_t st) {
    const int nbw = (WT == 2) ? (int)(K / kQK8) : (int)(K / kQK);
    const int64_t estride = N * (int64_t)nbw * GemmCfg<WT>::BB;
    const int64_t max_tiles = (T * top_k + kGroupBM - 1) / kGroupBM + E;
    if (max_tiles == 0) return hipSuccess;
    GroupArgs ga;
    ga.tiles = ws.tiles;
    ga.ntiles = ws.ntiles;
    ga.list = ws.list;
    ga.top_k = (int)top_k;
    ga.per_row = per_row;
    ga.expert_stride = estride;
    int64_t per = kMaxGridY;  // routed tiles per launch
    const int64_t rb = g_row_block;
    if (rb > 0) per = std::min(per, std::max<int64_t>(1, rb / kGroupBM));
    for (int64_t t0 = 0; t0 < max_tiles; t0 += per) {
        ga.tile_base = (int)t0;
        dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)std::min(per, max_tiles - t0));
        gemm_kernel<WT, 2, kGroupBM / 32, true><<<grid, 256, 0, st>>>(
            W, (int)N, (int)K, E * estride, (const int8_t*)aqs, ad, (const int16_t*)aux, (int)T, Y, N * 1, ga);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemm_grouped(int wtype, const uint8_t* W, int64_t E, int64_t N, int64_t K, const void* act_qs,
                               const void* act_d, const void* act_aux, int64_t T, int64_t top_k, int per_row,
                               int tile_rows, RouteWs ws, float* Y, hipStream_t st) {
    if (wtype != 2)
        return launch_gemm_kq_grouped(wtype, W, E, N, K, act_qs, act_d, act_aux, T, top_k, per_row, tile_rows, ws, Y,
                                      st);
    if (tile_rows != kGroupBM) return hipErrorInvalidValue;
    return launch_gemm_grouped_t<2>(W, E, N, K, act_qs, act_d, act_aux, T, top_k, per_row, ws, Y, st);
}

}  // namespace vqk
