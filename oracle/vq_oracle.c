/*
 * vq_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * block-quantized matmul (Q4_K / Q6_K / Q8_0 weights x Q8_K / Q8_1
 * activations).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library and never calls it.
 *
 * Sources (the pages):
 *   [P1] vllm.cpp PR #3035 "scope a cooperative activation share for the WMMA
 *        kernels" -- the BlockQ8_K activation super-block shared by all warps.
 *   [P2] vllm.cpp PR #2890 "fuse silu-mul with Q8_K quant epilogue" -- commit
 *        "QuantizeQ8KKWarpCoop" (amax scan, iscale=-127/mx, nearest int, clamp
 *        127, bsums), commit "gamma predicate + amax-seed fix" (amax seeded at
 *        0, zero block), commit "kROCM keep-quant provider" (Y = X*W^T, integer
 *        dots in the CPU accumulation order, NMSE 1e-6, f64 dequant band 5e-4).
 *   [P3] strix-llama.cpp PR #18 "Optimize ROCM Prefill and Decode" -- commits
 *        "mul_mat_vec_q_fq" (Q8_1: amax, IEEE division, roundf), "generic
 *        mul_mat_vec_q_fq" (Q8_1 block sum in butterfly order), "warp reduce
 *        via DPP" (xor 16/8/4/2/1 pairing), "weighted expert sum" (explicit
 *        mul then add, no FMA), "routed-compact" (per-expert row lists).
 *
 * Where the pages leave a step open the plainest reading is taken; every such
 * reading is listed beside the function that takes it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Floating point is IEEE binary32 with round-to-nearest-even; no FMA
 * contraction; every product and sum below is rounded on its own.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK_K 256   /* super-block length of Q4_K, Q6_K and Q8_K */
#define QK8 32     /* block length of Q8_0 and Q8_1 */

#define Q4K_BYTES 144
#define Q5K_BYTES 176
#define Q6K_BYTES 210
#define Q8_0_BYTES 34

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary32, written out from the IEEE 754 encodings.           */
/* Rounding to binary16 is round-to-nearest, ties-to-even; subnormals kept.  */
/* ------------------------------------------------------------------------ */

uint16_t oracle_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) {
        if (ax == 0x7F800000u) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u | ((ax >> 13) & 0x3FFu));
    }
    int e = (int)(ax >> 23) - 127;
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    if (e >= -14) {
        uint32_t mant = ax & 0x7FFFFFu;
        uint32_t h = ((uint32_t)(e + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may reach inf: correct */
        return (uint16_t)(sign | h);
    }
    if (e < -25) return sign;
    /* value = sig * 2^(e-23); in units of 2^-24 that is sig * 2^(e+1) */
    uint32_t sig = (ax & 0x7FFFFFu) | 0x800000u;
    int shift = -(e + 1); /* 14..24 */
    uint32_t h = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) h += 1u;
    return (uint16_t)(sign | h);
}

float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    uint32_t x;
    if (e == 0) {
        float v = (float)m * 5.9604644775390625e-8f; /* m * 2^-24, exact */
        memcpy(&x, &v, 4);
        x |= sign;
    } else if (e == 31) {
        x = sign | 0x7F800000u | (m << 13);
    } else {
        x = sign | ((e + 112u) << 23) | (m << 13);
    }
    float f;
    memcpy(&f, &x, 4);
    return f;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ------------------------------------------------------------------------ */
/* Block layouts (this library's own byte layouts; the pages give the fields */
/* but no bit positions).                                                     */
/*                                                                            */
/* Q4_K, 144 bytes per 256 weights:                                           */
/*   [0,2) d (binary16)   [2,4) dmin (binary16)   [4,16) scales   [16,144) qs */
/*   scales byte j (j<8): bits 0-5 = sc_j, bits 6-7 = bits 0-1 of m_j         */
/*   scales byte 8+(j>>1), nibble (j&1): bits 2-5 of m_j                      */
/*   qs byte 32c+l (c<4, l<32): low nibble = element 64c+l,                   */
/*                              high nibble = element 64c+32+l                */
/*   value_i = d*sc_{i/32}*q_i - dmin*m_{i/32}                                */
/* Q6_K, 210 bytes per 256 weights:                                           */
/*   [0,128) ql   [128,192) qh   [192,208) int8 sc[16]   [208,210) d          */
/*   element e, half h=e/128, r=e%128: low 4 bits are nibble r/64 of          */
/*   ql[64h + r%64]; high 2 bits are bit pair r/32 of qh[32h + r%32]          */
/*   value_e = d*sc_{e/16}*(q_e - 32)                                         */
/* Q8_0, 34 bytes per 32 weights: [0,2) d (binary16), [2,34) int8 qs          */
/*   value_i = d*q_i                                                          */
/* Q5_K, 176 bytes per 256 weights (the pages name Q5_K but give no layout;   */
/* this one is a Q4_K block plus a plane of fifth bits):                      */
/*   [0,16) d, dmin and scales exactly as Q4_K   [16,48) qh   [48,176) qs as  */
/*   the Q4_K nibbles; bit j of qh byte l is bit 4 of element 32j+l, so       */
/*   q_i = nibble_i | qhbit_i << 4 in 0..31; value_i = d*sc*q_i - dmin*m      */
/* ------------------------------------------------------------------------ */

typedef struct {
    float d, dmin;
    int sc[8], m[8];
    int q[256];
} q4k_fields;

typedef struct {
    float d;
    int sc[16];
    int q[256]; /* 0..63, zero point 32 */
} q6k_fields;

static void q4k_unpack(const uint8_t* b, q4k_fields* f) {
    f->d = oracle_f16_to_f32(rd16(b));
    f->dmin = oracle_f16_to_f32(rd16(b + 2));
    const uint8_t* s = b + 4;
    for (int j = 0; j < 8; ++j) {
        f->sc[j] = s[j] & 63;
        int hi4 = (s[8 + (j >> 1)] >> (4 * (j & 1))) & 15;
        f->m[j] = (s[j] >> 6) | (hi4 << 2);
    }
    const uint8_t* qs = b + 16;
    for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 32; ++l) {
            f->q[64 * c + l] = qs[32 * c + l] & 15;
            f->q[64 * c + 32 + l] = qs[32 * c + l] >> 4;
        }
}

static void q4k_pack(const q4k_fields* f, uint16_t d16, uint16_t dmin16, uint8_t* b) {
    memset(b, 0, Q4K_BYTES);
    wr16(b, d16);
    wr16(b + 2, dmin16);
    uint8_t* s = b + 4;
    for (int j = 0; j < 8; ++j) {
        s[j] = (uint8_t)((f->sc[j] & 63) | ((f->m[j] & 3) << 6));
        s[8 + (j >> 1)] |= (uint8_t)(((f->m[j] >> 2) & 15) << (4 * (j & 1)));
    }
    uint8_t* qs = b + 16;
    for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 32; ++l)
            qs[32 * c + l] = (uint8_t)((f->q[64 * c + l] & 15) | ((f->q[64 * c + 32 + l] & 15) << 4));
}

/* Q5_K: the Q4_K header and nibbles, then the fifth bit of every element. */
static void q5k_unpack(const uint8_t* b, q4k_fields* f) {
    uint8_t as_q4k[Q4K_BYTES];
    memcpy(as_q4k, b, 16);
    memcpy(as_q4k + 16, b + 48, 128);
    q4k_unpack(as_q4k, f);
    const uint8_t* qh = b + 16;
    for (int e = 0; e < 256; ++e) f->q[e] |= ((qh[e % 32] >> (e / 32)) & 1) << 4;
}

static void q5k_pack(const q4k_fields* f, uint16_t d16, uint16_t dmin16, uint8_t* b) {
    uint8_t as_q4k[Q4K_BYTES];
    q4k_pack(f, d16, dmin16, as_q4k);  /* keeps the low four bits of each q */
    memset(b, 0, Q5K_BYTES);
    memcpy(b, as_q4k, 16);
    memcpy(b + 48, as_q4k + 16, 128);
    uint8_t* qh = b + 16;
    for (int e = 0; e < 256; ++e) qh[e % 32] |= (uint8_t)(((f->q[e] >> 4) & 1) << (e / 32));
}

static void q6k_unpack(const uint8_t* b, q6k_fields* f) {
    const uint8_t* ql = b;
    const uint8_t* qh = b + 128;
    for (int j = 0; j < 16; ++j) f->sc[j] = (int)(int8_t)b[192 + j];
    f->d = oracle_f16_to_f32(rd16(b + 208));
    for (int e = 0; e < 256; ++e) {
        int h = e / 128, r = e % 128;
        int lo = (ql[64 * h + r % 64] >> (4 * (r / 64))) & 15;
        int hi = (qh[32 * h + r % 32] >> (2 * (r / 32))) & 3;
        f->q[e] = lo | (hi << 4);
    }
}

static void q6k_pack(const q6k_fields* f, uint16_t d16, uint8_t* b) {
    memset(b, 0, Q6K_BYTES);
    uint8_t* ql = b;
    uint8_t* qh = b + 128;
    for (int e = 0; e < 256; ++e) {
        int h = e / 128, r = e % 128;
        ql[64 * h + r % 64] |= (uint8_t)((f->q[e] & 15) << (4 * (r / 64)));
        qh[32 * h + r % 32] |= (uint8_t)(((f->q[e] >> 4) & 3) << (2 * (r / 32)));
    }
    for (int j = 0; j < 16; ++j) b[192 + j] = (uint8_t)(int8_t)f->sc[j];
    wr16(b + 208, d16);
}

/* Decoders exposed for the tests (block fields and dequantized values). */
void oracle_q4k_fields(const uint8_t* blk, float* d_dmin, int32_t* sc, int32_t* m, int32_t* q) {
    q4k_fields f;
    q4k_unpack(blk, &f);
    d_dmin[0] = f.d;
    d_dmin[1] = f.dmin;
    for (int j = 0; j < 8; ++j) { sc[j] = f.sc[j]; m[j] = f.m[j]; }
    for (int i = 0; i < 256; ++i) q[i] = f.q[i];
}

void oracle_q5k_fields(const uint8_t* blk, float* d_dmin, int32_t* sc, int32_t* m, int32_t* q) {
    q4k_fields f;
    q5k_unpack(blk, &f);
    d_dmin[0] = f.d;
    d_dmin[1] = f.dmin;
    for (int j = 0; j < 8; ++j) { sc[j] = f.sc[j]; m[j] = f.m[j]; }
    for (int i = 0; i < 256; ++i) q[i] = f.q[i];
}

void oracle_q6k_fields(const uint8_t* blk, float* d, int32_t* sc, int32_t* q) {
    q6k_fields f;
    q6k_unpack(blk, &f);
    d[0] = f.d;
    for (int j = 0; j < 16; ++j) sc[j] = f.sc[j];
    for (int i = 0; i < 256; ++i) q[i] = f.q[i];
}

/* Builders from fields (for hand-made test blocks). */
void oracle_q4k_build(uint16_t d16, uint16_t dmin16, const int32_t* sc, const int32_t* m,
                      const int32_t* q, uint8_t* blk) {
    q4k_fields f;
    for (int j = 0; j < 8; ++j) { f.sc[j] = sc[j]; f.m[j] = m[j]; }
    for (int i = 0; i < 256; ++i) f.q[i] = q[i];
    q4k_pack(&f, d16, dmin16, blk);
}

void oracle_q5k_build(uint16_t d16, uint16_t dmin16, const int32_t* sc, const int32_t* m,
                      const int32_t* q, uint8_t* blk) {
    q4k_fields f;
    for (int j = 0; j < 8; ++j) { f.sc[j] = sc[j]; f.m[j] = m[j]; }
    for (int i = 0; i < 256; ++i) f.q[i] = q[i];
    q5k_pack(&f, d16, dmin16, blk);
}

void oracle_q6k_build(uint16_t d16, const int32_t* sc, const int32_t* q, uint8_t* blk) {
    q6k_fields f;
    for (int j = 0; j < 16; ++j) f.sc[j] = sc[j];
    for (int i = 0; i < 256; ++i) f.q[i] = q[i];
    q6k_pack(&f, d16, blk);
}

/* ------------------------------------------------------------------------ */
/* Weight encoders (test-data generation; the matmul only ever reads bytes). */
/* The pages name the formats but not an encoder; the rules below are the    */
/* plainest min/max scale fit, all in binary32, with d and dmin rounded to   */
/* binary16 before the sub-block scales are fitted against them.             */
/* ------------------------------------------------------------------------ */

/* Q4_K (qmax 15) and Q5_K (qmax 31): per sub-block j of 32: lo=min(0,min w),
 * hi=max w, s=(hi-lo)/qmax, o=-lo; d=f16(max s/63), dmin=f16(max o/63);
 * sc=clamp(rint(s/d),0,63), m=clamp(rint(o/dmin),0,63);
 * q=clamp(rint((w+dmin*m)/(d*sc)),0,qmax); a zero divisor gives 0. */
static void fit_min_blocks(const float* w, int qmax, q4k_fields* f, uint16_t* d16_out,
                           uint16_t* dmin16_out) {
    float s[8], o[8];
    for (int j = 0; j < 8; ++j) {
        float lo = 0.0f, hi = w[32 * j];
        for (int i = 0; i < 32; ++i) {
            float v = w[32 * j + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        float span = hi - lo;
        s[j] = span / (float)qmax;
        o[j] = -lo;
    }
    float maxs = s[0], maxo = o[0];
    for (int j = 1; j < 8; ++j) {
        if (s[j] > maxs) maxs = s[j];
        if (o[j] > maxo) maxo = o[j];
    }
    uint16_t d16 = oracle_f32_to_f16(maxs / 63.0f);
    uint16_t dmin16 = oracle_f32_to_f16(maxo / 63.0f);
    float d = oracle_f16_to_f32(d16), dmin = oracle_f16_to_f32(dmin16);
    for (int j = 0; j < 8; ++j) {
        f->sc[j] = (d != 0.0f) ? clampi((int)rintf(s[j] / d), 0, 63) : 0;
        f->m[j] = (dmin != 0.0f) ? clampi((int)rintf(o[j] / dmin), 0, 63) : 0;
        float off = dmin * (float)f->m[j];
        float div = d * (float)f->sc[j];
        for (int i = 0; i < 32; ++i) {
            int q = 0;
            if (div != 0.0f) {
                float num = w[32 * j + i] + off;
                q = clampi((int)rintf(num / div), 0, qmax);
            }
            f->q[32 * j + i] = q;
        }
    }
    *d16_out = d16;
    *dmin16_out = dmin16;
}

static void encode_q4k_block(const float* w, uint8_t* blk) {
    q4k_fields f;
    uint16_t d16, dmin16;
    fit_min_blocks(w, 15, &f, &d16, &dmin16);
    q4k_pack(&f, d16, dmin16, blk);
}

static void encode_q5k_block(const float* w, uint8_t* blk) {
    q4k_fields f;
    uint16_t d16, dmin16;
    fit_min_blocks(w, 31, &f, &d16, &dmin16);
    q5k_pack(&f, d16, dmin16, blk);
}

/* Q6_K: per sub-block j of 16: s=max|w|/31; d=f16(max s/127);
 * sc=clamp(rint(s/d),0,127); q=clamp(rint(w/(d*sc)),-32,31)+32;
 * a zero divisor gives the signed quant 0 (stored 32). */
static void encode_q6k_block(const float* w, uint8_t* blk) {
    float s[16];
    for (int j = 0; j < 16; ++j) {
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) {
            float a = fabsf(w[16 * j + i]);
            if (a > amax) amax = a;
        }
        s[j] = amax / 31.0f;
    }
    float maxs = s[0];
    for (int j = 1; j < 16; ++j)
        if (s[j] > maxs) maxs = s[j];
    uint16_t d16 = oracle_f32_to_f16(maxs / 127.0f);
    float d = oracle_f16_to_f32(d16);
    q6k_fields f;
    for (int j = 0; j < 16; ++j) {
        f.sc[j] = (d != 0.0f) ? clampi((int)rintf(s[j] / d), 0, 127) : 0;
        float div = d * (float)f.sc[j];
        for (int i = 0; i < 16; ++i) {
            int q = 0;
            if (div != 0.0f) q = clampi((int)rintf(w[16 * j + i] / div), -32, 31);
            f.q[16 * j + i] = q + 32;
        }
    }
    q6k_pack(&f, d16, blk);
}

/* Q8_0: the Q8_1 rule (amax/127, per-element IEEE division, roundf) with the
 * quant clamped to [-127,127]; d stored as binary16. */
static void encode_q8_0_block(const float* w, uint8_t* blk) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(w[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    wr16(blk, oracle_f32_to_f16(d));
    for (int i = 0; i < 32; ++i) {
        int q = 0;
        if (amax != 0.0f) q = clampi((int)roundf(w[i] / d), -127, 127);
        blk[2 + i] = (uint8_t)(int8_t)q;
    }
}

/* type codes shared with the Python wrapper: 0 = Q4_K, 1 = Q6_K, 2 = Q8_0,
 * 5 = Q5_K */
void oracle_quantize_weights(int type, const float* W, int64_t N, int64_t K, uint8_t* out) {
    if (type == 5) {
        int64_t nb = K / QK_K;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < nb; ++b)
                encode_q5k_block(W + n * K + b * QK_K, out + (n * nb + b) * Q5K_BYTES);
    } else if (type == 0) {
        int64_t nb = K / QK_K;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < nb; ++b)
                encode_q4k_block(W + n * K + b * QK_K, out + (n * nb + b) * Q4K_BYTES);
    } else if (type == 1) {
        int64_t nb = K / QK_K;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < nb; ++b)
                encode_q6k_block(W + n * K + b * QK_K, out + (n * nb + b) * Q6K_BYTES);
    } else {
        int64_t nb = K / QK8;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < nb; ++b)
                encode_q8_0_block(W + n * K + b * QK8, out + (n * nb + b) * Q8_0_BYTES);
    }
}

/* ------------------------------------------------------------------------ */
/* Activation quantizers.                                                   */
/* ------------------------------------------------------------------------ */

/* Q8_K, one super-block of 256 ([P2] QuantizeQ8KKWarpCoop and the amax-seed
 * fix):
 *   1. amax=0, mx=0; scan ascending; if |x_i| > amax then amax=|x_i|, mx=x_i.
 *      Strict '>' keeps the first occurrence and never selects a NaN.
 *   2. amax == 0 gives the zero block (d=0, q=0, bsums=0).
 *   3. iscale = -127/mx, correctly rounded binary32 division.
 *   4. q_i = min(127, nearest-int(iscale*x_i)); nearest-int read as
 *      ties-to-even (rint) on the binary32 product.
 *   5. d = 1/iscale (reading: the stored scale is the reciprocal of the
 *      quantizing scale, so d is signed and q(mx) = -127).
 *   6. bsum_j = sum of q over elements 16j..16j+15.
 * Blocks holding Inf, or NaN mixed with numbers, are outside the contract:
 * the quant is then defined here as 0 only to keep the C well defined. */
static void quant_q8k_block(const float* x, int8_t* qs, float* d, int16_t* bsums) {
    float amax = 0.0f, mx = 0.0f;
    for (int i = 0; i < QK_K; ++i) {
        float ax = fabsf(x[i]);
        if (ax > amax) { amax = ax; mx = x[i]; }
    }
    if (amax == 0.0f) {
        memset(qs, 0, QK_K);
        *d = 0.0f;
        for (int j = 0; j < 16; ++j) bsums[j] = 0;
        return;
    }
    float iscale = -127.0f / mx;
    for (int i = 0; i < QK_K; ++i) {
        float v = iscale * x[i];
        float r = rintf(v);
        int q = (r == r && fabsf(r) < 1e9f) ? (int)r : 0;
        if (q > 127) q = 127;
        qs[i] = (int8_t)q;
    }
    *d = 1.0f / iscale;
    for (int j = 0; j < 16; ++j) {
        int s = 0;
        for (int i = 0; i < 16; ++i) s += qs[16 * j + i];
        bsums[j] = (int16_t)s;
    }
}

/* X fp32 [M][ldx], K % 256 == 0.  Output planes: qs int8 [M][K],
 * d fp32 [M][K/256], bsums int16 [M][K/16]. */
void oracle_quantize_q8k(const float* X, int64_t M, int64_t K, int64_t ldx,
                         int8_t* qs, float* d, int16_t* bsums) {
    int64_t nb = K / QK_K;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < nb; ++b)
            quant_q8k_block(X + m * ldx + b * QK_K, qs + m * K + b * QK_K, d + m * nb + b,
                            bsums + (m * nb + b) * 16);
}

/* Q8_1, one block of 32 ([P3] mul_mat_vec_q_fq and its generic extension):
 *   amax = max |x_i| (NaN never selected); d = amax/127 (IEEE division);
 *   q_i = 0 if amax == 0, else roundf(x_i/d) (per-element IEEE division,
 *   halves away from zero), computed with the binary32 d;
 *   s = binary32 sum of x in xor-butterfly order: v_i <- x_i, then for
 *   o = 16, 8, 4, 2, 1: v_i <- v_i + v_(i xor o); s = v_0.
 *   d and s are stored as binary16 (nearest even). */
static void quant_q8_1_block(const float* x, int8_t* qs, uint16_t* d16, uint16_t* s16) {
    float amax = 0.0f;
    for (int i = 0; i < QK8; ++i) {
        float ax = fabsf(x[i]);
        if (ax > amax) amax = ax;
    }
    float d = amax / 127.0f;
    for (int i = 0; i < QK8; ++i) {
        int q = 0;
        if (amax != 0.0f) {
            float r = roundf(x[i] / d);
            q = (r == r && fabsf(r) < 1e9f) ? (int)r : 0;
        }
        qs[i] = (int8_t)q;
    }
    float v[QK8], nv[QK8];
    for (int i = 0; i < QK8; ++i) v[i] = x[i];
    for (int o = 16; o >= 1; o >>= 1) {
        for (int i = 0; i < QK8; ++i) nv[i] = v[i] + v[i ^ o];
        for (int i = 0; i < QK8; ++i) v[i] = nv[i];
    }
    *d16 = oracle_f32_to_f16(d);
    *s16 = oracle_f32_to_f16(v[0]);
}

/* X fp32 [M][ldx], K % 32 == 0.  Output planes: qs int8 [M][K],
 * d binary16 [M][K/32], s binary16 [M][K/32]. */
void oracle_quantize_q8_1(const float* X, int64_t M, int64_t K, int64_t ldx,
                          int8_t* qs, uint16_t* d, uint16_t* s) {
    int64_t nb = K / QK8;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < nb; ++b)
            quant_q8_1_block(X + m * ldx + b * QK8, qs + m * K + b * QK8, d + m * nb + b,
                             s + m * nb + b);
}

/* ------------------------------------------------------------------------ */
/* Dots.  Y[m][n] = sum over blocks b ascending of c_b, in binary32 from 0.  */
/* The integer sums are exact int32; only the scale combine rounds.          */
/* ([P2] kROCM provider: integer dots in the CPU accumulation order.)       */
/* ------------------------------------------------------------------------ */

/* Q4_K x Q8_K, one super-block:
 *   I_j = sum_{i in sub-block j} q_i*a_i; S = sum_j sc_j*I_j;
 *   Mn = sum_j m_j*(bsum_2j + bsum_2j+1);
 *   c = da*(d*f32(S) - dmin*f32(Mn)). */
static float dot_q4k_q8k_block(const q4k_fields* f, const int8_t* a, float da, const int16_t* bs,
                               int32_t* I_out) {
    int32_t S = 0, Mn = 0;
    for (int j = 0; j < 8; ++j) {
        int32_t I = 0;
        for (int i = 0; i < 32; ++i) I += f->q[32 * j + i] * (int32_t)a[32 * j + i];
        if (I_out) I_out[j] = I;
        S += f->sc[j] * I;
        Mn += f->m[j] * ((int32_t)bs[2 * j] + (int32_t)bs[2 * j + 1]);
    }
    float t1 = f->d * (float)S;
    float t2 = f->dmin * (float)Mn;
    float t3 = t1 - t2;
    return da * t3;
}

/* Q6_K x Q8_K, one super-block:
 *   I_j = sum_{i in sub-block j of 16} (q_i-32)*a_i; S = sum_j sc_j*I_j;
 *   c = da*(d*f32(S)). */
static float dot_q6k_q8k_block(const q6k_fields* f, const int8_t* a, float da, int32_t* I_out) {
    int32_t S = 0;
    for (int j = 0; j < 16; ++j) {
        int32_t I = 0;
        for (int i = 0; i < 16; ++i) I += (f->q[16 * j + i] - 32) * (int32_t)a[16 * j + i];
        if (I_out) I_out[j] = I;
        S += f->sc[j] * I;
    }
    float t1 = f->d * (float)S;
    return da * t1;
}

/* Q8_0 x Q8_1, one block of 32: I = sum qw_i*qa_i; c = (dw*da)*f32(I). */
static float dot_q8_0_q8_1_block(const uint8_t* blk, const int8_t* a, float da, int32_t* I_out) {
    float dw = oracle_f16_to_f32(rd16(blk));
    const int8_t* qw = (const int8_t*)(blk + 2);
    int32_t I = 0;
    for (int i = 0; i < QK8; ++i) I += (int32_t)qw[i] * (int32_t)a[i];
    if (I_out) I_out[0] = I;
    float s = dw * da;
    return s * (float)I;
}

/* One output: row n of W against activation row m. */
static float dot_row(int type, const uint8_t* wrow, int64_t K, const int8_t* qs_row,
                     const void* d_row, const void* aux_row) {
    float y = 0.0f;
    if (type == 5) {
        /* Q5_K: the Q4_K definition with q in 0..31 */
        const float* da = (const float*)d_row;
        const int16_t* bs = (const int16_t*)aux_row;
        q4k_fields f;
        for (int64_t b = 0; b < K / QK_K; ++b) {
            q5k_unpack(wrow + b * Q5K_BYTES, &f);
            float c = dot_q4k_q8k_block(&f, qs_row + b * QK_K, da[b], bs + b * 16, NULL);
            y = y + c;
        }
    } else if (type == 0) {
        const float* da = (const float*)d_row;
        const int16_t* bs = (const int16_t*)aux_row;
        q4k_fields f;
        for (int64_t b = 0; b < K / QK_K; ++b) {
            q4k_unpack(wrow + b * Q4K_BYTES, &f);
            float c = dot_q4k_q8k_block(&f, qs_row + b * QK_K, da[b], bs + b * 16, NULL);
            y = y + c;
        }
    } else if (type == 1) {
        const float* da = (const float*)d_row;
        q6k_fields f;
        for (int64_t b = 0; b < K / QK_K; ++b) {
            q6k_unpack(wrow + b * Q6K_BYTES, &f);
            float c = dot_q6k_q8k_block(&f, qs_row + b * QK_K, da[b], NULL);
            y = y + c;
        }
    } else {
        const uint16_t* da16 = (const uint16_t*)d_row;
        for (int64_t b = 0; b < K / QK8; ++b) {
            float da = oracle_f16_to_f32(da16[b]);
            float c = dot_q8_0_q8_1_block(wrow + b * Q8_0_BYTES, qs_row + b * QK8, da, NULL);
            y = y + c;
        }
    }
    return y;
}

static int64_t row_bytes(int type, int64_t K) {
    if (type == 5) return (K / QK_K) * Q5K_BYTES;
    if (type == 0) return (K / QK_K) * Q4K_BYTES;
    if (type == 1) return (K / QK_K) * Q6K_BYTES;
    return (K / QK8) * Q8_0_BYTES;
}

/* Y[m][n] for m < M, n < N (Y row stride ldy).  Activation planes as produced
 * by the quantizers: qs [M][K]; for Q8_K d fp32 [M][K/256] and bsums int16
 * [M][K/16]; for Q8_1 d binary16 [M][K/32] (its s is not read by Q8_0).
 * nthreads splits the output rows over threads; the arithmetic of each
 * output is unchanged. */
void oracle_gemm(int type, const uint8_t* W, int64_t N, int64_t K, const int8_t* qs,
                 const void* d, const int16_t* bsums, int64_t M, float* Y, int64_t ldy,
                 int nthreads) {
    int64_t rb = row_bytes(type, K);
    int64_t nbd = (type == 2) ? K / QK8 : K / QK_K;
    int64_t total = M * N;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t idx = 0; idx < total; ++idx) {
        int64_t m = idx / N, n = idx % N;
        const void* drow = (type == 2) ? (const void*)((const uint16_t*)d + m * nbd)
                                       : (const void*)((const float*)d + m * nbd);
        const void* aux = (type == 0 || type == 5) ? (const void*)(bsums + m * (K / 16)) : NULL;
        Y[m * ldy + n] = dot_row(type, W + n * rb, K, qs + m * K, drow, aux);
    }
}

/* Selected outputs only: out[i] = Y[ms[i]][ns[i]] (for sampled checks at full
 * size). */
void oracle_gemm_sampled(int type, const uint8_t* W, int64_t N, int64_t K, const int8_t* qs,
                         const void* d, const int16_t* bsums, const int64_t* ms,
                         const int64_t* ns, int64_t count, float* out, int nthreads) {
    int64_t rb = row_bytes(type, K);
    int64_t nbd = (type == 2) ? K / QK8 : K / QK_K;
    (void)N;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        const void* drow = (type == 2) ? (const void*)((const uint16_t*)d + m * nbd)
                                       : (const void*)((const float*)d + m * nbd);
        const void* aux = (type == 0 || type == 5) ? (const void*)(bsums + m * (K / 16)) : NULL;
        out[i] = dot_row(type, W + n * rb, K, qs + m * K, drow, aux);
    }
}

/* The exact int32 sub-block sums I_j of one (weight block, activation block)
 * pair: 8 values for Q4_K and Q5_K, 16 for Q6_K, 1 for Q8_0. */
void oracle_subblock_sums(int type, const uint8_t* wblk, const int8_t* a, int32_t* I_out) {
    if (type == 5) {
        q4k_fields f;
        q5k_unpack(wblk, &f);
        int16_t bs[16] = {0};
        dot_q4k_q8k_block(&f, a, 1.0f, bs, I_out);
    } else if (type == 0) {
        q4k_fields f;
        q4k_unpack(wblk, &f);
        int16_t bs[16] = {0};
        dot_q4k_q8k_block(&f, a, 1.0f, bs, I_out);
    } else if (type == 1) {
        q6k_fields f;
        q6k_unpack(wblk, &f);
        dot_q6k_q8k_block(&f, a, 1.0f, I_out);
    } else {
        dot_q8_0_q8_1_block(wblk, a, 1.0f, I_out);
    }
}

/* ------------------------------------------------------------------------ */
/* Routed experts ([P3] routed-compact MUL_MAT_ID and weighted expert sum). */
/* ------------------------------------------------------------------------ */

/* counts[e] = #{(t,s): ids[t][s] == e}; offsets[0..E] = exclusive prefix sum
 * (offsets[E] = T*top_k); list = pair indices t*top_k+s grouped by expert,
 * ascending (t,s) inside each expert (stable compaction). */
void oracle_route(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, int32_t* counts,
                  int32_t* offsets, int32_t* list) {
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < T * top_k; ++p) counts[ids[p]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e) pos[e] = offsets[e];
    for (int64_t p = 0; p < T * top_k; ++p) list[pos[ids[p]]++] = (int32_t)p;
    free(pos);
}

/* Y[t][s][n] = dot(W_{ids[t][s]} row n, x_t) for Q8_K activations; W is
 * [E][N] rows of K/256 blocks. */
void oracle_gemm_grouped(int type, const uint8_t* W, int64_t E, int64_t N, int64_t K,
                         const int8_t* qs, const void* d, const int16_t* bsums, int64_t T,
                         const int32_t* ids, int64_t top_k, int per_row, float* Y, int nthreads) {
    int64_t rb = row_bytes(type, K);
    int64_t nbd = (type == 2) ? K / QK8 : K / QK_K;
    int64_t total = T * top_k * N;
    (void)E;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t idx = 0; idx < total; ++idx) {
        int64_t p = idx / N, n = idx % N;
        /* broadcast arm: the pair's token row; per-row arm: the pair's own row */
        int64_t a = per_row ? p : p / top_k;
        int64_t e = ids[p];
        const uint8_t* wrow = W + (e * N + n) * rb;
        const void* drow = (type == 2) ? (const void*)((const uint16_t*)d + a * nbd)
                                       : (const void*)((const float*)d + a * nbd);
        const void* aux = (type == 0 || type == 5) ? (const void*)(bsums + a * (K / 16)) : NULL;
        Y[idx] = dot_row(type, wrow, K, qs + a * K, drow, aux);
    }
}

/* Ysum[t][n] = (((w0*y0 + w1*y1) + w2*y2) + ...) + w_{k-1}*y_{k-1}: slots
 * ascending, each product and each sum rounded on its own (no FMA). */
void oracle_weighted_sum(const float* Y, const float* w, int64_t T, int64_t top_k, int64_t N,
                         float* Ysum) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            float acc = w[t * top_k] * Y[(t * top_k) * N + n];
            for (int64_t s = 1; s < top_k; ++s) {
                float p = w[t * top_k + s] * Y[(t * top_k + s) * N + n];
                acc = acc + p;
            }
            Ysum[t * N + n] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Producers whose output feeds the activation quantizer ([P2] commits       */
/* "Norm epilogue" (RMSNorm row kernel emitting the row's Q8_K blocks) and    */
/* "SiLU-mul quant" (silu(gate)*up emitting Q8_K)).  The pages name the       */
/* operations, not their formulas; the textbook definitions are taken, in    */
/* binary64 from the binary32 inputs:                                        */
/*   RMSNorm: y_i = x_i / sqrt(mean_j(x_j^2) + eps) * gamma_i                */
/*   SiLU-mul: y_i = g_i / (1 + exp(-g_i)) * u_i  (silu(g) = g*sigmoid(g))   */
/* The fused producer's quantized bytes are checked against                  */
/* oracle_quantize_q8k / _q8_1 applied to the producer's own binary32        */
/* output (the pages' byte-identity with the unfused path).                  */
/* ------------------------------------------------------------------------ */
void oracle_rmsnorm(const float* X, const float* gamma, int64_t M, int64_t K, int64_t ldx, double eps,
                    double* Y) {
    for (int64_t m = 0; m < M; ++m) {
        const float* x = X + m * ldx;
        double ss = 0.0;
        for (int64_t i = 0; i < K; ++i) ss += (double)x[i] * (double)x[i];
        const double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t i = 0; i < K; ++i) Y[m * K + i] = (double)x[i] * r * (double)gamma[i];
    }
}

void oracle_silu_mul(const float* G, const float* U, int64_t M, int64_t K, int64_t ldx, double* Y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t i = 0; i < K; ++i) {
            const double g = (double)G[m * ldx + i];
            Y[m * K + i] = g / (1.0 + exp(-g)) * (double)U[m * ldx + i];
        }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
