// vq_internal.h -- launchers between the host API (vq_api.hip) and the kernel
// files.  Every launcher assumes the host has already validated its
// arguments (types, shapes, alignment, aliasing) and returns the
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vqk {

// Per calling thread: the failure reporting of the kernels launched by the
// current call (set by the API before its launches).
struct DebugCtx {
    int wait_polls = 1 << 20;          // bound of the decode GEMV loaders' wait
    unsigned int* err_word = nullptr;  // the current device's error word
};
extern thread_local DebugCtx g_dbg;

// Debug check of the routed-expert ids: bit 2 of the error word for an id
// outside [0, E), bit 4 for an id repeated within a token.
hipError_t launch_check_ids(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, unsigned int* err_word,
                            hipStream_t st);

// Routed-expert GEMM tiles: the routing scan writes its tile table in units
// of a per-call tile height and the grouped GEMM consumes it.  The Q8_0
// grouped GEMM keeps 96-row tiles (four waves of 32 weight rows x 48
// activation rows); the K-quant one takes 32, 64, 96 or 128 rows from the
// rows per expert (grouped_tile_rows).  The tile table is sized for the
// smallest height.
constexpr int kGroupTileRows = 96;
constexpr int kGroupMinTileRows = 32;

// Planar activation buffers (include/vq.h).
struct ActQ8K {
    int8_t* qs;      // [M][K]
    float* d;        // [M][K/256]
    int16_t* bsums;  // [M][K/16]
};
struct ActQ81 {
    int8_t* qs;      // [M][K]
    uint16_t* d;     // [M][K/32] binary16
    uint16_t* s;     // [M][K/32] binary16
};

// Producers with the quantizer as epilogue: kind 0 RMSNorm (B = gamma),
// kind 1 SiLU-mul (A = gate, B = up); act 0 Q8_K (o8k), 1 Q8_1 (o81).
hipError_t launch_produce_quant(int kind, int act, const float* A, const float* B, int64_t lda, int64_t M,
                                int64_t K, float eps, float* Y, int64_t ldy, ActQ8K o8k, ActQ81 o81,
                                hipStream_t st);
hipError_t launch_quantize_q8k(const float* X, int64_t M, int64_t K, int64_t ldx, ActQ8K out,
                               hipStream_t st);
hipError_t launch_quantize_q8_1(const float* X, int64_t M, int64_t K, int64_t ldx, ActQ81 out,
                                hipStream_t st);
hipError_t launch_quantize_weights(int wtype, const float* W, int64_t N, int64_t K, uint8_t* out,
                                   hipStream_t st);

constexpr int kMaxDevices = 64;
// Compute units of the current device (cached per device).
int num_cus();

// Prefill GEMM row blocking: one launch covers at most this many activation
// rows (0: as many as keep the launch's activation bytes below 2^31).
void set_gemm_row_block(int64_t rows);
int64_t gemm_row_block();  // the calling thread's cap (0: none)

// Decode GEMV with the fused activation quantizer.  xq_out may be null.
hipError_t launch_gemv(int wtype, const uint8_t* W, int64_t N, int64_t K, const float* x,
                       float* y, uint8_t* xq_out, hipStream_t st);
size_t gemv_lds_bytes(int wtype, int64_t N, int64_t K, int mb);
// Small batches (M <= max_m <= kSkinnyMaxM) of pre-quantized activations run
// on the GEMV kernel, which streams the weights once for all M rows (in
// groups of rows above 8).
constexpr int kSkinnyMaxM = 64;
bool gemm_skinny_ok(int wtype, int64_t N, int64_t K, int64_t M, int64_t max_m);
hipError_t launch_gemm_skinny(int wtype, const uint8_t* W, int64_t N, int64_t K, const uint8_t* xq, int64_t M,
                              int64_t d_off, int64_t aux_off, float* Y, int64_t ldy, hipStream_t st);

// Prefill GEMM of the K-quant weights (wtype 0 Q4_K, 1 Q6_K, 5 Q5_K) on
// Q8_K activations; ws/ws_bytes: split-K workspace (may be null).
hipError_t launch_gemm_kq(int wtype, const uint8_t* W, int64_t N, int64_t K, const void* aqs, const void* ad,
                          const void* aux, int64_t M, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                          hipStream_t st);
int gemm_kq_splits(int wtype, int64_t M, int64_t N, int64_t K);
size_t gemm_kq_ws_bytes(int wtype, int64_t M, int64_t N, int64_t K);
size_t gemm_kq_call_ws_bytes(int wtype, int64_t M, int64_t N, int64_t K);  // over the row blocks

// Prefill GEMM on pre-quantized activations (Q8_0 x Q8_1).
hipError_t launch_gemm(int wtype, const uint8_t* W, int64_t N, int64_t K, const void* act_qs,
                       const void* act_d, const void* act_aux, int64_t M, float* Y, int64_t ldy,
                       hipStream_t st);

// Streaming floor of the decode GEMV's launch (measurement only).
// int8 MFMA ceiling (one launch of 2 workgroups per CU); ops_out gets its int8 operations.
hipError_t launch_mfma_probe(int64_t iters, uint32_t* sink, int64_t* ops_out, hipStream_t st);
hipError_t launch_stream_probe(int wtype, const uint8_t* W, int64_t N, int64_t K, uint32_t* sink, int64_t* grid_out,
                               hipStream_t st);

// Routed experts.
struct RouteWs {
    int32_t* counts;   // [E]
    int32_t* offsets;  // [E+1]
    int32_t* list;     // [T*top_k]
    int32_t* chunk;    // [nchunks][E] per-chunk counts, then offsets
    int32_t* rank;     // [T*top_k] rank of each pair among its chunk's pairs of the same expert
    int32_t* tiles;    // tile table
    int32_t* ntiles;   // [1]
};
size_t route_ws_layout(int64_t E, int64_t T, int64_t top_k, RouteWs* ws, uint8_t* base);
// Routed tile height of the grouped GEMM for a call (a multiple of 32).
int grouped_tile_rows(int wtype, int64_t E, int64_t T, int64_t top_k, int64_t K, int per_row);
hipError_t launch_route(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, int tile_rows, RouteWs ws,
                        hipStream_t st);
hipError_t launch_gemm_grouped(int wtype, const uint8_t* W, int64_t E, int64_t N, int64_t K, const void* act_qs,
                               const void* act_d, const void* act_aux, int64_t T, int64_t top_k, int per_row,
                               int tile_rows, RouteWs ws, float* Y, hipStream_t st);
// K-quant routed-expert GEMM on the MFMA core of the dense K-quant GEMM.
hipError_t launch_gemm_kq_grouped(int wtype, const uint8_t* W, int64_t E, int64_t N, int64_t K, const void* aqs,
                                  const void* ad, const void* aux, int64_t T, int64_t top_k, int per_row,
                                  int tile_rows, RouteWs ws, float* Y, hipStream_t st);
hipError_t launch_weighted_sum(const float* Y, const float* w, int64_t T, int64_t top_k, int64_t N,
                               float* Ysum, hipStream_t st);

}  // namespace vqk
