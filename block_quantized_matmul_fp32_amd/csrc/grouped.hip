// grouped.hip -- routing / compaction for the routed-expert grouped GEMM and
// the weighted expert sum, for gfx950.
//
// Pages: strix-llama.cpp PR #18, commits "routed-compact" (token-expert pairs
// grouped per expert, MUL_MAT_ID tiles sized from the rows of each expert
// instead of the total pair count, which left 50-87% of every tile as
// padding) and "weighted expert sum" (slot-ordered explicit multiply then
// add, no FMA contraction, no scratch spills, four adjacent channels per
// thread with float4 accesses).
//
// Routing is integer bookkeeping with one answer: counts per expert, the
// exclusive prefix offsets, and the pair indices t*top_k+s listed per expert
// in ascending (t, s) order.  It is built without atomics in three small
// launches (per-chunk counts, one scan workgroup that also writes the tile
// table, per-chunk placement), so the list is deterministic; the tile table
// stays on the device, so the grouped GEMM needs no host synchronisation.
#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

constexpr int kRouteChunk = 64;   // tokens per routing chunk
constexpr int kTileRows = kGroupTileRows;

size_t route_ws_layout(int64_t E, int64_t T, int64_t top_k, RouteWs* ws, uint8_t* base) {
    const int64_t nchunks = (T + kRouteChunk - 1) / kRouteChunk;
    const int64_t max_tiles = (T * top_k + kTileRows - 1) / kTileRows + E;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t o_counts = take(sizeof(int32_t) * (size_t)E);
    const size_t o_offsets = take(sizeof(int32_t) * (size_t)(E + 1));
    const size_t o_list = take(sizeof(int32_t) * (size_t)(T * top_k));
    const size_t o_chunk = take(sizeof(int32_t) * (size_t)(nchunks * E));
    const size_t o_tiles = take(sizeof(int32_t) * 4 * (size_t)max_tiles);
    const size_t o_ntiles = take(sizeof(int32_t) * 4);
    if (ws) {
        ws->counts = (int32_t*)(base + o_counts);
        ws->offsets = (int32_t*)(base + o_offsets);
        ws->list = (int32_t*)(base + o_list);
        ws->chunk = (int32_t*)(base + o_chunk);
        ws->tiles = (int32_t*)(base + o_tiles);
        ws->ntiles = (int32_t*)(base + o_ntiles);
    }
    return off;
}

// Per chunk of 64 tokens: chunk[c][e] = number of pairs of the chunk routed to e.
__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids, int T,
                                                          int top_k, int E, int32_t* __restrict__ chunk) {
    __shared__ int32_t sid[kRouteChunk * 16];
    const int c = blockIdx.x;
    const int t0 = c * kRouteChunk;
    const int np = min(kRouteChunk, T - t0) * top_k;
    for (int i = threadIdx.x; i < np; i += 256) sid[i] = ids[(int64_t)t0 * top_k + i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        int cnt = 0;
        for (int i = 0; i < np; ++i) cnt += (sid[i] == e);
        chunk[(int64_t)c * E + e] = cnt;
    }
}

// One workgroup: per-expert scan over chunks (chunk[c][e] becomes the
// exclusive offset of the chunk inside the expert), counts, expert offsets,
// and the tile table (expert, first list slot, rows).
__global__ __launch_bounds__(1024) void route_scan_kernel(int nchunks, int E, int32_t* __restrict__ chunk,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles) {
    __shared__ int32_t sc[1024];
    __shared__ int32_t st[1024];
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        for (int c = 0; c < nchunks; ++c) {
            const int v = chunk[(int64_t)c * E + e];
            chunk[(int64_t)c * E + e] = total;
            total += v;
        }
        counts[e] = total;
    }
    const int nt = (e < E) ? (total + kTileRows - 1) / kTileRows : 0;
    sc[e] = (e < E) ? total : 0;
    st[e] = nt;
    __syncthreads();
    // inclusive Hillis-Steele scans of counts and tile counts
    for (int o = 1; o < 1024; o <<= 1) {
        const int a = (e >= o) ? sc[e - o] : 0;
        const int b = (e >= o) ? st[e - o] : 0;
        __syncthreads();
        sc[e] += a;
        st[e] += b;
        __syncthreads();
    }
    if (e < E) {
        const int off = sc[e] - total;
        offsets[e] = off;
        if (e == E - 1) offsets[E] = sc[e];
        int tbase = st[e] - nt;
        for (int i = 0; i < nt; ++i) {
            tiles[4 * (tbase + i) + 0] = e;
            tiles[4 * (tbase + i) + 1] = off + i * kTileRows;
            tiles[4 * (tbase + i) + 2] = min(kTileRows, total - i * kTileRows);
            tiles[4 * (tbase + i) + 3] = 0;
        }
        if (e == E - 1) ntiles[0] = st[e];
    }
}

// Per chunk: list[offsets[e] + chunk offset + k] = pair index, ascending.
__global__ __launch_bounds__(256) void route_place_kernel(const int32_t* __restrict__ ids, int T, int top_k,
                                                          int E, const int32_t* __restrict__ chunk,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ list) {
    __shared__ int32_t sid[kRouteChunk * 16];
    const int c = blockIdx.x;
    const int t0 = c * kRouteChunk;
    const int np = min(kRouteChunk, T - t0) * top_k;
    for (int i = threadIdx.x; i < np; i += 256) sid[i] = ids[(int64_t)t0 * top_k + i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        int pos = offsets[e] + chunk[(int64_t)c * E + e];
        for (int i = 0; i < np; ++i)
            if (sid[i] == e) list[pos++] = t0 * top_k + i;
    }
}

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, RouteWs ws,
                        hipStream_t st) {
    const int nchunks = (int)((T + kRouteChunk - 1) / kRouteChunk);
    if (nchunks > 0)
        route_count_kernel<<<nchunks, 256, 0, st>>>(ids, (int)T, (int)top_k, (int)E, ws.chunk);
    route_scan_kernel<<<1, 1024, 0, st>>>(nchunks, (int)E, ws.chunk, ws.counts, ws.offsets, ws.tiles,
                                          ws.ntiles);
    if (nchunks > 0)
        route_place_kernel<<<nchunks, 256, 0, st>>>(ids, (int)T, (int)top_k, (int)E, ws.chunk, ws.offsets,
                                                    ws.list);
    return hipGetLastError();
}

// Ysum[t][n..n+3] = (((w0*y0 + w1*y1) + w2*y2) + ...): one thread per four
// adjacent channels.
__global__ __launch_bounds__(256) void weighted_sum_kernel(const float* __restrict__ Y,
                                                           const float* __restrict__ w, int T, int top_k,
                                                           int N, float* __restrict__ Ysum) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int n4 = N / 4;
    if (q >= (int64_t)T * n4) return;
    const int64_t t = q / n4;
    const int n = (int)(q - t * n4) * 4;
    const float* yp = Y + t * top_k * (int64_t)N + n;
    const float* wp = w + t * top_k;
    float4 v = *(const float4*)yp;
    float w0 = wp[0];
    float a0 = w0 * v.x, a1 = w0 * v.y, a2 = w0 * v.z, a3 = w0 * v.w;
    for (int s = 1; s < top_k; ++s) {
        const float4 u = *(const float4*)(yp + (int64_t)s * N);
        const float ws = wp[s];
        const float p0 = ws * u.x, p1 = ws * u.y, p2 = ws * u.z, p3 = ws * u.w;
        a0 = a0 + p0; a1 = a1 + p1; a2 = a2 + p2; a3 = a3 + p3;
    }
    *(float4*)(Ysum + t * (int64_t)N + n) = make_float4(a0, a1, a2, a3);
}

hipError_t launch_weighted_sum(const float* Y, const float* w, int64_t T, int64_t top_k, int64_t N,
                               float* Ysum, hipStream_t st) {
    const int64_t total = T * (N / 4);
    if (total == 0) return hipSuccess;
    weighted_sum_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(Y, w, (int)T, (int)top_k, (int)N,
                                                                        Ysum);
    return hipGetLastError();
}

}  // namespace vqk
