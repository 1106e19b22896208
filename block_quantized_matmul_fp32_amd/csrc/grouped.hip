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
// in ascending (t, s) order.  It is built without atomics, so the list is
// deterministic.  A call of up to 8192 pairs is routed by one workgroup in
// one launch (route_one_kernel below); larger calls take two launches (up to
// 64 chunks) or three, which spread the ballot work (the bulk of the
// routing's instructions) over one CU per chunk:
//  * four waves per chunk of 64 tokens, each walking a quarter of the
//    chunk's pairs 64 at a time; the lanes holding the same expert are found
//    with one ballot per bit of the expert id, which gives each pair its rank
//    among the quarter's earlier pairs of that expert and the quarter's
//    per-expert counts, and the quarters' counts then give the ranks in the
//    chunk and the chunk's per-expert counts;
//  * up to 64 chunks: one workgroup per chunk sums the chunk table, scans
//    it over experts and places the chunk's pairs (workgroup 0 writes the
//    counts, offsets and tile table);
//  * more chunks: one workgroup scans the per-chunk counts over chunks and
//    experts and writes the tile table, then one thread per pair writes it
//    to its list slot.
// The tile table stays on the device, so the grouped GEMM needs no host
// synchronisation.  Pairs whose id is outside [0, E) are neither counted nor
// placed.
#include "vq_device.h"
#include "vq_internal.h"

// Every binary32 expression in this file is evaluated as written: no
// multiply-add contraction (the fixed-order definitions round each product
// and each sum on their own).
#pragma clang fp contract(off)

namespace vqk {

constexpr int kRouteChunk = 64;   // tokens per routing chunk

size_t route_ws_layout(int64_t E, int64_t T, int64_t top_k, RouteWs* ws, uint8_t* base) {
    const int64_t nchunks = (T + kRouteChunk - 1) / kRouteChunk;
    const int64_t max_tiles = (T * top_k + kGroupMinTileRows - 1) / kGroupMinTileRows + E;
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
    const size_t o_rank = take(sizeof(int32_t) * (size_t)(T * top_k));
    const size_t o_tiles = take(sizeof(int32_t) * 4 * (size_t)max_tiles);
    const size_t o_ntiles = take(sizeof(int32_t) * 4);
    if (ws) {
        ws->counts = (int32_t*)(base + o_counts);
        ws->offsets = (int32_t*)(base + o_offsets);
        ws->list = (int32_t*)(base + o_list);
        ws->chunk = (int32_t*)(base + o_chunk);
        ws->rank = (int32_t*)(base + o_rank);
        ws->tiles = (int32_t*)(base + o_tiles);
        ws->ntiles = (int32_t*)(base + o_ntiles);
    }
    return off;
}

constexpr int kIdBits = 11;  // expert ids < 1024, plus 64 distinct keys for pairs not routed

// One workgroup of kCountWaves waves per chunk of kRouteChunk tokens:
// rank[p] = number of earlier pairs of the chunk with the same expert,
// chunk[c][e] = the chunk's pairs of e.  Wave w takes the contiguous pair
// range [w L, (w + 1) L) of the chunk (L a multiple of 64) and ranks its
// pairs among the range's earlier pairs (ballot-per-id-bit groups, as in
// route_one_kernel), counting per expert in its own LDS row; then the
// counts are turned into each wave's exclusive offset inside the expert
// (wave order is pair order), and a pair's rank is its rank in the range
// plus its wave's offset.  Same ranks and counts as one wave walking the
// whole chunk, in a quarter of the rounds.  Grouped calls take top_k <= 16,
// so a chunk holds at most 1024 pairs and a wave at most 4 rounds.
constexpr int kCountWaves = 4;
constexpr int kCountThreads = 64 * kCountWaves;
constexpr int kCountMaxPairs = kRouteChunk * 16;
constexpr int kCountMaxRounds = kCountMaxPairs / kCountThreads;
__global__ __launch_bounds__(kCountThreads) void route_count_kernel(const int32_t* __restrict__ ids, int T,
                                                                    int top_k, int E, int32_t* __restrict__ chunk,
                                                                    int32_t* __restrict__ rank) {
    __shared__ int32_t cnt[kCountWaves * 1024];  // [wave][expert]: count, then the wave's offset
    __shared__ int32_t lrank[kCountMaxPairs];     // rank inside the wave's range, or -1 (not routed)
    __shared__ int16_t lexp[kCountMaxPairs];      // the pair's expert
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x;
    const int64_t p0 = (int64_t)c * kRouteChunk * top_k;
    const int np = min(kRouteChunk, T - c * kRouteChunk) * top_k;
    for (int i = tid; i < kCountWaves * E; i += kCountThreads) cnt[i] = 0;
    __syncthreads();
    const int L = 64 * ((np + kCountThreads - 1) / kCountThreads);
    const int a = min(w * L, np), b = min(a + L, np);
    int32_t* cw = cnt + w * E;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // the range's ids are requested up front, so the rounds do not each wait
    // on a global load
    int idv[kCountMaxRounds];
#pragma unroll
    for (int k = 0; k < kCountMaxRounds; ++k) {
        const int i = a + 64 * k + lane;
        idv[k] = (i < b) ? ids[p0 + i] : -1;
    }
#pragma unroll
    for (int k = 0; k < kCountMaxRounds; ++k) {
        if (a + 64 * k >= b) break;  // uniform
        const int i = a + 64 * k + lane;
        const int e = idv[k];
        const bool ok = (i < b) && e >= 0 && e < E;
        const int key = ok ? e : 1024 + lane;  // a pair not routed matches no other lane
        uint64_t same = ~0ull;
#pragma unroll
        for (int bit = 0; bit < kIdBits; ++bit) {
            const uint64_t set = __ballot((key >> bit) & 1);
            same &= ((key >> bit) & 1) ? set : ~set;
        }
        // the wave's LDS operations run in order, so this round reads what
        // the previous round's group leaders wrote
        const int before = ok ? cw[e] : 0;
        if (i < b) {
            lrank[i] = ok ? before + __popcll(same & below) : -1;
            lexp[i] = (int16_t)(ok ? e : 0);
        }
        // the highest lane of each expert's group advances the count
        if (ok && (same >> lane) == 1ull) cw[e] = before + __popcll(same);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kCountThreads) {
        int run = 0;
#pragma unroll
        for (int u = 0; u < kCountWaves; ++u) {
            const int v = cnt[u * E + e];
            cnt[u * E + e] = run;
            run += v;
        }
        chunk[(int64_t)c * E + e] = run;
    }
    __syncthreads();
    for (int i = tid; i < np; i += kCountThreads) {
        const int lr = lrank[i];
        if (lr >= 0) rank[p0 + i] = lr + cnt[(i / L) * E + lexp[i]];
    }
}

// One workgroup: chunk[c][e] becomes the exclusive offset of chunk c inside
// expert e; counts, expert offsets and the tile table (expert, first list
// slot, rows).  kScanThreads / E threads share one expert's chunks.
constexpr int kScanThreads = 1024;
constexpr int64_t kScanStageCells = 12288;  // chunk-table cells staged in LDS (48 KiB)
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(int nchunks, int E, int tile_rows,
                                                                  int32_t* __restrict__ chunk,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ tiles,
                                                                  int32_t* __restrict__ ntiles) {
    extern __shared__ int32_t cstage[];  // the chunk table, when it fits (dynamic LDS)
    __shared__ int32_t part[kScanThreads];
    __shared__ int32_t sc[1024];
    __shared__ int32_t st[1024];
    const int tid = threadIdx.x;
    const int tpe = kScanThreads / E;  // threads per expert (>= 1 for E <= 1024)
    const int e = tid / tpe, q = tid % tpe;
    const bool own = e < E;
    const int len = (nchunks + tpe - 1) / tpe;
    const int c0 = min(nchunks, q * len), c1 = min(nchunks, c0 + len);
    const int64_t ncell = (int64_t)nchunks * E;
    // Staged: one coalesced copy into LDS, the two passes over it there, one
    // coalesced copy back (instead of two rounds of strided global reads).
    const bool staged = ncell <= kScanStageCells;
    int32_t* tab = staged ? cstage : chunk;
    if (staged) {
        // all of a thread's loads in flight before its first LDS store
        constexpr int kMaxPer = (int)((kScanStageCells + kScanThreads - 1) / kScanThreads);
        int32_t v[kMaxPer];
#pragma unroll
        for (int k = 0; k < kMaxPer; ++k) {
            const int64_t i = tid + (int64_t)k * kScanThreads;
            v[k] = (i < ncell) ? chunk[i] : 0;
        }
#pragma unroll
        for (int k = 0; k < kMaxPer; ++k) {
            const int64_t i = tid + (int64_t)k * kScanThreads;
            if (i < ncell) cstage[i] = v[k];
        }
        __syncthreads();
    }
    int sum = 0;
    if (own)
        for (int c = c0; c < c1; ++c) sum += tab[(int64_t)c * E + e];
    part[tid] = sum;
    __syncthreads();
    int base = 0, total = 0;
    if (own) {
        for (int k = 0; k < tpe; ++k) {
            const int v = part[e * tpe + k];
            base += (k < q) ? v : 0;
            total += v;
        }
        int run = base;
        for (int c = c0; c < c1; ++c) {
            const int v = tab[(int64_t)c * E + e];
            tab[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    if (staged) {
        __syncthreads();
        for (int64_t i = tid; i < ncell; i += kScanThreads) chunk[i] = cstage[i];
    }
    const bool lead = own && q == 0;
    if (lead) counts[e] = total;
    if (tid < 1024) {
        const int ex = tid;
        sc[ex] = 0;
        st[ex] = 0;
    }
    __syncthreads();
    const int nt = lead ? (total + tile_rows - 1) / tile_rows : 0;
    if (lead) {
        sc[e] = total;
        st[e] = nt;
    }
    __syncthreads();
    // inclusive scans of counts and tile counts over experts (index = tid):
    // within each wave by shuffles, then the earlier waves' totals added
    {
        __shared__ int32_t wsc[kScanThreads / 64], wst[kScanThreads / 64];
        const int lane = tid & 63, w = tid >> 6;
        int a = sc[tid], b = st[tid];
        for (int o = 1; o < 64; o <<= 1) {
            const int ua = __shfl_up(a, o, 64), ub = __shfl_up(b, o, 64);
            if (lane >= o) { a += ua; b += ub; }
        }
        if (lane == 63) { wsc[w] = a; wst[w] = b; }
        __syncthreads();
        for (int k = 0; k < w; ++k) { a += wsc[k]; b += wst[k]; }
        sc[tid] = a;
        st[tid] = b;
        __syncthreads();
    }
    if (lead) {
        const int off = sc[e] - total;
        offsets[e] = off;
        if (e == E - 1) offsets[E] = sc[e];
        const int tbase = st[e] - nt;
        for (int i = 0; i < nt; ++i) {
            tiles[4 * (tbase + i) + 0] = e;
            tiles[4 * (tbase + i) + 1] = off + i * tile_rows;
            tiles[4 * (tbase + i) + 2] = min(tile_rows, total - i * tile_rows);
            tiles[4 * (tbase + i) + 3] = 0;
        }
        if (e == E - 1) ntiles[0] = st[e];
    }
}

// One workgroup routes a whole call of up to kOneMaxPairs pairs in a single
// launch (no chunk table and no second or third launch).  Wave v of the 16
// takes the contiguous pair range [v L, (v + 1) L), L = 64 rounds:
//  * count: per round of 64 pairs, the ballot-per-id-bit groups give each
//    pair its rank among the wave's earlier pairs of its expert (kept in
//    rank[]) and advance the wave's per-expert count in LDS;
//  * scan: one thread per expert turns the 16 wave counts into the waves'
//    exclusive offsets inside the expert (wave order is pair order) and the
//    expert's total; totals and tile counts are scanned over experts, and the
//    counts, offsets and tile table are written;
//  * place: each wave walks its pairs again, list[offset(e) + wave offset(e)
//    + rank] = pair index.
// Per-wave counts and offsets stay below 2^16 (at most kOneMaxPairs pairs).
// Every round costs each wave about 140 instructions, and the 16 waves share
// one CU's four SIMDs (about 1.3 us per round of 1024 pairs measured), so
// above kOneMaxPairs the three-launch path, with one CU per chunk, is faster.
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int64_t kOneMaxPairs = 8192;
constexpr int kOneIdBatch = 8;  // rounds whose ids are requested together
__global__ __launch_bounds__(kOneThreads) void route_one_kernel(const int32_t* __restrict__ ids, int npairs, int E,
                                                                int tile_rows, int32_t* __restrict__ rank,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ list,
                                                                int32_t* __restrict__ tiles,
                                                                int32_t* __restrict__ ntiles) {
    __shared__ uint16_t wcnt[kOneWaves * 1024];  // [wave][expert]: count, then the wave's offset
    __shared__ int32_t eoff[1024];               // exclusive offset of each expert in the list
    __shared__ int32_t wsc[kOneWaves], wst[kOneWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int v = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < kOneWaves * E; i += kOneThreads) wcnt[i] = 0;
    __syncthreads();
    const int rounds = (npairs + kOneThreads - 1) / kOneThreads;
    const int p0 = v * rounds * 64;
    uint16_t* cnt = wcnt + v * E;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int idv[kOneIdBatch];
    for (int r0 = 0; r0 < rounds; r0 += kOneIdBatch) {
#pragma unroll
        for (int k = 0; k < kOneIdBatch; ++k) {
            const int p = p0 + 64 * (r0 + k) + lane;
            idv[k] = (r0 + k < rounds && p < npairs) ? ids[p] : -1;
        }
#pragma unroll
        for (int k = 0; k < kOneIdBatch; ++k) {
            if (r0 + k >= rounds) break;  // uniform
            const int p = p0 + 64 * (r0 + k) + lane;
            const int e = idv[k];
            const bool ok = p < npairs && e >= 0 && e < E;
            const int key = ok ? e : 1024 + lane;  // a pair not routed matches no other lane
            uint64_t same = ~0ull;
#pragma unroll
            for (int b = 0; b < kIdBits; ++b) {
                const uint64_t set = __ballot((key >> b) & 1);
                same &= ((key >> b) & 1) ? set : ~set;
            }
            // the wave's LDS operations run in order, so this round reads what
            // the previous round's group leaders wrote
            const int before = ok ? (int)cnt[e] : 0;
            if (ok) rank[p] = before + __popcll(same & below);
            if (ok && (same >> lane) == 1ull) cnt[e] = (uint16_t)(before + __popcll(same));
        }
    }
    __syncthreads();
    int total = 0;
    if (tid < E) {
        int c[kOneWaves];  // all 16 counts read before the first offset is written
#pragma unroll
        for (int u = 0; u < kOneWaves; ++u) c[u] = wcnt[u * E + tid];
#pragma unroll
        for (int u = 0; u < kOneWaves; ++u) {
            wcnt[u * E + tid] = (uint16_t)total;
            total += c[u];
        }
        counts[tid] = total;
    }
    const int nt = (tid < E) ? (total + tile_rows - 1) / tile_rows : 0;
    // inclusive scans of the totals and tile counts over experts (index =
    // tid): within each wave by shuffles, then the earlier waves' sums added
    int a = total, b = nt;
    for (int o = 1; o < 64; o <<= 1) {
        const int ua = __shfl_up(a, o, 64), ub = __shfl_up(b, o, 64);
        if (lane >= o) {
            a += ua;
            b += ub;
        }
    }
    if (lane == 63) {
        wsc[v] = a;
        wst[v] = b;
    }
    __syncthreads();
    for (int k = 0; k < v; ++k) {
        a += wsc[k];
        b += wst[k];
    }
    if (tid < E) {
        const int off = a - total;
        eoff[tid] = off;
        offsets[tid] = off;
        if (tid == E - 1) {
            offsets[E] = a;
            ntiles[0] = b;
        }
        const int tbase = b - nt;
        for (int i = 0; i < nt; ++i) {
            tiles[4 * (tbase + i) + 0] = tid;
            tiles[4 * (tbase + i) + 1] = off + i * tile_rows;
            tiles[4 * (tbase + i) + 2] = min(tile_rows, total - i * tile_rows);
            tiles[4 * (tbase + i) + 3] = 0;
        }
    }
    __syncthreads();  // expert offsets and wave offsets visible
    for (int r0 = 0; r0 < rounds; r0 += kOneIdBatch) {
        // The batch's ids and ranks (this thread's own stores above) are
        // loaded unconditionally (pair index clamped into the call) and every
        // slot is computed before the first list store, so the stores do not
        // wait on each other.
        int rkv[kOneIdBatch], dst[kOneIdBatch];
#pragma unroll
        for (int k = 0; k < kOneIdBatch; ++k) {
            const int p = min(p0 + 64 * (r0 + k) + lane, npairs - 1);
            idv[k] = ids[p];
            rkv[k] = rank[p];
        }
#pragma unroll
        for (int k = 0; k < kOneIdBatch; ++k) {
            const int p = p0 + 64 * (r0 + k) + lane;
            const int e = idv[k];
            const bool ok = r0 + k < rounds && p < npairs && e >= 0 && e < E;
            const int ec = ok ? e : 0;
            dst[k] = ok ? eoff[ec] + (int)cnt[ec] + rkv[k] : -1;
        }
#pragma unroll
        for (int k = 0; k < kOneIdBatch; ++k)
            if (dst[k] >= 0) list[dst[k]] = p0 + 64 * (r0 + k) + lane;
    }
}

// Calls of more than kOneMaxPairs pairs in at most kFuseMaxChunks chunks:
// after the count launch, one workgroup per chunk c sums the chunk table over
// chunks for every expert (the expert's total, and its pairs in the chunks
// before c), scans the totals over experts and places its own chunk's pairs:
// list[offset(e) + pairs of e in chunks < c + rank] = pair index.  Workgroup
// 0 also writes the counts, the offsets and the tile table.  Every workgroup
// reads the whole table (nchunks x E cells, at most 256 KiB), which takes the
// place of the single-workgroup scan launch and the separate place launch.
constexpr int kFuseThreads = 256;
constexpr int kFuseMaxChunks = 64;
constexpr int kFuseBatch = 32;  // chunk rows whose loads are in flight together
__global__ __launch_bounds__(kFuseThreads) void route_scan_place_kernel(
    const int32_t* __restrict__ ids, int T, int top_k, int E, int tile_rows, const int32_t* __restrict__ chunk,
    const int32_t* __restrict__ rank, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ list, int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    __shared__ int32_t sTot[1024];  // expert totals
    __shared__ int32_t sOff[1024];  // list offset of expert e, then plus its pairs in chunks before c
    __shared__ int32_t wsum[kFuseThreads / 64], wnt[kFuseThreads / 64];
    const int tid = threadIdx.x, c = blockIdx.x, nchunks = gridDim.x;
    // strided ownership for the sums over chunks: experts tid + 256 j
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    for (int c0 = 0; c0 < nchunks; c0 += kFuseBatch) {
        int v[4][kFuseBatch];
#pragma unroll
        for (int k = 0; k < kFuseBatch; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = tid + kFuseThreads * j, cc = c0 + k;
                v[j][k] = (e < E && cc < nchunks) ? chunk[(int64_t)cc * E + e] : 0;
            }
#pragma unroll
        for (int k = 0; k < kFuseBatch; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                tot[j] += v[j][k];
                pre[j] += (c0 + k < c) ? v[j][k] : 0;
            }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + kFuseThreads * j;
        if (e < E) sTot[e] = tot[j];
    }
    __syncthreads();
    // contiguous ownership for the scans over experts: experts 4 tid .. 4 tid + 3
    int a[4], nt[4], sa = 0, snt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        a[q] = (e < E) ? sTot[e] : 0;
        nt[q] = (a[q] + tile_rows - 1) / tile_rows;
        sa += a[q];
        snt += nt[q];
    }
    const int lane = tid & 63, w = tid >> 6;
    int ia = sa, int_ = snt;
    for (int o = 1; o < 64; o <<= 1) {
        const int ua = __shfl_up(ia, o, 64), ub = __shfl_up(int_, o, 64);
        if (lane >= o) {
            ia += ua;
            int_ += ub;
        }
    }
    if (lane == 63) {
        wsum[w] = ia;
        wnt[w] = int_;
    }
    __syncthreads();
    int ea = ia - sa, en = int_ - snt;  // exclusive prefixes of this thread's first expert
    int all_a = 0, all_n = 0;
    for (int k = 0; k < kFuseThreads / 64; ++k) {
        ea += (k < w) ? wsum[k] : 0;
        en += (k < w) ? wnt[k] : 0;
        all_a += wsum[k];
        all_n += wnt[k];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        if (e < E) {
            sOff[e] = ea;
            if (c == 0) {
                counts[e] = a[q];
                offsets[e] = ea;
                for (int i = 0; i < nt[q]; ++i) {
                    tiles[4 * (en + i) + 0] = e;
                    tiles[4 * (en + i) + 1] = ea + i * tile_rows;
                    tiles[4 * (en + i) + 2] = min(tile_rows, a[q] - i * tile_rows);
                    tiles[4 * (en + i) + 3] = 0;
                }
            }
            ea += a[q];
            en += nt[q];
        }
    }
    if (c == 0 && tid == 0) {
        offsets[E] = all_a;
        ntiles[0] = all_n;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + kFuseThreads * j;
        if (e < E) sOff[e] += pre[j];
    }
    __syncthreads();
    const int64_t p0 = (int64_t)c * kRouteChunk * top_k;
    const int64_t p1 = (int64_t)min(T, (c + 1) * kRouteChunk) * top_k;
    for (int64_t p = p0 + tid; p < p1; p += kFuseThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) list[sOff[e] + rank[p]] = (int32_t)p;
    }
}

// One thread per pair: list[offsets[e] + chunk offset + rank] = pair index.
__global__ __launch_bounds__(256) void route_place_kernel(const int32_t* __restrict__ ids, int64_t npairs,
                                                          int top_k, int E, const int32_t* __restrict__ chunk,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ rank,
                                                          int32_t* __restrict__ list) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= npairs) return;
    const int e = ids[p];
    if (e < 0 || e >= E) return;
    const int64_t c = (p / top_k) / kRouteChunk;
    list[offsets[e] + chunk[c * E + e] + rank[p]] = (int32_t)p;
}

// One thread per token: its top_k ids in [0, E) and distinct.
__global__ __launch_bounds__(256) void check_ids_kernel(const int32_t* __restrict__ ids, int64_t T, int top_k,
                                                        int E, unsigned int* __restrict__ err_word) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const int32_t* row = ids + t * top_k;
    unsigned int bits = 0;
    for (int i = 0; i < top_k; ++i) {
        const int e = row[i];
        if (e < 0 || e >= E) bits |= 2u;
        for (int j = 0; j < i; ++j)
            if (row[j] == e) bits |= 4u;
    }
    if (bits) __hip_atomic_fetch_or(err_word, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_check_ids(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, unsigned int* err_word,
                            hipStream_t st) {
    if (T <= 0) return hipSuccess;
    check_ids_kernel<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(ids, T, (int)top_k, (int)E, err_word);
    return hipGetLastError();
}

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t top_k, int64_t E, int tile_rows, RouteWs ws,
                        hipStream_t st) {
    if (tile_rows < kGroupMinTileRows) return hipErrorInvalidValue;
    // the count kernel's LDS holds 16 pairs per token and ids below 1024
    if (top_k < 1 || top_k > 16 || E < 1 || E > 1024) return hipErrorInvalidValue;
    const int64_t npairs_all = T * top_k;
    if (npairs_all <= kOneMaxPairs) {
        route_one_kernel<<<1, kOneThreads, 0, st>>>(ids, (int)npairs_all, (int)E, tile_rows, ws.rank, ws.counts,
                                                    ws.offsets, ws.list, ws.tiles, ws.ntiles);
        return hipGetLastError();
    }
    const int nchunks = (int)((T + kRouteChunk - 1) / kRouteChunk);
    if (nchunks > 0)
        route_count_kernel<<<nchunks, kCountThreads, 0, st>>>(ids, (int)T, (int)top_k, (int)E, ws.chunk, ws.rank);
    if (nchunks > 0 && nchunks <= kFuseMaxChunks) {
        route_scan_place_kernel<<<nchunks, kFuseThreads, 0, st>>>(ids, (int)T, (int)top_k, (int)E, tile_rows,
                                                                 ws.chunk, ws.rank, ws.counts, ws.offsets, ws.list,
                                                                 ws.tiles, ws.ntiles);
        return hipGetLastError();
    }
    const int64_t ncell = (int64_t)nchunks * E;
    const size_t stage = (ncell <= kScanStageCells) ? (size_t)ncell * 4 : 0;
    route_scan_kernel<<<1, kScanThreads, stage, st>>>(nchunks, (int)E, tile_rows, ws.chunk, ws.counts, ws.offsets, ws.tiles,
                                                      ws.ntiles);
    const int64_t npairs = T * top_k;
    if (npairs > 0)
        route_place_kernel<<<(unsigned)((npairs + 255) / 256), 256, 0, st>>>(ids, npairs, (int)top_k, (int)E,
                                                                             ws.chunk, ws.offsets, ws.rank,
                                                                             ws.list);
    return hipGetLastError();
}

// Ysum[t][n..n+3] = (((w0*y0 + w1*y1) + w2*y2) + ...): one thread per four
// adjacent channels.
constexpr int kSumPre = 8;  // slots whose loads are all issued before the first product
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
    // the first kSumPre slots' channels and weights requested before the
    // first product; later slots (top_k > kSumPre) follow one at a time
    float4 u[kSumPre];
    float ws[kSumPre];
#pragma unroll
    for (int s = 0; s < kSumPre; ++s) {
        if (s < top_k) {
            u[s] = *(const float4*)(yp + (int64_t)s * N);
            ws[s] = wp[s];
        }
    }
    float a0 = ws[0] * u[0].x, a1 = ws[0] * u[0].y, a2 = ws[0] * u[0].z, a3 = ws[0] * u[0].w;
#pragma unroll
    for (int s = 1; s < kSumPre; ++s) {
        if (s < top_k) {
            const float p0 = ws[s] * u[s].x, p1 = ws[s] * u[s].y, p2 = ws[s] * u[s].z, p3 = ws[s] * u[s].w;
            a0 = a0 + p0; a1 = a1 + p1; a2 = a2 + p2; a3 = a3 + p3;
        }
    }
    for (int s = kSumPre; s < top_k; ++s) {
        const float4 v = *(const float4*)(yp + (int64_t)s * N);
        const float wv = wp[s];
        const float p0 = wv * v.x, p1 = wv * v.y, p2 = wv * v.z, p3 = wv * v.w;
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
