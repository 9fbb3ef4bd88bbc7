// epdc_kernels.hpp -- gfx950 (CDNA4) kernels of the MoE dispatch/combine hot
// path: routing histogram + scan + stable in-tile ranks, slot assignment fused
// with the payload scatter (bf16/raw copy, OCP E4M3 or MXFP4 quantization on
// the fly), and the gather combine.
//
// What is computed follows MORI's EpDispatchCombineOp methods (MORI
// "Communication APIs" page, MORI-EP section, methods table) on one GPU with
// the destination ranks as contiguous segments of one receive buffer; the
// count is produced by the dispatch kernels themselves (same page, "AsyncLL v2
// SDMA overlap" section).  Gather combine in BF16 with FP32 accumulation and
// the FP8/FP4 formats are the ones the "Choosing an EP API and backend" page
// lists for gfx950 ("EP paths" table and EPv2 restrictions list).
//
// Work is data movement, so nothing here uses MFMA: one wavefront (64 lanes)
// owns one token row, rows move as 16-byte vectors per lane, and the routing
// uses wave ballots instead of atomics so the slot order is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epdc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kRouteThreads = 1024;                 // one pair per thread
constexpr int kRouteWaves = kRouteThreads / kWave;  // 16
constexpr int kRouteTile = kRouteThreads;           // pairs per routing tile
constexpr int kMaxExperts = 512;
constexpr int kMaxTopk = 16;

// Control words at the start of the workspace.
enum { kCtrlError = 1, kCtrlTicket0 = 2, kCtrlTicket1 = 3, kCtrlWords = 64 };

// ---------------------------------------------------------------------------
// Small wave helpers
// ---------------------------------------------------------------------------

__device__ inline int lanes_below(uint64_t mask)
{
    // number of set bits of `mask` in lanes below this one
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ inline int wave_inclusive_sum(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int u = __shfl_up(v, d, kWave);
        if (lane >= d)
            v += u;
    }
    return v;
}

__device__ inline int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ inline float read_lane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Routing: histogram, exclusive scan, stable in-tile ranks
// ---------------------------------------------------------------------------
//
// Pair p = t*K + k belongs to tile p / kRouteTile.  k_route_rank ranks each
// tile in one block: inside a wave, lanes with the same expert are found by
// ballots over the bits of the expert id (a match-any), the rank inside the
// wave is the number of matching lower lanes, and the rank inside the tile
// adds the counts of the same expert in lower waves.  The block writes the
// tile's expert histogram as one row of a [tiles x experts] table, and the
// last block to finish (route_scan_body) turns the table into expert_off =
// exclusive scan of the expert totals and, in place of each count, the first
// slot of that expert's run inside that tile.  Slot of pair p =
// table[tile(p)][e] + rank_in_tile[p]: experts ascending, pairs in ascending
// p inside an expert.  With a single tile the rank kernel scans its own
// histogram; with a small table the scatter blocks scan it themselves
// (kRouteTableScan below).  The last-block hand-off uses device-scope stores
// and loads for the table rows and a device-scope ticket, not agent-scope
// fences: those compile to an L2 writeback / invalidate across the XCDs and
// made an earlier form of this scheme slower than a second launch.

struct RouteArgs {
    const int32_t *indices;  // [n_pairs]
    int32_t n_pairs;
    int32_t num_experts;
    int32_t num_ranks;
    int32_t key_bits;        // bits that hold any key < num_experts
    int32_t topk;            // pairs per token
    int32_t key_div;         // 0: the key is the expert id; > 0: unit keys (below)
    int32_t tiles;           // ceil(n_pairs / kRouteTile), >= 1
    int32_t *tile_table;     // [tiles][E]: counts, then first slot per (tile, e)
    uint16_t *tile_cnt16;    // or NULL; else [E][tiles_pad8] 16-bit counts (scatter-side scan)
    int32_t tiles_pad8;      // tiles rounded up to a multiple of 8
    int32_t *rank_in_tile;   // [n_pairs], -1 for an invalid id
    int32_t *expert_off;     // [E+1]
    int32_t *rank_off;       // [R+1]
    int32_t *recv_count;     // [R]
    uint32_t *ctrl;          // [kCtrlWords]
    int32_t ticket_word;     // ctrl word counting finished rank blocks (table path, several tiles)
};

// LDS ints k_route_rank needs for E experts.
__host__ __device__ inline int route_lds_ints(int E) { return kRouteWaves * E + E + 1; }

// Exclusive prefix sum over the block (kRouteThreads threads, one value each).
__device__ inline int block_exclusive_sum(int v, int *wave_tot /* kRouteWaves+1 */, int *total)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int incl = wave_inclusive_sum(v, lane);
    if (lane == kWave - 1)
        wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int t = lane < kRouteWaves ? wave_tot[lane] : 0;
        int ti = wave_inclusive_sum(t, lane);
        if (lane < kRouteWaves)
            wave_tot[lane] = ti - t;
        if (lane == kRouteWaves - 1)
            wave_tot[kRouteWaves] = ti;
    }
    __syncthreads();
    *total = wave_tot[kRouteWaves];
    return wave_tot[wave] + incl - v;
}

// expert_off from the expert totals (thread e < E holds total e), plus
// rank_off / recv_count; eoff: LDS [E+1] (filled in every block); only a
// block with `publish` writes the global arrays.
__device__ inline void write_offsets(int E, int R, int col_total, int *eoff, int *wave_tot,
                                     int32_t *expert_off, int32_t *rank_off, int32_t *recv_count,
                                     bool publish)
{
    const int tid = threadIdx.x;
    int total;
    const int excl = block_exclusive_sum(col_total, wave_tot, &total);
    if (tid < E)
        eoff[tid] = excl;
    if (tid == 0)
        eoff[E] = total;
    __syncthreads();
    if (!publish)
        return;
    if (tid <= E)
        expert_off[tid] = eoff[tid];
    const int per_rank = E / R;
    if (tid <= R)
        rank_off[tid] = eoff[tid * per_rank];
    if (tid < R)
        recv_count[tid] = eoff[(tid + 1) * per_rank] - eoff[tid * per_rank];
}

// Stable ranks of one tile of pairs, one pair per thread of a kRouteThreads
// block.  Thread `tid` holds pair p (p >= n_pairs: no pair).  Returns its
// expert (-1: none or an id outside [0, E), which raises the error flag when
// `flag_errors`), its rank among the tile's pairs with the same expert, and
// for threads x < E the tile's count of expert x.  wave_cnt: LDS
// [kRouteWaves][E].
struct TileRank {
    int e, rank, col_total;
};

// Routing key of pair p, or -1 for no row.  key_div == 0: the expert id,
// valid in [0, E).  key_div > 0 (units of the rank-deduplicated dispatch, E
// = number of ranks, key_div = experts per rank): the pair's destination
// rank id / key_div for the pair with the smallest k among the token's pairs
// on that rank (it opens the unit), -1 for the token's other pairs there; ids
// outside [0, key_div * E) have no key either way.
__device__ inline int route_key(const int32_t *indices, int p, int E, int topk, int key_div,
                                bool &bad_id)
{
    const int v = indices[p];
    bad_id = false;
    if (key_div == 0) {
        if (v >= 0 && v < E)
            return v;
        bad_id = true;
        return -1;
    }
    const int limit = key_div * E;
    if (v < 0 || v >= limit)
        return -1;
    const int r = v / key_div;
    const int k = p % topk;
    for (int j = 1; j <= k; ++j) {
        const int u = indices[p - j];
        if (u >= 0 && u < limit && u / key_div == r)
            return -1;
    }
    return r;
}

__device__ inline TileRank rank_tile(const int32_t *indices, int n_pairs, int E, int key_bits,
                                     int topk, int key_div, int p, int32_t *wave_cnt,
                                     uint32_t *ctrl, bool flag_errors)
{
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads)
        wave_cnt[i] = 0;

    int e = -1;
    if (p < n_pairs) {
        bool bad_id;
        e = route_key(indices, p, E, topk, key_div, bad_id);
        if (bad_id && flag_errors)
            atomicOr(&ctrl[kCtrlError], 1u);
    }
    const bool valid = e >= 0;

    // match-any over the expert id bits
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < key_bits; ++bit) {
        const bool one = (e >> bit) & 1;
        const uint64_t ones = __ballot(one);
        match &= one ? ones : ~ones;
    }
    const int rank_in_wave = lanes_below(match);

    __syncthreads();  // wave_cnt cleared
    if (valid && rank_in_wave == 0)
        wave_cnt[wave * E + e] = __popcll(match);
    __syncthreads();

    // per expert: exclusive prefix over the waves (independent LDS loads
    // first), and the tile total; E <= kRouteThreads: one expert per thread
    TileRank r;
    r.col_total = 0;
    if (tid < E) {
        int c[kRouteWaves];
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w)
            c[w] = wave_cnt[w * E + tid];
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            wave_cnt[w * E + tid] = run;
            run += c[w];
        }
        r.col_total = run;
    }
    __syncthreads();
    r.e = e;
    r.rank = valid ? wave_cnt[wave * E + e] + rank_in_wave : -1;
    return r;
}

__device__ inline void route_scan_body(const RouteArgs &a);

template <bool SINGLE_TILE>
__device__ inline void route_rank_body(const RouteArgs &a)
{
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_wave_tot[kRouteWaves + 1];

    const int tid = threadIdx.x;
    const int E = a.num_experts;
    const int tile = blockIdx.x;
    const int p = tile * kRouteTile + tid;
    int32_t *wave_cnt = lds;                     // [kRouteWaves][E]
    int32_t *eoff = lds + kRouteWaves * E;       // [E+1] (single tile)

    const TileRank r = rank_tile(a.indices, a.n_pairs, E, a.key_bits, a.topk, a.key_div, p,
                                 wave_cnt, a.ctrl, a.key_div == 0);
    if (p < a.n_pairs)
        a.rank_in_tile[p] = r.rank;
    if (!SINGLE_TILE) {
        if (a.tile_cnt16) {
            // by expert, 16 bits per tile (a tile holds at most 1024 pairs):
            // the scatter blocks read one expert's tiles with 16-byte loads
            if (tid < E) {
                uint16_t *row = a.tile_cnt16 + (size_t)tid * a.tiles_pad8;
                row[tile] = (uint16_t)r.col_total;
                if (tile == a.tiles - 1)
                    for (int b = a.tiles; b < a.tiles_pad8; ++b)
                        row[b] = 0;
            }
        } else {
            // Last-block scan (ctrl[ticket_word] is the ticket).  The
            // histogram row goes out with device-scope stores (visible to
            // every XCD without an L2 writeback); each
            // thread waits for its stores to complete before the block takes
            // a ticket, so the block that draws the last ticket finds every
            // row in place and reads them with device-scope loads.  No block
            // waits for another.
            if (tid < E)
                __hip_atomic_store(&a.tile_table[(size_t)tile * E + tid], r.col_total,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            __shared__ int s_last;
            if (tid == 0)
                s_last = __hip_atomic_fetch_add(&a.ctrl[a.ticket_word], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) ==
                         (uint32_t)(a.tiles - 1);
            __syncthreads();
            if (s_last) {
                route_scan_body(a);
                if (tid == 0)
                    __hip_atomic_store(&a.ctrl[a.ticket_word], 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    } else {
        // the only tile: its histogram is the whole histogram
        write_offsets(E, a.num_ranks, r.col_total, eoff, s_wave_tot, a.expert_off, a.rank_off,
                      a.recv_count, true);
        if (tid < E)
            a.tile_table[tid] = eoff[tid];
    }
}

template <bool SINGLE_TILE>
__global__ __launch_bounds__(kRouteThreads) void k_route_rank(RouteArgs a)
{
    route_rank_body<SINGLE_TILE>(a);
}

// Both routing levels of the rank-deduplicated dispatch in one launch:
// blockIdx.y = 0 routes the pairs to experts, 1 the units to ranks.
template <bool SINGLE_TILE>
__global__ __launch_bounds__(kRouteThreads) void k_route_rank2(RouteArgs a, RouteArgs b)
{
    route_rank_body<SINGLE_TILE>(blockIdx.y == 0 ? a : b);
}

// The scan of the tile table by one block (the last rank block).  Column
// chunks of up to kScanRegs tiles stay in registers between the two passes;
// longer columns are re-read from memory.
constexpr int kScanRegs = 16;

// Table reads of the scan: device-scope loads, since the last rank block
// reads rows other blocks wrote with device-scope stores during the launch.
__device__ inline int32_t table_load(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void route_scan_body(const RouteArgs &a)
{
    __shared__ int32_t part[kRouteThreads];
    __shared__ int32_t eoff[kMaxExperts + 1];
    __shared__ int32_t s_wave_tot[kRouteWaves + 1];

    const int tid = threadIdx.x;
    const int E = a.num_experts;
    const int B = a.tiles;
    int G = kRouteThreads / E;  // threads per expert column, >= 1 since E <= 512
    if (G > B)
        G = B;
    const int chunk = (B + G - 1) / G;
    const bool in_regs = chunk <= kScanRegs;
    const int g = tid / E, col = tid - (tid / E) * E;
    const int b0 = g * chunk;
    const int b1 = min(B, b0 + chunk);

    int vals[kScanRegs];
    if (tid < G * E) {
        int sum = 0;
        if (in_regs) {
#pragma unroll
            for (int r = 0; r < kScanRegs; ++r)
                vals[r] = (b0 + r < b1) ? table_load(&a.tile_table[(size_t)(b0 + r) * E + col]) : 0;
#pragma unroll
            for (int r = 0; r < kScanRegs; ++r)
                sum += vals[r];
        } else {
            for (int b = b0; b < b1; ++b)
                sum += table_load(&a.tile_table[(size_t)b * E + col]);
        }
        part[tid] = sum;
    }
    __syncthreads();

    int col_total = 0;
    if (tid < E) {
        int run = 0;
        for (int gg = 0; gg < G; ++gg) {
            const int c = part[gg * E + tid];
            part[gg * E + tid] = run;
            run += c;
        }
        col_total = run;
    }
    write_offsets(E, a.num_ranks, col_total, eoff, s_wave_tot, a.expert_off, a.rank_off,
                  a.recv_count, true);

    if (tid < G * E) {
        int run = eoff[col] + part[tid];
        if (in_regs) {
#pragma unroll
            for (int r = 0; r < kScanRegs; ++r)
                if (b0 + r < b1) {
                    a.tile_table[(size_t)(b0 + r) * E + col] = run;
                    run += vals[r];
                }
        } else {
            for (int b = b0; b < b1; ++b) {
                const size_t i = (size_t)b * E + col;
                const int c = table_load(&a.tile_table[i]);
                a.tile_table[i] = run;
                run += c;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Dispatch scatter: one wave per (token, row segment)
// ---------------------------------------------------------------------------
//
// A wave owns a segment of one token row (seg_vecs 16-byte input vectors, a
// whole number of passes): it reads each vector once, quantizes it if asked,
// and writes it to the token's K received rows.  Several waves per token keep
// the grid many waves deep, so the kernel is bound by HBM throughput rather
// than by the latency of one wave walking a whole row.  Every wave of a token derives
// the same K slots; the wave of segment 0 records them and carries the small
// per-slot rows (weights, indices, scales).

struct ScatterArgs {
    int32_t num_tokens;
    int32_t n_pairs;             // num_tokens * topk: every slot is below this
    int32_t topk;
    int32_t num_experts;
    int32_t hidden;              // bf16 elements per row (quantizing kernels)
    int32_t segs;                // row segments per token
    int32_t seg_vecs;            // input vectors per segment (a multiple of 64*CH)
    int32_t work_waves;          // waves per block that take a (token, segment)
    const int32_t *indices;      // [T, K]
    const int32_t *tile_table;   // first slot per (tile, expert)
    const int32_t *rank_in_tile; // [T*K]
    int32_t *slot_of;            // [T*K]
    int32_t *src_pos;            // [N_cap]
    const uint8_t *input;        // [T, in_row_vecs*16]
    int32_t in_row_vecs;         // 16-byte vectors per input row
    uint8_t *out;                // [N_cap, out row]
    const float *weights;        // [T, K] or NULL
    float *out_weights;          // [N_cap, K]
    int32_t *out_indices;        // [N_cap, K] or NULL
    const uint8_t *scales;       // carried [T, scale_words*4] or NULL
    uint8_t *out_scales;         // [N_cap, scale row] or NULL
    int32_t scale_words;         // 4-byte words per carried scale row
    uint32_t *ctrl;              // error flag
    // routing outputs, written by the scatter itself when it routes inline
    int32_t key_bits;
    int32_t num_ranks;
    int32_t *expert_off;         // [E+1]
    int32_t *rank_off;           // [R+1]
    int32_t *recv_count;         // [R]
    // rank-deduplicated dispatch ("units": one row per (token, rank)) and
    // its conversion to the expert layout
    int32_t key_div;                   // experts per rank
    const int32_t *unit_table;         // [tiles][R]: first unit row per (tile, rank)
    const int32_t *unit_rank_in_tile;  // [T*K]: rank among the tile's unit openers, or -1
    int32_t *unit_of;                  // [T*K]: unit row of each pair, -1 for none
    int32_t *unit_src;                 // [U_cap]: token of each unit row
    const int32_t *row_count;          // device count of input rows (units), or NULL
    int32_t unit_rows_max;             // num_tokens * min(K, R): every unit row is below
    int32_t num_src_tokens;            // tokens of the recorded dispatch (conversion)
    int32_t tiles;                     // routing tiles (kRouteTableScan)
    const uint16_t *tile_cnt16;        // [E][tiles_pad8] tile counts (kRouteTableScan)
    int32_t tiles_pad8;
    int32_t xcd_order;                 // 1: (token, segment) items in XCD order (xcd_item)
    int32_t cached_stores;             // 1: ordinary row stores that stay in the L2 (small batches)
    int32_t scale_stage;               // 1: MXFP4 scale bytes staged in LDS, stored as words
};

// ---- inline routing for a single tile (num_tokens * K <= kRouteTile) ----
//
// With at most one routing tile there is nothing to scan across blocks, so
// the scatter launch routes by itself and dispatch is one launch.  Its blocks
// have kRouteThreads threads: every block ranks the whole tile (one pair per
// thread, the same match-any ranks as k_route_rank) and scans the histogram
// into expert offsets, all in LDS, then its first work_waves waves copy their
// (token, segment) pieces (fewer copying waves per block spread the copies
// over more CUs).  Block 0 publishes expert_off / rank_off / recv_count and
// raises the error flag.  Two block barriers in all: each wave clears its own
// row of counts (a wave's LDS operations complete in order), and the copying
// waves assemble each pair's slot from the LDS tables instead of waiting for
// a table of slots.

struct InlineRouteLds {
    int32_t wave_cnt[kRouteWaves * kMaxExperts];  // [wave][e]: count, then prefix over waves
    int32_t ebase[kMaxExperts];                   // exclusive scan inside e's 64-expert group
    int32_t grp_tot[kMaxExperts / kWave];         // total of each 64-expert group
    int32_t e_of[kRouteTile];                     // expert of each pair, -1 for none
    int32_t rank_w[kRouteTile];                   // rank among the same expert in its wave
};

// First slot of expert e (e == E: the number of valid pairs).
__device__ inline int inline_expert_off(const InlineRouteLds &l, int E, int e)
{
    int s = e < E ? l.ebase[e] : 0;
    const int groups = e < E ? e / kWave : (E + kWave - 1) / kWave;
    for (int g = 0; g < groups; ++g)
        s += l.grp_tot[g];
    return s;
}

__device__ inline void inline_route(const ScatterArgs &a, InlineRouteLds &l)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int E = a.num_experts;
    int e = -1;
    if (tid < a.n_pairs) {
        const int v = a.indices[tid];
        if (v >= 0 && v < E)
            e = v;
        else if (blockIdx.x == 0)
            atomicOr(&a.ctrl[kCtrlError], 1u);
    }
    for (int i = lane; i < E; i += kWave)
        l.wave_cnt[wave * E + i] = 0;
    const bool valid = e >= 0;
    uint64_t match = __ballot(valid);  // match-any over the expert id bits
    for (int bit = 0; bit < a.key_bits; ++bit) {
        const bool one = (e >> bit) & 1;
        const uint64_t ones = __ballot(one);
        match &= one ? ones : ~ones;
    }
    const int rank_in_wave = lanes_below(match);
    if (valid && rank_in_wave == 0)
        l.wave_cnt[wave * E + e] = __popcll(match);
    l.e_of[tid] = e;
    l.rank_w[tid] = rank_in_wave;
    __syncthreads();
    if (wave * kWave < E) {  // whole waves, one expert per thread
        int total = 0;
        if (tid < E) {
            int c[kRouteWaves];
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w)
                c[w] = l.wave_cnt[w * E + tid];
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) {
                l.wave_cnt[w * E + tid] = total;
                total += c[w];
            }
        }
        const int incl = wave_inclusive_sum(total, lane);
        if (tid < E)
            l.ebase[tid] = incl - total;
        if (lane == kWave - 1)
            l.grp_tot[wave] = incl;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        const int R = a.num_ranks;
        const int per_rank = E / R;
        if (tid <= E)
            a.expert_off[tid] = inline_expert_off(l, E, tid);
        if (tid <= R)
            a.rank_off[tid] = inline_expert_off(l, E, tid * per_rank);
        if (tid < R)
            a.recv_count[tid] = inline_expert_off(l, E, (tid + 1) * per_rank) -
                                inline_expert_off(l, E, tid * per_rank);
    }
}

// Slot of this lane's pair (lanes < K): the expert's first slot, plus the
// pairs of that expert in lower waves, plus those in lower lanes of its wave.
__device__ inline int pair_slot_inline(const ScatterArgs &a, const InlineRouteLds &l, int t,
                                       int lane, bool record)
{
    int s = -1;
    if (lane < a.topk) {
        const int p = t * a.topk + lane;
        const int e = l.e_of[p];
        if (e >= 0)
            s = inline_expert_off(l, a.num_experts, e) +
                l.wave_cnt[(p / kWave) * a.num_experts + e] + l.rank_w[p];
        if (record) {
            if (s >= 0)
                a.src_pos[s] = p;
            a.slot_of[p] = s;
        }
    }
    return s;
}

// Slot of this lane's pair (lanes < K) from the routing table of the
// two-launch route; `record` also stores slot_of / src_pos.
__device__ inline int pair_slot(const ScatterArgs &a, int t, int lane, bool record)
{
    int s = -1;
    if (lane < a.topk) {
        const int p = t * a.topk + lane;
        const int r = a.rank_in_tile[p];
        if (r >= 0) {
            const int e = a.indices[p];
            s = a.tile_table[(size_t)(p / kRouteTile) * a.num_experts + e] + r;
            if ((unsigned)s >= (unsigned)a.n_pairs) {
                // cannot happen for a consistent routing table; never write out of bounds
                if (record)
                    atomicOr(&a.ctrl[kCtrlError], 2u);
                s = -1;
            } else if (record) {
                a.src_pos[s] = p;
            }
        }
        if (record)
            a.slot_of[p] = s;
    }
    return s;
}

// Copy the token's weights / indices / carried-scale rows to each of its
// slots.  All lanes execute the shuffles; stores are predicated.
__device__ inline void carry_small_rows(const ScatterArgs &a, int t, int slot, int lane)
{
    const int K = a.topk;
    const int kk = K * K;
    for (int base = 0; base < kk; base += kWave) {
        const int q = base + lane;
        const int k = min(q / K, K - 1);
        const int j = q - (q / K) * K;
        const int s = __shfl(slot, k, kWave);
        if (q < kk && s >= 0) {
            if (a.out_weights)
                a.out_weights[(size_t)s * K + j] = a.weights[(size_t)t * K + j];
            if (a.out_indices)
                a.out_indices[(size_t)s * K + j] = a.indices[(size_t)t * K + j];
        }
    }
    if (a.scales) {
        const int W = a.scale_words;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.scales) + (size_t)t * W;
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.out_scales);
        const int n = K * W;
        for (int base = 0; base < n; base += kWave) {
            const int q = base + lane;
            const int k = min(q / W, K - 1);
            const int j = q - (q / W) * W;
            const int s = __shfl(slot, k, kWave);
            if (q < n && s >= 0)
                dst[(size_t)s * W + j] = src[j];
        }
    }
}

// Token, segment and K slots of this wave; false if the wave has no work.
struct ScatterWave {
    int lane, t, base, end, slot;
};

// Work item of wave w of block b (W waves per block) when items are dealt
// to the XCDs one at a time.  The dispatcher hands a launch's blocks to the
// chip's eight XCDs in turn, block b to XCD b % 8, so item j runs on XCD
// j % 8 whatever the block size.  A scatter and a combine that both number
// (token, segment) items this way run the two waves of one item on the same
// XCD, where the combine finds the rows the scatter just wrote in that XCD's
// L2 instead of fetching them across the chip.  The grid is a multiple of
// kXcds blocks; items past the end have no work.
constexpr int kXcds = 8;

__device__ inline int xcd_item(int b, int W, int w)
{
    return kXcds * ((b / kXcds) * W + w) + b % kXcds;
}

// Token, segment and range of this wave; false if it has no work.
__device__ inline bool scatter_wave_range(const ScatterArgs &a, int row_vecs, ScatterWave &w,
                                          int &seg)
{
    w.lane = threadIdx.x & (kWave - 1);
    w.slot = -1;
    const int wave = threadIdx.x / kWave;
    if (wave >= a.work_waves)
        return false;
    const int wv = a.xcd_order ? xcd_item(blockIdx.x, a.work_waves, wave)
                               : blockIdx.x * a.work_waves + wave;
    if (wv >= a.num_tokens * a.segs)
        return false;
    // the grid covers the row capacity; rows past the device count have no work
    if (a.row_count && wv / a.segs >= *a.row_count)
        return false;
    w.t = wv / a.segs;
    seg = wv - w.t * a.segs;
    w.base = seg * a.seg_vecs;
    w.end = min(row_vecs, w.base + a.seg_vecs);
    return true;
}

__device__ inline InlineRouteLds &inline_route_lds()
{
    __shared__ InlineRouteLds l;
    return l;
}

// Where a scatter launch takes its slots from.
enum {
    kRouteTable = 0,   // the tile table of the two-launch route
    kRouteInline = 1,  // routes the single tile itself (kRouteThreads-thread blocks)
    kRouteReplay = 2,  // slot_of of a dispatch recorded earlier (routing replay)
    kRouteUnits = 3,        // rank-deduplicated: one row per (token, rank), from the unit table
    kRouteConvert = 4,      // a wave per unit row: its pairs' expert rows (standard-MoE layout)
    kRouteUnitsReplay = 5,  // unit rows of a rank-deduplicated dispatch recorded earlier
    kRouteTableScan = 6     // tile histograms scanned by each block (not by the last rank block)
};

// ---- the scan folded into the scatter, for small tile tables ----
//
// Each block turns the tile histograms k_route_rank wrote into the bases of
// the (at most two) tiles its tokens fall in: expert totals summed over all
// tiles, their exclusive scan, plus the counts of the earlier tiles.  Every
// block reads the whole table, so the host uses this only while the table
// is small; there it beats the scan by the last rank block.
// Largest tile table (tiles x experts entries) the scatter blocks scan, and
// the most table entries all blocks of one launch may read together.
constexpr int kFusedScanMaxEntries = 8192;
constexpr int64_t kFusedScanMaxReads = int64_t(1) << 24;
constexpr int kScanMaxLoads = 8;  // 16-byte loads per expert row: at most 64 tiles

struct ScanLds {
    int32_t base[2][kMaxExperts];
    int32_t eoff[kMaxExperts + 1];
};

__device__ inline ScanLds &scan_lds()
{
    __shared__ ScanLds l;
    return l;
}

__device__ inline void block_tile_bases(const ScatterArgs &a, ScanLds &l, int tile0)
{
    const int E = a.num_experts;
    const int nthr = blockDim.x;
    const int n16 = a.tiles_pad8 / 8;  // 16-byte loads per expert row (<= kScanMaxLoads)
    for (int e = threadIdx.x; e < E; e += nthr) {
        const u32x4 *row = reinterpret_cast<const u32x4 *>(a.tile_cnt16 + (size_t)e * a.tiles_pad8);
        u32x4 v[kScanMaxLoads];
#pragma unroll
        for (int j = 0; j < kScanMaxLoads; ++j)  // independent loads in flight
            v[j] = j < n16 ? row[j] : u32x4{0u, 0u, 0u, 0u};
        int total = 0, pre = 0, c0 = 0;
#pragma unroll
        for (int j = 0; j < kScanMaxLoads; ++j) {
            const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const int c = (int)((wd[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
                const int b = 8 * j + h;
                total += c;
                if (b < tile0)
                    pre += c;
                else if (b == tile0)
                    c0 = c;
            }
        }
        l.eoff[e] = total;
        l.base[0][e] = pre;
        l.base[1][e] = pre + c0;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {  // exclusive scan of the totals by one wave
        const int lane = threadIdx.x;
        const int per = (E + kWave - 1) / kWave;
        const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
        int sum = 0;
        for (int e = e0; e < e1; ++e)
            sum += l.eoff[e];
        int incl = sum;
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(incl, d, kWave);
            if (lane >= d)
                incl += v;
        }
        int run = incl - sum;
        for (int e = e0; e < e1; ++e) {
            const int c = l.eoff[e];
            l.eoff[e] = run;
            run += c;
        }
        if (lane == kWave - 1)
            l.eoff[E] = incl;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += nthr) {
        l.base[0][e] += l.eoff[e];
        l.base[1][e] += l.eoff[e];
    }
    if (blockIdx.x == 0) {  // publish the offsets and the counts
        const int R = a.num_ranks;
        const int per_rank = E / R;
        for (int e = threadIdx.x; e <= E; e += nthr)
            a.expert_off[e] = l.eoff[e];
        for (int r = threadIdx.x; r <= R; r += nthr)
            a.rank_off[r] = l.eoff[r * per_rank];
        for (int r = threadIdx.x; r < R; r += nthr)
            a.recv_count[r] = l.eoff[(r + 1) * per_rank] - l.eoff[r * per_rank];
    }
    __syncthreads();
}

// Slot of this lane's pair from the block's bases (tile0 = the block's first tile).
__device__ inline int pair_slot_scan(const ScatterArgs &a, const ScanLds &l, int tile0, int t,
                                     int lane, bool record)
{
    int s = -1;
    if (lane < a.topk) {
        const int p = t * a.topk + lane;
        const int r = a.rank_in_tile[p];
        if (r >= 0) {
            const int e = a.indices[p];
            s = l.base[p / kRouteTile - tile0][e] + r;
            if ((unsigned)s >= (unsigned)a.n_pairs) {
                if (record)
                    atomicOr(&a.ctrl[kCtrlError], 2u);
                s = -1;
            } else if (record) {
                a.src_pos[s] = p;
            }
        }
        if (record)
            a.slot_of[p] = s;
    }
    return s;
}

// Rank-deduplicated dispatch: the pair's expert slot is recorded as in
// kRouteTable (the conversion and the combine use it), and the wave writes
// the token's row once per unit: the unit opener (smallest k of the token on
// that rank) holds the unit row, the token's other pairs on the rank take the
// opener's row as their unit.
__device__ inline int unit_slot(const ScatterArgs &a, int t, int lane, bool record)
{
    const int K = a.topk;
    const int R = a.num_ranks;
    int rank = -1, us = -1;
    if (lane < K) {
        const int p = t * K + lane;
        const int v = a.indices[p];
        if (v >= 0 && v < a.num_experts)
            rank = v / a.key_div;
        const int ur = a.unit_rank_in_tile[p];
        if (ur >= 0 && rank >= 0) {
            us = a.unit_table[(size_t)(p / kRouteTile) * R + rank] + ur;
            if ((unsigned)us >= (unsigned)a.unit_rows_max) {
                if (record)
                    atomicOr(&a.ctrl[kCtrlError], 2u);
                us = -1;
            }
        }
    }
    // the unit of every pair: the row of the opener on the same rank
    int unit = -1;
    for (int j = 0; j < K; ++j) {
        const int rj = read_lane(rank, j);
        const int uj = read_lane(us, j);
        if (unit < 0 && rank >= 0 && rj == rank && uj >= 0)
            unit = uj;
    }
    if (record && lane < K) {
        a.unit_of[t * K + lane] = unit;
        if (us >= 0)
            a.unit_src[us] = t;
    }
    return us;
}

// Conversion of unit rows to the expert layout: the wave's row is unit u of
// token unit_src[u]; lane k's slot is the expert row of pair k when that pair
// belongs to u.
__device__ inline int convert_slot(const ScatterArgs &a, int u, int lane)
{
    if (lane >= a.topk)
        return -1;
    const int t = a.unit_src[u];
    if ((unsigned)t >= (unsigned)a.num_src_tokens) {
        atomicOr(&a.ctrl[kCtrlError], 2u);
        return -1;
    }
    const int p = t * a.topk + lane;
    if (a.unit_of[p] != u)
        return -1;
    const int s = a.slot_of[p];
    return (unsigned)s < (unsigned)a.n_pairs ? s : -1;
}

// The K slots of the wave's token (lane k holds pair k's slot), recorded by
// the segment-0 wave, which also carries the small rows.  With kRouteInline
// the whole block routes the tile first, waves without work included.
// Called after the wave's first loads are in flight, so their latency
// overlaps the routing.
template <int MODE>
__device__ inline void route_wave(const ScatterArgs &a, bool has_work, int seg, ScatterWave &w)
{
    if constexpr (MODE == kRouteInline) {
        InlineRouteLds &l = inline_route_lds();
        inline_route(a, l);
        if (has_work)
            w.slot = pair_slot_inline(a, l, w.t, w.lane, seg == 0);
    } else if constexpr (MODE == kRouteTableScan) {
        // every wave of the block takes part in the block's scan
        ScanLds &l = scan_lds();
        const int tile0 = (int)(((int64_t)blockIdx.x * a.work_waves / a.segs) * a.topk / kRouteTile);
        block_tile_bases(a, l, tile0);
        if (has_work)
            w.slot = pair_slot_scan(a, l, tile0, w.t, w.lane, seg == 0);
    } else if constexpr (MODE == kRouteUnits) {
        if (has_work) {  // wave-uniform: the shuffles in unit_slot see the whole wave
            if (seg == 0)
                (void)pair_slot(a, w.t, w.lane, true);
            w.slot = unit_slot(a, w.t, w.lane, seg == 0);
        }
    } else if constexpr (MODE == kRouteConvert) {
        if (has_work)
            w.slot = convert_slot(a, w.t, w.lane);
    } else if constexpr (MODE == kRouteUnitsReplay) {
        if (has_work) {  // wave-uniform
            int u = -1;
            if (w.lane < a.topk) {
                u = a.unit_of[w.t * a.topk + w.lane];
                if ((unsigned)u >= (unsigned)a.unit_rows_max)
                    u = -1;
            }
            int opener = u >= 0;  // the first of the token's pairs in the unit writes it
            for (int j = 0; j < a.topk; ++j) {
                const int uj = read_lane(u, j);
                if (j < w.lane && uj == u)
                    opener = 0;
            }
            w.slot = opener ? u : -1;
        }
    } else if constexpr (MODE == kRouteReplay) {
        if (has_work && w.lane < a.topk) {
            const int s = a.slot_of[w.t * a.topk + w.lane];
            // a recorded slot is -1 or in range; a workspace edited since is not trusted
            if (s >= a.n_pairs || s < -1) {
                if (seg == 0)
                    atomicOr(&a.ctrl[kCtrlError], 2u);
            } else {
                w.slot = s;
            }
        }
    } else {
        if (has_work)
            w.slot = pair_slot(a, w.t, w.lane, seg == 0);
    }
    if (has_work && seg == 0)
        carry_small_rows(a, w.t, w.slot, w.lane);
}

// ---- row stores of the scatter kernels ----
//
// Large batches write payload rows with buffer stores of device scope (the
// sc1 cache-policy bit) through a resource that covers the one destination
// row, so a store past the row is dropped by the hardware and any
// receive-buffer size works (offsets stay below one row).  On gfx950 this
// streams the 1->K copies of 16-byte vectors 3-4% faster than ordinary
// global stores (headline bf16 copy 80.0-81.4 -> 77.8 us, FP8 51.1-51.8 ->
// 50.2 us; nontemporal stores are much slower, 111 us).  It does not pay
// where the reader wants the rows in the writer's L2: a batch whose rows fit
// the L2s (cached_stores; at the decode shape the combine took 3.9 -> 5.6 us
// after device-scope stores) keeps ordinary stores, and so do the MXFP4
// kernel's 4-byte stores (77.5-80.1 -> 81.1 us).
// Fourth descriptor word: DATA_FORMAT = 32 bits (bits 15-18 = 4); untyped
// MUBUF accesses need a nonzero data format on gfx9-family parts.
constexpr int kBufferDword3 = 0x00020000;
constexpr int kStoreDeviceScope = 16;      // cache policy: sc1

__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(uint8_t *base, size_t row_bytes, int row)
{
    return __builtin_amdgcn_make_buffer_rsrc(base + (size_t)row * row_bytes, 0, (int)row_bytes,
                                             kBufferDword3);
}

__device__ inline void store_row16(__amdgpu_buffer_rsrc_t r, int byte_off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kStoreDeviceScope);
}

// bf16 or raw rows: 16-byte nontemporal loads once, K rows of 16-byte stores
// (row_rsrc / store_row16 above).
template <int CH, int MODE = kRouteTable>
__global__ __launch_bounds__(MODE == kRouteInline ? kRouteThreads : 256) void k_scatter_copy(ScatterArgs a)
{
    const int V = a.in_row_vecs;
    ScatterWave w;
    int seg = 0;
    const bool has_work = scatter_wave_range(a, V, w, seg);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.input) + (size_t)(has_work ? w.t : 0) * V;
    u32x4 v[CH];
    auto load = [&](int b) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int j = b + w.lane + kWave * i;
            if (j < w.end)
                v[i] = __builtin_nontemporal_load(src + j);
        }
    };
    if (has_work)
        load(w.base);
    route_wave<MODE>(a, has_work, seg, w);
    if (!has_work)
        return;
    for (int b = w.base; b < w.end; b += kWave * CH) {
        if (b != w.base)
            load(b);
        for (int k = 0; k < a.topk; ++k) {
            const int s = read_lane(w.slot, k);
            if (s < 0)
                continue;
            if (a.cached_stores) {
                u32x4 *dst = reinterpret_cast<u32x4 *>(a.out) + (size_t)s * V;
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int j = b + w.lane + kWave * i;
                    if (j < w.end)
                        dst[j] = v[i];
                }
            } else {
                const __amdgpu_buffer_rsrc_t dst = row_rsrc(a.out, (size_t)V * 16, s);
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int j = b + w.lane + kWave * i;
                    if (j < w.end)
                        store_row16(dst, j * 16, v[i]);
                }
            }
        }
    }
}

// OCP E4M3 with one fp32 scale per 128 elements.  Each lane quantizes two
// adjacent input vectors (16 elements) per pass, so a block is 8 lanes and
// every copy is one 16-byte store per lane (1 KiB per store instruction).
// Segments are whole numbers of 128-vector passes and rows whole numbers of
// 16-vector blocks, so the 8 lanes of a block are all in or all out.
constexpr int kFp8PassVecs = 2 * kWave;

__device__ inline void quant_fp8_pass(const u32x4 *src, int b, int end, int lane, u32x4 &code,
                                      float &scale)
{
    const int j = b + 2 * lane;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (j < end) {
        v0 = __builtin_nontemporal_load(src + j);
        v1 = __builtin_nontemporal_load(src + j + 1);
    }
    const float x[16] = {bf16_lo(v0.x), bf16_hi(v0.x), bf16_lo(v0.y), bf16_hi(v0.y),
                         bf16_lo(v0.z), bf16_hi(v0.z), bf16_lo(v0.w), bf16_hi(v0.w),
                         bf16_lo(v1.x), bf16_hi(v1.x), bf16_lo(v1.y), bf16_hi(v1.y),
                         bf16_lo(v1.z), bf16_hi(v1.z), bf16_lo(v1.w), bf16_hi(v1.w)};
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
        m = fmaxf(m, fabsf(x[q]));
    m = fmaxf(m, __shfl_xor(m, 1, kWave));
    m = fmaxf(m, __shfl_xor(m, 2, kWave));
    m = fmaxf(m, __shfl_xor(m, 4, kWave));
    float s = 0.0f;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    if (m != 0.0f) {
        s = m / 448.0f;  // IEEE division, round to nearest
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i] / s, x[4 * i + 1] / s, 0u, false);
            c[i] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i + 2] / s, x[4 * i + 3] / s, c[i], true);
        }
    }
    code = u32x4{c[0], c[1], c[2], c[3]};
    scale = s;
}

template <int MODE = kRouteTable>
__global__ __launch_bounds__(MODE == kRouteInline ? kRouteThreads : 256) void k_scatter_fp8(ScatterArgs a)
{
    const int V = a.hidden / 8;          // 8 bf16 per vector
    const int nblk = a.hidden / 128;     // scales per row
    ScatterWave w;
    int seg = 0;
    const bool has_work = scatter_wave_range(a, V, w, seg);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.input) + (size_t)(has_work ? w.t : 0) * V;
    u32x4 code;
    float scale;
    if (has_work)
        quant_fp8_pass(src, w.base, w.end, w.lane, code, scale);
    route_wave<MODE>(a, has_work, seg, w);
    if (!has_work)
        return;
    for (int b = w.base; b < w.end; b += kFp8PassVecs) {
        if (b != w.base)
            quant_fp8_pass(src, b, w.end, w.lane, code, scale);
        const int j = b + 2 * w.lane;
        for (int k = 0; k < a.topk; ++k) {
            const int s = read_lane(w.slot, k);
            if (s < 0)
                continue;
            if (j < w.end) {
                if (a.cached_stores)
                    reinterpret_cast<u32x4 *>(a.out + (size_t)s * a.hidden)[j >> 1] = code;
                else
                    store_row16(row_rsrc(a.out, (size_t)a.hidden, s), (j >> 1) * 16, code);
                if ((w.lane & 7) == 0)
                    reinterpret_cast<float *>(a.out_scales)[(size_t)s * nblk + (j >> 4)] = scale;
            }
        }
    }
}

// MXFP4: E2M1 pairs via v_cvt_scalef32_pk_fp4_f32, one E8M0 scale per 32
// elements (4 lanes x 8 elements, CH vectors per lane per pass, lanes on
// consecutive vectors).  Unlike the FP8 kernel it keeps 4-byte stores: a
// 16-byte-store layout (4 adjacent vectors per lane) measured 108 us against
// 79 us at 16384 x 4096, whose 1:2 read/write mix already runs at the
// mixed-traffic ceiling of about 5.4 TB/s.
template <int CH>
__device__ inline void quant_mxfp4_pass(const u32x4 *src, int b, int end, int lane,
                                        uint32_t *code, uint32_t *sbyte)
{
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int j = b + lane + kWave * i;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < end)
            v = __builtin_nontemporal_load(src + j);
        float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            m = fmaxf(m, fabsf(x[q]));
        m = fmaxf(m, __shfl_xor(m, 1, kWave));
        m = fmaxf(m, __shfl_xor(m, 2, kWave));
        // E8M0 byte = floor(log2 amax) - 2 + 127, clamped at 0: the fp32
        // exponent field minus 2 (0 for zero or subnormal amax)
        const uint32_t ef = (__float_as_uint(m) >> 23) & 0xFFu;
        const uint32_t sb = ef > 2u ? ef - 2u : 0u;
        const float scale = __uint_as_float(sb << 23);  // only its exponent field is used
        uint32_t q = 0;
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[0], x[1], scale, 0);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[2], x[3], scale, 1);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[4], x[5], scale, 2);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[6], x[7], scale, 3);
        code[i] = q;
        sbyte[i] = sb;
    }
}

// Scale bytes of a segment, staged per wave (scale_stage): one byte per
// 4 vectors, so a stage holds segments of up to 4 * kMxStageBytes vectors.
// Storing them as words after the wave's passes replaces 1-byte stores
// from every fourth lane, which cost 5-15 us of an 82-88 us scatter at
// 16384 x 4096 for 17 MB of scales (one wave per row then writes each scale
// row as one whole 128-byte line per copy).
constexpr int kMxStageBytes = 512;

__device__ inline uint32_t *mx_scale_stage(int wave)
{
    __shared__ uint32_t stage[kRouteWaves][kMxStageBytes / 4];
    return stage[wave];
}

template <int CH, int MODE = kRouteTable>
__global__ __launch_bounds__(MODE == kRouteInline ? kRouteThreads : 256) void k_scatter_mxfp4(ScatterArgs a)
{
    const int V = a.hidden / 8;
    const int nblk = a.hidden / 32;
    ScatterWave w;
    int seg = 0;
    const bool has_work = scatter_wave_range(a, V, w, seg);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.input) + (size_t)(has_work ? w.t : 0) * V;
    uint32_t code[CH];
    uint32_t sbyte[CH];
    if (has_work)
        quant_mxfp4_pass<CH>(src, w.base, w.end, w.lane, code, sbyte);
    route_wave<MODE>(a, has_work, seg, w);
    if (!has_work)
        return;
    uint32_t *stage = mx_scale_stage(threadIdx.x / kWave);
    uint8_t *stage8 = reinterpret_cast<uint8_t *>(stage);
    for (int b = w.base; b < w.end; b += kWave * CH) {
        if (b != w.base)
            quant_mxfp4_pass<CH>(src, b, w.end, w.lane, code, sbyte);
        if (a.scale_stage) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int j = b + w.lane + kWave * i;
                if (j < w.end && (w.lane & 3) == 0)
                    stage8[(j - w.base) >> 2] = (uint8_t)sbyte[i];
            }
        }
        for (int k = 0; k < a.topk; ++k) {
            const int s = read_lane(w.slot, k);
            if (s < 0)
                continue;
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.out + (size_t)s * (a.hidden / 2));
            uint8_t *dsc = a.out_scales + (size_t)s * nblk;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int j = b + w.lane + kWave * i;
                if (j < w.end) {
                    dst[j] = code[i];
                    if (!a.scale_stage && (w.lane & 3) == 0)
                        dsc[j >> 2] = (uint8_t)sbyte[i];
                }
            }
        }
    }
    if (a.scale_stage) {
        // the wave's own LDS writes above complete before these reads
        const int words = (w.end - w.base) >> 4;
        for (int k = 0; k < a.topk; ++k) {
            const int s = read_lane(w.slot, k);
            if (s < 0)
                continue;
            uint32_t *dsc =
                reinterpret_cast<uint32_t *>(a.out_scales + (size_t)s * nblk + (w.base >> 2));
            for (int m = w.lane; m < words; m += kWave)
                dsc[m] = stage[m];
        }
    }
}

// ---------------------------------------------------------------------------
// Combine: one wave per (token, row segment), K rows double buffered
// ---------------------------------------------------------------------------
//
// A wave owns kCombineSeg 16-byte vectors per lane (a 2 KiB segment of a
// bf16 row) of one token: it streams the segment of its K received rows in k
// order, loading row k+1 while it accumulates row k, and writes the bf16
// segment.  Splitting rows into segments gives several waves per token,
// which measured faster than one wave walking the whole row.

constexpr int kCombineSeg = 2;
constexpr int kCombineSegVecs = kWave * kCombineSeg;

struct CombineArgs {
    int32_t num_tokens;
    int32_t topk;
    int32_t row_vecs;        // 16-byte vectors per bf16 row (H/8)
    int32_t segs;            // ceil(row_vecs / seg_vecs)
    const int32_t *slot_of;  // [T*K]
    const uint8_t *input;    // [rows, H] bf16
    const float *weights;    // [rows, K] or NULL
    uint8_t *output;         // [T, H] bf16
    float *out_weights;      // [T, K] or NULL
    // unit modes (rank-deduplicated path)
    const int32_t *unit_of;    // [T*K]
    const int32_t *unit_src;   // [U_cap]
    const int32_t *row_count;  // device count of output rows (units), or NULL
    int32_t n_pairs;           // expert rows of the recorded dispatch
    int32_t num_src_tokens;    // tokens of the recorded dispatch
    int32_t in_rows_max;       // rows of the unit-row input
    int32_t xcd_order;         // 1: (row, segment) items in XCD order (xcd_item)
    int32_t seg_vecs;          // vectors per row segment (<= kWave * CH)
    int32_t cached_stores;     // 1: ordinary output stores that stay in the L2
    int32_t recent_input;      // 1: the input rows were just written (cache-allocating output stores)
    int32_t stage_rows;        // k_combine_staged: output rows per block
    // (Large batches keep nontemporal output stores in every mode: for the
    // expert->unit conversion, whose output is 40% of its bytes, device-scope
    // stores made the deduplicated headline step 404 -> 409 us and ordinary
    // ones 414 us.)
};

// What a combine wave sums.
enum {
    kCombinePairs = 0,     // token t: its K expert rows, weighted (the gather combine)
    kCombineUnitsIn = 1,   // unit u: the expert rows of its pairs, weighted
    kCombineUnitsOut = 2   // token t: its distinct unit rows in ascending order, unweighted
};

__device__ inline uint32_t pack_bf16_rne(float lo, float hi)
{
    const bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);  // v_cvt_pk_bf16_f32
    return __builtin_bit_cast(uint32_t, b);
}

__device__ inline void accumulate_row(float *acc, float w, u32x4 x)
{
#pragma clang fp contract(off)
    acc[0] = acc[0] + w * bf16_lo(x.x);
    acc[1] = acc[1] + w * bf16_hi(x.x);
    acc[2] = acc[2] + w * bf16_lo(x.y);
    acc[3] = acc[3] + w * bf16_hi(x.y);
    acc[4] = acc[4] + w * bf16_lo(x.z);
    acc[5] = acc[5] + w * bf16_hi(x.z);
    acc[6] = acc[6] + w * bf16_lo(x.w);
    acc[7] = acc[7] + w * bf16_hi(x.w);
}

// The wave's terms in summation order, compacted to the front lanes: lane
// i < n holds the input row (cs) of the i-th term and the index k of its pair
// (ck); n is wave-uniform.  Pairs and units-in terms are the token's pairs in
// k order that have a row (terms without one add nothing); units-out terms
// are the token's distinct unit rows, ascending.  Also writes the returned
// weights that need no term weight (missing pairs, units-out).  Cross-lane
// reads use v_readlane (the lane index is uniform), not LDS permutes.
template <int MODE>
__device__ inline int combine_slots(const CombineArgs &a, int row, int sg, int lane, int K,
                                    int &cs, int &ck)
{
    cs = -1;
    ck = 0;
    if constexpr (MODE == kCombineUnitsOut) {
        int u = -1;
        if (lane < K) {
            u = a.unit_of[row * K + lane];
            if ((unsigned)u >= (unsigned)a.in_rows_max)
                u = -1;
            if (a.out_weights && sg == 0)
                a.out_weights[row * K + lane] =
                    u < 0 ? 0.0f : (a.weights ? a.weights[(size_t)u * K + lane] : 1.0f);
        }
        // the first lane holding a unit opens it; openers are ordered by unit row
        int opener = u >= 0;
        for (int j = 0; j < K; ++j) {
            const int uj = read_lane(u, j);
            if (j < lane && uj == u)
                opener = 0;
        }
        int pos = 0;
        for (int j = 0; j < K; ++j) {
            const int oj = read_lane(opener, j);
            const int uj = read_lane(u, j);
            if (oj && uj < u)
                ++pos;
        }
        for (int j = 0; j < K; ++j) {
            const int oj = read_lane(opener, j);
            const int pj = read_lane(pos, j);
            const int uj = read_lane(u, j);
            if (oj && pj == lane) {
                cs = uj;
                ck = j;
            }
        }
        return __popcll(__ballot(opener));
    } else {
        int s = -1;
        if (lane < K) {
            if constexpr (MODE == kCombinePairs) {
                s = a.slot_of[row * K + lane];
            } else {
                const int t = a.unit_src[row];
                if ((unsigned)t < (unsigned)a.num_src_tokens) {
                    const int p = t * K + lane;
                    const int s0 = a.slot_of[p];
                    if (a.unit_of[p] == row && (unsigned)s0 < (unsigned)a.n_pairs)
                        s = s0;
                }
            }
            if (MODE == kCombinePairs && s < 0 && a.out_weights && sg == 0)
                a.out_weights[row * K + lane] = 0.0f;
        }
        const uint64_t have = __ballot(s >= 0);
        if (have == (uint64_t(1) << K) - 1) {  // every pair has a row: already compact
            cs = s;
            ck = lane;
        } else {
            const int r = s >= 0 ? lanes_below(have) : kWave;
            for (int j = 0; j < K; ++j) {
                const int rj = read_lane(r, j);
                const int sj = read_lane(s, j);
                if (rj == lane) {
                    cs = sj;
                    ck = j;
                }
            }
        }
        return __popcll(have);
    }
}

// CH vectors per lane of row s's segment [base, end) (rows of V vectors).
template <int CH>
__device__ inline void load_segment(const u32x4 *in, int s, int V, int base, int end, int lane,
                                    u32x4 *dst)
{
    const u32x4 *row = in + (size_t)s * V;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int j = base + lane + kWave * i;
        dst[i] = j < end ? __builtin_nontemporal_load(row + j) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Sum of NT rows, lane k < NT holding the k-th slot and weight, all NT rows'
// segments requested at once.  NT is a compile-time count so no load sits
// behind a branch and the wait counters stay exact.
template <int NT, int CH>
__device__ inline void sum_rows(const u32x4 *in, int V, int base, int end, int lane, int my_slot,
                                float my_w, float (&acc)[CH][8])
{
    // the rows are requested before the weights are read, so the rows' loads
    // never wait for the weights' (which depend on the slots)
    u32x4 buf[NT][CH];
#pragma unroll
    for (int k = 0; k < NT; ++k)
        load_segment<CH>(in, read_lane(my_slot, k), V, base, end, lane, buf[k]);
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const float w = read_lane_f(my_w, k);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            accumulate_row(acc[i], w, buf[k][i]);
    }
}

// sum_rows for the wave-uniform count n in [1, KT] (nothing for n == 0).
template <int KT, int CH, int NT = 1>
__device__ inline void sum_rows_n(int n, const u32x4 *in, int V, int base, int end, int lane,
                                  int my_slot, float my_w, float (&acc)[CH][8])
{
    if constexpr (NT <= KT) {
        if (n == NT)
            sum_rows<NT, CH>(in, V, base, end, lane, my_slot, my_w, acc);
        else
            sum_rows_n<KT, CH, NT + 1>(n, in, V, base, end, lane, my_slot, my_w, acc);
    }
}

// KT = K known at compile time (double-buffered), or 0: runtime K <= kMaxTopk.
// CH 16-byte vectors per lane per segment; segments are seg_vecs <= 64*CH
// vectors.
template <int KT, int CH = kCombineSeg, int MODE = kCombinePairs>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wv = a.xcd_order ? xcd_item(blockIdx.x, wpb, threadIdx.x / kWave)
                               : blockIdx.x * wpb + threadIdx.x / kWave;
    if (wv >= a.num_tokens * a.segs)
        return;
    const int t = wv / a.segs;  // output row: a token, or a unit for kCombineUnitsIn
    const int sg = wv - t * a.segs;
    const int K = KT > 0 ? KT : a.topk;
    if (a.row_count && t >= *a.row_count)
        return;

    int my_slot, my_k;
    const int n = combine_slots<MODE>(a, t, sg, lane, K, my_slot, my_k);
    // term weights: requested now, read only after the rows' loads are issued
    float my_w = 0.0f;
    if (lane < n)
        my_w = (MODE == kCombineUnitsOut || !a.weights) ? 1.0f
                                                        : a.weights[(size_t)my_slot * K + my_k];
    const int V = a.row_vecs;
    const int base = sg * a.seg_vecs;
    const int end = min(V, base + a.seg_vecs);
    u32x4 *out = reinterpret_cast<u32x4 *>(a.output) + (size_t)t * V;
    const u32x4 *in = reinterpret_cast<const u32x4 *>(a.input);
    float acc[CH][8];
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[i][q] = 0.0f;

    if constexpr (KT > 0) {
        // n == 0 leaves the sum at +0
        sum_rows_n<KT, CH>(n, in, V, base, end, lane, my_slot, my_w, acc);
    } else {
        for (int k = 0; k < n; ++k) {
            u32x4 buf[CH];
            load_segment<CH>(in, read_lane(my_slot, k), V, base, end, lane, buf);
            const float wk = read_lane_f(my_w, k);
#pragma unroll
            for (int i = 0; i < CH; ++i)
                accumulate_row(acc[i], wk, buf[i]);
        }
    }

    if (MODE == kCombinePairs && a.out_weights && sg == 0 && lane < n)
        a.out_weights[t * K + my_k] = my_w;

    // Nontemporal output stores by default: device-scope or ordinary stores
    // of the output slow this read-dominated kernel down by 7-12% when its
    // input rows come from HBM (measured on gfx950).  When the input rows were
    // written just before (recent_input: the caller says so), part of them sit
    // dirty in the MALL and are written back while the combine reads them;
    // stores that allocate in the caches are then faster: buffer stores with
    // no policy bits by 6-7%, device-scope ones by 5-6%.  Outputs that the
    // next kernel reads from this XCD's L2 (cached_stores) take the same
    // stores.  They are buffer stores because an ordinary global store in
    // one branch and a nontemporal one in the other would be merged by the
    // compiler into one store without the nontemporal hint.
    const __amdgpu_buffer_rsrc_t orow = row_rsrc(a.output, (size_t)V * 16, t);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int j = base + lane + kWave * i;
        const u32x4 v = {pack_bf16_rne(acc[i][0], acc[i][1]), pack_bf16_rne(acc[i][2], acc[i][3]),
                         pack_bf16_rne(acc[i][4], acc[i][5]), pack_bf16_rne(acc[i][6], acc[i][7])};
        if (j < end) {
            if (a.cached_stores || a.recent_input)
                __builtin_amdgcn_raw_buffer_store_b128(v, orow, j * 16, 0, 0);
            else
                __builtin_nontemporal_store(v, out + j);
        }
    }
}

// Staged gather combine, for inputs that come from HBM (the op's default
// hint) in rows whose byte size is not a power of two.  A block takes
// stage_rows consecutive tokens; each of its waves computes a run of
// consecutive (token, segment) items exactly as k_combine does, into LDS,
// and after a barrier the whole block writes the group's rows, which are
// contiguous in the output, as one run of nontemporal 16-byte stores.  The
// sums are k_combine's (same terms, same order), so the outputs are
// bit-identical; what changes is when and in what pieces the output bytes
// reach HBM.  Measured on gfx950 over bf16 rows of 2880 to 8192 elements
// (cold inputs, 4096-65536 tokens, top-8): 6-7% faster than k_combine at
// hidden 7168, equal at 2880, 3072, 5120 and 6144, and up to 20% slower at
// 4096 and 8192, hence the restriction to rows that are not a power of two.
template <int KT, int CH>
__global__ __launch_bounds__(512) void k_combine_staged(CombineArgs a)
{
    extern __shared__ u32x4 stage[];  // [stage_rows * row_vecs]
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int V = a.row_vecs;
    const int K = KT > 0 ? KT : a.topk;
    const u32x4 *in = reinterpret_cast<const u32x4 *>(a.input);
    const int t0 = blockIdx.x * a.stage_rows;
    const int gt = min(a.stage_rows, a.num_tokens - t0);
    const int items = gt * a.segs;
    const int per = (items + nw - 1) / nw;  // wave w: items [w*per, w*per + per)
    for (int q = 0; q < per; ++q) {
        const int it = w * per + q;
        if (it >= items)
            break;
        const int tl = it / a.segs;
        const int sg = it - tl * a.segs;
        const int t = t0 + tl;
        int my_slot, my_k;
        const int n = combine_slots<kCombinePairs>(a, t, sg, lane, K, my_slot, my_k);
        float my_w = 0.0f;
        if (lane < n)
            my_w = a.weights ? a.weights[(size_t)my_slot * K + my_k] : 1.0f;
        const int base = sg * a.seg_vecs;
        const int end = min(V, base + a.seg_vecs);
        float acc[CH][8];
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[i][e] = 0.0f;
        if constexpr (KT > 0) {
            sum_rows_n<KT, CH>(n, in, V, base, end, lane, my_slot, my_w, acc);
        } else {
            for (int k = 0; k < n; ++k) {
                u32x4 buf[CH];
                load_segment<CH>(in, read_lane(my_slot, k), V, base, end, lane, buf);
                const float wk = read_lane_f(my_w, k);
#pragma unroll
                for (int i = 0; i < CH; ++i)
                    accumulate_row(acc[i], wk, buf[i]);
            }
        }
        if (a.out_weights && sg == 0 && lane < n)
            a.out_weights[t * K + my_k] = my_w;
        u32x4 *row = stage + (size_t)tl * V;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int j = base + lane + kWave * i;
            if (j < end)
                row[j] = u32x4{pack_bf16_rne(acc[i][0], acc[i][1]),
                               pack_bf16_rne(acc[i][2], acc[i][3]),
                               pack_bf16_rne(acc[i][4], acc[i][5]),
                               pack_bf16_rne(acc[i][6], acc[i][7])};
        }
    }
    __syncthreads();
    u32x4 *out = reinterpret_cast<u32x4 *>(a.output) + (size_t)t0 * V;
    const int nv = gt * V;
    for (int j = threadIdx.x; j < nv; j += blockDim.x)
        __builtin_nontemporal_store(stage[j], out + j);
}

// ---------------------------------------------------------------------------
// Scatter combine: the expert side pushes, the token side reduces
// ---------------------------------------------------------------------------
//
// Push: one wave per (received row s, 2 KiB segment) multiplies the bf16 row
// by its weight in fp32 and writes the products to the fp32 staging row of
// the pair it came from (src_token_pos[s]); no two rows share a staging row,
// so there are no atomics and no order to fix.  Reduce: one wave per
// (token, segment) adds the token's staging rows in k order.  The products
// and the order are the gather combine's, so the result is bit-identical to
// it; the staging round trip costs 4 extra bytes per element each way, which
// is what a one-sided push across GPUs would pay on the link instead.

struct PushArgs {
    int32_t rows;               // grid rows (received-row capacity of the call)
    const int32_t *row_count;   // device count of received rows
    int32_t topk;
    int32_t row_vecs;           // 16-byte vectors per bf16 row (H/8)
    int32_t segs;
    int32_t n_pairs;
    const int32_t *src_pos;     // [rows]: pair of each received row
    const int32_t *slot_of;     // [T*K]
    const uint8_t *input;       // [rows, H] bf16
    const float *weights;       // [rows, K] or NULL
    float *staging;             // [T*K, H] fp32
    uint8_t *output;            // [T, H] bf16
    float *out_weights;         // [T, K] or NULL
    int32_t num_tokens;
    int32_t cached_stores;      // 1: ordinary staging stores that stay in the L2 (small batches)
};

// Both kernels work on 4-element pieces (8 bytes of bf16, 16 bytes of fp32),
// lane l on pieces base + l + 64 i, so every staging load and store
// instruction covers 1 KiB of one row.  With 16-byte bf16 vectors per lane
// each lane wrote two fp32 vectors 32 bytes apart and read them back the
// same way; contiguous pieces took the headline push + reduce from 454 to
// 450 us.  The push then writes a large staging buffer with device-scope
// stores like the scatter (row_rsrc; 446 us) and one that fits the L2s with
// ordinary stores (the decode-shaped step took 26.7 us with them against
// 28.3 us with device scope).
template <int CH>
__global__ __launch_bounds__(256) void k_combine_push(PushArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (wv >= a.rows * a.segs)
        return;
    const int s = wv / a.segs;
    const int sg = wv - s * a.segs;
    if (s >= *a.row_count)
        return;
    const int p = a.src_pos[s];
    if ((unsigned)p >= (unsigned)a.n_pairs)
        return;
    const int K = a.topk;
    const float w = a.weights ? a.weights[(size_t)s * K + p % K] : 1.0f;
    constexpr int PC = 2 * CH;        // pieces per lane per segment
    const int P = 2 * a.row_vecs;     // pieces per row
    const int base = sg * kWave * PC;
    const u32x2 *row = reinterpret_cast<const u32x2 *>(a.input) + (size_t)s * P;
    const __amdgpu_buffer_rsrc_t dst =
        row_rsrc(reinterpret_cast<uint8_t *>(a.staging), (size_t)P * 16, p);
    u32x2 v[PC];
#pragma unroll
    for (int i = 0; i < PC; ++i) {
        const int h = base + lane + kWave * i;
        if (h < P)
            v[i] = __builtin_nontemporal_load(row + h);
    }
#pragma unroll
    for (int i = 0; i < PC; ++i) {
        const int h = base + lane + kWave * i;
        if (h < P) {
#pragma clang fp contract(off)
            const f32x4 prod = {w * bf16_lo(v[i].x), w * bf16_hi(v[i].x), w * bf16_lo(v[i].y),
                                w * bf16_hi(v[i].y)};
            if (a.cached_stores)
                reinterpret_cast<f32x4 *>(a.staging)[(size_t)p * P + h] = prod;
            else
                store_row16(dst, h * 16, __builtin_bit_cast(u32x4, prod));
        }
    }
}

// Sum of NT staging rows (lane k < NT holds the k-th pair), double buffered;
// PC pieces per lane starting at piece `base`.
template <int NT, int PC>
__device__ inline void sum_staged(const f32x4 *st, int P, int base, int lane, int my_pair,
                                  float (&acc)[PC][4])
{
    int pr[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k)
        pr[k] = read_lane(my_pair, k);
    f32x4 buf[2][PC];
    auto load = [&](int p, f32x4 (&d)[PC]) {
        const f32x4 *r = st + (size_t)p * P;
#pragma unroll
        for (int i = 0; i < PC; ++i) {
            const int h = base + lane + kWave * i;
            d[i] = h < P ? __builtin_nontemporal_load(r + h) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    load(pr[0], buf[0]);
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        if (k + 1 < NT)
            load(pr[k + 1], buf[(k + 1) & 1]);
#pragma unroll
        for (int i = 0; i < PC; ++i) {
#pragma clang fp contract(off)
            acc[i][0] = acc[i][0] + buf[k & 1][i].x;
            acc[i][1] = acc[i][1] + buf[k & 1][i].y;
            acc[i][2] = acc[i][2] + buf[k & 1][i].z;
            acc[i][3] = acc[i][3] + buf[k & 1][i].w;
        }
    }
}

template <int KT, int PC, int NT = 1>
__device__ inline void sum_staged_n(int n, const f32x4 *st, int P, int base, int lane,
                                    int my_pair, float (&acc)[PC][4])
{
    if constexpr (NT <= KT) {
        if (n == NT)
            sum_staged<NT, PC>(st, P, base, lane, my_pair, acc);
        else
            sum_staged_n<KT, PC, NT + 1>(n, st, P, base, lane, my_pair, acc);
    }
}

// KT = K known at compile time (double buffered), or 0: runtime K.
template <int KT, int CH>
__global__ __launch_bounds__(256) void k_combine_reduce(PushArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (wv >= a.num_tokens * a.segs)
        return;
    const int t = wv / a.segs;
    const int sg = wv - t * a.segs;
    const int K = KT > 0 ? KT : a.topk;
    int my_pair = -1;
    if (lane < K) {
        const int p = t * K + lane;
        const int s = a.slot_of[p];
        if (s >= 0)
            my_pair = p;
        if (a.out_weights && sg == 0)
            a.out_weights[p] = s < 0 ? 0.0f : (a.weights ? a.weights[(size_t)s * K + lane] : 1.0f);
    }
    // pairs with a row to the front lanes, in k order
    const uint64_t have = __ballot(my_pair >= 0);
    const int n = __popcll(have);
    const int r = my_pair >= 0 ? lanes_below(have) : kWave;
    int cp = -1;
    for (int j = 0; j < K; ++j) {
        const int pj = read_lane(my_pair, j);
        if (read_lane(r, j) == lane)
            cp = pj;
    }
    constexpr int PC = 2 * CH;     // pieces per lane per segment
    const int P = 2 * a.row_vecs;  // pieces per row
    const int base = sg * kWave * PC;
    float acc[PC][4];
#pragma unroll
    for (int i = 0; i < PC; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc[i][q] = 0.0f;
    const f32x4 *st = reinterpret_cast<const f32x4 *>(a.staging);
    if constexpr (KT > 0) {
        sum_staged_n<KT, PC>(n, st, P, base, lane, cp, acc);
    } else {
        for (int k = 0; k < n; ++k)  // one row at a time
            sum_staged<1, PC>(st, P, base, lane, read_lane(cp, k), acc);
    }
    u32x2 *out = reinterpret_cast<u32x2 *>(a.output) + (size_t)t * P;
#pragma unroll
    for (int i = 0; i < PC; ++i) {
        const int h = base + lane + kWave * i;
        if (h < P)
            __builtin_nontemporal_store(
                u32x2{pack_bf16_rne(acc[i][0], acc[i][1]), pack_bf16_rne(acc[i][2], acc[i][3])},
                out + h);
    }
}

// ---------------------------------------------------------------------------
// Debug check of combine's indices against the recorded routing
// ---------------------------------------------------------------------------
//
// combine(input, weights, indices) takes the indices in the received layout
// (MORI "Communication APIs" page, MORI-EP section, methods table).  The op
// keeps the routing of the last dispatch, so the indices are redundant; when
// the caller asks for the check, every received row s < n_valid must hold,
// in entry k of its indices row, the expert that row belongs to, where k is
// the k of the pair the row came from (src_pos[s] mod K) and the expert is
// the one whose run of rows [expert_off[e], expert_off[e+1]) contains s.
// A mismatch raises bit 4 of the device error flag; the check writes
// nothing else.  One thread per row of the capacity of the call.

struct CheckArgs {
    int32_t n_pairs;             // num_tokens * K of the recorded dispatch
    int32_t topk;
    int32_t num_experts;
    const int32_t *expert_off;   // [E+1]
    const int32_t *src_pos;      // [n_valid]
    const int32_t *indices;      // [rows, K] received layout
    uint32_t *ctrl;
};

__global__ __launch_bounds__(256) void k_check_indices(CheckArgs a)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    const int E = a.num_experts;
    const int n_valid = a.expert_off[E];
    if (s >= a.n_pairs || s >= n_valid)
        return;
    const int p = a.src_pos[s];
    bool bad = (unsigned)p >= (unsigned)a.n_pairs;
    if (!bad) {
        // the expert e with expert_off[e] <= s < expert_off[e+1]: the last
        // e in [0, E) whose first row is <= s (empty experts share an offset
        // with the next one, so the last such e is the non-empty one)
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.expert_off[mid] <= s)
                lo = mid;
            else
                hi = mid - 1;
        }
        bad = a.indices[(size_t)s * a.topk + p % a.topk] != lo;
    }
    if (bad)
        atomicOr(&a.ctrl[kCtrlError], 4u);
}

}  // namespace epdc
