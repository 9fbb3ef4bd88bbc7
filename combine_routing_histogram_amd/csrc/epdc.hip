// epdc.hip -- host side of the C ABI declared in include/epdc.h: argument
// checks, workspace layout, kernel selection and launch, per-kernel event
// timing.  Every step of dispatch and combine runs in the kernels of
// epdc_kernels.hpp; the host enqueues them on the caller's stream and never
// waits, except in epdc_create (control words cleared once),
// epdc_get_device_error and epdc_profile_end.
#include "epdc.h"
#include "epdc_kernels.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace epdc;

namespace {

thread_local std::string g_last_error;

epdc_status fail(epdc_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

epdc_status ok()
{
    g_last_error.clear();
    return EPDC_SUCCESS;
}

// Largest row (elements): rows are addressed with 32-bit byte offsets, and an
// fp32 staging row is 4H bytes.
constexpr int kMaxHidden = 1 << 24;

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Device workspace: control words, routing tables and the per-pair arrays.
struct Layout {
    size_t ctrl, tile_table, rank_in_tile, expert_off, rank_off, slot_of, src_pos;
    // rank-deduplicated dispatch: the unit routing and the pairs' rank counts
    size_t unit_table, unit_rank_in_tile, unit_off, unit_of, unit_src, pair_recv;
    size_t tile_cnt16;  // [E][<= 8 * kScanMaxLoads] 16-bit tile counts
    size_t total;
    int64_t n_cap;
    int64_t u_cap;  // max_tokens * min(topk, num_ranks)
    int64_t tiles_max;
};

int units_per_token(const epdc_config &c) { return c.topk < c.num_ranks ? c.topk : c.num_ranks; }

epdc_status check_config(const epdc_config *c)
{
    if (!c)
        return fail(EPDC_ERR_INVALID_ARGS, "config is NULL");
    if (c->max_tokens < 0)
        return fail(EPDC_ERR_INVALID_ARGS, "max_tokens must be >= 0");
    if (c->hidden <= 0 || c->hidden % 8 != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "hidden must be a positive multiple of 8");
    if (c->hidden > kMaxHidden)
        return fail(EPDC_ERR_INVALID_ARGS, "hidden must be <= 2^24");
    if (c->topk < 1 || c->topk > kMaxTopk)
        return fail(EPDC_ERR_INVALID_ARGS, "topk must be in [1, %d]", kMaxTopk);
    if (c->num_experts < 1 || c->num_experts > kMaxExperts)
        return fail(EPDC_ERR_INVALID_ARGS, "num_experts must be in [1, %d]", kMaxExperts);
    if (c->num_ranks < 1 || c->num_experts % c->num_ranks != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "num_ranks must divide num_experts");
    if ((int64_t)c->max_tokens * c->topk > (int64_t)(1 << 30))
        return fail(EPDC_ERR_INVALID_ARGS, "max_tokens*topk must be <= 2^30");
    if (c->input_kind != EPDC_IN_BF16 && c->input_kind != EPDC_IN_RAW)
        return fail(EPDC_ERR_INVALID_ARGS, "unknown input_kind %d", c->input_kind);
    if (c->scale_row_bytes < 0 || c->scale_row_bytes % 4 != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "scale_row_bytes must be a non-negative multiple of 4");
    switch (c->quant) {
    case EPDC_QUANT_NONE:
        break;
    case EPDC_QUANT_FP8_E4M3_B128:
        if (c->hidden % 128 != 0)
            return fail(EPDC_ERR_INVALID_ARGS, "FP8 block-128 quantization needs hidden %% 128 == 0");
        break;
    case EPDC_QUANT_MXFP4_B32:
        if (c->hidden % 32 != 0)
            return fail(EPDC_ERR_INVALID_ARGS, "MXFP4 quantization needs hidden %% 32 == 0");
        break;
    default:
        return fail(EPDC_ERR_INVALID_ARGS, "unknown quant %d", c->quant);
    }
    if (c->quant != EPDC_QUANT_NONE) {
        if (c->input_kind != EPDC_IN_BF16)
            return fail(EPDC_ERR_INVALID_ARGS, "quantization needs bf16 input");
        if (c->scale_row_bytes != 0)
            return fail(EPDC_ERR_INVALID_ARGS, "scale_row_bytes must be 0 when dispatch quantizes");
    }
    if (c->input_kind == EPDC_IN_RAW && (c->raw_row_bytes <= 0 || c->raw_row_bytes % 16 != 0 ||
                                         c->raw_row_bytes > 2 * kMaxHidden))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "raw_row_bytes must be a positive multiple of 16, at most 2^25");
    return EPDC_SUCCESS;
}

Layout layout_for(const epdc_config &c)
{
    Layout l{};
    l.n_cap = (int64_t)c.max_tokens * c.topk;
    l.tiles_max = l.n_cap > 0 ? (l.n_cap + kRouteTile - 1) / kRouteTile : 1;
    size_t off = 0;
    l.ctrl = off;
    off += align256(sizeof(uint32_t) * kCtrlWords);
    l.tile_table = off;
    off += align256(sizeof(int32_t) * (size_t)l.tiles_max * c.num_experts);
    l.rank_in_tile = off;
    off += align256(sizeof(int32_t) * (size_t)l.n_cap);
    l.expert_off = off;
    off += align256(sizeof(int32_t) * (size_t)(c.num_experts + 1));
    l.rank_off = off;
    off += align256(sizeof(int32_t) * (size_t)(c.num_ranks + 1));
    l.slot_of = off;
    off += align256(sizeof(int32_t) * (size_t)l.n_cap);
    l.src_pos = off;
    off += align256(sizeof(int32_t) * (size_t)l.n_cap);
    l.u_cap = (int64_t)c.max_tokens * units_per_token(c);
    l.unit_table = off;
    off += align256(sizeof(int32_t) * (size_t)l.tiles_max * c.num_ranks);
    l.unit_rank_in_tile = off;
    off += align256(sizeof(int32_t) * (size_t)l.n_cap);
    l.unit_off = off;
    off += align256(sizeof(int32_t) * (size_t)(c.num_ranks + 1));
    l.unit_of = off;
    off += align256(sizeof(int32_t) * (size_t)l.n_cap);
    l.unit_src = off;
    off += align256(sizeof(int32_t) * (size_t)l.u_cap);
    l.pair_recv = off;
    off += align256(sizeof(int32_t) * (size_t)c.num_ranks);
    l.tile_cnt16 = off;
    off += align256(sizeof(uint16_t) * 8 * kScanMaxLoads * (size_t)c.num_experts);
    l.total = off;
    return l;
}

void row_bytes_for(const epdc_config &c, size_t *payload, size_t *scales)
{
    switch (c.quant) {
    case EPDC_QUANT_FP8_E4M3_B128:
        *payload = (size_t)c.hidden;
        *scales = sizeof(float) * (size_t)(c.hidden / 128);
        return;
    case EPDC_QUANT_MXFP4_B32:
        *payload = (size_t)c.hidden / 2;
        *scales = (size_t)c.hidden / 32;
        return;
    default:
        *payload = c.input_kind == EPDC_IN_RAW ? (size_t)c.raw_row_bytes : 2 * (size_t)c.hidden;
        *scales = (size_t)c.scale_row_bytes;
        return;
    }
}

const char *const kKernelNames[EPDC_NUM_KERNELS] = {
    "k_route_rank", "k_route_scan", "k_scatter_copy", "k_scatter_fp8", "k_scatter_mxfp4",
    "k_combine", "k_units_to_experts", "k_experts_to_units", "k_combine_units",
    "k_combine_push", "k_combine_reduce", "k_check_indices"};

// Workspace of the ops made by epdc_create_static, for callers that cannot
// allocate device memory.  Each device the library runs on holds its own copy
// for the life of the process.  In host code `scratch` names a host-side
// stand-in, not device memory: the host only ever uses the per-device
// address hipGetSymbolAddress returns for it (static_workspace below).
constexpr size_t kStaticWorkspaceBytes = EPDC_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (the current device), looked up
// once per device.
epdc_status static_workspace(int dev, void **ptr)
{
    if (dev < 0 || dev >= kMaxDevices)
        return fail(EPDC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(EPDC_ERR_GPU_OP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return EPDC_SUCCESS;
}

}  // namespace

struct epdc_op {
    epdc_config cfg;
    int device;
    uint8_t *ws;
    Layout lay;
    int key_bits;
    int unit_key_bits;
    bool routed;
    bool units_routed;  // the last dispatch was rank-deduplicated
    int32_t last_tokens;
    int32_t debug;          // EPDC_DEBUG_* bits (epdc_set_debug)
    int32_t combine_hint;   // EPDC_COMBINE_INPUT_* (epdc_set_combine_hint)
    bool static_ws;         // the workspace is the library's `scratch` (epdc_create_static)
    // split-phase completion markers (timing disabled), made on first use
    hipEvent_t ev_dispatch, ev_combine;
    bool dispatch_sent, combine_sent;
    // per-kernel timing
    bool profiling;
    int ev_cap, ev_used;
    std::vector<hipEvent_t> ev;  // 2 per launch
    std::vector<int> ev_kernel;

    uint32_t *ctrl() const { return reinterpret_cast<uint32_t *>(ws + lay.ctrl); }
    int32_t *i32(size_t off) const { return reinterpret_cast<int32_t *>(ws + off); }
};

namespace {

// The op over each device's `scratch` (epdc_create_static): one per device,
// since all of them would share the one workspace; each create re-configures
// it in place, so the handle always describes what the workspace holds.
// Guarded by g_scratch_mu.
epdc_op g_static_ops[kMaxDevices];

// Release the events an op holds (timing and split-phase markers).
void release_events(epdc_op *op)
{
    for (hipEvent_t ev : op->ev)
        (void)hipEventDestroy(ev);
    op->ev.clear();
    op->ev_kernel.clear();
    op->ev_cap = op->ev_used = 0;
    op->profiling = false;
    if (op->ev_dispatch)
        (void)hipEventDestroy(op->ev_dispatch);
    if (op->ev_combine)
        (void)hipEventDestroy(op->ev_combine);
    op->ev_dispatch = op->ev_combine = nullptr;
}

// Launch `f` on `st`, bracketed by timing events when profiling.
template <typename F>
epdc_status launch(epdc_op *op, hipStream_t st, int kernel_id, F &&f)
{
    const bool prof = op->profiling && op->ev_used < op->ev_cap;
    hipError_t ev_err = hipSuccess;
    if (prof)
        ev_err = hipEventRecord(op->ev[2 * op->ev_used], st);
    f();
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "%s launch failed: %s", kKernelNames[kernel_id],
                    hipGetErrorString(err));
    if (prof) {
        if (ev_err == hipSuccess)
            ev_err = hipEventRecord(op->ev[2 * op->ev_used + 1], st);
        if (ev_err != hipSuccess)
            return fail(EPDC_ERR_GPU_OP, "hipEventRecord: %s", hipGetErrorString(ev_err));
        op->ev_kernel[op->ev_used] = kernel_id;
        ++op->ev_used;
    }
    return EPDC_SUCCESS;
}

// How a scatter launch splits token rows: CH 16-byte vectors per lane per
// pass, segments of seg_vecs vectors (a multiple of 64*CH), one wave each.
struct ScatterPlan {
    int ch, seg_vecs, segs;
};

ScatterPlan make_plan(int ch, int row_vecs, int max_segs)
{
    const int pass = kWave * ch;
    const int passes = (row_vecs + pass - 1) / pass;
    int segs = max_segs < passes ? max_segs : passes;
    if (segs < 1)
        segs = 1;
    const int per_seg = (passes + segs - 1) / segs;
    ScatterPlan p;
    p.ch = ch;
    p.seg_vecs = per_seg * pass;
    p.segs = (passes + per_seg - 1) / per_seg;
    return p;
}

// Measured on MI355X in the dispatch -> combine loop:
// the bf16 copy streams best with one wave per token once there are enough
// tokens to fill the chip; the quantizing kernels and small batches need more,
// shorter waves per token to hide their per-wave latency.
ScatterPlan plan_scatter(int quant, int tokens, int row_vecs, bool inline_route)
{
    switch (quant) {
    case EPDC_QUANT_FP8_E4M3_B128:  // 2 adjacent vectors per lane per pass
        return make_plan(kFp8PassVecs / kWave, row_vecs, 1 << 20);
    case EPDC_QUANT_MXFP4_B32:      // 2 vectors per lane per pass
        // many tokens: one wave per row up to the scale stage (kMxStageBytes)
        return tokens >= 2048 && !inline_route
                   ? make_plan(2, row_vecs, (row_vecs + 4 * kMxStageBytes - 1) / (4 * kMxStageBytes))
                   : make_plan(2, row_vecs, 1 << 20);
    default:
        return tokens >= 2048 && !inline_route ? make_plan(8, row_vecs, 1)
                                               : make_plan(2, row_vecs, 1 << 20);
    }
}

// Grid of one-wave work items: 4 waves per block once there are enough waves
// to fill the chip with such blocks, else single-wave blocks spread over more
// CUs.
int waves_per_block(int64_t waves) { return waves >= 4096 ? 4 : 1; }

epdc_status grid_for_waves(int64_t waves, int *grid, int *block)
{
    if (waves <= 0 || waves > (int64_t)0x7FFFFFFF - 64)
        return fail(EPDC_ERR_INVALID_ARGS, "work of %lld waves does not fit one launch",
                    (long long)waves);
    const int wpb = waves_per_block(waves);
    *grid = (int)((waves + wpb - 1) / wpb);
    *block = wpb * kWave;
    return EPDC_SUCCESS;
}

// Blocks of wpb waves for `waves` one-wave items; in XCD order (xcd_item)
// a whole number of rounds of kXcds blocks.
int blocks_for(int64_t waves, int wpb, bool xcd_order)
{
    if (!xcd_order)
        return (int)((waves + wpb - 1) / wpb);
    const int64_t round = (int64_t)kXcds * wpb;
    return (int)(kXcds * ((waves + round - 1) / round));
}

// Items in XCD order for a batch of at most one routing tile.  The scatter
// of such a batch (inline routing or its replay) and the gather combine
// after it split rows into the same 2 KiB segments, so the two waves of a
// (token, segment) share an XCD; larger batches keep launch order (their
// rows do not fit the L2s anyway).
bool one_tile_xcd_order(int64_t n_pairs) { return n_pairs > 0 && n_pairs <= kRouteTile; }

// Rows a scatter writes that fit the eight XCDs' 4 MB L2s together are
// written with ordinary stores, which leave them there for the kernel that
// reads them next; larger batches use device-scope stores (row_rsrc).
constexpr int64_t kL2ResidentBytes = int64_t(32) << 20;

// Segment width of the XCD-local layout of a small rank-deduplicated bf16
// batch, or 0.  Its four kernels number their rows differently (token, unit,
// expert row), so XCD order alone cannot pair a writer wave with its reader.
// With a multiple of 8 segments per row it does not need to: item
// row * segs + s runs on XCD s mod 8 in every kernel, so each kernel of the
// chain finds the rows segment s of the previous one wrote in its own L2.
// Rows need at least 512 vectors (hidden >= 4096) so that a segment keeps
// at least 64 vectors, one per lane.
int dedup_local_seg_vecs(const epdc_config &c, int64_t tokens)
{
    if (c.quant != EPDC_QUANT_NONE || c.input_kind != EPDC_IN_BF16)
        return 0;
    const int V = c.hidden / 8;
    if (V < kXcds * kWave || tokens * c.topk * 2 * (int64_t)c.hidden > kL2ResidentBytes)
        return 0;
    const int per_round = kXcds * kCombineSegVecs;
    const int segs = kXcds * ((V + per_round - 1) / per_round);
    return (V + segs - 1) / segs;
}

// Plan, grid and launch of the scatter kernel for the op's payload kind;
// sa holds everything but the plan fields.
// local_seg_vecs > 0: the XCD-local layout (dedup_local_seg_vecs), rows in
// segments of that many vectors, items in XCD order.
epdc_status launch_scatter(epdc_op *op, hipStream_t st, ScatterArgs &sa, int mode,
                           int local_seg_vecs = 0)
{
    const epdc_config &c = op->cfg;
    const int num_tokens = sa.num_tokens;
    const bool inline_route = mode == kRouteInline;
    const int quant = mode == kRouteConvert ? (int)EPDC_QUANT_NONE : c.quant;
    const int in_vecs = quant == EPDC_QUANT_NONE ? sa.in_row_vecs : c.hidden / 8;
    ScatterPlan plan = plan_scatter(quant, num_tokens, in_vecs, inline_route);
    if (local_seg_vecs > 0) {
        plan.ch = 2;  // one pass of up to 128 vectors per segment
        plan.seg_vecs = local_seg_vecs;
        plan.segs = (in_vecs + local_seg_vecs - 1) / local_seg_vecs;
        sa.xcd_order = 1;
    }
    sa.segs = plan.segs;
    sa.seg_vecs = plan.seg_vecs;
    // word-aligned scale rows and segments that fit the stage
    sa.scale_stage = quant == EPDC_QUANT_MXFP4_B32 && c.hidden % 128 == 0 &&
                     plan.seg_vecs <= 4 * kMxStageBytes;
    {
        size_t payload, scales;
        row_bytes_for(c, &payload, &scales);
        if (mode == kRouteConvert)
            payload = (size_t)sa.in_row_vecs * 16;
        const bool unit_rows = mode == kRouteUnits || mode == kRouteUnitsReplay;
        const int64_t rows = unit_rows ? sa.unit_rows_max : sa.n_pairs;
        sa.cached_stores = rows * (int64_t)payload <= kL2ResidentBytes;
    }
    int grid, block;
    const int64_t waves = (int64_t)num_tokens * sa.segs;
    if (inline_route) {
        // kRouteThreads threads per block for the ranking; about 256 blocks
        // share the copies (waves <= 1024 * 64 here: at most one tile of pairs)
        sa.work_waves =
            (int)std::min<int64_t>(kRouteWaves, std::max<int64_t>(1, (waves + 255) / 256));
        grid = blocks_for(waves, sa.work_waves, sa.xcd_order);
        block = kRouteThreads;
    } else {
        epdc_status s = grid_for_waves(waves, &grid, &block);
        if (s != EPDC_SUCCESS)
            return s;
        sa.work_waves = block / kWave;
        grid = blocks_for(waves, sa.work_waves, sa.xcd_order);
    }
    // the table-scanning blocks locate their tiles from launch-order items
    if (sa.xcd_order && mode == kRouteTableScan)
        return fail(EPDC_ERR_INVALID_ARGS, "XCD item order cannot scan the tile table");
    if (mode == kRouteConvert)  // unit rows to expert rows: bytes, whatever the payload
        return launch(op, st, EPDC_KERNEL_UNITS_TO_EXPERTS, [&] {
            if (plan.ch == 8)
                k_scatter_copy<8, kRouteConvert><<<grid, block, 0, st>>>(sa);
            else
                k_scatter_copy<2, kRouteConvert><<<grid, block, 0, st>>>(sa);
        });
    switch (c.quant) {
    case EPDC_QUANT_FP8_E4M3_B128:
        return launch(op, st, EPDC_KERNEL_SCATTER_FP8, [&] {
            switch (mode) {
            case kRouteInline: k_scatter_fp8<kRouteInline><<<grid, block, 0, st>>>(sa); break;
            case kRouteReplay: k_scatter_fp8<kRouteReplay><<<grid, block, 0, st>>>(sa); break;
            case kRouteUnits: k_scatter_fp8<kRouteUnits><<<grid, block, 0, st>>>(sa); break;
            case kRouteTableScan:
                k_scatter_fp8<kRouteTableScan><<<grid, block, 0, st>>>(sa);
                break;
            case kRouteUnitsReplay:
                k_scatter_fp8<kRouteUnitsReplay><<<grid, block, 0, st>>>(sa);
                break;
            default: k_scatter_fp8<><<<grid, block, 0, st>>>(sa); break;
            }
        });
    case EPDC_QUANT_MXFP4_B32:
        return launch(op, st, EPDC_KERNEL_SCATTER_MXFP4, [&] {
            switch (mode) {
            case kRouteInline: k_scatter_mxfp4<2, kRouteInline><<<grid, block, 0, st>>>(sa); break;
            case kRouteReplay: k_scatter_mxfp4<2, kRouteReplay><<<grid, block, 0, st>>>(sa); break;
            case kRouteUnits: k_scatter_mxfp4<2, kRouteUnits><<<grid, block, 0, st>>>(sa); break;
            case kRouteTableScan:
                k_scatter_mxfp4<2, kRouteTableScan><<<grid, block, 0, st>>>(sa);
                break;
            case kRouteUnitsReplay:
                k_scatter_mxfp4<2, kRouteUnitsReplay><<<grid, block, 0, st>>>(sa);
                break;
            default: k_scatter_mxfp4<2><<<grid, block, 0, st>>>(sa); break;
            }
        });
    default:
        return launch(op, st, EPDC_KERNEL_SCATTER, [&] {
            const bool wide = plan.ch == 8;
            switch (mode) {
            case kRouteInline: k_scatter_copy<2, kRouteInline><<<grid, block, 0, st>>>(sa); break;
            case kRouteReplay:
                if (wide)
                    k_scatter_copy<8, kRouteReplay><<<grid, block, 0, st>>>(sa);
                else
                    k_scatter_copy<2, kRouteReplay><<<grid, block, 0, st>>>(sa);
                break;
            case kRouteUnits:
                if (wide)
                    k_scatter_copy<8, kRouteUnits><<<grid, block, 0, st>>>(sa);
                else
                    k_scatter_copy<2, kRouteUnits><<<grid, block, 0, st>>>(sa);
                break;
            case kRouteUnitsReplay:
                if (wide)
                    k_scatter_copy<8, kRouteUnitsReplay><<<grid, block, 0, st>>>(sa);
                else
                    k_scatter_copy<2, kRouteUnitsReplay><<<grid, block, 0, st>>>(sa);
                break;
            case kRouteTableScan:
                if (wide)
                    k_scatter_copy<8, kRouteTableScan><<<grid, block, 0, st>>>(sa);
                else
                    k_scatter_copy<2, kRouteTableScan><<<grid, block, 0, st>>>(sa);
                break;
            default:
                if (wide)
                    k_scatter_copy<8><<<grid, block, 0, st>>>(sa);
                else
                    k_scatter_copy<2><<<grid, block, 0, st>>>(sa);
                break;
            }
        });
    }
}

template <int KT, int MODE>
void launch_combine(int grid, int block, size_t lds, hipStream_t st, const CombineArgs &a)
{
    k_combine<KT, kCombineSeg, MODE><<<grid, block, lds, st>>>(a);
}

// A gather combine over at least this many bytes of cold input rows runs
// with fewer waves per CU: its launch reserves LDS that the kernel does not
// use (kCombineLdsReserve, so at most two 4-wave blocks share a CU's
// 160 KiB).  Measured on gfx950 with top-8 bf16 rows: 1-2% faster at 0.75 GiB
// of input, 3-4% at 1-1.3 GiB, 5-6% at 2 GiB; equal or up to 3% slower
// below 0.5 GiB.
constexpr int64_t kCombineFewWavesBytes = int64_t(768) << 20;
constexpr size_t kCombineLdsReserve = size_t(64) << 10;

// A combine of rows written just before (the RECENT hint) in the plain CU
// order reserves LDS the same way for at most three 4-wave blocks per CU.  At
// 4096 x 7168 top-8 after the scatter (five runs each, gfx950): the kernel up
// to 2 us faster with the steps back to back (97.4-97.8 against 97.6-100.1
// us), the step 1 us faster after a 512 MiB read and with layers stepped in
// turn, equal after a 512 MiB write.
constexpr size_t kCombineRecentLdsReserve = size_t(48) << 10;

// One wave per (row, 2 KiB segment) over `rows` output rows; with
// local_seg_vecs > 0 the XCD-local layout (dedup_local_seg_vecs).
template <int MODE>
epdc_status launch_combine_mode(epdc_op *op, hipStream_t st, int kernel_id, CombineArgs &ca,
                                int64_t rows, int local_seg_vecs = 0, size_t lds = 0)
{
    const epdc_config &c = op->cfg;
    ca.topk = c.topk;
    ca.row_vecs = c.hidden / 8;
    ca.seg_vecs = kCombineSegVecs;
    if (local_seg_vecs > 0) {
        ca.seg_vecs = local_seg_vecs;
        ca.xcd_order = 1;
        ca.cached_stores = 1;
    }
    ca.segs = (ca.row_vecs + ca.seg_vecs - 1) / ca.seg_vecs;
    ca.num_tokens = (int32_t)rows;
    int grid, block;
    epdc_status s = grid_for_waves(rows * ca.segs, &grid, &block);
    if (s != EPDC_SUCCESS)
        return s;
    grid = blocks_for(rows * ca.segs, block / kWave, ca.xcd_order);
    return launch(op, st, kernel_id, [&] {
        switch (c.topk) {
        case 1: launch_combine<1, MODE>(grid, block, lds, st, ca); break;
        case 2: launch_combine<2, MODE>(grid, block, lds, st, ca); break;
        case 4: launch_combine<4, MODE>(grid, block, lds, st, ca); break;
        case 6: launch_combine<6, MODE>(grid, block, lds, st, ca); break;
        case 8: launch_combine<8, MODE>(grid, block, lds, st, ca); break;
        default: launch_combine<0, MODE>(grid, block, lds, st, ca); break;
        }
    });
}

// The staged gather combine (k_combine_staged): groups of up to four rows
// per 8-wave block, 1 KiB segments, a row group of at most 64 KiB of LDS.
constexpr int kCombineStageBytes = 64 << 10;
constexpr int kCombineStageMaxRows = 4;
constexpr int kCombineStageWaves = 8;
constexpr int kCombineStageSeg = 1;

template <int KT>
void launch_combine_staged(int grid, int block, size_t lds, hipStream_t st, const CombineArgs &a)
{
    k_combine_staged<KT, kCombineStageSeg><<<grid, block, lds, st>>>(a);
}

// Rows per block for the staged combine, or 0 where the plain one runs: the
// staged form takes large batches of cold input in rows whose byte size is
// not a power of two (k_combine_staged).
int combine_stage_rows(const epdc_config &c, const CombineArgs &ca)
{
    if (ca.recent_input || ca.xcd_order || ca.cached_stores)
        return 0;
    const int64_t row_bytes = (int64_t)(c.hidden / 8) * 16;
    if (row_bytes > kCombineStageBytes || (row_bytes & (row_bytes - 1)) == 0)
        return 0;
    const int64_t g = kCombineStageBytes / row_bytes;
    return (int)(g < kCombineStageMaxRows ? g : kCombineStageMaxRows);
}

epdc_status launch_combine_staged_mode(epdc_op *op, hipStream_t st, CombineArgs &ca, int64_t rows,
                                       int stage_rows)
{
    const epdc_config &c = op->cfg;
    ca.topk = c.topk;
    ca.row_vecs = c.hidden / 8;
    ca.seg_vecs = kWave * kCombineStageSeg;
    ca.segs = (ca.row_vecs + ca.seg_vecs - 1) / ca.seg_vecs;
    ca.num_tokens = (int32_t)rows;
    ca.stage_rows = stage_rows;
    const int grid = (int)((rows + stage_rows - 1) / stage_rows);
    const int block = kCombineStageWaves * kWave;
    const size_t lds = (size_t)stage_rows * ca.row_vecs * 16;
    return launch(op, st, EPDC_KERNEL_COMBINE, [&] {
        switch (c.topk) {
        case 1: launch_combine_staged<1>(grid, block, lds, st, ca); break;
        case 2: launch_combine_staged<2>(grid, block, lds, st, ca); break;
        case 4: launch_combine_staged<4>(grid, block, lds, st, ca); break;
        case 6: launch_combine_staged<6>(grid, block, lds, st, ca); break;
        case 8: launch_combine_staged<8>(grid, block, lds, st, ca); break;
        default: launch_combine_staged<0>(grid, block, lds, st, ca); break;
        }
    });
}

// The debug check of combine's indices (k_check_indices), when the op has it
// switched on and the caller passed indices.
epdc_status check_combine_indices(epdc_op *op, hipStream_t st, const int32_t *indices)
{
    if (!(op->debug & EPDC_DEBUG_CHECK_INDICES) || !indices)
        return EPDC_SUCCESS;
    if (!aligned(indices, 4))
        return fail(EPDC_ERR_INVALID_ARGS, "indices must be 4-byte aligned");
    const epdc_config &c = op->cfg;
    CheckArgs ca = {};
    ca.n_pairs = op->last_tokens * c.topk;
    ca.topk = c.topk;
    ca.num_experts = c.num_experts;
    ca.expert_off = op->i32(op->lay.expert_off);
    ca.src_pos = op->i32(op->lay.src_pos);
    ca.indices = indices;
    ca.ctrl = op->ctrl();
    const int grid = (ca.n_pairs + 255) / 256;
    return launch(op, st, EPDC_KERNEL_CHECK_INDICES,
                  [&] { k_check_indices<<<grid, 256, 0, st>>>(ca); });
}

}  // namespace

extern "C" {

epdc_status epdc_workspace_bytes(const epdc_config *cfg, size_t *bytes)
{
    epdc_status s = check_config(cfg);
    if (s != EPDC_SUCCESS)
        return s;
    if (!bytes)
        return fail(EPDC_ERR_INVALID_ARGS, "bytes is NULL");
    *bytes = layout_for(*cfg).total;
    return ok();
}

epdc_status epdc_row_bytes(const epdc_config *cfg, size_t *payload_bytes, size_t *scale_bytes)
{
    epdc_status s = check_config(cfg);
    if (s != EPDC_SUCCESS)
        return s;
    if (!payload_bytes || !scale_bytes)
        return fail(EPDC_ERR_INVALID_ARGS, "output pointer is NULL");
    row_bytes_for(*cfg, payload_bytes, scale_bytes);
    return ok();
}

}  // extern "C"

namespace {

// Create an op on the current device over `workspace` (>= layout total bytes).
epdc_status create_on(const epdc_config *cfg, void *workspace, bool static_ws, epdc_op **op)
{
    const Layout lay = layout_for(*cfg);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "hipGetDevice: %s", hipGetErrorString(e));
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(EPDC_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950",
                    dev, prop.gcnArchName);
    std::unique_lock<std::mutex> lock(g_scratch_mu, std::defer_lock);
    if (static_ws) {
        const epdc_status s = static_workspace(dev, &workspace);
        if (s != EPDC_SUCCESS)
            return s;
        lock.lock();  // after static_workspace, which takes the same mutex
    }
    // the sticky error flag and the other control words start at zero
    e = hipMemset(static_cast<uint8_t *>(workspace) + lay.ctrl, 0, sizeof(uint32_t) * kCtrlWords);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "clearing control words: %s", hipGetErrorString(e));

    epdc_op *o;
    if (static_ws) {
        o = &g_static_ops[dev];
        release_events(o);
    } else {
        o = new epdc_op();
    }
    o->cfg = *cfg;
    o->ev_dispatch = o->ev_combine = nullptr;
    o->dispatch_sent = o->combine_sent = false;
    o->device = dev;
    o->ws = static_cast<uint8_t *>(workspace);
    o->lay = lay;
    int bits = 0;
    while ((1 << bits) < cfg->num_experts)
        ++bits;
    o->key_bits = bits;
    bits = 0;
    while ((1 << bits) < cfg->num_ranks)
        ++bits;
    o->unit_key_bits = bits;
    o->routed = false;
    o->units_routed = false;
    o->last_tokens = 0;
    o->debug = 0;
    o->combine_hint = EPDC_COMBINE_INPUT_COLD;
    o->static_ws = static_ws;
    o->profiling = false;
    o->ev_cap = o->ev_used = 0;
    *op = o;
    return ok();
}

// The split phases' completion marker, created on the first send.
epdc_status send_event(hipEvent_t *ev)
{
    if (*ev)
        return EPDC_SUCCESS;
    const hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (e != hipSuccess) {
        *ev = nullptr;
        return fail(EPDC_ERR_GPU_OP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
    }
    return EPDC_SUCCESS;
}

}  // namespace

extern "C" {

epdc_status epdc_create(const epdc_config *cfg, void *workspace, size_t workspace_bytes,
                        epdc_op **op)
{
    epdc_status s = check_config(cfg);
    if (s != EPDC_SUCCESS)
        return s;
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    *op = nullptr;
    const Layout lay = layout_for(*cfg);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "workspace must be a 256-byte aligned device pointer");
    if (workspace_bytes < lay.total)
        return fail(EPDC_ERR_INVALID_ARGS, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    lay.total);
    return create_on(cfg, workspace, false, op);
}

epdc_status epdc_create_static(const epdc_config *cfg, epdc_op **op)
{
    epdc_status s = check_config(cfg);
    if (s != EPDC_SUCCESS)
        return s;
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    *op = nullptr;
    const Layout lay = layout_for(*cfg);
    if (lay.total > kStaticWorkspaceBytes)
        return fail(EPDC_ERR_INVALID_ARGS,
                    "this config needs %zu bytes of workspace; the library's static workspace "
                    "holds %zu (use epdc_create with a caller workspace)",
                    lay.total, kStaticWorkspaceBytes);
    return create_on(cfg, nullptr, true, op);
}

epdc_status epdc_destroy(epdc_op *op)
{
    if (!op)
        return ok();
    if (op->static_ws) {  // the device's static op: forget its state, keep the object
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        release_events(op);
        op->routed = op->units_routed = false;
        op->dispatch_sent = op->combine_sent = false;
        op->last_tokens = 0;
        return ok();
    }
    release_events(op);
    delete op;
    return ok();
}

}  // extern "C"

namespace {

// Pair dispatch (dedup = false) or rank-deduplicated dispatch (dedup = true).
epdc_status dispatch_impl(epdc_op *op, void *stream, int32_t num_tokens, const void *input,
                          const float *weights, const void *scales, const int32_t *indices,
                          void *out, float *out_weights, void *out_scales, int32_t *out_indices,
                          int32_t *recv_count, bool dedup)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    const epdc_config &c = op->cfg;
    if (num_tokens < 0 || num_tokens > c.max_tokens)
        return fail(EPDC_ERR_INVALID_ARGS, "num_tokens %d outside [0, %d]", num_tokens,
                    c.max_tokens);
    if (!out || !recv_count)
        return fail(EPDC_ERR_INVALID_ARGS, "out and recv_count are required");
    const bool quant = c.quant != EPDC_QUANT_NONE;
    if (num_tokens > 0) {  // with no tokens no row is read or written
        if (!input || !indices)
            return fail(EPDC_ERR_INVALID_ARGS, "input and indices are required");
        if ((weights == nullptr) != (out_weights == nullptr))
            return fail(EPDC_ERR_INVALID_ARGS,
                        "weights and out_weights must both be given or both NULL");
        if (quant) {
            if (scales)
                return fail(EPDC_ERR_INVALID_ARGS, "scales must be NULL: dispatch produces them");
            if (!out_scales)
                return fail(EPDC_ERR_INVALID_ARGS,
                            "out_scales is required when dispatch quantizes");
        } else if (scales) {
            if (c.scale_row_bytes == 0)
                return fail(EPDC_ERR_INVALID_ARGS, "scales given but scale_row_bytes is 0");
            if (!out_scales)
                return fail(EPDC_ERR_INVALID_ARGS, "out_scales is required to carry scales");
        }
    }

    if (!aligned(input, 16) || !aligned(out, 16) || !aligned(weights, 4) ||
        !aligned(indices, 4) || !aligned(scales, 4) || !aligned(out_weights, 4) ||
        !aligned(out_scales, 4) || !aligned(out_indices, 4) || !aligned(recv_count, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/out must be 16-byte aligned, the other arrays 4-byte aligned");

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int n_pairs = num_tokens * c.topk;
    const int tiles = n_pairs > 0 ? (n_pairs + kRouteTile - 1) / kRouteTile : 1;

    RouteArgs ra = {};
    ra.indices = indices;
    ra.n_pairs = n_pairs;
    ra.num_experts = c.num_experts;
    ra.num_ranks = c.num_ranks;
    ra.key_bits = op->key_bits;
    ra.topk = c.topk;
    ra.key_div = 0;
    ra.tiles = tiles;
    ra.tile_table = op->i32(op->lay.tile_table);
    ra.rank_in_tile = op->i32(op->lay.rank_in_tile);
    ra.expert_off = op->i32(op->lay.expert_off);
    ra.rank_off = op->i32(op->lay.rank_off);
    ra.recv_count = dedup ? op->i32(op->lay.pair_recv) : recv_count;
    ra.ctrl = op->ctrl();
    const size_t lds = sizeof(int32_t) * (size_t)route_lds_ints(c.num_experts);
    epdc_status s = EPDC_SUCCESS;
    bool inline_route = false;
    // A small tile table is scanned by every scatter block instead of by the
    // last rank block, while all blocks together read at most
    // kFusedScanMaxReads entries: for 32 tiles x 256 experts over the 1024
    // blocks of the bf16 copy at 4096 tokens the dispatch phase measured
    // 109.5 us against 112.5-112.9 us with the last-block scan; the same
    // table over the 7168 blocks of the FP8 scatter cost 9-23 us more than
    // scanning it once.
    bool fused_scan = false;
    if (!dedup && tiles > 1 && tiles <= 8 * kScanMaxLoads &&
        (int64_t)tiles * c.num_experts <= kFusedScanMaxEntries) {
        // the per-block scan costs each block a few us of latency: only
        // worth it while the scatter has few blocks
        const int in_vecs = c.quant == EPDC_QUANT_NONE
                                ? (c.input_kind == EPDC_IN_RAW ? c.raw_row_bytes / 16 : c.hidden / 8)
                                : c.hidden / 8;
        const ScatterPlan plan = plan_scatter(c.quant, num_tokens, in_vecs, false);
        const int64_t waves = (int64_t)num_tokens * plan.segs;
        const int wpb = waves_per_block(waves);
        const int64_t blocks = (waves + wpb - 1) / wpb;
        fused_scan = blocks * tiles * c.num_experts <= kFusedScanMaxReads;
    }
    const int tiles_pad8 = (tiles + 7) & ~7;
    ra.tile_cnt16 = fused_scan ? reinterpret_cast<uint16_t *>(op->ws + op->lay.tile_cnt16) : nullptr;
    ra.tiles_pad8 = tiles_pad8;
    // Otherwise, with several tiles, the last rank block to finish scans the
    // table (k_route_rank, ticket_word): no second launch.
    ra.ticket_word = !fused_scan && tiles > 1 ? kCtrlTicket0 : 0;
    if (dedup) {
        // the unit level: keys = destination ranks of the pairs that open a
        // unit; its offsets are both the expert and the rank offsets (one key
        // per rank), and its counts are the caller's recv_count
        RouteArgs rb = ra;
        rb.num_experts = c.num_ranks;
        rb.key_bits = op->unit_key_bits;
        rb.key_div = c.num_experts / c.num_ranks;
        rb.tile_table = op->i32(op->lay.unit_table);
        rb.rank_in_tile = op->i32(op->lay.unit_rank_in_tile);
        rb.expert_off = op->i32(op->lay.unit_off);
        rb.rank_off = op->i32(op->lay.unit_off);
        rb.recv_count = recv_count;
        rb.ticket_word = tiles > 1 ? kCtrlTicket1 : 0;
        if (tiles == 1) {
            s = launch(op, st, EPDC_KERNEL_ROUTE, [&] {
                k_route_rank2<true><<<dim3(1, 2), kRouteThreads, lds, st>>>(ra, rb);
            });
        } else {
            s = launch(op, st, EPDC_KERNEL_ROUTE, [&] {
                k_route_rank2<false><<<dim3(tiles, 2), kRouteThreads, lds, st>>>(ra, rb);
            });
        }
    } else {
        // One tile with tokens: the scatter launch below routes by itself.
        inline_route = tiles == 1 && num_tokens > 0;
        if (inline_route) {
            // no route launch
        } else if (tiles == 1) {
            s = launch(op, st, EPDC_KERNEL_ROUTE, [&] {
                k_route_rank<true><<<1, kRouteThreads, lds, st>>>(ra);
            });
        } else {
            s = launch(op, st, EPDC_KERNEL_ROUTE, [&] {
                k_route_rank<false><<<tiles, kRouteThreads, lds, st>>>(ra);
            });
        }
    }
    if (s != EPDC_SUCCESS)
        return s;

    if (num_tokens == 0) {
        op->routed = true;
        op->units_routed = dedup;
        op->last_tokens = 0;
        return ok();
    }

    ScatterArgs sa = {};
    sa.num_tokens = num_tokens;
    sa.n_pairs = n_pairs;
    sa.topk = c.topk;
    sa.num_experts = c.num_experts;
    sa.hidden = c.hidden;
    sa.indices = indices;
    sa.tile_table = ra.tile_table;
    sa.rank_in_tile = ra.rank_in_tile;
    sa.slot_of = op->i32(op->lay.slot_of);
    sa.src_pos = op->i32(op->lay.src_pos);
    sa.input = static_cast<const uint8_t *>(input);
    sa.in_row_vecs = c.input_kind == EPDC_IN_RAW ? c.raw_row_bytes / 16 : c.hidden / 8;
    sa.out = static_cast<uint8_t *>(out);
    sa.weights = weights;
    sa.out_weights = out_weights;
    sa.out_indices = out_indices;
    sa.scales = quant ? nullptr : static_cast<const uint8_t *>(scales);
    sa.out_scales = static_cast<uint8_t *>(out_scales);
    sa.scale_words = c.scale_row_bytes / 4;
    sa.ctrl = op->ctrl();
    sa.key_bits = op->key_bits;
    sa.num_ranks = c.num_ranks;
    sa.expert_off = ra.expert_off;
    sa.rank_off = ra.rank_off;
    sa.recv_count = recv_count;
    if (dedup) {
        sa.key_div = c.num_experts / c.num_ranks;
        sa.unit_table = op->i32(op->lay.unit_table);
        sa.unit_rank_in_tile = op->i32(op->lay.unit_rank_in_tile);
        sa.unit_of = op->i32(op->lay.unit_of);
        sa.unit_src = op->i32(op->lay.unit_src);
        sa.unit_rows_max = num_tokens * units_per_token(c);
    }

    sa.tiles = tiles;
    sa.tile_cnt16 = ra.tile_cnt16;
    sa.tiles_pad8 = tiles_pad8;
    sa.xcd_order = inline_route && one_tile_xcd_order(n_pairs);
    s = launch_scatter(op, st, sa,
                       dedup ? kRouteUnits
                             : (inline_route ? kRouteInline
                                             : (fused_scan ? kRouteTableScan : kRouteTable)),
                       dedup ? dedup_local_seg_vecs(c, num_tokens) : 0);
    if (s != EPDC_SUCCESS)
        return s;
    op->routed = true;
    op->units_routed = dedup;
    op->last_tokens = num_tokens;
    return ok();
}

}  // namespace

extern "C" {

epdc_status epdc_dispatch(epdc_op *op, void *stream, int32_t num_tokens, const void *input,
                          const float *weights, const void *scales, const int32_t *indices,
                          void *out, float *out_weights, void *out_scales, int32_t *out_indices,
                          int32_t *recv_count)
{
    return dispatch_impl(op, stream, num_tokens, input, weights, scales, indices, out,
                         out_weights, out_scales, out_indices, recv_count, false);
}

epdc_status epdc_dispatch_dedup(epdc_op *op, void *stream, int32_t num_tokens, const void *input,
                                const float *weights, const void *scales, const int32_t *indices,
                                void *out, float *out_weights, void *out_scales,
                                int32_t *out_indices, int32_t *recv_count)
{
    return dispatch_impl(op, stream, num_tokens, input, weights, scales, indices, out,
                         out_weights, out_scales, out_indices, recv_count, true);
}

epdc_status epdc_get_unit_routing(epdc_op *op, const int32_t **unit_off, const int32_t **unit_of,
                                  const int32_t **unit_src)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->units_routed)
        return fail(EPDC_ERR_BAD_STATE, "no rank-deduplicated dispatch recorded");
    if (unit_off)
        *unit_off = op->i32(op->lay.unit_off);
    if (unit_of)
        *unit_of = op->i32(op->lay.unit_of);
    if (unit_src)
        *unit_src = op->i32(op->lay.unit_src);
    return ok();
}

epdc_status epdc_units_to_experts(epdc_op *op, void *stream, const void *input,
                                  const float *in_weights, const void *in_scales,
                                  const int32_t *in_indices, void *out, float *out_weights,
                                  void *out_scales, int32_t *out_indices)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->units_routed)
        return fail(EPDC_ERR_BAD_STATE, "the conversion needs a rank-deduplicated dispatch first");
    const epdc_config &c = op->cfg;
    const int T = op->last_tokens;
    if (T == 0)
        return ok();
    if (!input || !out)
        return fail(EPDC_ERR_INVALID_ARGS, "input and out are required");
    if ((in_weights == nullptr) != (out_weights == nullptr) ||
        (in_scales == nullptr) != (out_scales == nullptr) ||
        (in_indices == nullptr) != (out_indices == nullptr))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "each carried array needs both its input and its output, or neither");
    size_t payload, scale_bytes;
    row_bytes_for(c, &payload, &scale_bytes);
    if (in_scales && (scale_bytes == 0 || scale_bytes % 4 != 0))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "scale rows of %zu bytes cannot be converted (need a positive multiple of 4)",
                    scale_bytes);
    if (!aligned(input, 16) || !aligned(out, 16) || !aligned(in_weights, 4) ||
        !aligned(in_scales, 4) || !aligned(in_indices, 4) || !aligned(out_weights, 4) ||
        !aligned(out_scales, 4) || !aligned(out_indices, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/out must be 16-byte aligned, the other arrays 4-byte aligned");

    ScatterArgs sa = {};
    sa.num_tokens = T * units_per_token(c);  // the grid covers the unit capacity
    sa.row_count = op->i32(op->lay.unit_off) + c.num_ranks;
    sa.n_pairs = T * c.topk;
    sa.topk = c.topk;
    sa.num_experts = c.num_experts;
    sa.hidden = c.hidden;
    sa.input = static_cast<const uint8_t *>(input);
    sa.in_row_vecs = (int)(payload / 16);
    sa.out = static_cast<uint8_t *>(out);
    sa.weights = in_weights;
    sa.out_weights = out_weights;
    sa.indices = in_indices;
    sa.out_indices = out_indices;
    sa.scales = static_cast<const uint8_t *>(in_scales);
    sa.out_scales = static_cast<uint8_t *>(out_scales);
    sa.scale_words = in_scales ? (int)(scale_bytes / 4) : 0;
    sa.slot_of = op->i32(op->lay.slot_of);
    sa.unit_of = op->i32(op->lay.unit_of);
    sa.unit_src = op->i32(op->lay.unit_src);
    sa.num_src_tokens = T;
    sa.num_ranks = c.num_ranks;
    sa.ctrl = op->ctrl();
    const epdc_status s = launch_scatter(op, static_cast<hipStream_t>(stream), sa, kRouteConvert,
                                         dedup_local_seg_vecs(c, T));
    return s == EPDC_SUCCESS ? ok() : s;
}

epdc_status epdc_experts_to_units(epdc_op *op, void *stream, const void *input,
                                  const float *weights, void *output)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->units_routed)
        return fail(EPDC_ERR_BAD_STATE, "the conversion needs a rank-deduplicated dispatch first");
    const epdc_config &c = op->cfg;
    const int T = op->last_tokens;
    if (T == 0)
        return ok();
    if (!input || !output)
        return fail(EPDC_ERR_INVALID_ARGS, "input and output are required");
    if (!aligned(input, 16) || !aligned(output, 16) || !aligned(weights, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/output must be 16-byte aligned, weights 4-byte aligned");
    CombineArgs ca = {};
    ca.slot_of = op->i32(op->lay.slot_of);
    ca.input = static_cast<const uint8_t *>(input);
    ca.weights = weights;
    ca.output = static_cast<uint8_t *>(output);
    ca.unit_of = op->i32(op->lay.unit_of);
    ca.unit_src = op->i32(op->lay.unit_src);
    ca.row_count = op->i32(op->lay.unit_off) + c.num_ranks;
    ca.n_pairs = T * c.topk;
    ca.num_src_tokens = T;
    const epdc_status s = launch_combine_mode<kCombineUnitsIn>(
        op, static_cast<hipStream_t>(stream), EPDC_KERNEL_EXPERTS_TO_UNITS, ca,
        (int64_t)T * units_per_token(c), dedup_local_seg_vecs(c, T));
    return s == EPDC_SUCCESS ? ok() : s;
}

epdc_status epdc_combine_units(epdc_op *op, void *stream, const void *input,
                               const float *unit_weights, void *output, float *out_weights)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->units_routed)
        return fail(EPDC_ERR_BAD_STATE, "combine_units needs a rank-deduplicated dispatch first");
    const epdc_config &c = op->cfg;
    const int T = op->last_tokens;
    if (T == 0)
        return ok();
    if (!input || !output)
        return fail(EPDC_ERR_INVALID_ARGS, "input and output are required");
    if (!aligned(input, 16) || !aligned(output, 16) || !aligned(unit_weights, 4) ||
        !aligned(out_weights, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/output must be 16-byte aligned, weights 4-byte aligned");
    CombineArgs ca = {};
    ca.input = static_cast<const uint8_t *>(input);
    ca.weights = unit_weights;
    ca.output = static_cast<uint8_t *>(output);
    ca.out_weights = out_weights;
    ca.unit_of = op->i32(op->lay.unit_of);
    ca.in_rows_max = T * units_per_token(c);
    const epdc_status s = launch_combine_mode<kCombineUnitsOut>(
        op, static_cast<hipStream_t>(stream), EPDC_KERNEL_COMBINE_UNITS, ca, T,
        dedup_local_seg_vecs(c, T));
    return s == EPDC_SUCCESS ? ok() : s;
}

epdc_status epdc_combine(epdc_op *op, void *stream, const void *input, const float *weights,
                         const int32_t *indices, void *output, float *out_weights)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->routed)
        return fail(EPDC_ERR_BAD_STATE, "combine needs a dispatch first (none since create/reset)");
    const epdc_config &c = op->cfg;
    const int T = op->last_tokens;
    if (T == 0)
        return ok();
    if (!input || !output)
        return fail(EPDC_ERR_INVALID_ARGS, "input and output are required");
    if (!aligned(input, 16) || !aligned(output, 16) || !aligned(weights, 4) ||
        !aligned(out_weights, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/output must be 16-byte aligned, weights 4-byte aligned");

    // the op keeps the routing of the last dispatch; indices are only checked
    epdc_status s = check_combine_indices(op, static_cast<hipStream_t>(stream), indices);
    if (s != EPDC_SUCCESS)
        return s;
    CombineArgs ca = {};
    ca.slot_of = op->i32(op->lay.slot_of);
    ca.input = static_cast<const uint8_t *>(input);
    ca.weights = weights;
    ca.output = static_cast<uint8_t *>(output);
    ca.out_weights = out_weights;
    ca.xcd_order = one_tile_xcd_order((int64_t)T * c.topk);
    ca.recent_input = op->combine_hint == EPDC_COMBINE_INPUT_RECENT;
    const int stage_rows = combine_stage_rows(c, ca);
    size_t lds_reserve = 0;  // unused LDS that caps the blocks per CU
    if (!ca.xcd_order && ca.recent_input)
        lds_reserve = kCombineRecentLdsReserve;
    else if (!ca.xcd_order && (int64_t)T * c.topk * c.hidden * 2 >= kCombineFewWavesBytes)
        lds_reserve = kCombineLdsReserve;
    if (stage_rows > 0)
        s = launch_combine_staged_mode(op, static_cast<hipStream_t>(stream), ca, T, stage_rows);
    else
        s = launch_combine_mode<kCombinePairs>(op, static_cast<hipStream_t>(stream),
                                               EPDC_KERNEL_COMBINE, ca, T, 0, lds_reserve);
    return s == EPDC_SUCCESS ? ok() : s;
}

epdc_status epdc_combine_scatter(epdc_op *op, void *stream, const void *input,
                                 const float *weights, const int32_t *indices, float *staging,
                                 void *output, float *out_weights)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->routed)
        return fail(EPDC_ERR_BAD_STATE, "combine needs a dispatch first (none since create/reset)");
    const epdc_config &c = op->cfg;
    const int T = op->last_tokens;
    if (T == 0)
        return ok();
    if (!input || !staging || !output)
        return fail(EPDC_ERR_INVALID_ARGS, "input, staging and output are required");
    if (!aligned(input, 16) || !aligned(staging, 16) || !aligned(output, 16) ||
        !aligned(weights, 4) || !aligned(out_weights, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/staging/output must be 16-byte aligned, weights 4-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the op keeps the routing of the last dispatch; indices are only checked
    epdc_status s = check_combine_indices(op, st, indices);
    if (s != EPDC_SUCCESS)
        return s;
    constexpr int CH = kCombineSeg;
    PushArgs pa = {};
    pa.rows = T * c.topk;
    pa.row_count = op->i32(op->lay.expert_off) + c.num_experts;
    pa.topk = c.topk;
    pa.row_vecs = c.hidden / 8;
    pa.segs = (pa.row_vecs + kWave * CH - 1) / (kWave * CH);
    pa.n_pairs = T * c.topk;
    pa.src_pos = op->i32(op->lay.src_pos);
    pa.slot_of = op->i32(op->lay.slot_of);
    pa.input = static_cast<const uint8_t *>(input);
    pa.weights = weights;
    pa.staging = staging;
    pa.output = static_cast<uint8_t *>(output);
    pa.out_weights = out_weights;
    pa.num_tokens = T;
    pa.cached_stores = (int64_t)pa.n_pairs * c.hidden * 4 <= kL2ResidentBytes;
    int grid, block;
    s = grid_for_waves((int64_t)pa.rows * pa.segs, &grid, &block);
    if (s == EPDC_SUCCESS)
        s = launch(op, st, EPDC_KERNEL_COMBINE_PUSH,
                   [&] { k_combine_push<CH><<<grid, block, 0, st>>>(pa); });
    if (s == EPDC_SUCCESS)
        s = grid_for_waves((int64_t)T * pa.segs, &grid, &block);
    if (s == EPDC_SUCCESS)
        s = launch(op, st, EPDC_KERNEL_COMBINE_REDUCE, [&] {
            switch (c.topk) {
            case 1: k_combine_reduce<1, CH><<<grid, block, 0, st>>>(pa); break;
            case 2: k_combine_reduce<2, CH><<<grid, block, 0, st>>>(pa); break;
            case 4: k_combine_reduce<4, CH><<<grid, block, 0, st>>>(pa); break;
            case 6: k_combine_reduce<6, CH><<<grid, block, 0, st>>>(pa); break;
            case 8: k_combine_reduce<8, CH><<<grid, block, 0, st>>>(pa); break;
            default: k_combine_reduce<0, CH><<<grid, block, 0, st>>>(pa); break;
            }
        });
    return s == EPDC_SUCCESS ? ok() : s;
}

epdc_status epdc_dispatch_replay(epdc_op *op, void *stream, const void *input,
                                 const float *weights, const void *scales, void *out,
                                 float *out_weights, void *out_scales)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->routed)
        return fail(EPDC_ERR_BAD_STATE, "routing replay needs a dispatch first");
    const epdc_config &c = op->cfg;
    const int T = op->last_tokens;
    if (T == 0)
        return ok();
    if (!input || !out)
        return fail(EPDC_ERR_INVALID_ARGS, "input and out are required");
    if ((weights == nullptr) != (out_weights == nullptr))
        return fail(EPDC_ERR_INVALID_ARGS, "weights and out_weights must both be given or both NULL");
    const bool quant = c.quant != EPDC_QUANT_NONE;
    if (quant && (scales || !out_scales))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "quantizing replay produces the scales: scales NULL, out_scales required");
    if (!quant && scales && (c.scale_row_bytes == 0 || !out_scales))
        return fail(EPDC_ERR_INVALID_ARGS, "carried scales need scale_row_bytes and out_scales");
    if (!aligned(input, 16) || !aligned(out, 16) || !aligned(weights, 4) || !aligned(scales, 4) ||
        !aligned(out_weights, 4) || !aligned(out_scales, 4))
        return fail(EPDC_ERR_INVALID_ARGS,
                    "input/out must be 16-byte aligned, the other arrays 4-byte aligned");

    ScatterArgs sa = {};
    sa.num_tokens = T;
    sa.n_pairs = T * c.topk;
    sa.topk = c.topk;
    sa.num_experts = c.num_experts;
    sa.hidden = c.hidden;
    sa.slot_of = op->i32(op->lay.slot_of);
    sa.input = static_cast<const uint8_t *>(input);
    sa.in_row_vecs = c.input_kind == EPDC_IN_RAW ? c.raw_row_bytes / 16 : c.hidden / 8;
    sa.out = static_cast<uint8_t *>(out);
    sa.weights = weights;
    sa.out_weights = out_weights;
    sa.out_indices = nullptr;  // the recorded dispatch already carried the indices
    sa.scales = quant ? nullptr : static_cast<const uint8_t *>(scales);
    sa.out_scales = static_cast<uint8_t *>(out_scales);
    sa.scale_words = c.scale_row_bytes / 4;
    sa.ctrl = op->ctrl();
    int mode = kRouteReplay;
    int local_seg_vecs = 0;
    if (op->units_routed) {  // replay the unit rows of a rank-deduplicated dispatch
        sa.unit_of = op->i32(op->lay.unit_of);
        sa.unit_rows_max = T * units_per_token(c);
        mode = kRouteUnitsReplay;
        local_seg_vecs = dedup_local_seg_vecs(c, T);
    } else {
        sa.xcd_order = one_tile_xcd_order(sa.n_pairs);
    }
    epdc_status s =
        launch_scatter(op, static_cast<hipStream_t>(stream), sa, mode, local_seg_vecs);
    return s == EPDC_SUCCESS ? ok() : s;
}

epdc_status epdc_dispatch_send(epdc_op *op, void *stream, int32_t num_tokens, const void *input,
                               const float *weights, const void *scales, const int32_t *indices,
                               void *out, float *out_weights, void *out_scales,
                               int32_t *out_indices, int32_t *recv_count)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    epdc_status s = send_event(&op->ev_dispatch);
    if (s != EPDC_SUCCESS)
        return s;
    s = epdc_dispatch(op, stream, num_tokens, input, weights, scales, indices, out, out_weights,
                      out_scales, out_indices, recv_count);
    if (s != EPDC_SUCCESS)
        return s;
    const hipError_t e = hipEventRecord(op->ev_dispatch, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "hipEventRecord: %s", hipGetErrorString(e));
    op->dispatch_sent = true;
    return ok();
}

epdc_status epdc_dispatch_recv(epdc_op *op, void *stream)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->dispatch_sent)
        return fail(EPDC_ERR_BAD_STATE, "dispatch_recv without a dispatch_send");
    const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), op->ev_dispatch, 0);
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
    op->dispatch_sent = false;
    return ok();
}

epdc_status epdc_combine_send(epdc_op *op, void *stream, const void *input, const float *weights,
                              const int32_t *indices, void *output, float *out_weights)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    epdc_status s = send_event(&op->ev_combine);
    if (s != EPDC_SUCCESS)
        return s;
    s = epdc_combine(op, stream, input, weights, indices, output, out_weights);
    if (s != EPDC_SUCCESS)
        return s;
    const hipError_t e = hipEventRecord(op->ev_combine, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "hipEventRecord: %s", hipGetErrorString(e));
    op->combine_sent = true;
    return ok();
}

epdc_status epdc_combine_recv(epdc_op *op, void *stream)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->combine_sent)
        return fail(EPDC_ERR_BAD_STATE, "combine_recv without a combine_send");
    const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), op->ev_combine, 0);
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
    op->combine_sent = false;
    return ok();
}

epdc_status epdc_get_dispatch_src_token_pos(epdc_op *op, const int32_t **dev_ptr, int32_t *count)
{
    if (!op || !dev_ptr || !count)
        return fail(EPDC_ERR_INVALID_ARGS, "NULL argument");
    if (!op->routed)
        return fail(EPDC_ERR_BAD_STATE, "no dispatch recorded");
    *dev_ptr = op->i32(op->lay.src_pos);
    *count = op->last_tokens * op->cfg.topk;
    return ok();
}

epdc_status epdc_get_routing(epdc_op *op, const int32_t **expert_off, const int32_t **rank_off,
                             const int32_t **slot_of)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (!op->routed)
        return fail(EPDC_ERR_BAD_STATE, "no dispatch recorded");
    if (expert_off)
        *expert_off = op->i32(op->lay.expert_off);
    if (rank_off)
        *rank_off = op->i32(op->lay.rank_off);
    if (slot_of)
        *slot_of = op->i32(op->lay.slot_of);
    return ok();
}

epdc_status epdc_get_offsets(epdc_op *op, const int32_t **expert_off, const int32_t **rank_off)
{
    return epdc_get_routing(op, expert_off, rank_off, nullptr);
}

epdc_status epdc_set_debug(epdc_op *op, int32_t flags)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (flags & ~EPDC_DEBUG_CHECK_INDICES)
        return fail(EPDC_ERR_INVALID_ARGS, "unknown debug flags 0x%x", (unsigned)flags);
    op->debug = flags;
    return ok();
}

epdc_status epdc_set_combine_hint(epdc_op *op, int32_t hint)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    if (hint != EPDC_COMBINE_INPUT_COLD && hint != EPDC_COMBINE_INPUT_RECENT)
        return fail(EPDC_ERR_INVALID_ARGS, "unknown combine hint %d", hint);
    op->combine_hint = hint;
    return ok();
}

epdc_status epdc_get_device_error(epdc_op *op, void *stream, int32_t *flag)
{
    if (!op || !flag)
        return fail(EPDC_ERR_INVALID_ARGS, "NULL argument");
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t v = 0;
    hipError_t e = hipStreamSynchronize(st);
    if (e == hipSuccess)
        e = hipMemcpy(&v, op->ctrl() + kCtrlError, sizeof v, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        e = hipMemset(op->ctrl() + kCtrlError, 0, sizeof v);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "reading the device error flag: %s", hipGetErrorString(e));
    *flag = (int32_t)v;
    return ok();
}

epdc_status epdc_reset(epdc_op *op)
{
    if (!op)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL");
    op->routed = false;
    op->units_routed = false;
    op->last_tokens = 0;
    op->dispatch_sent = op->combine_sent = false;
    return ok();
}

const char *epdc_last_error(void) { return g_last_error.c_str(); }

const char *epdc_kernel_name(int32_t kernel_id)
{
    if (kernel_id < 0 || kernel_id >= EPDC_NUM_KERNELS)
        return nullptr;
    return kKernelNames[kernel_id];
}

epdc_status epdc_profile_begin(epdc_op *op, int32_t max_launches)
{
    if (!op || max_launches <= 0)
        return fail(EPDC_ERR_INVALID_ARGS, "op is NULL or max_launches <= 0");
    for (hipEvent_t ev : op->ev)
        (void)hipEventDestroy(ev);
    op->ev.assign(2 * (size_t)max_launches, nullptr);
    op->ev_kernel.assign((size_t)max_launches, -1);
    for (auto &ev : op->ev) {
        // no system-scope release at the timestamps: the write-back it does
        // would be timed as part of the kernel it follows
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
        if (e != hipSuccess) {
            op->profiling = false;
            return fail(EPDC_ERR_GPU_OP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
        }
    }
    op->ev_cap = max_launches;
    op->ev_used = 0;
    op->profiling = true;
    return ok();
}

epdc_status epdc_profile_end(epdc_op *op, float *ms, int32_t *launches)
{
    if (!op || !ms || !launches)
        return fail(EPDC_ERR_INVALID_ARGS, "NULL argument");
    if (!op->profiling)
        return fail(EPDC_ERR_BAD_STATE, "profiling was not started");
    for (int k = 0; k < EPDC_NUM_KERNELS; ++k) {
        ms[k] = 0.0f;
        launches[k] = 0;
    }
    epdc_status st = EPDC_SUCCESS;
    if (op->ev_used > 0) {
        hipError_t e = hipEventSynchronize(op->ev[2 * op->ev_used - 1]);
        for (int i = 0; e == hipSuccess && i < op->ev_used; ++i) {
            float t = 0.0f;
            e = hipEventElapsedTime(&t, op->ev[2 * i], op->ev[2 * i + 1]);
            ms[op->ev_kernel[i]] += t;
            launches[op->ev_kernel[i]] += 1;
        }
        if (e != hipSuccess)
            st = fail(EPDC_ERR_GPU_OP, "reading timing events: %s", hipGetErrorString(e));
    }
    for (hipEvent_t ev : op->ev)
        (void)hipEventDestroy(ev);
    op->ev.clear();
    op->ev_kernel.clear();
    op->ev_cap = op->ev_used = 0;
    op->profiling = false;
    return st == EPDC_SUCCESS ? ok() : st;
}

}  // extern "C"
