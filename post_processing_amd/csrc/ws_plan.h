// ws_plan.h -- host-side planning for a pipeline lane: configuration checks,
// exact sampling taps, launch geometry and the lane state machine.
//
// Plain C++17 with no HIP dependency, so the same code the library runs can
// be compiled and tested on a host without a GPU.
//
// Sampling rule (WarpStream TRT article, fused-preprocess passage: every
// destination pixel takes a centre-aligned source coordinate and its four
// bilinear neighbours; half-pixel centres, align_corners=false, edge clamp):
//     src(d) = (d + 1/2) * S / R - 1/2 = ((2d + 1) S - R) / (2R)
// clamped below at 0, i0 = floor(src), w = src - i0, i1 = min(i0 + 1, S - 1).
// It is evaluated here in 64-bit integers, so the tap indices are exact and
// each weight is the exact fraction rounded once to FP32.  (A float
// evaluation of (d + 0.5) * scale - 0.5 is off by up to ~1e-4 px at
// 1080 -> 224, which alone moves outputs by ~5e-4.)
//
// Letterbox (yolo.cu README: the raw frame is letterboxed on the GPU):
// r = min(Dw/W, Dh/H) as a fraction; region Rw = floor(W r + 1/2),
// Rh = floor(H r + 1/2), each at least 1; left = floor((Dw - Rw) / 2),
// top = floor((Dh - Rh) / 2); the frame is resampled onto the region with the
// rule above per axis and every other cell holds the pad byte value.
#pragma once

#include <cmath>
#include <cstddef>
#include <algorithm>
#include <cstdint>

#include "ws.h"

namespace ws {

// One sampling tap along an axis: the two source indices and the weight of
// the second.
struct Tap {
    int32_t i0;
    int32_t i1;
    float w;
};

struct Region {
    int32_t left, top, w, h;
};

// Exact tap for destination index d of an axis resampling S source samples
// onto R destination samples.
inline Tap axis_tap(int64_t S, int64_t R, int64_t d) {
    int64_t num = (2 * d + 1) * S - R;
    const int64_t den = 2 * R;
    if (num < 0) num = 0;
    const int64_t i0 = num / den;
    const int64_t rem = num - i0 * den;
    Tap t;
    t.i0 = (int32_t)i0;
    t.i1 = (int32_t)(i0 + 1 < S ? i0 + 1 : S - 1);
    t.w = (float)((double)rem / (double)den);
    return t;
}

inline Region letterbox_region(int64_t W, int64_t H, int64_t Dw, int64_t Dh) {
    // r = min(Dw/W, Dh/H); compare Dw*H against Dh*W to pick the binding axis.
    int64_t rn, rd;  // r = rn / rd
    if (Dw * H <= Dh * W) { rn = Dw; rd = W; } else { rn = Dh; rd = H; }
    // floor(X * rn / rd + 1/2) = floor((2 X rn + rd) / (2 rd))
    int64_t rw = (2 * W * rn + rd) / (2 * rd);
    int64_t rh = (2 * H * rn + rd) / (2 * rd);
    if (rw < 1) rw = 1;
    if (rh < 1) rh = 1;
    if (rw > Dw) rw = Dw;
    if (rh > Dh) rh = Dh;
    Region g;
    g.w = (int32_t)rw;
    g.h = (int32_t)rh;
    g.left = (int32_t)((Dw - rw) / 2);
    g.top = (int32_t)((Dh - rh) / 2);
    return g;
}

inline Region lane_region(const ws_lane_config& c) {
    if (c.resize_mode == WS_RESIZE_LETTERBOX)
        return letterbox_region(c.src_w, c.src_h, c.dst_w, c.dst_h);
    Region g;
    g.left = 0;
    g.top = 0;
    g.w = c.dst_w;
    g.h = c.dst_h;
    return g;
}

// ---------------------------------------------------------------------------
// Configuration checks.

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Detection anchors: cells of the stride-8, -16 and -32 grids over the
// network input (its sides must be multiples of 32).
constexpr int kDetStrides[3] = {8, 16, 32};

inline int64_t det_anchor_count(int64_t net_w, int64_t net_h) {
    int64_t a = 0;
    for (int s : kDetStrides) a += (net_w / s) * (net_h / s);
    return a;
}

inline int validate_detection(const ws_lane_config* c) {
    if (c->det_classes == 0) return c->det_head_dev ? WS_E_INVALID_ARG : WS_OK;
    if (c->det_classes < 0 || c->det_classes > WS_DET_MAX_CLASSES) return WS_E_INVALID_ARG;
    if (c->batch != 1) return WS_E_INVALID_ARG;          // one head per frame, batch-1 lanes
    if (c->dst_w % 32 != 0 || c->dst_h % 32 != 0) return WS_E_INVALID_ARG;
    if (det_anchor_count(c->dst_w, c->dst_h) > WS_DET_MAX_ANCHORS) return WS_E_INVALID_ARG;
    if (c->det_max_det < 1 || c->det_max_det > WS_DET_MAX_DET) return WS_E_INVALID_ARG;
    if (!(c->det_conf >= 0.0f && c->det_conf < 1.0f)) return WS_E_INVALID_ARG;
    if (!(c->det_iou >= 0.0f && c->det_iou <= 1.0f)) return WS_E_INVALID_ARG;
    if (c->det_agnostic != 0 && c->det_agnostic != 1) return WS_E_INVALID_ARG;
    if (c->det_reserved != 0) return WS_E_INVALID_ARG;
    if (!aligned16(c->det_head_dev)) return WS_E_INVALID_ARG;
    return WS_OK;
}

inline int validate_config(const ws_lane_config* c) {
    if (!c) return WS_E_INVALID_ARG;
    if (c->device < 0) return WS_E_INVALID_ARG;
    if (c->batch < 1 || c->batch > WS_MAX_BATCH) return WS_E_INVALID_ARG;
    if (c->src_w < 1 || c->src_h < 1 || c->dst_w < 1 || c->dst_h < 1) return WS_E_INVALID_ARG;
    if (c->src_w > WS_MAX_SIDE || c->src_h > WS_MAX_SIDE || c->dst_w > WS_MAX_SIDE ||
        c->dst_h > WS_MAX_SIDE)
        return WS_E_INVALID_ARG;
    if (c->resize_mode != WS_RESIZE_BILINEAR && c->resize_mode != WS_RESIZE_LETTERBOX)
        return WS_E_INVALID_ARG;
    if (c->input_mode != WS_INPUT_MAPPED_HOST && c->input_mode != WS_INPUT_DEVICE &&
        c->input_mode != WS_INPUT_COPY)
        return WS_E_INVALID_ARG;
    if (!(c->pad_value >= 0.0 && c->pad_value <= 255.0)) return WS_E_INVALID_ARG;
    for (int i = 0; i < 3; ++i) {
        if (!std::isfinite(c->mean[i])) return WS_E_INVALID_ARG;
        if (!(std::isfinite(c->std[i]) && c->std[i] > 0.0)) return WS_E_INVALID_ARG;
    }
    if (c->num_scores < 0) return WS_E_INVALID_ARG;
    if (c->num_scores > 0) {
        const int kmax = c->num_scores < WS_MAX_K ? c->num_scores : WS_MAX_K;
        if (c->k < 1 || c->k > kmax) return WS_E_INVALID_ARG;
    } else if (c->k != 0) {
        return WS_E_INVALID_ARG;
    }
    if (c->use_graph != 0 && c->use_graph != 1) return WS_E_INVALID_ARG;
    if (c->wait_mode != WS_WAIT_SPIN && c->wait_mode != WS_WAIT_BLOCK) return WS_E_INVALID_ARG;
    if (c->input_dev && c->input_mode != WS_INPUT_DEVICE) return WS_E_INVALID_ARG;
    if (!aligned16(c->input_dev) || !aligned16(c->scores_dev) || !aligned16(c->tensor_dev))
        return WS_E_INVALID_ARG;
    if (c->scores_dev && c->num_scores == 0) return WS_E_INVALID_ARG;
    if (c->rows_per_group < 0 || c->rows_per_group > 64) return WS_E_INVALID_ARG;
    if (c->topk_chunk < 0 || (c->topk_chunk % 1024) != 0) return WS_E_INVALID_ARG;
    if (c->num_scores > WS_MAX_SCORES) return WS_E_INVALID_ARG;
    if (c->pixels_per_thread != 0 && c->pixels_per_thread != 1 && c->pixels_per_thread != 2 &&
        c->pixels_per_thread != 4)
        return WS_E_INVALID_ARG;
    if (c->tensor_dtype != WS_DTYPE_F32 && c->tensor_dtype != WS_DTYPE_F16 &&
        c->tensor_dtype != WS_DTYPE_BF16)
        return WS_E_INVALID_ARG;
    if (c->channel_order != WS_CHANNELS_RGB && c->channel_order != WS_CHANNELS_BGR)
        return WS_E_INVALID_ARG;
    if (c->autotune != 0 && c->autotune != 1) return WS_E_INVALID_ARG;
    if (c->cache_policy != WS_CACHE_AUTO && c->cache_policy != WS_CACHE_KEEP &&
        c->cache_policy != WS_CACHE_STREAM)
        return WS_E_INVALID_ARG;
    if (c->reserved != 0) return WS_E_INVALID_ARG;
    return validate_detection(c);
}

// ---------------------------------------------------------------------------
// Launch geometry.

constexpr int kMaxPreBlock = 512;          // preprocess threads per workgroup (staged)
constexpr int kMaxGatherBlock = 1024;      // preprocess threads per workgroup (gather)
constexpr int kMaxLdsBytes = 156 * 1024;   // gfx950: 160 KiB LDS per workgroup, less static use
constexpr int kTopkBatch = 1024;           // scores one wave takes per round
constexpr int kTopkMaxWaves = 4;           // one wave per SIMD of a CU
constexpr int kTopkSingleGroupMax = 8192;  // up to here one workgroup, no hand-off
constexpr int kTopkLargeN = 196608;        // beyond: 8 Ki scores per workgroup
constexpr int kDetDecodeBlock = 64;        // detection decode: anchors per workgroup

struct Plan {
    Region region;
    // Source byte span [span_lo, span_lo + span) of each source row that the
    // region's horizontal taps touch.
    int64_t span_lo = 0, span = 0;
    int32_t slot_bytes = 0;        // LDS bytes per staged source row (16-multiple)
    int32_t pixels_per_thread = 1; // adjacent output columns per thread (1, 2, 4)
    bool streaming = false;        // gather kernel: non-temporal loads and stores
    int32_t threads_per_row = 0;   // ceil(dst_w / pixels_per_thread)
    int32_t rows_per_group = 1;
    int32_t pre_block = 64;
    int32_t pre_groups = 0;
    int32_t groups_per_frame = 0;
    int32_t lds_bytes = 0;
    // Top-K
    int32_t topk_groups = 0;
    int32_t topk_chunk = 0;
    int32_t topk_waves = 0;        // wave64s per Top-K workgroup
    int32_t topk_keys_per_lane = 0;// scores per lane per batch: 16, or 32 when a wave's share is larger
    // Sizes
    size_t frame_bytes = 0, input_bytes = 0, tensor_bytes = 0;
    // Detection (det_anchors == 0: no detection stage)
    int32_t det_anchors = 0;
    int32_t det_level_end[3] = {0, 0, 0};  // anchor index where each grid ends
    int32_t det_grid_w[3] = {0, 0, 0};     // cells per row of each grid
    int32_t det_decode_groups = 0;         // decode workgroups, 64 anchors each
    int32_t det_sort_cap = 0;              // power of two >= max(anchors, 64): keys sorted in LDS
    size_t det_head_bytes = 0;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int32_t lds_for_rows(int32_t rows, int32_t slot_bytes) {
    return 2 * rows * slot_bytes + 16;
}

// Returns WS_OK and fills *p, or WS_E_INVALID_ARG if the shape cannot be
// staged (a source row span larger than LDS allows).
inline int make_plan(const ws_lane_config& c, Plan* p) {
    p->region = lane_region(c);
    const Region& g = p->region;
    const int64_t W = c.src_w, H = c.src_h, Dw = c.dst_w, Dh = c.dst_h;

    // Pixels per thread: 1 by default, which runs as the gather kernel (each
    // thread reads its taps straight from global memory, no row staging).
    // Measured on MI355X it beat the LDS-staged kernels with 2 or 4 columns
    // per thread everywhere: one 1920x1080 frame 3.9 -> 2.5 us, a 640x640
    // letterbox 4.8 -> 4.3 us, 64 frames of 1280x720 27.3 -> 22.5 us, and
    // mapped host input 59.4 -> 55.8 us.  2 and 4 (staged) stay selectable.
    int32_t px = c.pixels_per_thread;
    if (px == 0) px = 1;
    p->pixels_per_thread = px;
    const bool staged = px > 1;   // only the staged kernels hold source rows in LDS

    // The byte span of a source row that the region's horizontal taps read.
    const Tap first = axis_tap(W, g.w, 0);
    const Tap last = axis_tap(W, g.w, g.w - 1);
    p->span_lo = 3 * (int64_t)first.i0;
    p->span = 3 * (int64_t)last.i1 + 3 - p->span_lo;
    // A staged row starts at its 16-byte-aligned address below the span, so it
    // needs up to 15 extra bytes in front.
    p->slot_bytes = staged ? (int32_t)(ceil_div(p->span + 15, 16) * 16) : 0;
    if (staged && lds_for_rows(1, p->slot_bytes) > kMaxLdsBytes) return WS_E_INVALID_ARG;

    p->threads_per_row = (int32_t)ceil_div(Dw, px);
    const int32_t q = p->threads_per_row;

    int32_t rows = c.rows_per_group;
    if (rows == 0) {
        // The gather kernel: one row per workgroup, the most workgroups in
        // flight (its threads walk a workgroup's rows one after another).
        // The staged kernels, measured on MI355X: one row, or two once the
        // tensor has 320+ rows (fewer, fuller groups), with tiny rows packed
        // so a workgroup holds at least one full wave.
        if (!staged) {
            rows = 1;
        } else {
            rows = (px == 4 || Dh < 320) ? 1 : 2;
            while (rows < Dh && (int64_t)(rows + 1) * q <= 64) ++rows;
            while (rows > 1 && lds_for_rows(rows, p->slot_bytes) > kMaxLdsBytes / 2) --rows;
        }
    }
    if (rows > Dh) rows = (int32_t)Dh;
    if (staged && lds_for_rows(rows, p->slot_bytes) > kMaxLdsBytes) return WS_E_INVALID_ARG;
    p->rows_per_group = rows;
    // The staged kernels spread a workgroup's rows over its threads (up to
    // 512).  The gather kernel gives each thread one column of all its rows,
    // with workgroups of up to 1024 threads, so a 640-wide row takes one pass.
    const int64_t threads = staged ? (int64_t)rows * q : q;
    // A batch of device-resident frames is streamed through once per launch:
    // non-temporal frame loads and tensor stores keep it from displacing what
    // the last-level cache holds (64 x 1280x720 -> 224, measured on MI355X:
    // 28.8 -> 25.4 us per launch with the batches evicted between launches,
    // 22.0 -> 22.3 us for the same batch replayed).  Single frames, whose
    // producer may just have written them and whose tensor the next stage
    // reads, keep ordinary loads and stores.
    p->streaming = !staged && c.input_mode == WS_INPUT_DEVICE &&
                      (c.cache_policy == WS_CACHE_STREAM ||
                       (c.cache_policy == WS_CACHE_AUTO && c.batch >= WS_STREAM_MIN_BATCH));
    const int64_t block_cap = staged ? kMaxPreBlock : kMaxGatherBlock;
    p->pre_block = (int32_t)std::min<int64_t>(block_cap, ceil_div(threads, 64) * 64);
    p->groups_per_frame = (int32_t)ceil_div(Dh, rows);
    const int64_t groups = (int64_t)c.batch * p->groups_per_frame;
    if (groups > 0x7fffffff) return WS_E_INVALID_ARG;
    p->pre_groups = (int32_t)groups;
    p->lds_bytes = staged ? lds_for_rows(rows, p->slot_bytes) : 0;

    if (c.num_scores > 0) {
        // Up to 8 Ki scores one workgroup does everything, so no merge kernel
        // is needed: up to 4 Ki its waves take one 1024-score batch each,
        // beyond that four waves take 2048 (32 per lane) in one round.  Past
        // 8 Ki, 4-wave workgroups of 4 Ki scores, or 8 Ki past 192 Ki scores
        // so that the merge kernel folds fewer lists.  (Measured on MI355X,
        // Top-K stage with the fold merge: 672,000 scores 9.4 us with 8 Ki
        // chunks, 11.0 with 16 Ki, 12.1 with 4 Ki; 262,144 scores 8.0 us with
        // 8 Ki, 8.4 with 4 Ki; 131,072 scores 7.6 us with 4 Ki, 8.7 with 8 Ki;
        // 65,536 scores 7.1 us with 4 Ki, 7.4 with 8 Ki;
        // 21,843 scores 6.9 us with 4 Ki, 9.1 with one workgroup; 8,192
        // scores 5.0 us with one workgroup, 6.6 with two.)
        int64_t chunk = c.topk_chunk;
        if (chunk == 0) {
            if (c.num_scores <= kTopkSingleGroupMax / 2)
                chunk = ceil_div(c.num_scores, kTopkBatch) * kTopkBatch;
            else if (c.num_scores <= kTopkSingleGroupMax)
                chunk = kTopkSingleGroupMax;
            else
                chunk = c.num_scores <= kTopkLargeN ? kTopkSingleGroupMax / 2 : kTopkSingleGroupMax;
        }
        p->topk_chunk = (int32_t)chunk;
        p->topk_waves = (int32_t)std::min<int64_t>(kTopkMaxWaves, chunk / kTopkBatch);
        p->topk_groups = (int32_t)ceil_div(c.num_scores, chunk);
        // A wave whose share is 2 Ki scores or more takes them 32 per lane
        // per batch: one selection pass instead of two.
        p->topk_keys_per_lane = chunk / p->topk_waves >= 2 * kTopkBatch ? 32 : 16;
    }

    if (c.det_classes > 0) {
        int32_t end = 0;
        for (int l = 0; l < 3; ++l) {
            const int s = kDetStrides[l];
            p->det_grid_w[l] = (int32_t)(Dw / s);
            end += (int32_t)((Dw / s) * (Dh / s));
            p->det_level_end[l] = end;
        }
        p->det_anchors = end;
        p->det_decode_groups = (int32_t)ceil_div(end, kDetDecodeBlock);
        int32_t cap = 64;
        while (cap < end) cap <<= 1;
        p->det_sort_cap = cap;
        p->det_head_bytes = (size_t)(4 * WS_DET_REG_MAX + c.det_classes) * (size_t)end * 4u;
    }

    p->frame_bytes = (size_t)W * (size_t)H * 3u;
    p->input_bytes = p->frame_bytes * (size_t)c.batch;
    p->tensor_bytes = (size_t)c.batch * 3u * (size_t)Dw * (size_t)Dh *
                      (c.tensor_dtype == WS_DTYPE_F32 ? 4u : 2u);
    return WS_OK;
}

// Keys of Top-K partial lists a plan needs: one sorted list of K keys per
// workgroup when the scores span several workgroups, else none.
inline int64_t topk_scratch_keys(const Plan& p, int32_t k) {
    return p.topk_groups > 1 ? (int64_t)p.topk_groups * k : 0;
}

// ---------------------------------------------------------------------------
// Lane state machine: READY --submit--> IN_FLIGHT --wait--> READY.
// A busy lane rejects a second submit (no hidden queue); a wait with nothing
// in flight is an error.  Destroy is legal in both states.

enum class LaneState : int { Ready = 0, InFlight = 1 };

inline int begin_submit(LaneState s) { return s == LaneState::Ready ? WS_OK : WS_E_STATE; }
inline int begin_wait(LaneState s) { return s == LaneState::InFlight ? WS_OK : WS_E_STATE; }

inline const char* status_str(int s) {
    switch (s) {
        case WS_OK: return "WS_OK";
        case WS_E_INVALID_ARG: return "WS_E_INVALID_ARG";
        case WS_E_STATE: return "WS_E_STATE";
        case WS_E_NO_MAP_HOST: return "WS_E_NO_MAP_HOST";
        case WS_E_OOM: return "WS_E_OOM";
        case WS_E_CAPTURE: return "WS_E_CAPTURE";
        case WS_E_HIP: return "WS_E_HIP";
        case WS_E_NO_DEVICE: return "WS_E_NO_DEVICE";
        default: return "WS_E_UNKNOWN";
    }
}

}  // namespace ws
