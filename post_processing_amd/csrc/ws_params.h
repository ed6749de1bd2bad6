// ws_params.h -- kernel parameters from a lane configuration, its plan and
// the buffers the kernels read and write.  Host code shared by the lane
// runtime and the allocation-free entry point; internal to the library.
#pragma once

#include "ws.h"
#include "ws_kernels.h"
#include "ws_plan.h"

namespace ws {

// Preprocess parameters: the frame(s) at `in`, the tensor at `tensor`.
inline void fill_pre_params(const ws_lane_config& c, const Plan& P, const uint8_t* in,
                            void* tensor, PreParams* out) {
    PreParams& q = *out;
    q = PreParams{};
    q.src = in;
    q.dst = tensor;
    q.frame_bytes = (int64_t)P.frame_bytes;
    q.total_bytes = (int64_t)P.input_bytes;
    q.src_w = c.src_w;
    q.src_h = c.src_h;
    q.dst_w = c.dst_w;
    q.dst_h = c.dst_h;
    q.left = P.region.left;
    q.top = P.region.top;
    q.reg_w = P.region.w;
    q.reg_h = P.region.h;
    q.inv_den_x = (float)(1.0 / (2.0 * P.region.w));
    q.inv_den_y = (float)(1.0 / (2.0 * P.region.h));
    q.magic_x = (uint32_t)((1ull << 32) / (2ull * (uint64_t)P.region.w) + 1);
    q.magic_y = (uint32_t)((1ull << 32) / (2ull * (uint64_t)P.region.h) + 1);
    q.span_lo = (int32_t)P.span_lo;
    q.slot_chunks = P.slot_bytes / 16;
    q.pixels_per_thread = P.pixels_per_thread;
    q.streaming = P.streaming ? 1 : 0;
    q.threads_per_row = P.threads_per_row;
    q.rows_per_group = P.rows_per_group;
    q.groups_per_frame = P.groups_per_frame;
    q.vec = (c.dst_w % P.pixels_per_thread) == 0;
    q.dtype = c.tensor_dtype;
    for (int i = 0; i < 3; ++i)   // output plane i reads byte i (RGB) or byte 2 - i (BGR)
        q.shift[i] = 8u * (uint32_t)(c.channel_order == WS_CHANNELS_BGR ? 2 - i : i);
    for (int i = 0; i < 3; ++i) {
        q.a[i] = (float)(1.0 / (255.0 * c.std[i]));
        q.b[i] = (float)(-c.mean[i] / c.std[i]);
        q.padv[i] = (float)((c.pad_value / 255.0 - c.mean[i]) / c.std[i]);
    }
}

// Top-K parameters: scores at `scores`, the partial lists at `partials`
// (room for P.topk_groups * k keys when P.topk_groups > 1), the K result
// pairs at `result` (device-visible).
inline void fill_topk_params(const ws_lane_config& c, const Plan& P, const float* scores,
                             uint64_t* partials, uint2* result, TopkParams* out) {
    TopkParams& t = *out;
    t = TopkParams{};
    t.scores = scores;
    t.n = c.num_scores;
    t.k = c.k;
    t.chunk = P.topk_chunk;
    t.groups = P.topk_groups;
    t.waves = P.topk_waves;
    t.keys_per_lane = P.topk_keys_per_lane;
    t.partials = partials;
    t.result = result;
}

}  // namespace ws
