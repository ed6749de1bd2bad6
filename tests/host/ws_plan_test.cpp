// Host-only driver for the lane planning code (ws_plan.h): compiled with g++
// and no HIP by tests/test_host_logic.py.
//   ws_plan_test taps S R           -> "i0 i1 w" per destination index
//   ws_plan_test letterbox W H Dw Dh -> "left top w h"
//   ws_plan_test plan <cfg fields>   -> launch geometry
//   ws_plan_test selftest            -> config validation + state machine checks
//   ws_plan_test layout              -> "struct field offset" for the ABI structs
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ws_bench.h"
#include "ws_plan.h"

static int failures = 0;
#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static ws_lane_config good() {
    ws_lane_config c;
    std::memset(&c, 0, sizeof c);
    c.batch = 1;
    c.src_w = 1920;
    c.src_h = 1080;
    c.dst_w = 224;
    c.dst_h = 224;
    c.resize_mode = WS_RESIZE_BILINEAR;
    c.input_mode = WS_INPUT_DEVICE;
    c.pad_value = 114;
    for (int i = 0; i < 3; ++i) {
        c.mean[i] = 0.5;
        c.std[i] = 0.25;
    }
    c.num_scores = 1000;
    c.k = 5;
    c.use_graph = 1;
    return c;
}

static int selftest() {
    ws_lane_config c = good();
    CHECK(ws::validate_config(&c) == WS_OK);
    CHECK(ws::validate_config(nullptr) == WS_E_INVALID_ARG);
#define BAD(field, value)                                     \
    do {                                                      \
        ws_lane_config b = good();                            \
        b.field = value;                                      \
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);   \
    } while (0)
    BAD(batch, 0);
    BAD(batch, WS_MAX_BATCH + 1);
    BAD(src_w, 0);
    BAD(dst_h, -3);
    BAD(src_h, WS_MAX_SIDE + 1);
    BAD(resize_mode, 2);
    BAD(input_mode, 7);
    BAD(pad_value, -1.0);
    BAD(pad_value, 256.0);
    BAD(k, 0);
    BAD(k, WS_MAX_K + 1);
    BAD(num_scores, -1);
    BAD(use_graph, 2);
    BAD(wait_mode, 9);
    BAD(rows_per_group, 65);
    BAD(topk_chunk, 1000);
    BAD(pixels_per_thread, 3);
    BAD(tensor_dtype, 3);
    BAD(channel_order, 2);
    BAD(autotune, 2);
    BAD(cache_policy, 3);
    BAD(cache_policy, -1);
    BAD(reserved, 1);
    {
        // detection: a valid 640x640 detection lane, then each field out of range
        ws_lane_config d = good();
        d.dst_w = d.dst_h = 640;
        d.det_classes = 80;
        d.det_max_det = 300;
        d.det_conf = 0.25f;
        d.det_iou = 0.45f;
        CHECK(ws::validate_config(&d) == WS_OK);
        ws::Plan p;
        CHECK(ws::make_plan(d, &p) == WS_OK);
        CHECK(p.det_anchors == 8400 && p.det_level_end[0] == 6400 && p.det_level_end[1] == 8000);
        CHECK(p.det_grid_w[0] == 80 && p.det_grid_w[1] == 40 && p.det_grid_w[2] == 20);
        CHECK(p.det_decode_groups == 132);
        CHECK(p.det_head_bytes == (size_t)144 * 8400 * 4);
#define BAD_DET(field, value)                                 \
    do {                                                      \
        ws_lane_config b = d;                                 \
        b.field = value;                                      \
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);   \
    } while (0)
        BAD_DET(det_classes, -1);
        BAD_DET(det_classes, WS_DET_MAX_CLASSES + 1);
        BAD_DET(batch, 2);
        BAD_DET(dst_w, 650);
        BAD_DET(dst_h, 2048);           // 2048 x 640: more than 16384 anchors
        BAD_DET(det_max_det, 0);
        BAD_DET(det_max_det, WS_DET_MAX_DET + 1);
        BAD_DET(det_conf, -0.1f);
        BAD_DET(det_conf, 1.0f);
        BAD_DET(det_iou, 1.5f);
        BAD_DET(det_agnostic, 2);
        BAD_DET(det_reserved, 1);
        BAD_DET(det_head_dev, (const float*)8);
        ws_lane_config z = good();
        z.det_head_dev = (const float*)64;      // a head without a detection stage
        CHECK(ws::validate_config(&z) == WS_E_INVALID_ARG);
        d.dst_w = 1024;
        d.dst_h = 512;                          // 8192 + 2048 + 512 anchors
        CHECK(ws::validate_config(&d) == WS_OK);
    }
    BAD(num_scores, WS_MAX_SCORES + 1);
    {
        ws_lane_config b = good();
        b.std[1] = 0.0;
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);
        b = good();
        b.mean[2] = 1.0 / 0.0;
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);
        b = good();
        b.num_scores = 3;
        b.k = 4;  // K > N
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);
        b.k = 3;
        CHECK(ws::validate_config(&b) == WS_OK);
        b = good();
        b.num_scores = 0;
        b.k = 0;  // no Top-K stage
        CHECK(ws::validate_config(&b) == WS_OK);
        b.k = 1;
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);
        b = good();
        b.input_dev = reinterpret_cast<const uint8_t*>(uintptr_t(0x1008));  // misaligned
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);
        b.input_dev = reinterpret_cast<const uint8_t*>(uintptr_t(0x1000));
        CHECK(ws::validate_config(&b) == WS_OK);
        b.input_mode = WS_INPUT_MAPPED_HOST;  // a device input in mapped mode
        CHECK(ws::validate_config(&b) == WS_E_INVALID_ARG);
    }
    // State machine: submit only when READY, wait only when IN_FLIGHT.
    CHECK(ws::begin_submit(ws::LaneState::Ready) == WS_OK);
    CHECK(ws::begin_submit(ws::LaneState::InFlight) == WS_E_STATE);
    CHECK(ws::begin_wait(ws::LaneState::InFlight) == WS_OK);
    CHECK(ws::begin_wait(ws::LaneState::Ready) == WS_E_STATE);
    CHECK(std::strcmp(ws::status_str(WS_E_STATE), "WS_E_STATE") == 0);
    CHECK(std::strcmp(ws::status_str(12345), "WS_E_UNKNOWN") == 0);
    // Plans: every lane shape the workloads use is feasible.
    ws::Plan p;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(p.pre_groups == 224 && p.pixels_per_thread == 1 && p.threads_per_row == 224);
    CHECK(p.span_lo == 3 * 3);  // first tap of 1920 -> 224: (1920 - 224) / 448 -> column 3
    c.batch = 64;
    c.src_w = 1280;
    c.src_h = 720;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(p.pixels_per_thread == 1 && p.rows_per_group == 1 && p.pre_groups == 64 * 224);
    CHECK(p.rows_per_group * p.threads_per_row <= p.pre_block);
    CHECK(p.lds_bytes <= ws::kMaxLdsBytes);
    c = good();
    c.src_w = WS_MAX_SIDE;
    c.dst_w = WS_MAX_SIDE;
    CHECK(ws::make_plan(c, &p) == WS_OK);  // widest rows, gather kernel: no LDS
    CHECK(p.lds_bytes == 0 && p.slot_bytes == 0);
    c.pixels_per_thread = 2;
    CHECK(ws::make_plan(c, &p) == WS_OK);  // widest rows still stage
    CHECK(p.lds_bytes > 0 && p.lds_bytes <= ws::kMaxLdsBytes);
    // 3840 -> 384 with seven rows per workgroup: the staged kernels would
    // need more LDS than a workgroup holds and are refused; the gather kernel
    // holds none, so the same geometry is accepted.
    c = good();
    c.src_w = 3840;
    c.src_h = 2160;
    c.dst_w = 384;
    c.dst_h = 384;
    c.rows_per_group = 7;
    c.pixels_per_thread = 2;
    CHECK(ws::make_plan(c, &p) == WS_E_INVALID_ARG);
    c.pixels_per_thread = 4;
    CHECK(ws::make_plan(c, &p) == WS_E_INVALID_ARG);
    c.pixels_per_thread = 1;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    // One thread per output column, each walking the workgroup's seven rows.
    CHECK(p.rows_per_group == 7 && p.lds_bytes == 0 && p.pre_block == 384);
    // Cache policy: non-temporal frame loads and tensor stores for
    // device-resident batches of 8 or more frames (or when asked), ordinary
    // ones otherwise; the staged kernels never stream.
    c = good();
    CHECK(ws::make_plan(c, &p) == WS_OK && !p.streaming);
    c.batch = WS_STREAM_MIN_BATCH;
    CHECK(ws::make_plan(c, &p) == WS_OK && p.streaming);
    c.cache_policy = WS_CACHE_KEEP;
    CHECK(ws::make_plan(c, &p) == WS_OK && !p.streaming);
    c.input_mode = WS_INPUT_MAPPED_HOST;
    c.cache_policy = WS_CACHE_STREAM;
    CHECK(ws::make_plan(c, &p) == WS_OK && !p.streaming);
    c = good();
    c.cache_policy = WS_CACHE_STREAM;
    CHECK(ws::make_plan(c, &p) == WS_OK && p.streaming);
    c.pixels_per_thread = 2;
    CHECK(ws::make_plan(c, &p) == WS_OK && !p.streaming);
    c = good();
    c.num_scores = 672000;
    c.k = 32;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(p.topk_groups * (int64_t)p.topk_chunk >= 672000);
    CHECK(p.topk_chunk % 1024 == 0);
    CHECK(p.topk_keys_per_lane == 32);      // 2 Ki scores per wave: one pass of 32 per lane
    c.num_scores = 21843;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(p.topk_keys_per_lane == 16 && p.topk_groups == 6);
    c.num_scores = 1000;
    c.k = 5;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(p.topk_keys_per_lane == 16 && p.topk_groups == 1 && p.topk_waves == 1);
    // Partial-list keys the allocation-free entry point keeps in its 1 MiB
    // scratch: none for one workgroup; groups x K beyond.
    const int64_t scratch_keys = WS_NOALLOC_SCRATCH_BYTES / 8;
    CHECK(ws::topk_scratch_keys(p, c.k) == 0);
    c.k = 32;
    c.num_scores = 672000;   // 83 workgroups of 8 Ki scores
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(ws::topk_scratch_keys(p, c.k) == 83 * 32);
    c.num_scores = 4096 * 8192;   // the most scores whose lists fit at K = 32
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(ws::topk_scratch_keys(p, c.k) == scratch_keys);
    c.num_scores = 4096 * 8192 + 1;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(ws::topk_scratch_keys(p, c.k) > scratch_keys);
    c.num_scores = 40000000;
    CHECK(ws::make_plan(c, &p) == WS_OK);
    CHECK(ws::topk_scratch_keys(p, c.k) == 4883 * 32 && 4883 * 32 > scratch_keys);
    std::printf("%d failures\n", failures);
    return failures == 0 ? 0 : 1;
}

static int layout() {
    std::printf("ws_lane_config sizeof %zu\n", sizeof(ws_lane_config));
    std::printf("ws_lane_config device %zu\n", offsetof(ws_lane_config, device));
    std::printf("ws_lane_config batch %zu\n", offsetof(ws_lane_config, batch));
    std::printf("ws_lane_config src_w %zu\n", offsetof(ws_lane_config, src_w));
    std::printf("ws_lane_config src_h %zu\n", offsetof(ws_lane_config, src_h));
    std::printf("ws_lane_config dst_w %zu\n", offsetof(ws_lane_config, dst_w));
    std::printf("ws_lane_config dst_h %zu\n", offsetof(ws_lane_config, dst_h));
    std::printf("ws_lane_config resize_mode %zu\n", offsetof(ws_lane_config, resize_mode));
    std::printf("ws_lane_config input_mode %zu\n", offsetof(ws_lane_config, input_mode));
    std::printf("ws_lane_config pad_value %zu\n", offsetof(ws_lane_config, pad_value));
    std::printf("ws_lane_config mean %zu\n", offsetof(ws_lane_config, mean));
    std::printf("ws_lane_config std %zu\n", offsetof(ws_lane_config, std));
    std::printf("ws_lane_config num_scores %zu\n", offsetof(ws_lane_config, num_scores));
    std::printf("ws_lane_config k %zu\n", offsetof(ws_lane_config, k));
    std::printf("ws_lane_config use_graph %zu\n", offsetof(ws_lane_config, use_graph));
    std::printf("ws_lane_config wait_mode %zu\n", offsetof(ws_lane_config, wait_mode));
    std::printf("ws_lane_config input_dev %zu\n", offsetof(ws_lane_config, input_dev));
    std::printf("ws_lane_config scores_dev %zu\n", offsetof(ws_lane_config, scores_dev));
    std::printf("ws_lane_config tensor_dev %zu\n", offsetof(ws_lane_config, tensor_dev));
    std::printf("ws_lane_config rows_per_group %zu\n", offsetof(ws_lane_config, rows_per_group));
    std::printf("ws_lane_config topk_chunk %zu\n", offsetof(ws_lane_config, topk_chunk));
    std::printf("ws_lane_config pixels_per_thread %zu\n", offsetof(ws_lane_config, pixels_per_thread));
    std::printf("ws_lane_config tensor_dtype %zu\n", offsetof(ws_lane_config, tensor_dtype));
    std::printf("ws_lane_config channel_order %zu\n", offsetof(ws_lane_config, channel_order));
    std::printf("ws_lane_config autotune %zu\n", offsetof(ws_lane_config, autotune));
    std::printf("ws_lane_config det_classes %zu\n", offsetof(ws_lane_config, det_classes));
    std::printf("ws_lane_config det_max_det %zu\n", offsetof(ws_lane_config, det_max_det));
    std::printf("ws_lane_config det_conf %zu\n", offsetof(ws_lane_config, det_conf));
    std::printf("ws_lane_config det_iou %zu\n", offsetof(ws_lane_config, det_iou));
    std::printf("ws_lane_config det_agnostic %zu\n", offsetof(ws_lane_config, det_agnostic));
    std::printf("ws_lane_config det_reserved %zu\n", offsetof(ws_lane_config, det_reserved));
    std::printf("ws_lane_config det_head_dev %zu\n", offsetof(ws_lane_config, det_head_dev));
    std::printf("ws_lane_config cache_policy %zu\n", offsetof(ws_lane_config, cache_policy));
    std::printf("ws_lane_config reserved %zu\n", offsetof(ws_lane_config, reserved));
    std::printf("ws_lane_view sizeof %zu\n", sizeof(ws_lane_view));
    std::printf("ws_lane_view input_host %zu\n", offsetof(ws_lane_view, input_host));
    std::printf("ws_lane_view input_dev %zu\n", offsetof(ws_lane_view, input_dev));
    std::printf("ws_lane_view tensor_dev %zu\n", offsetof(ws_lane_view, tensor_dev));
    std::printf("ws_lane_view scores_dev %zu\n", offsetof(ws_lane_view, scores_dev));
    std::printf("ws_lane_view result_host %zu\n", offsetof(ws_lane_view, result_host));
    std::printf("ws_lane_view input_bytes %zu\n", offsetof(ws_lane_view, input_bytes));
    std::printf("ws_lane_view tensor_bytes %zu\n", offsetof(ws_lane_view, tensor_bytes));
    std::printf("ws_lane_view det_head_dev %zu\n", offsetof(ws_lane_view, det_head_dev));
    std::printf("ws_lane_view det_result_host %zu\n", offsetof(ws_lane_view, det_result_host));
    std::printf("ws_topk_entry sizeof %zu\n", sizeof(ws_topk_entry));
    std::printf("ws_topk_entry score %zu\n", offsetof(ws_topk_entry, score));
    std::printf("ws_topk_entry index %zu\n", offsetof(ws_topk_entry, index));
    std::printf("ws_lane_plan sizeof %zu\n", sizeof(ws_lane_plan));
    std::printf("ws_lane_plan pre_groups %zu\n", offsetof(ws_lane_plan, pre_groups));
    std::printf("ws_lane_plan pre_block %zu\n", offsetof(ws_lane_plan, pre_block));
    std::printf("ws_lane_plan rows_per_group %zu\n", offsetof(ws_lane_plan, rows_per_group));
    std::printf("ws_lane_plan pre_lds_bytes %zu\n", offsetof(ws_lane_plan, pre_lds_bytes));
    std::printf("ws_lane_plan topk_groups %zu\n", offsetof(ws_lane_plan, topk_groups));
    std::printf("ws_lane_plan topk_block %zu\n", offsetof(ws_lane_plan, topk_block));
    std::printf("ws_lane_plan topk_chunk %zu\n", offsetof(ws_lane_plan, topk_chunk));
    std::printf("ws_lane_plan graph_nodes %zu\n", offsetof(ws_lane_plan, graph_nodes));
    std::printf("ws_lane_plan pixels_per_thread %zu\n", offsetof(ws_lane_plan, pixels_per_thread));
    std::printf("ws_lane_plan det_anchors %zu\n", offsetof(ws_lane_plan, det_anchors));
    std::printf("ws_lane_plan det_decode_groups %zu\n", offsetof(ws_lane_plan, det_decode_groups));
    std::printf("ws_lane_plan topk_keys_per_lane %zu\n", offsetof(ws_lane_plan, topk_keys_per_lane));
    std::printf("ws_lane_plan streaming %zu\n", offsetof(ws_lane_plan, streaming));
    std::printf("ws_det sizeof %zu\n", sizeof(ws_det));
    std::printf("ws_det x1 %zu\n", offsetof(ws_det, x1));
    std::printf("ws_det y1 %zu\n", offsetof(ws_det, y1));
    std::printf("ws_det x2 %zu\n", offsetof(ws_det, x2));
    std::printf("ws_det y2 %zu\n", offsetof(ws_det, y2));
    std::printf("ws_det score %zu\n", offsetof(ws_det, score));
    std::printf("ws_det class_id %zu\n", offsetof(ws_det, class_id));
    std::printf("ws_det_result sizeof %zu\n", sizeof(ws_det_result));
    std::printf("ws_det_result count %zu\n", offsetof(ws_det_result, count));
    std::printf("ws_det_result candidates %zu\n", offsetof(ws_det_result, candidates));
    std::printf("ws_det_result det %zu\n", offsetof(ws_det_result, det));
    return 0;
}

int main(int argc, char** argv) {
    if (argc == 2 && !std::strcmp(argv[1], "layout")) return layout();
    if (argc >= 2 && !std::strcmp(argv[1], "selftest")) return selftest();
    if (argc == 4 && !std::strcmp(argv[1], "taps")) {
        const long S = std::atol(argv[2]), R = std::atol(argv[3]);
        for (long d = 0; d < R; ++d) {
            const ws::Tap t = ws::axis_tap(S, R, d);
            std::printf("%d %d %.9g\n", t.i0, t.i1, (double)t.w);
        }
        return 0;
    }
    if (argc == 6 && !std::strcmp(argv[1], "letterbox")) {
        const ws::Region g = ws::letterbox_region(std::atol(argv[2]), std::atol(argv[3]),
                                                  std::atol(argv[4]), std::atol(argv[5]));
        std::printf("%d %d %d %d\n", g.left, g.top, g.w, g.h);
        return 0;
    }
    std::fprintf(stderr, "usage: ws_plan_test selftest | taps S R | letterbox W H Dw Dh\n");
    return 2;
}
