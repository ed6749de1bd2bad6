// ws_detect.h -- launch parameters and launcher of the detection kernels
// (ws_detect.hip).  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "ws.h"

namespace ws {

constexpr int kDetDecodeAnchors = 64;   // anchors per decode workgroup (one wave's lanes)
constexpr int kDetMaxGroups = WS_DET_MAX_ANCHORS / kDetDecodeAnchors;

// Detection decode + greedy NMS over a YOLO-style head (layout in ws.h).
//
// Hand-off between the two kernels: decode workgroup g writes how many of
// its 64 anchors are candidates to counts[g], and their keys and boxes to
// slots g * 64 + q, q = 0, 1, ... in anchor order.  A slot therefore orders
// candidates exactly as their anchors do.  Each candidate also takes a place
// among the frame's candidates of its class from cls_counts[class] (one
// counter in any-class mode), written to offs[slot]; the suppression kernel
// reads the counters and sets them back to zero for the next frame.  Every
// decode launch rewrites every count in counts.
struct DetParams {
    const float* head;       // [4 * 16 + nc][anchors], 16-byte aligned
    int32_t anchors;         // A <= WS_DET_MAX_ANCHORS
    int32_t nc;
    int32_t level_end[3];    // anchor index where the stride-8/16/32 grids end
    int32_t grid_w[3];       // cells per row of each grid
    float conf;              // candidate: best probability > conf
    float iou;               // suppression: IoU > iou (binary32 IoU), decided as below
    double iou_mid;          // midpoint of iou and the next binary32 above it
    int32_t iou_tie_up;      // an IoU exactly at iou_mid rounds up (iou's significand is odd)
    int32_t max_det;
    int32_t agnostic;
    int32_t groups;          // decode workgroups: ceil(anchors / 64) <= kDetMaxGroups
    float4* boxes;           // [groups * 64] network-input xyxy by slot
    uint64_t* keys;          // [groups * 64] candidate keys by slot
    uint32_t* counts;        // [groups] candidates per decode workgroup
    uint32_t* cls_counts;    // [nc, or 1 in any-class mode] candidates per class, zero between frames
    uint16_t* offs;          // [groups * 64] each candidate's place in its class, by slot
    int32_t sort_cap;        // keys the suppression kernel's LDS holds: a power of two >= anchors
    float left, top;         // image region origin in the network input
    float sx, sy;            // source pixels per network pixel (binary32 of W/rw, H/rh)
    float src_w, src_h;      // clip bounds
    ws_det_result* out;      // device view of the mapped result slot
};

// Decode (one workgroup per 64 anchors) then suppression (one workgroup), in
// stream order.
hipError_t launch_detect(const DetParams& p, hipStream_t stream);
// Dynamic LDS of the suppression kernel for a lane's sizes; 0 if no
// workgroup size fits (never for sizes within the ws.h limits).
int det_nms_lds_bytes(int sort_cap, int max_det, int nc, bool any_class);
// Raise the suppression kernels' dynamic LDS limit (once per process).
hipError_t set_detect_attributes();

}  // namespace ws
