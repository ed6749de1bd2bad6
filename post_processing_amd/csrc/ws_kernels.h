// ws_kernels.h -- launch parameters and launchers of the preprocess and
// Top-K kernels (ws_preprocess.hip, ws_topk.hip); detection's are in
// ws_detect.h.
// Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "ws.h"

namespace ws {

// Fused preprocess: RGB8 HWC frames -> resample -> normalise -> FP32 NCHW.
struct PreParams {
    const uint8_t* src;     // [batch][src_h][src_w][3], 16-byte aligned base
    void* dst;              // [batch][3][dst_h][dst_w] of FP32 / FP16 / BF16
    int32_t dtype;          // WS_DTYPE_*
    uint32_t shift[3];      // bit offset of output channel c's byte in a pixel
    int64_t frame_bytes;    // 3 * src_w * src_h
    int64_t total_bytes;    // batch * frame_bytes (bound of every staged load)
    int32_t src_w, src_h;
    int32_t dst_w, dst_h;
    int32_t left, top;      // resampled region inside the tensor
    int32_t reg_w, reg_h;
    float inv_den_x;        // 1 / (2 reg_w)
    float inv_den_y;        // 1 / (2 reg_h)
    uint32_t magic_x;       // floor(2^32 / (2 reg_w)) + 1: division by 2 reg_w as a multiply
    uint32_t magic_y;       // floor(2^32 / (2 reg_h)) + 1
    int32_t span_lo;        // first staged byte of a source row
    int32_t slot_chunks;    // 16-byte chunks per staged row
    int32_t pixels_per_thread;  // PX: 1, 2 or 4 adjacent output columns
    int32_t streaming;          // gather kernel: non-temporal frame loads and tensor stores
    int32_t threads_per_row;    // ceil(dst_w / PX)
    int32_t rows_per_group;
    int32_t groups_per_frame;
    int32_t vec;            // dst_w % PX == 0: each thread's columns form an aligned vector
    float a[3];             // 1 / (255 std[c])
    float b[3];             // -mean[c] / std[c]
    float padv[3];          // (pad / 255 - mean[c]) / std[c]
};

// Exact Top-K over FP32 scores; G workgroups each select their chunk's top K;
// for G > 1 a one-workgroup merge kernel selects from the G partial lists.
struct TopkParams {
    const float* scores;     // [n], 16-byte aligned
    int64_t n;
    int32_t k;
    int32_t chunk;           // scores per workgroup, multiple of 1024
    int32_t keys_per_lane;   // scores per lane per batch: 16 or 32
    int32_t groups;
    int32_t waves;           // wave64s per workgroup, 1..4
    uint64_t* partials;      // [groups][k] order keys (groups > 1)
    uint2* result;           // [k] {score bits, index}, device view of the slot
};

hipError_t launch_preprocess(const PreParams& p, int groups, int block, int lds_bytes,
                             hipStream_t stream);
hipError_t launch_topk(const TopkParams& p, hipStream_t stream);
// Raise the dynamic LDS limit of the staged preprocess kernels.
hipError_t set_preprocess_attributes();
constexpr int kTopkMaxThreads = 256;   // 4 wave64s: one per SIMD

}  // namespace ws
