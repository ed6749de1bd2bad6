// ws_runtime.hip -- lane runtime behind the C ABI in ws.h / ws_bench.h.
//
// Every resource a lane uses is created in ws_create_lane and released in
// ws_destroy (WarpStream TRT article, lane and initialisation passages); the
// per-frame calls only record events, replay the graph and wait.  What a lane
// holds is the ws_lane struct below.  Whether the device can map pinned host
// memory is checked before the first mapped allocation, and a device that
// cannot is reported as an error.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstring>
#include <limits>
#include <new>
#include <thread>
#include <vector>

#include "ws.h"
#include "ws_bench.h"
#include "ws_detect.h"
#include "ws_kernels.h"
#include "ws_params.h"
#include "ws_plan.h"

namespace ws {
hipError_t set_kernel_attributes();
}

struct ws_lane {
    ws_lane_config cfg;
    ws::Plan plan;
    ws::LaneState state = ws::LaneState::Ready;
    int device = 0;
    hipStream_t stream = nullptr;
    hipEvent_t ev_start = nullptr;
    hipEvent_t ev_done = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    uint8_t* in_host = nullptr;        // mapped input slot (host view)
    uint8_t* in_own = nullptr;         // lane-owned device input
    const uint8_t* in_dev = nullptr;   // what the kernel reads
    void* tensor = nullptr;
    bool own_tensor = false;
    float* scores = nullptr;
    bool own_scores = false;
    ws_topk_entry* res_host = nullptr;  // mapped result slot (host view)
    uint2* res_dev = nullptr;           // its device view
    uint64_t* partials = nullptr;
    float* det_head = nullptr;
    bool own_det_head = false;
    float4* det_boxes = nullptr;
    uint64_t* det_keys = nullptr;
    uint32_t* det_counts = nullptr;
    uint32_t* det_cls_counts = nullptr;
    uint16_t* det_offs = nullptr;
    ws_det_result* det_host = nullptr;  // mapped detection result slot
    ws_det_result* det_dev = nullptr;   // its device view
    ws::PreParams pre{};
    ws::TopkParams tk{};
    ws::DetParams det{};
    int nodes = 0;
    int last_err = 0;
};

static_assert(ws::kDetDecodeBlock == ws::kDetDecodeAnchors, "decode grid and kernel agree");

namespace {

// Benchmark aid: streams over a buffer larger than the last-level cache so
// that the next kernel starts with cold caches.  Reads accumulate into a
// value stored only through a pointer the host passes as NULL, which keeps
// the loads without writing anything.
__global__ __launch_bounds__(256) void cache_flush_kernel(uint4* buf, size_t n16, int32_t write,
                                                          uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        if (write) {
            buf[i] = make_uint4(0u, 0u, 0u, 0u);
        } else {
            const uint4 v = buf[i];
            acc += v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (sink != nullptr && acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

// Benchmark aid: a kernel that does no work, for timing the launch path.  It
// stores only when `tag` is a value no caller passes, which keeps it a real
// dispatch with an argument.
__global__ __launch_bounds__(256) void launch_probe_kernel(uint32_t* sink, int32_t tag) {
    if (tag == INT32_MIN && sink != nullptr) sink[blockIdx.x] = (uint32_t)tag;
}

int fail(ws_lane* L, hipError_t e, int code) {
    if (L) L->last_err = (int)e;
    return code;
}

// The per-frame launch sequence, in stream order: (copy mode) the frame's
// host-to-device copy, preprocess, Top-K, detection decode + NMS.
hipError_t launch_all(ws_lane* L) {
    hipError_t e = hipSuccess;
    if (L->cfg.input_mode == WS_INPUT_COPY)
        e = hipMemcpyAsync(L->in_own, L->in_host, L->plan.input_bytes, hipMemcpyHostToDevice,
                           L->stream);
    if (e != hipSuccess) return e;
    e = ws::launch_preprocess(L->pre, L->plan.pre_groups, L->plan.pre_block, L->plan.lds_bytes,
                              L->stream);
    if (e != hipSuccess) return e;
    if (L->cfg.num_scores > 0) e = ws::launch_topk(L->tk, L->stream);
    if (e != hipSuccess) return e;
    if (L->plan.det_anchors > 0) e = ws::launch_detect(L->det, L->stream);
    return e;
}

void release(ws_lane* L) {
    if (!L) return;
    if (L->stream) hipStreamSynchronize(L->stream);
    if (L->exec) hipGraphExecDestroy(L->exec);
    if (L->graph) hipGraphDestroy(L->graph);
    if (L->ev_start) hipEventDestroy(L->ev_start);
    if (L->ev_done) hipEventDestroy(L->ev_done);
    if (L->stream) hipStreamDestroy(L->stream);
    if (L->in_host) hipHostFree(L->in_host);
    if (L->in_own) hipFree(L->in_own);
    if (L->own_tensor && L->tensor) hipFree(L->tensor);
    if (L->own_scores && L->scores) hipFree(L->scores);
    if (L->res_host) hipHostFree(L->res_host);
    if (L->partials) hipFree(L->partials);
    if (L->own_det_head && L->det_head) hipFree(L->det_head);
    if (L->det_boxes) hipFree(L->det_boxes);
    if (L->det_keys) hipFree(L->det_keys);
    if (L->det_counts) hipFree(L->det_counts);
    if (L->det_cls_counts) hipFree(L->det_cls_counts);
    if (L->det_offs) hipFree(L->det_offs);
    if (L->det_host) hipHostFree(L->det_host);
    delete L;
}

int dev_alloc(ws_lane* L, void** p, size_t bytes) {
    hipError_t e = hipMalloc(p, bytes < 16 ? 16 : bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(L, e, WS_E_OOM);
    }
    return WS_OK;
}

// Pinned, mapped, coherent host memory and its device address.
int mapped_alloc(ws_lane* L, void** host, void** dev, size_t bytes) {
    hipError_t e = hipHostMalloc(host, bytes < 16 ? 16 : bytes,
                                 hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) {
        *host = nullptr;
        return fail(L, e, WS_E_OOM);
    }
    std::memset(*host, 0, bytes < 16 ? 16 : bytes);
    e = hipHostGetDevicePointer(dev, *host, 0);
    if (e != hipSuccess) return fail(L, e, WS_E_NO_MAP_HOST);
    return WS_OK;
}

#define WS_TRY(expr)                 \
    do {                             \
        const int rc_ = (expr);      \
        if (rc_ != WS_OK) return rc_; \
    } while (0)

#define WS_HIP(expr, code)                                 \
    do {                                                   \
        const hipError_t e_ = (expr);                      \
        if (e_ != hipSuccess) return fail(L, e_, (code));  \
    } while (0)

// Kernel parameters from the lane's config and current plan (fixed for the
// lane's lifetime once construction ends).
void fill_params(ws_lane* L) {
    const ws_lane_config& c = L->cfg;
    const ws::Plan& P = L->plan;
    ws::fill_pre_params(c, P, L->in_dev, L->tensor, &L->pre);
    ws::fill_topk_params(c, P, L->scores, L->partials, L->res_dev, &L->tk);
    ws::DetParams& d = L->det;
    d.head = L->det_head;
    d.anchors = P.det_anchors;
    d.nc = c.det_classes;
    for (int i = 0; i < 3; ++i) {
        d.level_end[i] = P.det_level_end[i];
        d.grid_w[i] = P.det_grid_w[i];
    }
    d.conf = c.det_conf;
    d.iou = c.det_iou;
    {
        // The suppression test compares without dividing (ws_detect.hip,
        // iou_above): the midpoint of the threshold and its binary32
        // successor (exact in binary64), and which way a tie there rounds.
        const float t = c.det_iou;
        const float up = std::nextafter(t, std::numeric_limits<float>::infinity());
        d.iou_mid = ((double)t + (double)up) * 0.5;
        uint32_t tb = 0;
        std::memcpy(&tb, &t, sizeof tb);
        d.iou_tie_up = (int32_t)(tb & 1u);
    }
    d.max_det = c.det_max_det;
    d.agnostic = c.det_agnostic;
    d.boxes = L->det_boxes;
    d.keys = L->det_keys;
    d.groups = P.det_decode_groups;
    d.counts = L->det_counts;
    d.cls_counts = L->det_cls_counts;
    d.offs = L->det_offs;
    d.sort_cap = P.det_sort_cap;
    d.left = (float)P.region.left;
    d.top = (float)P.region.top;
    // Source pixels per network pixel inside the image region: the binary32
    // value of the float64 quotient.
    d.sx = (float)((double)c.src_w / (double)P.region.w);
    d.sy = (float)((double)c.src_h / (double)P.region.h);
    d.src_w = (float)c.src_w;
    d.src_h = (float)c.src_h;
    d.out = L->det_dev;
}

// Microseconds per launch of one stage on the lane's stream: the best of
// three timed runs of `reps` back-to-back launches (after two untimed
// launches), or a huge value on error.
double time_stage_us(ws_lane* L, int stage, int reps) {
    hipError_t e = hipSuccess;
    auto launch = [&]() {
        return stage == WS_STAGE_PREPROCESS
                   ? ws::launch_preprocess(L->pre, L->plan.pre_groups, L->plan.pre_block,
                                           L->plan.lds_bytes, L->stream)
                   : ws::launch_topk(L->tk, L->stream);
    };
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = launch();
    double best = 1e30;
    for (int trial = 0; trial < 3 && e == hipSuccess; ++trial) {
        e = hipEventRecord(L->ev_start, L->stream);
        for (int i = 0; i < reps && e == hipSuccess; ++i) e = launch();
        if (e == hipSuccess) e = hipEventRecord(L->ev_done, L->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(L->stream);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, L->ev_start, L->ev_done);
        if (e == hipSuccess) best = std::min(best, 1e3 * (double)ms / reps);
    }
    return e == hipSuccess ? best : 1e30;
}

// Construction-time autotune: time a few launch geometries on this lane's own
// buffers and keep the fastest (yolo.cu times its tile choices once at
// startup).  Geometry changes speed only, never results.  A candidate must
// beat the current choice by 2% to replace it, so timing noise does not move
// the lane off the heuristic plan.
int autotune(ws_lane* L) {
    const ws_lane_config base = L->cfg;
    const int kReps = 10;
    ws::Plan best = L->plan;
    double best_us = time_stage_us(L, WS_STAGE_PREPROCESS, kReps);
    for (int px : {1, 2, 4}) {
        for (int rows : {1, 2, 4}) {
            ws_lane_config c = base;
            c.pixels_per_thread = px;
            c.rows_per_group = rows;
            ws::Plan p;
            if (ws::make_plan(c, &p) != WS_OK) continue;
            // Every preprocess field of the candidate plan: the staged
            // kernels also need the row span and slot size, which the gather
            // kernel's plan leaves at zero.
            L->plan.span_lo = p.span_lo;
            L->plan.span = p.span;
            L->plan.slot_bytes = p.slot_bytes;
            L->plan.pixels_per_thread = p.pixels_per_thread;
            L->plan.threads_per_row = p.threads_per_row;
            L->plan.rows_per_group = p.rows_per_group;
            L->plan.pre_block = p.pre_block;
            L->plan.pre_groups = p.pre_groups;
            L->plan.groups_per_frame = p.groups_per_frame;
            L->plan.lds_bytes = p.lds_bytes;
            fill_params(L);
            const double us = time_stage_us(L, WS_STAGE_PREPROCESS, kReps);
            if (us < 0.98 * best_us) {
                best_us = us;
                best = L->plan;
            }
        }
    }
    L->plan = best;
    fill_params(L);
    if (base.num_scores > ws::kTopkSingleGroupMax) {
        double best_tk = time_stage_us(L, WS_STAGE_TOPK, kReps);
        for (int chunk : {1024, 2048, 4096, 8192, 16384}) {
            ws_lane_config c = base;
            c.topk_chunk = chunk;
            ws::Plan p;
            if (ws::make_plan(c, &p) != WS_OK) continue;
            L->plan.topk_chunk = p.topk_chunk;
            L->plan.topk_waves = p.topk_waves;
            L->plan.topk_groups = p.topk_groups;
            L->plan.topk_keys_per_lane = p.topk_keys_per_lane;
            fill_params(L);
            const double us = time_stage_us(L, WS_STAGE_TOPK, kReps);
            if (us < 0.98 * best_tk) {
                best_tk = us;
                best = L->plan;
            }
        }
        L->plan = best;
        fill_params(L);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? WS_OK : fail(L, e, WS_E_HIP);
}

int build(ws_lane* L) {
    const ws_lane_config& c = L->cfg;
    ws::Plan& P = L->plan;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || c.device >= ndev) return WS_E_NO_DEVICE;
    L->device = c.device;
    WS_HIP(hipSetDevice(c.device), WS_E_HIP);
    // Mapping must be enabled before use.  ROCm always allows it; the flag
    // call fails harmlessly once the device is active, so the capability and
    // the mapping itself are what decide.
    (void)hipSetDeviceFlags(hipDeviceMapHost);
    (void)hipGetLastError();
    int can_map = 0;
    WS_HIP(hipDeviceGetAttribute(&can_map, hipDeviceAttributeCanMapHostMemory, c.device),
           WS_E_HIP);
    if (!can_map) return WS_E_NO_MAP_HOST;

    WS_TRY(ws::make_plan(c, &P));
    // Raise the dynamic LDS limit for wide rows; only a plan that needs more
    // than the default 64 KiB depends on it succeeding.
    if (ws::set_kernel_attributes() != hipSuccess) {
        const hipError_t e = hipGetLastError();
        if (P.lds_bytes > 64 * 1024 || P.topk_keys_per_lane == 32) return fail(L, e, WS_E_HIP);
    }
    // The suppression kernel keeps every candidate key in LDS.
    if (P.det_anchors > 0) {
        // Every lane within the limits of ws.h fits (checked at compile time).
        if (ws::det_nms_lds_bytes(P.det_sort_cap, c.det_max_det, c.det_classes, c.det_agnostic != 0) == 0)
            return fail(L, hipSuccess, WS_E_INVALID_ARG);
        WS_HIP(ws::set_detect_attributes(), WS_E_HIP);
    }

    // ---- buffers ---------------------------------------------------------
    if (c.input_mode == WS_INPUT_MAPPED_HOST) {
        void *h = nullptr, *d = nullptr;
        WS_TRY(mapped_alloc(L, &h, &d, P.input_bytes));
        L->in_host = static_cast<uint8_t*>(h);
        L->in_dev = static_cast<const uint8_t*>(d);
    } else if (c.input_mode == WS_INPUT_COPY) {
        // Pinned host slot for the producer (the DMA engine reads it) and the
        // fixed device buffer the copy lands in.
        void* h = nullptr;
        const size_t hb = P.input_bytes < 16 ? 16 : P.input_bytes;
        hipError_t e = hipHostMalloc(&h, hb, hipHostMallocDefault);
        if (e != hipSuccess) return fail(L, e, WS_E_OOM);
        std::memset(h, 0, hb);
        L->in_host = static_cast<uint8_t*>(h);
        void* d = nullptr;
        WS_TRY(dev_alloc(L, &d, P.input_bytes));
        L->in_own = static_cast<uint8_t*>(d);
        L->in_dev = L->in_own;
    } else if (c.input_dev) {
        L->in_dev = c.input_dev;
    } else {
        void* d = nullptr;
        WS_TRY(dev_alloc(L, &d, P.input_bytes));
        L->in_own = static_cast<uint8_t*>(d);
        L->in_dev = L->in_own;
        WS_HIP(hipMemset(L->in_own, 0, P.input_bytes), WS_E_HIP);
    }
    if (c.tensor_dev) {
        L->tensor = c.tensor_dev;
    } else {
        void* d = nullptr;
        WS_TRY(dev_alloc(L, &d, P.tensor_bytes));
        L->tensor = d;
        L->own_tensor = true;
    }
    if (c.num_scores > 0) {
        if (c.scores_dev) {
            L->scores = const_cast<float*>(c.scores_dev);
        } else {
            void* d = nullptr;
            WS_TRY(dev_alloc(L, &d, (size_t)c.num_scores * sizeof(float)));
            L->scores = static_cast<float*>(d);
            L->own_scores = true;
            WS_HIP(hipMemset(L->scores, 0, (size_t)c.num_scores * sizeof(float)), WS_E_HIP);
        }
        void *h = nullptr, *d = nullptr;
        WS_TRY(mapped_alloc(L, &h, &d, (size_t)c.k * sizeof(ws_topk_entry)));
        L->res_host = static_cast<ws_topk_entry*>(h);
        L->res_dev = static_cast<uint2*>(d);
        void* pp = nullptr;
        // Room for the most workgroups any geometry can use (1024-score chunks).
        const size_t max_groups = ((size_t)c.num_scores + 1023) / 1024;
        WS_TRY(dev_alloc(L, &pp, max_groups * (size_t)c.k * sizeof(uint64_t)));
        L->partials = static_cast<uint64_t*>(pp);
    }

    if (P.det_anchors > 0) {
        const size_t A = (size_t)P.det_anchors;
        if (c.det_head_dev) {
            L->det_head = const_cast<float*>(c.det_head_dev);
        } else {
            void* d = nullptr;
            WS_TRY(dev_alloc(L, &d, P.det_head_bytes));
            L->det_head = static_cast<float*>(d);
            L->own_det_head = true;
            WS_HIP(hipMemset(L->det_head, 0, P.det_head_bytes), WS_E_HIP);
        }
        void *bx = nullptr, *ky = nullptr, *cn = nullptr;
        WS_TRY(dev_alloc(L, &bx, A * sizeof(float4)));
        L->det_boxes = static_cast<float4*>(bx);
        WS_TRY(dev_alloc(L, &ky, A * sizeof(uint64_t)));
        L->det_keys = static_cast<uint64_t*>(ky);
        const size_t G = (size_t)P.det_decode_groups;
        WS_TRY(dev_alloc(L, &cn, G * sizeof(uint32_t)));
        L->det_counts = static_cast<uint32_t*>(cn);
        WS_HIP(hipMemset(L->det_counts, 0, G * sizeof(uint32_t)), WS_E_HIP);
        // Class counters start at zero; the suppression kernel clears them
        // after every frame.
        const size_t ncc = c.det_agnostic ? 1u : (size_t)c.det_classes;
        void *cc = nullptr, *of = nullptr;
        WS_TRY(dev_alloc(L, &cc, ncc * sizeof(uint32_t)));
        L->det_cls_counts = static_cast<uint32_t*>(cc);
        WS_HIP(hipMemset(L->det_cls_counts, 0, ncc * sizeof(uint32_t)), WS_E_HIP);
        WS_TRY(dev_alloc(L, &of, G * 64u * sizeof(uint16_t)));
        L->det_offs = static_cast<uint16_t*>(of);
        void *h = nullptr, *d = nullptr;
        WS_TRY(mapped_alloc(L, &h, &d, sizeof(ws_det_result)));
        L->det_host = static_cast<ws_det_result*>(h);
        L->det_dev = static_cast<ws_det_result*>(d);
    }

    fill_params(L);
    L->nodes = 1 + (c.num_scores > 0 ? 1 : 0) + (c.input_mode == WS_INPUT_COPY ? 1 : 0) +
               (P.det_anchors > 0 ? 2 : 0);

    // ---- stream, events, warm-up, capture ---------------------------------
    WS_HIP(hipStreamCreateWithFlags(&L->stream, hipStreamNonBlocking), WS_E_HIP);
    WS_HIP(hipEventCreate(&L->ev_start), WS_E_HIP);
    WS_HIP(hipEventCreate(&L->ev_done), WS_E_HIP);

    if (c.autotune) WS_TRY(autotune(L));

    // Warm-up outside capture: loads code objects and touches every buffer.
    WS_HIP(launch_all(L), WS_E_HIP);
    WS_HIP(hipStreamSynchronize(L->stream), WS_E_HIP);

    if (c.use_graph) {
        WS_HIP(hipStreamBeginCapture(L->stream, hipStreamCaptureModeThreadLocal), WS_E_CAPTURE);
        const hipError_t le = launch_all(L);
        const hipError_t ce = hipStreamEndCapture(L->stream, &L->graph);
        if (le != hipSuccess) return fail(L, le, WS_E_CAPTURE);
        if (ce != hipSuccess) return fail(L, ce, WS_E_CAPTURE);
        WS_HIP(hipGraphInstantiate(&L->exec, L->graph, nullptr, nullptr, 0), WS_E_CAPTURE);
        WS_HIP(hipGraphUpload(L->exec, L->stream), WS_E_CAPTURE);
        WS_HIP(hipGraphLaunch(L->exec, L->stream), WS_E_HIP);
        WS_HIP(hipStreamSynchronize(L->stream), WS_E_HIP);
    }
    return WS_OK;
}

}  // namespace

extern "C" {

int ws_create_lane(const ws_lane_config* cfg, ws_lane** out, ws_lane_view* view) {
    if (!out) return WS_E_INVALID_ARG;
    *out = nullptr;
    const int v = ws::validate_config(cfg);
    if (v != WS_OK) return v;
    ws_lane* L = new (std::nothrow) ws_lane();
    if (!L) return WS_E_OOM;
    L->cfg = *cfg;
    const int rc = build(L);
    if (rc != WS_OK) {
        release(L);
        return rc;
    }
    if (view) {
        view->input_host = L->in_host;
        view->input_dev = L->in_dev;
        view->tensor_dev = L->tensor;
        view->scores_dev = L->scores;
        view->result_host = L->res_host;
        view->input_bytes = L->plan.input_bytes;
        view->tensor_bytes = L->plan.tensor_bytes;
        view->det_head_dev = L->det_head;
        view->det_result_host = L->det_host;
    }
    *out = L;
    return WS_OK;
}

int ws_submit(ws_lane* L) {
    if (!L) return WS_E_INVALID_ARG;
    if (ws::begin_submit(L->state) != WS_OK) return WS_E_STATE;
    hipError_t e = hipEventRecord(L->ev_start, L->stream);
    if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    e = L->cfg.use_graph ? hipGraphLaunch(L->exec, L->stream) : launch_all(L);
    if (e == hipSuccess) e = hipEventRecord(L->ev_done, L->stream);
    if (e != hipSuccess) {
        // Whatever was enqueued finishes before the lane is usable again.
        hipStreamSynchronize(L->stream);
        return fail(L, e, WS_E_HIP);
    }
    L->state = ws::LaneState::InFlight;
    return WS_OK;
}

int ws_wait(ws_lane* L, float* gpu_ms) {
    if (!L) return WS_E_INVALID_ARG;
    if (ws::begin_wait(L->state) != WS_OK) return WS_E_STATE;
    hipError_t e;
    if (L->cfg.wait_mode == WS_WAIT_SPIN) {
        while ((e = hipEventQuery(L->ev_done)) == hipErrorNotReady) {
        }
    } else {
        e = hipEventSynchronize(L->ev_done);
    }
    L->state = ws::LaneState::Ready;
    if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    if (gpu_ms) {
        e = hipEventElapsedTime(gpu_ms, L->ev_start, L->ev_done);
        if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    }
    return WS_OK;
}

int ws_destroy(ws_lane* L) {
    if (!L) return WS_OK;
    if (L->state == ws::LaneState::InFlight && L->ev_done) hipEventSynchronize(L->ev_done);
    release(L);
    return WS_OK;
}

const char* ws_status_str(int status) { return ws::status_str(status); }

int ws_lane_hip_error(const ws_lane* L) { return L ? L->last_err : 0; }

int ws_lane_describe(const ws_lane* L, ws_lane_plan* plan) {
    if (!L || !plan) return WS_E_INVALID_ARG;
    plan->pre_groups = L->plan.pre_groups;
    plan->pre_block = L->plan.pre_block;
    plan->rows_per_group = L->plan.rows_per_group;
    plan->pre_lds_bytes = L->plan.lds_bytes;
    plan->topk_groups = L->plan.topk_groups;
    plan->topk_block = 64 * L->plan.topk_waves;
    plan->topk_chunk = L->plan.topk_chunk;
    plan->graph_nodes = L->nodes;
    plan->pixels_per_thread = L->plan.pixels_per_thread;
    plan->det_anchors = L->plan.det_anchors;
    plan->det_decode_groups = L->plan.det_decode_groups;
    plan->topk_keys_per_lane = L->plan.topk_keys_per_lane;
    plan->streaming = L->plan.streaming ? 1 : 0;
    return WS_OK;
}

int ws_bench_replays(ws_lane* L, int32_t replays, float* gpu_ms, float* host_us,
                     float* submit_us, double* wall_s) {
    if (!L || replays < 0) return WS_E_INVALID_ARG;
    int rc = WS_OK;
    using clk = std::chrono::steady_clock;
    const auto t0 = clk::now();
    auto ts = t0;
    for (int32_t i = 0; i < replays && rc == WS_OK; ++i) {
        rc = ws_submit(L);
        if (submit_us) {
            submit_us[i] =
                (float)std::chrono::duration<double, std::micro>(clk::now() - ts).count();
        }
        if (rc == WS_OK) rc = ws_wait(L, gpu_ms ? &gpu_ms[i] : nullptr);
        if (host_us || submit_us) {
            const auto te = clk::now();
            if (host_us)
                host_us[i] = (float)std::chrono::duration<double, std::micro>(te - ts).count();
            ts = te;
        }
    }
    const auto t1 = std::chrono::steady_clock::now();
    if (wall_s) *wall_s = std::chrono::duration<double>(t1 - t0).count();
    return rc;
}

int ws_bench_lanes(ws_lane** lanes, int32_t nlanes, int32_t replays, float* gpu_ms,
                   double* wall_s) {
    if (!lanes || nlanes < 1 || replays < 0) return WS_E_INVALID_ARG;
    for (int32_t i = 0; i < nlanes; ++i)
        if (!lanes[i]) return WS_E_INVALID_ARG;
    std::atomic<int> ready{0};
    std::atomic<bool> go{false};
    std::vector<int> rcs((size_t)nlanes, WS_OK);
    std::vector<std::thread> threads;
    threads.reserve((size_t)nlanes);
    for (int32_t i = 0; i < nlanes; ++i) {
        threads.emplace_back([&, i]() {
            hipSetDevice(lanes[i]->device);
            ready.fetch_add(1);
            while (!go.load(std::memory_order_acquire)) {
            }
            rcs[(size_t)i] = ws_bench_replays(lanes[i], replays,
                                              gpu_ms ? gpu_ms + (size_t)i * replays : nullptr,
                                              nullptr, nullptr, nullptr);
        });
    }
    while (ready.load() < nlanes) {
    }
    const auto t0 = std::chrono::steady_clock::now();
    go.store(true, std::memory_order_release);
    for (auto& th : threads) th.join();
    const auto t1 = std::chrono::steady_clock::now();
    if (wall_s) *wall_s = std::chrono::duration<double>(t1 - t0).count();
    for (int rc : rcs)
        if (rc != WS_OK) return rc;
    return WS_OK;
}

namespace {

// One stage's kernels of lane L, on `stream`.
hipError_t launch_stage_on(ws_lane* L, int32_t stage, hipStream_t stream) {
    if (stage == WS_STAGE_PREPROCESS)
        return ws::launch_preprocess(L->pre, L->plan.pre_groups, L->plan.pre_block,
                                     L->plan.lds_bytes, stream);
    if (stage == WS_STAGE_TOPK) return ws::launch_topk(L->tk, stream);
    return ws::launch_detect(L->det, stream);
}

hipError_t launch_stage(ws_lane* L, int32_t stage) { return launch_stage_on(L, stage, L->stream); }

bool stage_present(const ws_lane* L, int32_t stage) {
    if (stage == WS_STAGE_PREPROCESS) return true;
    if (stage == WS_STAGE_TOPK) return L->cfg.num_scores > 0;
    if (stage == WS_STAGE_DETECT) return L->plan.det_anchors > 0;
    return false;
}

}  // namespace

int ws_bench_stage_cold(ws_lane* L, int32_t stage, void* flush, size_t flush_bytes,
                        int32_t flush_write, int32_t launches, float* ms) {
    if (!L || !flush || !ms || launches < 1 || flush_bytes < 16 || !ws::aligned16(flush))
        return WS_E_INVALID_ARG;
    if (!stage_present(L, stage) || (flush_write != 0 && flush_write != 1))
        return WS_E_INVALID_ARG;
    if (ws::begin_submit(L->state) != WS_OK) return WS_E_STATE;
    hipError_t e = hipSuccess;
    for (int32_t i = 0; i < launches && e == hipSuccess; ++i) {
        hipLaunchKernelGGL(cache_flush_kernel, dim3(4096), dim3(256), 0, L->stream,
                           static_cast<uint4*>(flush), flush_bytes / 16, flush_write,
                           static_cast<uint32_t*>(nullptr));
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(L->ev_start, L->stream);
        if (e == hipSuccess) e = launch_stage(L, stage);
        if (e == hipSuccess) e = hipEventRecord(L->ev_done, L->stream);
        const hipError_t se = hipStreamSynchronize(L->stream);
        if (e == hipSuccess) e = se;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], L->ev_start, L->ev_done);
    }
    if (e != hipSuccess) {
        hipStreamSynchronize(L->stream);
        return fail(L, e, WS_E_HIP);
    }
    return WS_OK;
}

int ws_bench_stage_rotate(ws_lane** lanes, int32_t nlanes, int32_t stage, int32_t warmup,
                          int32_t launches, double* ms_per_launch) {
    if (!lanes || nlanes < 1 || launches < 1 || warmup < 0 || !ms_per_launch)
        return WS_E_INVALID_ARG;
    for (int32_t i = 0; i < nlanes; ++i) {
        if (!lanes[i] || !stage_present(lanes[i], stage) || lanes[i]->device != lanes[0]->device)
            return WS_E_INVALID_ARG;
        if (ws::begin_submit(lanes[i]->state) != WS_OK) return WS_E_STATE;
    }
    ws_lane* L = lanes[0];
    hipError_t e = hipSuccess;
    for (int32_t i = 0; i < warmup && e == hipSuccess; ++i)
        e = launch_stage_on(lanes[i % nlanes], stage, L->stream);
    if (e == hipSuccess) e = hipEventRecord(L->ev_start, L->stream);
    for (int32_t i = 0; i < launches && e == hipSuccess; ++i)
        e = launch_stage_on(lanes[i % nlanes], stage, L->stream);
    if (e == hipSuccess) e = hipEventRecord(L->ev_done, L->stream);
    const hipError_t se = hipStreamSynchronize(L->stream);
    if (e == hipSuccess) e = se;
    if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, L->ev_start, L->ev_done);
    if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    *ms_per_launch = (double)ms / (double)launches;
    return WS_OK;
}

int ws_bench_stage(ws_lane* L, int32_t stage, int32_t launches, double* ms_per_launch) {
    if (!L || !ms_per_launch || launches < 1) return WS_E_INVALID_ARG;
    if (!stage_present(L, stage)) return WS_E_INVALID_ARG;
    if (ws::begin_submit(L->state) != WS_OK) return WS_E_STATE;
    hipError_t e = hipEventRecord(L->ev_start, L->stream);
    for (int32_t i = 0; i < launches && e == hipSuccess; ++i) e = launch_stage(L, stage);
    if (e == hipSuccess) e = hipEventRecord(L->ev_done, L->stream);
    const hipError_t se = hipStreamSynchronize(L->stream);
    if (e == hipSuccess) e = se;
    if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, L->ev_start, L->ev_done);
    if (e != hipSuccess) return fail(L, e, WS_E_HIP);
    *ms_per_launch = (double)ms / (double)launches;
    return WS_OK;
}

int ws_bench_launch_cost(int32_t device, int32_t nodes, int32_t form, int32_t warmup,
                         int32_t replays, float* launch_us, float* total_us, float* gpu_us,
                         int32_t* hip_error) {
    if (hip_error) *hip_error = 0;
    if (nodes < 1 || nodes > 8 || replays < 1 || warmup < 0 || !launch_us || !total_us ||
        !gpu_us || (form != WS_LAUNCH_GRAPH && form != WS_LAUNCH_DIRECT))
        return WS_E_INVALID_ARG;
    if (hipSetDevice(device) != hipSuccess) return WS_E_HIP;
    // The launch checks below read the thread's last error, which an earlier
    // call of this thread (a not-ready event query, say) may have left set.
    (void)hipGetLastError();
    constexpr int kGrid = 224;
    hipStream_t s = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t x = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    auto chain = [&]() {
        hipError_t r = hipSuccess;
        for (int32_t i = 0; i < nodes && r == hipSuccess; ++i) {
            hipLaunchKernelGGL(launch_probe_kernel, dim3(kGrid), dim3(256), 0, s, nullptr, i);
            r = hipGetLastError();
        }
        return r;
    };
    if (e == hipSuccess) e = chain();   // loads the code object outside any capture
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess && form != WS_LAUNCH_DIRECT) {
        e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
        if (e == hipSuccess) {
            const hipError_t le = chain();
            e = hipStreamEndCapture(s, &g);
            if (e == hipSuccess) e = le;
        }
        if (e == hipSuccess) e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
        if (e == hipSuccess) e = hipGraphUpload(x, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
    }
    using clk = std::chrono::steady_clock;
    const auto us = [](clk::time_point a, clk::time_point b) {
        return (float)std::chrono::duration<double, std::micro>(b - a).count();
    };
    for (int32_t it = 0; it < warmup + replays && e == hipSuccess; ++it) {
        (void)hipGetLastError();   // the previous round's not-ready queries
        const auto t0 = clk::now();
        e = hipEventRecord(e0, s);
        const auto ta = clk::now();
        if (e == hipSuccess) e = form == WS_LAUNCH_DIRECT ? chain() : hipGraphLaunch(x, s);
        const auto tb = clk::now();
        if (e == hipSuccess) e = hipEventRecord(e1, s);
        if (e != hipSuccess) break;
        while ((e = hipEventQuery(e1)) == hipErrorNotReady) {
        }
        const auto t2 = clk::now();
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && it >= warmup) {
            launch_us[it - warmup] = us(ta, tb);
            total_us[it - warmup] = us(t0, t2);
            gpu_us[it - warmup] = ms * 1e3f;
        }
    }
    if (s) hipStreamSynchronize(s);
    if (x) hipGraphExecDestroy(x);
    if (g) hipGraphDestroy(g);
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    if (s) hipStreamDestroy(s);
    if (hip_error) *hip_error = (int32_t)e;
    (void)hipGetLastError();   // leave no error behind for the caller's next call
    return e == hipSuccess ? WS_OK : WS_E_HIP;
}

}  // extern "C"
