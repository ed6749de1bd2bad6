// ws_noalloc.hip -- the allocation-free entry point (ws_run_noalloc in ws.h)
// for callers that cannot allocate: code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc.
//
// One frame of the per-frame launch sequence -- preprocess, then Top-K -- on
// the caller's stream and buffers.  The only memory beyond the caller's is
// the Top-K partial lists (one sorted list of K keys per workgroup when the
// scores span several workgroups), which live in the file-scope array
// `scratch` below: each GPU holds its own copy for the life of the process.
// In host code `scratch` names a host-side handle, not a device address, so
// the address every launch uses comes from hipGetSymbolAddress, taken once
// per device with that device current.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "ws.h"
#include "ws_kernels.h"
#include "ws_params.h"
#include "ws_plan.h"

namespace ws {
hipError_t set_kernel_attributes();
}

static constexpr size_t kScratchKeys = WS_NOALLOC_SCRATCH_BYTES / sizeof(uint64_t);

// Top-K partial lists of ws_run_noalloc: [groups][k] order keys, fully
// rewritten by the partial kernel of each call before the merge kernel reads
// them, so nothing needs clearing between calls.
static __device__ __align__(256) uint64_t scratch[kScratchKeys];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_setup_mu;
uint64_t* g_scratch[kMaxDevices] = {};

// Once per device, with that device current: the device address of
// `scratch` and the kernels' LDS limits.
hipError_t device_setup(int dev, uint64_t** out) {
    std::lock_guard<std::mutex> hold(g_setup_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        e = ws::set_kernel_attributes();
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<uint64_t*>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int ws_run_noalloc(const ws_lane_config* cfg, ws_topk_entry* result, void* stream) {
    const int v = ws::validate_config(cfg);
    if (v != WS_OK) return v;
    const ws_lane_config& c = *cfg;
    if (c.input_mode != WS_INPUT_DEVICE || !c.input_dev || !c.tensor_dev) return WS_E_INVALID_ARG;
    if (c.det_classes != 0 || c.autotune != 0) return WS_E_INVALID_ARG;
    if (c.num_scores > 0 && (!c.scores_dev || !result)) return WS_E_INVALID_ARG;
    if (c.num_scores == 0 && result) return WS_E_INVALID_ARG;
    if (((uintptr_t)result & 7u) != 0) return WS_E_INVALID_ARG;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || c.device >= ndev) return WS_E_NO_DEVICE;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WS_E_HIP;
    if (cur != c.device || cur < 0 || cur >= kMaxDevices) return WS_E_INVALID_ARG;
    ws::Plan P;
    if (ws::make_plan(c, &P) != WS_OK) return WS_E_INVALID_ARG;
    if (ws::topk_scratch_keys(P, c.k) > (int64_t)kScratchKeys) return WS_E_INVALID_ARG;
    uint64_t* scr = nullptr;
    if (device_setup(cur, &scr) != hipSuccess) return WS_E_HIP;

    const hipStream_t s = static_cast<hipStream_t>(stream);
    ws::PreParams pre;
    ws::fill_pre_params(c, P, c.input_dev, c.tensor_dev, &pre);
    hipError_t e = ws::launch_preprocess(pre, P.pre_groups, P.pre_block, P.lds_bytes, s);
    if (e == hipSuccess && c.num_scores > 0) {
        ws::TopkParams tk;
        ws::fill_topk_params(c, P, c.scores_dev, scr, reinterpret_cast<uint2*>(result), &tk);
        e = ws::launch_topk(tk, s);
    }
    return e == hipSuccess ? WS_OK : WS_E_HIP;
}
