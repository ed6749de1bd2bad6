// ws_detect.hip -- detection decode + greedy NMS for gfx950 (CDNA4, wave64).
//
// yolo.cu README: the end-to-end pipeline passage (DFL decode and NMS inside
// the frame's one graph launch), the "GPU-resident NMS" highlight (greedy
// suppression over the live candidates in score order; only the final boxes,
// about 7 KB, cross to pinned memory) and the embedding example (up to 300
// boxes in source-image coordinates).
//
// det_decode_kernel: one thread per anchor.  The best class is the first
//   maximum of the anchor's class probabilities; an anchor above the
//   confidence threshold decodes its four DFL distributions, stores its box
//   by anchor index and appends a 64-bit key to the candidate list (one
//   atomic per wave).  Key = probability bits (positive, so they order as
//   integers) : 0x3FFF - anchor : class, so a larger key is a higher score,
//   then a lower anchor.
// det_nms_kernel: one 1024-thread workgroup.  Each thread holds up to 16
//   candidates in registers (keys, and boxes up to 8 per thread).  Every round, the largest live key
//   in the workgroup is the next box in rank order that no kept box
//   suppressed -- exactly the next box greedy suppression keeps -- so the
//   round keeps it, writes it out, and every thread drops its candidates of
//   the same class whose IoU with it exceeds the threshold.  One barrier per
//   kept box; suppressed candidates are never sorted.
//
// All arithmetic that decides a result (DFL exponentials, boxes, IoU,
// mapping) is binary32 with one rounding per operation in a fixed order:
// fused multiply-add is switched off below, and division is IEEE (the
// library is built with correctly rounded fp32 division).
#include <hip/hip_runtime.h>

#include "ws_kernels.h"
#include "ws_lanes.h"

namespace ws {
namespace {

constexpr int kDecodeBlock = 256;
constexpr int kNmsBlock = 1024;
constexpr int kNmsWaves = kNmsBlock / 64;
constexpr int kBins = WS_DET_REG_MAX;

// e^x for x <= 0 (Cody & Waite, "Software Manual for the Elementary
// Functions", exp): x = n ln2 + r with ln 2 split into a 15-significant-bit
// high part (n * hi is exact for |n| < 512) and the rounded remainder, then
// e^r by its degree-7 Taylor polynomial (|r| <= ln2 / 2, truncation below
// 6e-9 relative) in Horner form, then scaling by 2^n.  Arguments below -80
// are raised to -80 so the result stays a normal number.
__device__ __forceinline__ float exp_nonpos(float x) {
#pragma clang fp contract(off)
    const float log2e = __uint_as_float(0x3FB8AA3Bu);
    const float ln2_hi = __uint_as_float(0x3F317200u);
    const float ln2_lo = __uint_as_float(0x35BFBE8Eu);
    x = fmaxf(x, -80.0f);
    const float n = rintf(x * log2e);
    const float r = (x - n * ln2_hi) - n * ln2_lo;
    float p = 1.0f / 5040.0f;
    p = p * r + 1.0f / 720.0f;
    p = p * r + 1.0f / 120.0f;
    p = p * r + 1.0f / 24.0f;
    p = p * r + 1.0f / 6.0f;
    p = p * r + 1.0f / 2.0f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    return ldexpf(p, (int)n);
}

// Expected bin index under the softmax of one side's 16 logits (bin b at
// q[b * A]): the maximum, the shifted exponentials, the weight sum and the
// index-weighted sum accumulated bin 0..15 in order, one division.
__device__ __forceinline__ float dfl_side(const float* __restrict__ q, int A) {
#pragma clang fp contract(off)
    float l[kBins];
#pragma unroll
    for (int b = 0; b < kBins; ++b) l[b] = q[(size_t)b * A];
    float m = l[0];
#pragma unroll
    for (int b = 1; b < kBins; ++b) m = fmaxf(m, l[b]);
    float s = exp_nonpos(l[0] - m);
    float num = 0.0f;
#pragma unroll
    for (int b = 1; b < kBins; ++b) {
        const float e = exp_nonpos(l[b] - m);
        s = s + e;
        num = num + (float)b * e;
    }
    return num / s;
}

// IoU of kept box a and candidate b (xyxy): areas, clipped intersection
// sides, intersection, union = (area_a + area_b) - inter, one division.  A
// zero union gives NaN, which suppresses nothing.
__device__ __forceinline__ float iou_xyxy(float4 a, float4 b) {
#pragma clang fp contract(off)
    const float area_a = (a.z - a.x) * (a.w - a.y);
    const float area_b = (b.z - b.x) * (b.w - b.y);
    const float iw = fmaxf(0.0f, fminf(a.z, b.z) - fmaxf(a.x, b.x));
    const float ih = fmaxf(0.0f, fminf(a.w, b.w) - fmaxf(a.y, b.y));
    const float inter = iw * ih;
    const float uni = (area_a + area_b) - inter;
    return inter / uni;
}

// Network-input pixels -> source pixels, clipped to [0, hi].
__device__ __forceinline__ float to_source(float v, float origin, float scale, float hi) {
#pragma clang fp contract(off)
    return fminf(fmaxf((v - origin) * scale, 0.0f), hi);
}

__global__ __launch_bounds__(kDecodeBlock) void det_decode_kernel(const DetParams p) {
#pragma clang fp contract(off)
    const int a = (int)blockIdx.x * kDecodeBlock + (int)threadIdx.x;
    const int lane = (int)threadIdx.x & 63;
    const int A = p.anchors;
    bool cand = false;
    uint64_t key = 0;
    if (a < A) {
        const float* __restrict__ pr = p.head + (size_t)(4 * kBins) * A + a;
        float best = -INFINITY;    // NaN never compares greater: it never wins
        int cls = 0;
        int c = 0;
        for (; c + 8 <= p.nc; c += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = pr[(size_t)(c + j) * A];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (v[j] > best) {
                    best = v[j];
                    cls = c + j;
                }
        }
        for (; c < p.nc; ++c) {
            const float v = pr[(size_t)c * A];
            if (v > best) {
                best = v;
                cls = c;
            }
        }
        cand = best > p.conf;
        if (cand) {
            const int level = a < p.level_end[0] ? 0 : (a < p.level_end[1] ? 1 : 2);
            const int cell = a - (level == 0 ? 0 : p.level_end[level - 1]);
            const int gw = p.grid_w[level];
            const float cx = (float)(cell % gw) + 0.5f;
            const float cy = (float)(cell / gw) + 0.5f;
            const float s = (float)(8 << level);
            const float* __restrict__ q = p.head + a;
            const float dl = dfl_side(q, A);
            const float dt = dfl_side(q + (size_t)kBins * A, A);
            const float dr = dfl_side(q + (size_t)(2 * kBins) * A, A);
            const float db = dfl_side(q + (size_t)(3 * kBins) * A, A);
            p.boxes[a] = make_float4((cx - dl) * s, (cy - dt) * s, (cx + dr) * s, (cy + db) * s);
            key = ((uint64_t)__float_as_uint(best) << 32) | ((uint64_t)(0x3FFF - a) << 16) |
                  (uint64_t)(uint32_t)cls;
        }
    }
    // Append the wave's candidates with one atomic.
    const uint64_t m = __ballot(cand);
    if (m != 0) {
        const int leader = __ffsll((unsigned long long)m) - 1;
        uint32_t base = 0;
        if (lane == leader) base = atomicAdd(p.counter, (uint32_t)__popcll(m));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
        if (cand) {
            const uint32_t idx = base + (uint32_t)lanes_below(m);
            if (idx < (uint32_t)A) p.keys[idx] = key;
        }
    }
}

// S candidates per thread.  REG_BOXES: boxes live in registers beside their
// keys (up to 8 per thread); otherwise only keys do and boxes are re-read from
// the anchor-indexed box buffer (L2-resident) when a test needs them -- the
// rare case of more than 8192 candidates.
template <int S, bool REG_BOXES>
__device__ __forceinline__ void nms_rounds(const DetParams& p, int n,
                                           uint64_t (*s_key)[kNmsWaves],
                                           float4 (*s_box)[kNmsWaves]) {
#pragma clang fp contract(off)
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float4* __restrict__ boxes = p.boxes;
    auto box_of = [boxes](uint64_t k) { return boxes[0x3FFF - (int)((k >> 16) & 0x3FFFu)]; };
    uint64_t key[S];
    float4 box[REG_BOXES ? S : 1];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int i = s * kNmsBlock + tid;
        key[s] = i < n ? p.keys[i] : 0;
        if constexpr (REG_BOXES) box[s] = key[s] ? box_of(key[s]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float thr = p.iou;
    int kept = 0;
    int buf = 0;
    while (kept < p.max_det) {
        // This thread's, then this wave's, largest live key.
        uint64_t best = 0;
        int bs = 0;
#pragma unroll
        for (int s = 0; s < S; ++s)
            if (key[s] > best) {
                best = key[s];
                bs = s;
            }
        uint64_t w = umax64(best, xor_lane64<32>(best, lane));
        w = umax64(w, xor_lane64<16>(w, lane));
        w = umax64(w, xor_lane64<8>(w, lane));
        w = umax64(w, xor_lane64<4>(w, lane));
        w = umax64(w, xor_lane64<2>(w, lane));
        w = umax64(w, xor_lane64<1>(w, lane));
        // Keys are unique, so exactly one lane holds a non-zero wave maximum.
        if (w != 0 ? best == w : lane == 0) {
            float4 bb = make_float4(0.f, 0.f, 0.f, 0.f);
            if (w != 0) {
                if constexpr (REG_BOXES) {
#pragma unroll
                    for (int s = 0; s < S; ++s)
                        if (s == bs) bb = box[s];
                } else {
                    bb = box_of(w);
                }
            }
            s_key[buf][wave] = w;
            s_box[buf][wave] = bb;
        }
        // Double-buffered: the next round writes the other half, and the one
        // after can only start once every thread has passed this barrier.
        __syncthreads();
        uint64_t g = 0;
        int gw = 0;
#pragma unroll
        for (int i = 0; i < kNmsWaves; ++i) {
            const uint64_t k = s_key[buf][i];
            if (k > g) {
                g = k;
                gw = i;
            }
        }
        if (g == 0) break;    // no live candidate left (uniform)
        const float4 kb = s_box[buf][gw];
        const uint32_t kc = (uint32_t)g & 0xFFFFu;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (key[s] == 0) continue;
            if (key[s] == g) {
                key[s] = 0;
            } else if (p.agnostic || ((uint32_t)key[s] & 0xFFFFu) == kc) {
                float4 b;
                if constexpr (REG_BOXES) b = box[s];
                else b = box_of(key[s]);
                if (iou_xyxy(kb, b) > thr) key[s] = 0;
            }
        }
        if (tid == 0) {
            ws_det d;
            d.x1 = to_source(kb.x, p.left, p.sx, p.src_w);
            d.y1 = to_source(kb.y, p.top, p.sy, p.src_h);
            d.x2 = to_source(kb.z, p.left, p.sx, p.src_w);
            d.y2 = to_source(kb.w, p.top, p.sy, p.src_h);
            d.score = __uint_as_float((uint32_t)(g >> 32));
            d.class_id = (int32_t)kc;
            p.out->det[kept] = d;
        }
        ++kept;
        buf ^= 1;
    }
    if (tid == 0) {
        p.out->count = kept;
        p.out->candidates = n;
    }
}

__global__ __launch_bounds__(kNmsBlock) void det_nms_kernel(const DetParams p) {
    __shared__ uint64_t s_key[2][kNmsWaves];
    __shared__ float4 s_box[2][kNmsWaves];
    __shared__ int s_n;
    if (threadIdx.x == 0) {
        const uint32_t c = *p.counter;
        s_n = (int)(c < (uint32_t)p.anchors ? c : (uint32_t)p.anchors);
        *p.counter = 0;    // ready for the next replay's decode
    }
    __syncthreads();
    const int n = s_n;    // uniform
    if (n <= kNmsBlock)
        nms_rounds<1, true>(p, n, s_key, s_box);
    else if (n <= 2 * kNmsBlock)
        nms_rounds<2, true>(p, n, s_key, s_box);
    else if (n <= 4 * kNmsBlock)
        nms_rounds<4, true>(p, n, s_key, s_box);
    else if (n <= 8 * kNmsBlock)
        nms_rounds<8, true>(p, n, s_key, s_box);
    else
        nms_rounds<16, false>(p, n, s_key, s_box);
}

static_assert(16 * kNmsBlock >= WS_DET_MAX_ANCHORS, "NMS registers must hold every anchor");

}  // namespace

hipError_t launch_detect(const DetParams& p, int decode_groups, hipStream_t stream) {
    hipLaunchKernelGGL(det_decode_kernel, dim3((unsigned)decode_groups), dim3(kDecodeBlock), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(det_nms_kernel, dim3(1), dim3(kNmsBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ws
