// ws_detect.hip -- detection decode + greedy NMS for gfx950 (CDNA4, wave64).
//
// yolo.cu README: the end-to-end pipeline passage (DFL decode and NMS inside
// the frame's one graph launch), the "GPU-resident NMS" highlight (greedy
// suppression over the live candidates in score order; only the final boxes,
// about 7 KB, cross to pinned memory) and the embedding example (up to 300
// boxes in source-image coordinates).
//
// det_decode_kernel (one workgroup per 64 anchors, four waves): wave w finds
//   each anchor's best class within the w-th quarter of the classes; the
//   anchors above the confidence threshold are compacted in LDS, their DFL
//   distances are computed one lane per (candidate, box side), and each
//   candidate's box is stored by anchor and its sort key appended to the
//   candidate list (one atomic per workgroup).
// det_nms_kernel (one workgroup of 16 waves, or 8 when 16 waves' kept-box
// lists do not fit LDS beside the keys):
//   1. sorts the candidate keys descending in LDS (bitonic: DPP exchanges
//      inside a wave, LDS exchanges across waves).  The key orders by class
//      first (unless boxes of any class suppress each other), then by
//      probability descending, then anchor ascending -- so each class is a
//      contiguous run in rank order;
//   2. resolves the runs in parallel, one wave per run: 64 candidates at a
//      time, each is tested against the run's boxes kept so far, then the
//      first live candidate is kept and suppresses the live ones after it,
//      and so on.  Boxes of different classes never interact, so this is
//      exactly greedy suppression restricted to each class, and a class's
//      run stops once it has max_det boxes;
//   3. re-sorts the kept boxes of all classes by probability descending,
//      anchor ascending -- the order in which plain greedy suppression over
//      all candidates keeps them -- and writes the first max_det.
//
// All arithmetic that decides a result (DFL exponentials, boxes, IoU,
// mapping) is binary32 with one rounding per operation in a fixed order:
// fused multiply-add is switched off below, and division is IEEE (the
// library is built with correctly rounded fp32 division).  The IoU
// threshold test reaches the same decision as dividing and comparing, by an
// exact comparison in binary64 (iou_above).
#include <hip/hip_runtime.h>

#include "ws_kernels.h"
#include "ws_lanes.h"

namespace ws {
namespace {

constexpr int kDecodeBlock = kDetDecodeAnchors;
constexpr int kDecodeParts = 4;               // class ranges per anchor, one wave each
constexpr int kDecodeThreads = kDecodeParts * kDecodeBlock;
// The suppression kernel runs with 1,024 threads when its LDS allows (more
// class runs in flight: each wave's run is a chain of dependent steps), else
// with kDetNmsThreads.
constexpr int kNmsWideThreads = 1024;
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

// Whether IoU(a, b) > t for kept box a and candidate b (xyxy), where the IoU
// is binary32: areas, clipped intersection sides, intersection, union =
// (area_a + area_b) - inter, each rounded once, then inter / union rounded
// once.  The division is not carried out.  With t+ the next binary32 above
// t and m their midpoint, the rounded quotient exceeds t exactly when
// inter / union > m, or equals m and the tie rounds up to t+ (t+ has the
// even significand, i.e. t's is odd).  inter and union are binary32 and m
// has 25 significant bits, so m * union is exact in binary64 and the test is
// exact.  A zero union (0 / 0 = NaN) and NaN boxes suppress nothing.
__device__ __forceinline__ bool iou_above(float4 a, float4 b, double mid, bool tie_up) {
#pragma clang fp contract(off)
    const float area_a = (a.z - a.x) * (a.w - a.y);
    const float area_b = (b.z - b.x) * (b.w - b.y);
    const float iw = fmaxf(0.0f, fminf(a.z, b.z) - fmaxf(a.x, b.x));
    const float ih = fmaxf(0.0f, fminf(a.w, b.w) - fmaxf(a.y, b.y));
    const float inter = iw * ih;
    const float uni = (area_a + area_b) - inter;
    const double bound = mid * (double)uni;
    const double in = (double)inter;
    // Bitwise, not short-circuit: every compare is evaluated, no branches.
    return (uni > 0.0f) & ((in > bound) | (tie_up & (in == bound)));
}

// Network-input pixels -> source pixels, clipped to [0, hi].
__device__ __forceinline__ float to_source(float v, float origin, float scale, float hi) {
#pragma clang fp contract(off)
    return fminf(fmaxf((v - origin) * scale, 0.0f), hi);
}

// ---------------------------------------------------------------------------
// Candidate keys.  Larger keys come first; every key is non-zero and unique
// (the anchor is in it), and bit 0 is free (it marks kept candidates).
//   by class:  [63:52] 4095 - class, [51:21] probability bits, [20:7] 16383 - anchor
//   any class: [63:33] probability bits, [32:19] 16383 - anchor, [18:7] class
// The probability is > conf >= 0, so its sign bit is clear and its bits order
// as integers.  The second layout is also the rank order of the output.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t make_key(bool any_class, uint32_t prob, int anchor, int cls) {
    const uint64_t pr = prob & 0x7FFFFFFFu;
    const uint64_t an = (uint64_t)(0x3FFF - anchor);
    if (any_class) return (pr << 33) | (an << 19) | ((uint64_t)cls << 7);
    return ((uint64_t)(0xFFF - cls) << 52) | (pr << 21) | (an << 7);
}

__device__ __forceinline__ int key_anchor(uint64_t k, bool any_class) {
    return 0x3FFF - (int)((k >> (any_class ? 19 : 7)) & 0x3FFFu);
}

__device__ __forceinline__ uint32_t key_group(uint64_t k, bool any_class) {
    return any_class ? 0u : (uint32_t)(k >> 52);
}

// A class-ordered key in rank layout (the "any class" layout).
__device__ __forceinline__ uint64_t to_rank_key(uint64_t k) {
    const uint64_t cls = 0xFFFu - (k >> 52);
    return (((k >> 7) & ((1ull << 45) - 1)) << 19) | (cls << 7);
}

__device__ __forceinline__ float4 readlane4(float4 v, int lane) {
    return make_float4(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.x), lane)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.y), lane)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.z), lane)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.w), lane)));
}

// Block sort of the candidate keys (bitonic network, descending): each wave
// sorts blocks of 64*K keys in registers (sort_block), and only distances of
// a whole block or more go through LDS.

// One stage (B, J) with J at least a block, through LDS: one thread per pair,
// four pairs loaded before any is stored.
template <int NT>
__device__ __forceinline__ void cx_pass_lds(uint64_t* s, int P, int B, int J, int tid) {
    const int pairs = P >> 1;
    for (int q0 = tid; q0 < pairs; q0 += 4 * NT) {
        int lo[4];
        uint64_t a[4], b[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int q = q0 + m * NT;
            lo[m] = ((q & ~(J - 1)) << 1) | (q & (J - 1));
            if (q < pairs) {
                a[m] = s[lo[m]];
                b[m] = s[lo[m] + J];
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int q = q0 + m * NT;
            if (q < pairs && (a[m] < b[m]) == ((lo[m] & B) == 0)) {
                s[lo[m]] = b[m];
                s[lo[m] + J] = a[m];
            }
        }
    }
}

// Sorts P keys descending into s[0, P), P a power of two with 64 <= P and
// P / (64 K) blocks.  The keys come from g[0, n) (zero past n) when g is
// given, else from s itself.  Ends with a barrier.
template <int NT, int K>
__device__ __forceinline__ void sort_desc_k(uint64_t* s, int P, int tid, const uint64_t* __restrict__ g,
                                            int n) {
    constexpr int Q = 64 * K;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blocks = P / Q;
    for (int b = wave; b < blocks; b += NT / 64) {
        uint64_t x[K];
        if (g) {
#pragma unroll
            for (int r = 0; r < K; ++r) {
                const int e = b * Q + r * 64 + lane;
                x[r] = e < n ? g[e] : 0;
            }
        } else {
#pragma unroll
            for (int r = 0; r < K; ++r) x[r] = s[b * Q + r * 64 + lane];
        }
        sort_block<K>(x, (b & 1) == 0, lane);
#pragma unroll
        for (int r = 0; r < K; ++r) s[b * Q + r * 64 + lane] = x[r];
    }
    __syncthreads();
    for (int B = 2 * Q; B <= P; B <<= 1) {
        for (int J = B >> 1; J >= Q; J >>= 1) {
            cx_pass_lds<NT>(s, P, B, J, tid);
            __syncthreads();
        }
        for (int b = wave; b < blocks; b += NT / 64) {
            uint64_t x[K];
#pragma unroll
            for (int r = 0; r < K; ++r) x[r] = s[b * Q + r * 64 + lane];
            cx_stages<K, 2 * Q, Q / 2>(x, ((b * Q) & B) == 0, lane);
#pragma unroll
            for (int r = 0; r < K; ++r) s[b * Q + r * 64 + lane] = x[r];
        }
        __syncthreads();
    }
}

// Block sizes: one block per wave up to 4096 keys (64 per lane at most 8),
// then several blocks of 512 per wave.
template <int NT>
__device__ __forceinline__ void sort_desc(uint64_t* s, int P, int tid, const uint64_t* __restrict__ g = nullptr,
                                          int n = 0) {
    if (P <= 512) sort_desc_k<NT, 1>(s, P, tid, g, n);
    else if (P == 1024) sort_desc_k<NT, 2>(s, P, tid, g, n);
    else if (P == 2048) sort_desc_k<NT, 4>(s, P, tid, g, n);
    else sort_desc_k<NT, 8>(s, P, tid, g, n);
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------
// Both detection kernels take the fields their first loads need as leading
// scalar and pointer arguments, which the library's kernarg preloading puts
// in scalar registers at wave launch, and read them from there; DetParams
// follows by value and is read in place (a local copy with its arrays
// indexed at run time would live in private memory).
__global__ __launch_bounds__(kDecodeThreads) void det_decode_kernel(
    const float* head, int32_t anchors, int32_t nc, const DetParams p) {
#pragma clang fp contract(off)
    __shared__ int s_anchor[kDecodeBlock];
    __shared__ int s_cls[kDecodeBlock];
    __shared__ uint32_t s_prob[kDecodeBlock];
    __shared__ float s_dist[kDecodeBlock][4];
    __shared__ float s_pbest[kDecodeParts][kDecodeBlock];
    __shared__ int s_pcls[kDecodeParts][kDecodeBlock];
    __shared__ int s_count;
    __shared__ uint32_t s_base;
    const int tid = (int)threadIdx.x;
    const int A = anchors;
    if (tid == 0) s_count = 0;

    // 1. Best class (first maximum; NaN never compares greater) and threshold.
    //    Wave w scans the w-th quarter of the classes of the group's anchors.
    const int a = (int)blockIdx.x * kDecodeBlock + (tid & (kDecodeBlock - 1));
    const int part = tid / kDecodeBlock;   // wave-uniform
    const int per = (nc + kDecodeParts - 1) / kDecodeParts;
    const int c_begin = min(nc, part * per);
    const int c_end = min(nc, c_begin + per);
    float best = -INFINITY;
    int cls = c_begin;
    if (a < A) {
        const float* __restrict__ pr = head + (size_t)(4 * kBins) * A + a;
        int c = c_begin;
        for (; c + 16 <= c_end; c += 16) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = pr[(size_t)(c + j) * A];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (v[j] > best) {
                    best = v[j];
                    cls = c + j;
                }
        }
        for (; c < c_end; ++c) {
            const float v = pr[(size_t)c * A];
            if (v > best) {
                best = v;
                cls = c;
            }
        }
    }
    s_pbest[part][tid & (kDecodeBlock - 1)] = best;
    s_pcls[part][tid & (kDecodeBlock - 1)] = cls;
    __syncthreads();
    if (part == 0 && a < A) {
        // Later ranges win only when strictly greater: ties keep the first.
        best = -INFINITY;
        cls = 0;
#pragma unroll
        for (int q = 0; q < kDecodeParts; ++q)
            if (s_pbest[q][tid] > best) {
                best = s_pbest[q][tid];
                cls = s_pcls[q][tid];
            }
        if (best > p.conf) {
            const int slot = atomicAdd(&s_count, 1);
            s_anchor[slot] = a;
            s_cls[slot] = cls;
            s_prob[slot] = __float_as_uint(best);
        }
    }
    __syncthreads();
    const int n = s_count;   // uniform
    if (n == 0) return;

    // 2. DFL distances, one lane per (candidate, side); each lane issues its
    //    16 loads before any arithmetic.
    for (int t = tid; t < 4 * n; t += kDecodeThreads) {
        const int q = t >> 2;
        const int side = t & 3;
        s_dist[q][side] = dfl_side(head + (size_t)(side * kBins) * A + s_anchor[q], A);
    }
    if (tid == 0) s_base = atomicAdd(p.counter, (uint32_t)n);
    __syncthreads();

    // 3. Boxes by anchor, keys appended to the candidate list.
    const uint32_t base = s_base;
    const bool any_class = p.agnostic != 0;
    for (int q = tid; q < n; q += kDecodeThreads) {
        const int aq = s_anchor[q];
        const int level = aq < p.level_end[0] ? 0 : (aq < p.level_end[1] ? 1 : 2);
        const int cell = aq - (level == 0 ? 0 : p.level_end[level - 1]);
        const int gw = p.grid_w[level];
        const float cx = (float)(cell % gw) + 0.5f;
        const float cy = (float)(cell / gw) + 0.5f;
        const float st = (float)(8 << level);
        p.boxes[aq] = make_float4((cx - s_dist[q][0]) * st, (cy - s_dist[q][1]) * st,
                                  (cx + s_dist[q][2]) * st, (cy + s_dist[q][3]) * st);
        const uint32_t idx = base + (uint32_t)q;   // < anchors: each anchor appears once
        if (idx < (uint32_t)A) p.keys[idx] = make_key(any_class, s_prob[q], aq, s_cls[q]);
    }
}

// ---------------------------------------------------------------------------
// Suppression
// ---------------------------------------------------------------------------

// Greedy suppression over one class's run s[s0 ..) (all of s when boxes of
// any class interact), by one wave.  With STAGED, s_box holds the boxes in
// sorted order in LDS; otherwise they are read by anchor from global memory.
// The choice is a template argument so that each instance loads from one
// address space (a run-time choice between the two pointers compiles to
// generic loads that wait on both memory counters).  Kept candidates get
// bit 0 set in s and their positions listed in kept_pos (capacity max_det).
// Returns how many were kept.
template <bool STAGED>
__device__ __forceinline__ int resolve_run(const DetParams& p, uint64_t* s, const float4* s_box, int n, int s0,
                           uint16_t* kept_pos, bool any_class, int lane) {
#pragma clang fp contract(off)
    const double mid = p.iou_mid;
    const bool tie_up = p.iou_tie_up != 0;
    uint32_t group = 0;
    int kept = 0;
    for (int c0 = s0; c0 < n; c0 += 64) {
        wave_lds_sync();   // kept_pos writes of the previous block are visible
        const int e = c0 + lane;
        const uint64_t key = e < n ? s[e] : 0;
        if (c0 == s0) group = key_group(readlane64(key, 0), any_class);   // the run's first key
        const bool valid = e < n && key_group(key, any_class) == group;
        const uint64_t vmask = __ballot(valid);
        if (vmask == 0) break;
        // Branches rather than a conditional over lvalues, which would give
        // the zero box a private-memory copy.
        float4 box = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) box = STAGED ? s_box[e] : p.boxes[key_anchor(key, any_class)];
        uint64_t alive = vmask;

        // Boxes of this run kept in earlier blocks, 64 at a time.
        for (int kb = 0; kb < kept && alive != 0; kb += 64) {
            const int kl = kb + lane;
            float4 kbox = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kl < kept)
                kbox = STAGED ? s_box[kept_pos[kl]]
                              : p.boxes[key_anchor(s[kept_pos[kl]], any_class)];
            const int lim = min(64, kept - kb);
            for (int t = 0; t < lim && alive != 0; ++t) {
                const bool sup = valid & iou_above(readlane4(kbox, t), box, mid, tie_up);
                alive &= ~(uint64_t)__ballot(sup);
            }
        }

        // This block: the first live candidate is the next kept box.
        uint64_t pending = alive;
        while (pending != 0) {
            const int i = __ffsll((unsigned long long)pending) - 1;
            if (lane == i) {
                kept_pos[kept] = (uint16_t)e;
                s[e] = key | 1u;
            }
            ++kept;
            if (kept == p.max_det) return kept;
            const bool sup = (lane > i) & iou_above(readlane4(box, i), box, mid, tie_up);
            alive &= ~(uint64_t)__ballot(sup);
            pending = alive & ~((2ull << i) - 1);   // candidates after i
        }
        if (vmask != ~0ull) break;   // the run ended inside this block
    }
    return kept;
}

// Up to this many kept boxes are placed by counting, not sorted.
constexpr int kRankByCountMax = 256;

// Number of the n keys of v (LDS) above x; sixteen loads are issued before
// their compares.
__device__ __forceinline__ int count_above(const uint64_t* v, int n, uint64_t x) {
    int r = 0;
    int j = 0;
    for (; j + 16 <= n; j += 16) {
        uint64_t t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] = v[j + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) r += t[u] > x ? 1 : 0;
    }
    for (; j < n; ++j) r += v[j] > x ? 1 : 0;
    return r;
}

template <int NT>
__global__ __launch_bounds__(NT) void det_nms_kernel(
    uint32_t* counter, uint64_t* keys, int32_t anchors, int32_t sort_cap, int32_t agnostic,
    int32_t max_det, const DetParams p) {
#pragma clang fp contract(off)
    constexpr int kNmsThreads = NT;
    constexpr int kNmsWaves = NT / 64;
    // Dynamic LDS: keys [sort_cap] | run starts [kDetRunCap] | kept positions
    // [kNmsWaves][max_det].
    extern __shared__ uint64_t s_dyn[];
    uint64_t* s = s_dyn;
    uint16_t* s_run = reinterpret_cast<uint16_t*>(s_dyn + sort_cap);
    uint16_t* s_kept = s_run + kDetRunCap;
    __shared__ int s_n, s_runs, s_total, s_next;

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool any_class = agnostic != 0;
    if (tid == 0) {
        // Written by the decode kernel's atomics: read as a device-scope
        // atomic (a vector load), never through the scalar cache.
        const uint32_t c = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_n = (int)(c < (uint32_t)anchors ? c : (uint32_t)anchors);
        *counter = 0;   // ready for the next replay's decode
        s_runs = 0;
        s_total = 0;
        s_next = kNmsWaves;
    }
    __syncthreads();
    const int n = s_n;   // uniform
    if (n == 0) {
        if (tid == 0) {
            p.out->count = 0;
            p.out->candidates = 0;
        }
        return;
    }

    // 1. Load and sort.
    int P = 64;
    while (P < n) P <<= 1;
    sort_desc<NT>(s, P, tid, keys, n);

    // 2. Class runs (one run of everything when any class suppresses any).
    for (int e = tid; e < n; e += kNmsThreads)
        if (e == 0 || key_group(s[e], any_class) != key_group(s[e - 1], any_class))
            s_run[atomicAdd(&s_runs, 1)] = (uint16_t)e;
    __syncthreads();
    const int runs = s_runs;

    // Longest runs first (up to 64 runs, by one wave): the run starts sorted
    // ascending give each run's length as the distance to the next start,
    // then (length, start) sorted descending is the order the waves take
    // them in.  A start is below 2^14 and a length at most 2^14, so both fit
    // one 32-bit key.
    if (!any_class && runs > 1 && runs <= 64) {   // uniform
        if (wave == 0) {
            const uint32_t start = lane < runs ? s_run[lane] : 0xFFFFu;
            const uint32_t asc = wave_sort<false>(start, lane);
            const uint32_t next = (uint32_t)__shfl_down((int)asc, 1);
            const uint32_t len = (lane + 1 < runs ? next : (uint32_t)n) - asc;
            const uint32_t key = lane < runs ? (len << 16) | asc : 0u;
            const uint32_t ord = wave_sort<true>(key, lane);
            if (lane < runs) s_run[lane] = (uint16_t)(ord & 0xFFFFu);
        }
        __syncthreads();
    }

    // 3. Boxes in sorted order, into the LDS the sort left free (when it fits),
    //    then greedy suppression, one wave per run.
    float4* s_box = nullptr;
    if ((int64_t)(sort_cap - P) * (int64_t)sizeof(uint64_t) >= (int64_t)n * (int64_t)sizeof(float4)) {
        s_box = reinterpret_cast<float4*>(s + P);   // P * 8 is a multiple of 512: 16-byte aligned
        for (int e = tid; e < n; e += kNmsThreads) s_box[e] = p.boxes[key_anchor(s[e], any_class)];
        __syncthreads();
    }
    uint16_t* kept_pos = s_kept + wave * max_det;
    int my_kept = 0;
    // Wave w takes run w first, then whichever run is next when it is done,
    // so long runs do not queue behind each other on one wave.  (With one
    // run, wave 0 resolves it and its kept list is read below.)
    auto next_run = [&]() -> int {
        int r = 0;
        if (lane == 0) r = atomicAdd(&s_next, 1);
        return __builtin_amdgcn_readfirstlane(r);
    };
    if (s_box) {
        for (int r = wave; r < runs; r = next_run())
            my_kept = resolve_run<true>(p, s, s_box, n, s_run[r], kept_pos, any_class, lane);
    } else {
        for (int r = wave; r < runs; r = next_run())
            my_kept = resolve_run<false>(p, s, s_box, n, s_run[r], kept_pos, any_class, lane);
    }
    __syncthreads();

    // 4. Kept boxes in rank order.  With one run, that is its kept list
    //    (wave 0 resolved it).  Otherwise gather the flagged keys of all runs;
    //    up to kRankByCountMax of them are placed by counting (keys are
    //    distinct, so a key's place is the number of kept keys above it),
    //    more are sorted.
    int total;
    if (any_class) {
        if (tid == 0) s_total = my_kept;
        __syncthreads();
        total = s_total;
    } else {
        // 512 positions at a time: every thread reads its key, then the
        // flagged ones are appended.  A slot is below the number of keys
        // flagged so far, hence below every position still to be read.
        for (int base = 0; base < n; base += kNmsThreads) {   // uniform
            const int e = base + tid;
            const uint64_t k = e < n ? s[e] : 0;
            __syncthreads();
            if (k & 1u) s[atomicAdd(&s_total, 1)] = to_rank_key(k);
        }
        __syncthreads();
        total = s_total;
        if (total > kRankByCountMax) {   // uniform
            int P2 = 64;
            while (P2 < total) P2 <<= 1;
            for (int e = total + tid; e < P2; e += kNmsThreads) s[e] = 0;
            __syncthreads();
            sort_desc<NT>(s, P2, tid);
        }
    }

    // 5. The first max_det, mapped to source pixels, to the mapped slot.
    const int count = min(total, max_det);
    auto emit = [&](uint64_t k, int q) {
        const float4 b = p.boxes[key_anchor(k, true)];
        ws_det d;
        d.x1 = to_source(b.x, p.left, p.sx, p.src_w);
        d.y1 = to_source(b.y, p.top, p.sy, p.src_h);
        d.x2 = to_source(b.z, p.left, p.sx, p.src_w);
        d.y2 = to_source(b.w, p.top, p.sy, p.src_h);
        d.score = __uint_as_float((uint32_t)(k >> 33));
        d.class_id = (int32_t)((k >> 7) & 0xFFFu);
        p.out->det[q] = d;
    };
    if (!any_class && total <= kRankByCountMax) {
        for (int t = tid; t < total; t += kNmsThreads) {
            const uint64_t x = s[t];
            const int r = count_above(s, total, x);
            if (r < count) emit(x, r);
        }
    } else {
        for (int q = tid; q < count; q += kNmsThreads)
            emit(any_class ? (s[s_kept[q]] & ~1ull) : s[q], q);
    }
    if (tid == 0) {
        p.out->count = count;
        p.out->candidates = n;
    }
}

static_assert(WS_DET_MAX_ANCHORS <= 16384, "anchors must fit the 14-bit key field");
static_assert(WS_DET_MAX_CLASSES <= 4096, "classes must fit the 12-bit key field");
static_assert(WS_DET_MAX_ANCHORS % kDetNmsThreads == 0 && WS_DET_MAX_ANCHORS % kNmsWideThreads == 0,
              "gather loop covers every key");

}  // namespace

namespace {
int nms_lds_bytes(int sort_cap, int max_det, int threads) {
    return sort_cap * (int)sizeof(uint64_t) + kDetRunCap * (int)sizeof(uint16_t) +
           (threads / 64) * max_det * (int)sizeof(uint16_t);
}

// Dynamic LDS one workgroup may take: 160 KiB on gfx950, less the kernel's
// few bytes of static LDS.
constexpr int kNmsLdsCap = 160 * 1024 - 64;

int nms_threads(int sort_cap, int max_det) {
    return nms_lds_bytes(sort_cap, max_det, kNmsWideThreads) <= kNmsLdsCap ? kNmsWideThreads
                                                                           : kDetNmsThreads;
}
}  // namespace

int det_nms_lds_bytes(int sort_cap, int max_det) {
    return nms_lds_bytes(sort_cap, max_det, nms_threads(sort_cap, max_det));
}

hipError_t set_detect_attributes() {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(det_nms_kernel<kDetNmsThreads>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        nms_lds_bytes(WS_DET_MAX_ANCHORS, WS_DET_MAX_DET, kDetNmsThreads));
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(det_nms_kernel<kNmsWideThreads>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kNmsLdsCap);
    return e;
}

hipError_t launch_detect(const DetParams& p, int decode_groups, hipStream_t stream) {
    hipLaunchKernelGGL(det_decode_kernel, dim3((unsigned)decode_groups), dim3(kDecodeThreads), 0,
                       stream, p.head, p.anchors, p.nc, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nt = nms_threads(p.sort_cap, p.max_det);
    const unsigned lds = (unsigned)nms_lds_bytes(p.sort_cap, p.max_det, nt);
    auto nms = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3(1), dim3(threads), lds, stream, p.counter, p.keys,
                           p.anchors, p.sort_cap, p.agnostic, p.max_det, p);
    };
    if (nt == kNmsWideThreads)
        nms(det_nms_kernel<kNmsWideThreads>, kNmsWideThreads);
    else
        nms(det_nms_kernel<kDetNmsThreads>, kDetNmsThreads);
    return hipGetLastError();
}

}  // namespace ws
