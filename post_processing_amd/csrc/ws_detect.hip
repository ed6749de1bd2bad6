// ws_detect.hip -- detection decode + greedy NMS for gfx950 (CDNA4, wave64).
//
// yolo.cu README: the end-to-end pipeline passage (DFL decode and NMS inside
// the frame's one graph launch), the "GPU-resident NMS" highlight (greedy
// suppression over the live candidates in score order; only the final boxes,
// about 7 KB, cross to pinned memory) and the embedding example (up to 300
// boxes in source-image coordinates).
//
// det_decode_kernel (one workgroup per 64 anchors, four waves): wave w finds
//   each anchor's best class within the w-th quarter of the classes (all of
//   a lane's loads in flight together); the anchors above the confidence
//   threshold are numbered in anchor order by a ballot, and the workgroup
//   writes its candidate count, their keys and boxes to its own 64 slots
//   (slot order is anchor order).  Wave 0 also gives each candidate its
//   place among the frame's candidates of its class: one atomic per class
//   present on that class's counter.  Waves 1-3 compute the DFL distances,
//   one lane per (candidate, box side).
// det_nms_kernel (one workgroup of 16 waves, or 8 when 16 waves' kept-box
// lists do not fit LDS beside the keys):
//   0. reads the class counters (and clears them for the next frame) and
//      the per-workgroup candidate counts, whose prefix sums number the
//      candidates;
//   1. class-aware mode: the class counts' prefix sums give each class's
//      start, so each class is a contiguous run; any-class mode: one run;
//   2. gathers every candidate's key (and box, when LDS has room) straight
//      to its class's start plus its place;
//   3. one wave resolves a class run of up to 512 candidates from its
//      registers by selection -- the largest live key is the next kept box
//      and suppresses the live candidates it overlaps -- switching to a sort
//      of the live keys once the run has kept eight boxes (runs longest
//      first, one wave each).  With any longer run, or when boxes of any
//      class suppress each other, the whole list is sorted by the workgroup
//      instead (bitonic; the key orders by class first in class-aware mode,
//      so runs stay contiguous) and resolved in rank order, 64 candidates at
//      a time: each is tested against the run's boxes kept so far, then the
//      first live candidate is kept and suppresses the live ones after it,
//      and so on.  The any-class run and any class run longer than 512 are
//      resolved by all waves together (each wave screens one block against
//      the kept boxes, then one wave settles the blocks in order).  Boxes of
//      different classes never interact, so class runs are independent;
//   4. orders the kept boxes of all classes by probability descending, anchor
//      ascending -- the order in which plain greedy suppression over all
//      candidates keeps them -- and writes the first max_det.
//
// All arithmetic that decides a result (DFL exponentials, boxes, IoU,
// mapping) is binary32 with one rounding per operation in a fixed order:
// fused multiply-add is switched off below, and division is IEEE (the
// library is built with correctly rounded fp32 division).  The IoU
// threshold test reaches the same decision as dividing and comparing, by an
// exact comparison in binary64 (iou_above).
#include <hip/hip_runtime.h>

#include "ws_detect.h"
#include "ws_lanes.h"
#include "ws_marks.h"

namespace ws {
namespace {

#ifdef WS_CLOCK_MARKS
// Phase marks of the detection kernels: the decode kernel's wave w of
// workgroup g writes slots (4 g + w) * 8 + phase, the suppression kernel's
// wave w slots kNmsMarks + 16 w + phase.
__device__ uint64_t g_marks[kMarkSlots];
#endif
constexpr int kNmsMarks = 1 << 16;
// Instrumented builds: per-wave totals (shader clock cycles, counts) of the
// suppression phases at kNmsProf + 8 w + {0 block loads, 1 screening
// (cooperative runs: every wave's part of each round), 2 settling
// (cooperative runs: wave 0's part of each round), 3 screening steps, 4 kept
// boxes, 5 blocks, 6 round barrier waits, 7 wave 0's screening within
// rounds}.
[[maybe_unused]] constexpr int kNmsProf = kNmsMarks + 4096;
#ifdef WS_CLOCK_MARKS
#define WS_PROF_T(v) const uint64_t v = __builtin_amdgcn_s_memtime()
#define WS_PROF_WAIT() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory")
#define WS_PROF_DECL uint64_t prof_[8] = {0, 0, 0, 0, 0, 0, 0, 0}
#define WS_PROF_ACC(slot_, val_) prof_[slot_] += (uint64_t)(val_)
#define WS_PROF_FLUSH()                                                                  \
    do {                                                                                 \
        if ((threadIdx.x & 63) == 0)                                                     \
            for (int q_ = 0; q_ < 8; ++q_) g_marks[kNmsProf + 8 * (threadIdx.x >> 6) + q_] += prof_[q_]; \
    } while (0)
#else
#define WS_PROF_T(v)
#define WS_PROF_WAIT()
#define WS_PROF_DECL
#define WS_PROF_ACC(slot_, val_)
#define WS_PROF_FLUSH()
#endif

constexpr int kDecodeBlock = kDetDecodeAnchors;
constexpr int kDecodeParts = 4;               // class ranges per anchor, one wave each
constexpr int kDecodeThreads = kDecodeParts * kDecodeBlock;
constexpr int kScanBatch = 32;                // class loads a lane keeps in flight
constexpr int kBins = WS_DET_REG_MAX;
// The suppression kernel runs with 1,024 threads when its LDS allows (more
// class runs in flight: each wave's run is a chain of dependent steps), else
// with 512.
constexpr int kNmsWide = 1024;
constexpr int kNmsNarrow = 512;
// Class runs up to this long are sorted by one wave in registers.
constexpr int kRunSortMax = 512;
// LDS of the suppression kernel, in 16-bit words: run starts (one per
// class, a sentinel, and 64 run lengths), prefix sums of the decode counts.
constexpr int kRunCap = WS_DET_MAX_CLASSES;
constexpr int kRunLen = kRunCap + 1;          // run lengths (ordered runs only) start here
constexpr int kRunSlots = kRunCap + 1 + 64 + 7;
constexpr int kPreSlots = kDetMaxGroups + 8;
// Long runs resolved by all waves: at most WS_DET_MAX_ANCHORS / 513.
constexpr int kCoopCap = 32;
// NaN boxes past the kept list of a run resolved by all waves.
constexpr int kCoopPad = 8;

static_assert(WS_DET_MAX_ANCHORS <= 16384, "slots must fit the 14-bit key field");
static_assert(WS_DET_MAX_CLASSES <= 4096, "classes must fit the 12-bit key field");
static_assert(WS_DET_MAX_ANCHORS % kNmsNarrow == 0 && WS_DET_MAX_ANCHORS % kNmsWide == 0,
              "bucketing registers cover every key");
static_assert(WS_DET_MAX_CLASSES % kNmsNarrow == 0 && WS_DET_MAX_CLASSES % kNmsWide == 0,
              "class prefix sums cover every class");
static_assert(kDetMaxGroups < kNmsNarrow, "one thread per decode workgroup count, and the total");
static_assert(WS_DET_MAX_ANCHORS / (kRunSortMax + 1) < kCoopCap, "long-run list capacity");
static_assert((kRunSlots * 2) % 16 == 0 && (kPreSlots * 2) % 16 == 0, "16-byte aligned regions");

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
__device__ __forceinline__ void dfl_load(const float* __restrict__ q, int A, float (&l)[kBins]) {
#pragma unroll
    for (int b = 0; b < kBins; ++b) l[b] = q[(size_t)b * A];
}

__device__ __forceinline__ float dfl_side(const float (&l)[kBins]) {
#pragma clang fp contract(off)
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

// Area of an xyxy box, binary32: (x2 - x1) * (y2 - y1).
__device__ __forceinline__ float box_area(float4 b) {
#pragma clang fp contract(off)
    return (b.z - b.x) * (b.w - b.y);
}

// Whether IoU(a, b) > t for kept box a and candidate b (xyxy) with their
// areas, where the IoU is binary32: areas, clipped intersection sides,
// intersection, union = (area_a + area_b) - inter, each rounded once, then
// inter / union rounded once.  The division is not carried out.  With t+
// the next binary32 above t and m their midpoint, the rounded quotient
// exceeds t exactly when inter / union > m, or equals m and the tie rounds
// up to t+ (t+ has the even significand, i.e. t's is odd).  inter and union
// are binary32 and m has 25 significant bits, so m * union is exact in
// binary64 and the test is exact.  A zero union (0 / 0 = NaN) and NaN boxes
// suppress nothing.
__device__ __forceinline__ bool iou_above(float4 a, float area_a, float4 b, float area_b, double mid,
                                          bool tie_up) {
#pragma clang fp contract(off)
    const float iw = fmaxf(0.0f, fminf(a.z, b.z) - fmaxf(a.x, b.x));
    const float ih = fmaxf(0.0f, fminf(a.w, b.w) - fmaxf(a.y, b.y));
    const float inter = iw * ih;
    const float uni = (area_a + area_b) - inter;
    const double bound = mid * (double)uni;
    const double in = (double)inter;
    // Bitwise, not short-circuit: every compare is evaluated, no branches.
    return (uni > 0.0f) & ((in > bound) | (tie_up & (in == bound)));
}

// v_min_f32 / v_max_f32 as written: the compiler would first quiet every
// operand it cannot prove canonical (one more instruction per value read
// from memory).  Boxes are results of arithmetic, never signalling NaNs, and
// on quiet NaNs these give what fminf / fmaxf give.
__device__ __forceinline__ float min_raw(float a, float b) {
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// iou_above with the tie rule fixed at compile time, for the screening
// loops.  Candidate boxes have x2 >= x1 and y2 >= y1 (the DFL distances are
// expectations over non-negative bins), so union >= 0, and union == 0 gives
// bound == 0 == inter, which "inter > bound" already rejects; only the tie
// case needs union > 0 spelled out.  NaN boxes compare false everywhere.
template <bool TIE>
__device__ __forceinline__ bool iou_above_fixed(float4 a, float area_a, float4 b, float area_b, double mid) {
#pragma clang fp contract(off)
    const float iw = max_raw(0.0f, min_raw(a.z, b.z) - max_raw(a.x, b.x));
    const float ih = max_raw(0.0f, min_raw(a.w, b.w) - max_raw(a.y, b.y));
    const float inter = iw * ih;
    const float uni = (area_a + area_b) - inter;
    const double bound = mid * (double)uni;
    const double in = (double)inter;
    if (TIE) return (in > bound) | ((in == bound) & (uni > 0.0f));
    return in > bound;
}

// Network-input pixels -> source pixels, clipped to [0, hi].
__device__ __forceinline__ float to_source(float v, float origin, float scale, float hi) {
#pragma clang fp contract(off)
    return fminf(fmaxf((v - origin) * scale, 0.0f), hi);
}

// ---------------------------------------------------------------------------
// Candidate keys.  Larger keys come first; every key is non-zero and unique
// (the slot is in it), and bit 0 is free (it marks kept candidates).
//   by class:  [63:52] 4095 - class, [51:21] probability bits, [20:7] 16383 - slot
//   any class: [63:33] probability bits, [32:19] 16383 - slot, [18:7] class
// The probability is > conf >= 0, so its sign bit is clear and its bits order
// as integers.  Slots order candidates as their anchors do, so the second
// layout is also the rank order of the output.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t make_key(bool any_class, uint32_t prob, int slot, int cls) {
    const uint64_t pr = prob & 0x7FFFFFFFu;
    const uint64_t sl = (uint64_t)(0x3FFF - slot);
    if (any_class) return (pr << 33) | (sl << 19) | ((uint64_t)cls << 7);
    return ((uint64_t)(0xFFF - cls) << 52) | (pr << 21) | (sl << 7);
}

__device__ __forceinline__ int key_slot(uint64_t k, bool any_class) {
    return 0x3FFF - (int)((k >> (any_class ? 19 : 7)) & 0x3FFFu);
}

// Class of a class-ordered key.
__device__ __forceinline__ int key_class(uint64_t k) { return 0xFFF - (int)(k >> 52); }

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

__device__ __forceinline__ float readlanef(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------------------
// Prefix sums
// ---------------------------------------------------------------------------

// Inclusive prefix sum across a wave64 by DPP: shifts of 1, 2, 4 and 8
// lanes inside each row of 16 (a lane with no source adds 0), then row 0's
// total to row 1 and row 2's to row 3 (row_bcast:15), then rows 0-1's total
// to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
    return v;
}

// Largest 64-bit value across a wave64 (every lane gets it).
__device__ __forceinline__ uint64_t wave_max64(uint64_t v, int lane) {
    v = umax64(v, xor_lane64<1>(v, lane));
    v = umax64(v, xor_lane64<2>(v, lane));
    v = umax64(v, xor_lane64<4>(v, lane));
    v = umax64(v, xor_lane64<8>(v, lane));
    v = umax64(v, xor_lane64<16>(v, lane));
    v = umax64(v, xor_lane64<32>(v, lane));
    return v;
}

// Largest 32-bit value across a wave64 (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v, int lane) {
    v = max(v, xor_lane32<1>(v, lane));
    v = max(v, xor_lane32<2>(v, lane));
    v = max(v, xor_lane32<4>(v, lane));
    v = max(v, xor_lane32<8>(v, lane));
    v = max(v, xor_lane32<16>(v, lane));
    return max(v, xor_lane32<32>(v, lane));
}

// Exclusive prefix sum of one value per thread over the workgroup, and the
// total (uniform).  Starts and ends with a barrier, so s_tot may be reused
// right after.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_tot, uint32_t& total, int tid) {
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint32_t incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) s_tot[wave] = incl;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t t = s_tot[w];
        base += w < wave ? t : 0u;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return base + incl - v;
}

// ---------------------------------------------------------------------------
// Sorting
// ---------------------------------------------------------------------------

// Block sort of keys in LDS (bitonic network, descending): each wave sorts
// blocks of 64*K keys in registers (sort_block), and only distances of a
// whole block or more go through LDS.

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

// Sorts s[0, P) descending, P a power of two with 64 <= P and P / (64 K)
// blocks.  Ends with a barrier.
template <int NT, int K>
__device__ __forceinline__ void sort_desc_k(uint64_t* s, int P, int tid) {
    constexpr int Q = 64 * K;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blocks = P / Q;
    for (int b = wave; b < blocks; b += NT / 64) {
        uint64_t x[K];
#pragma unroll
        for (int r = 0; r < K; ++r) x[r] = s[b * Q + r * 64 + lane];
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
__device__ __forceinline__ void sort_desc(uint64_t* s, int P, int tid) {
    if (P <= 512) sort_desc_k<NT, 1>(s, P, tid);
    else if (P == 1024) sort_desc_k<NT, 2>(s, P, tid);
    else if (P == 2048) sort_desc_k<NT, 4>(s, P, tid);
    else sort_desc_k<NT, 8>(s, P, tid);
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
    __shared__ uint16_t s_off[kDecodeBlock];
    __shared__ int s_n;
    const int tid = (int)threadIdx.x;
    const int lane = tid & (kDecodeBlock - 1);
    const int A = anchors;
    const int g = (int)blockIdx.x;
    [[maybe_unused]] const int mark = (g * 4 + (tid >> 6)) * 8;
    WS_MARK(mark + 0);

    // 1. Best class (first maximum; NaN never compares greater) and threshold.
    //    Wave w scans the w-th quarter of the classes of the group's anchors,
    //    up to kScanBatch loads in flight per lane (past the range a lane
    //    re-reads the range's last class and ignores it).
    const int a = g * kDecodeBlock + lane;
    const int part = tid / kDecodeBlock;   // wave-uniform
    const int per = (nc + kDecodeParts - 1) / kDecodeParts;
    const int c_begin = min(nc, part * per);
    const int c_end = min(nc, c_begin + per);
    float best = -INFINITY;
    int cls = c_begin;
    if (a < A) {
        const float* __restrict__ pr = head + (size_t)(4 * kBins) * A + a;
        for (int c0 = c_begin; c0 < c_end; c0 += kScanBatch) {
            float v[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) v[j] = pr[(size_t)min(c0 + j, c_end - 1) * A];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                if (c0 + j < c_end && v[j] > best) {
                    best = v[j];
                    cls = c0 + j;
                }
        }
    }
    WS_MARK(mark + 1);
    s_pbest[part][lane] = best;
    s_pcls[part][lane] = cls;
    __syncthreads();
    if (part == 0) {
        // Later ranges win only when strictly greater: ties keep the first.
        best = -INFINITY;
        cls = 0;
#pragma unroll
        for (int q = 0; q < kDecodeParts; ++q)
            if (s_pbest[q][lane] > best) {
                best = s_pbest[q][lane];
                cls = s_pcls[q][lane];
            }
        // Candidates numbered in anchor (lane) order.
        const bool cand = a < A && best > p.conf;
        const uint64_t m = __ballot(cand);
        if (cand) {
            const int q = lanes_below(m);
            s_anchor[q] = a;
            s_cls[q] = cls;
            s_prob[q] = __float_as_uint(best);
        }
        if (lane == 0) {
            const int n = __popcll(m);
            s_n = n;
            p.counts[g] = (uint32_t)n;
        }
    }
    __syncthreads();
    WS_MARK(mark + 2);
    const int n = s_n;   // uniform
    if (n == 0) return;

    const bool any_class = p.agnostic != 0;
    if (part == 0) {
        // 2a. Each candidate's place among the frame's candidates of its
        //     class (any-class mode: all are one class): the lanes sort
        //     (class, candidate) pairs, the first lane of each class takes
        //     that many places from the class's counter (one atomic per
        //     class present, all in one instruction), and the others follow
        //     it.  Overlaps the other waves' DFL loads.
        const bool v = lane < n;
        const uint32_t c = v ? (any_class ? 0u : (uint32_t)s_cls[lane]) : 0xFFFFu;
        const uint32_t e = wave_sort<false>((c << 6) | (uint32_t)lane, lane);
        const uint32_t ec = e >> 6;
        const bool ev = lane < n;   // invalid pairs sort last
        const uint32_t prev = (uint32_t)__shfl_up((int)ec, 1);
        const bool head = ev && (lane == 0 || prev != ec);
        const uint64_t heads = __ballot(head);
        const uint64_t above = heads & ~((2ull << lane) - 1);
        const int next = above ? __ffsll((unsigned long long)above) - 1 : n;
        uint32_t base = 0;
        if (head) base = atomicAdd(&p.cls_counts[ec], (uint32_t)(next - lane));
        const int mine = 63 - __clzll((long long)(heads & ((2ull << lane) - 1)));
        const uint32_t hb = (uint32_t)__shfl((int)base, mine);
        if (ev) s_off[e & 63u] = (uint16_t)(hb + (uint32_t)(lane - mine));
    } else {
        // 2b. DFL distances, one lane per (candidate, side), on waves 1-3:
        //     up to two pairs per lane, all 16 or 32 loads issued before any
        //     arithmetic.
        const int t0 = tid - kDecodeBlock;
        constexpr int kPairStride = kDecodeThreads - kDecodeBlock;
        const bool h0 = t0 < 4 * n, h1 = t0 + kPairStride < 4 * n;
        float l0[kBins], l1[kBins];
        if (h0) dfl_load(head + (size_t)((t0 & 3) * kBins) * A + s_anchor[t0 >> 2], A, l0);
        if (h1) {
            const int t1 = t0 + kPairStride;
            dfl_load(head + (size_t)((t1 & 3) * kBins) * A + s_anchor[t1 >> 2], A, l1);
        }
        if (h0) s_dist[t0 >> 2][t0 & 3] = dfl_side(l0);
        if (h1) s_dist[(t0 + kPairStride) >> 2][(t0 + kPairStride) & 3] = dfl_side(l1);
    }
    WS_MARK_AFTER_LOADS(mark + 3);
    __syncthreads();
    WS_MARK(mark + 4);

    // 3. Boxes, keys and class places to the group's slots.  The grid bounds
    //    are read with constant indices (scalar loads of the kernel
    //    arguments).
    const int le0 = p.level_end[0], le1 = p.level_end[1];
    const int gw0 = p.grid_w[0], gw1 = p.grid_w[1], gw2 = p.grid_w[2];
    for (int q = tid; q < n; q += kDecodeThreads) {
        const int aq = s_anchor[q];
        const int level = aq < le0 ? 0 : (aq < le1 ? 1 : 2);
        const int cell = aq - (level == 0 ? 0 : (level == 1 ? le0 : le1));
        const int gw = level == 0 ? gw0 : (level == 1 ? gw1 : gw2);
        const float cx = (float)(cell % gw) + 0.5f;
        const float cy = (float)(cell / gw) + 0.5f;
        const float st = (float)(8 << level);
        const int slot = g * kDecodeBlock + q;   // < anchors: q counts anchors of this group
        p.boxes[slot] = make_float4((cx - s_dist[q][0]) * st, (cy - s_dist[q][1]) * st,
                                    (cx + s_dist[q][2]) * st, (cy + s_dist[q][3]) * st);
        p.keys[slot] = make_key(any_class, s_prob[q], slot, s_cls[q]);
        p.offs[slot] = s_off[q];
    }
    WS_MARK(mark + 5);
}

// ---------------------------------------------------------------------------
// Suppression
// ---------------------------------------------------------------------------

// Box of sorted position e holding key k: staged in sorted order in LDS, or
// read by slot from global memory.  The choice is a template argument so
// that each instance loads from one address space (a run-time choice between
// the two pointers compiles to generic loads that wait on both memory
// counters).
template <bool STAGED>
__device__ __forceinline__ float4 box_at(const DetParams& p, const float4* s_box, int e, uint64_t k,
                                         bool any_class) {
    return STAGED ? s_box[e] : p.boxes[key_slot(k, any_class)];
}

// Tests the 64 candidates of one block (box and area per lane; alive: the
// live ones) against kept boxes k0 .. k1 - 1 of the run and returns the
// candidates still alive.  U kept boxes per step, all fetched before any
// test so that the U tests overlap (a last step short of U boxes repeats
// box k1 - 1, which changes nothing).  kept(j, box, area) gives kept box j
// and its area (wave-uniform j).
template <int U, bool TIE, bool PADDED, typename Kept>
__device__ __forceinline__ uint64_t screen_t(uint64_t alive, float4 box, float area, int k0, int k1, Kept kept,
                                            double mid, int& steps) {
    for (int k = k0; k < k1 && alive != 0; k += U) {
        ++steps;
        float4 a[U];
        float aa[U];
#pragma unroll
        for (int u = 0; u < U; ++u) kept(PADDED ? k + u : min(k + u, k1 - 1), a[u], aa[u]);
        bool sup = false;
#pragma unroll
        for (int u = 0; u < U; ++u) sup |= iou_above_fixed<TIE>(a[u], aa[u], box, area, mid);
        alive &= ~(uint64_t)__ballot(sup);
    }
    return alive;
}

// PADDED: kept(j) is defined (a box that suppresses nothing) up to k1 + U - 1,
// so a short last step reads past k1 instead of repeating box k1 - 1.
template <int U, bool PADDED = false, typename Kept>
__device__ __forceinline__ uint64_t screen(uint64_t alive, float4 box, float area, int k0, int k1, Kept kept,
                                          double mid, bool tie_up, int& steps) {
    return tie_up ? screen_t<U, true, PADDED>(alive, box, area, k0, k1, kept, mid, steps)
                  : screen_t<U, false, PADDED>(alive, box, area, k0, k1, kept, mid, steps);
}

// Greedy suppression of one run s[s0, s0 + len) by one wave, in rank order
// (s sorted descending).  kept_pos holds the positions of the kept0 boxes of
// the run kept before s0 (all ranked above it).  Kept candidates get bit 0
// set in s and their positions listed in kept_pos (capacity max_det).
// Returns how many the run keeps in all.
template <bool STAGED>
__device__ __forceinline__ int resolve_run(const DetParams& p, uint64_t* s, const float4* s_box, int s0, int len,
                           uint16_t* kept_pos, bool any_class, int lane, int kept0 = 0) {
#pragma clang fp contract(off)
    const double mid = p.iou_mid;
    const bool tie_up = p.iou_tie_up != 0;
    const int end = s0 + len;
    int kept = kept0;
    [[maybe_unused]] int steps = 0;
    WS_PROF_DECL;
    for (int c0 = s0; c0 < end; c0 += 64) {
        wave_lds_sync();   // kept_pos writes of the previous block are visible
        WS_PROF_T(t0);
        const int e = c0 + lane;
        const bool valid = e < end;
        const uint64_t key = valid ? s[e] : 0;
        // Branches rather than a conditional over lvalues, which would give
        // the zero box a private-memory copy.
        float4 box = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) box = box_at<STAGED>(p, s_box, e, key, any_class);
        const float area = box_area(box);
        uint64_t alive = __ballot(valid);
        WS_PROF_WAIT();
        WS_PROF_T(t1);

        // Boxes of this run kept in earlier blocks, 64 at a time in registers.
        for (int kb = 0; kb < kept && alive != 0; kb += 64) {
            const int kl = kb + lane;
            float4 kbox = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kl < kept) {
                const int pos = kept_pos[kl];
                kbox = STAGED ? s_box[pos] : p.boxes[key_slot(s[pos], any_class)];
            }
            const float karea = box_area(kbox);
            alive = screen<4>(alive, box, area, kb, min(kb + 64, kept),
                              [&](int j, float4& a, float& aa) {
                                  a = readlane4(kbox, j - kb);
                                  aa = readlanef(karea, j - kb);
                              },
                              mid, tie_up, steps);
        }
        WS_PROF_T(t2);

        // This block: the first live candidate is the next kept box.
        uint64_t pending = alive;
        bool full = false;
        while (pending != 0) {
            const int i = __ffsll((unsigned long long)pending) - 1;
            if (lane == i) {
                kept_pos[kept] = (uint16_t)e;
                s[e] = key | 1u;
            }
            ++kept;
            WS_PROF_ACC(4, 1);
            if (kept == p.max_det) {
                full = true;
                break;
            }
            const bool sup =
                (lane > i) & iou_above(readlane4(box, i), readlanef(area, i), box, area, mid, tie_up);
            alive &= ~(uint64_t)__ballot(sup);
            pending = alive & ~((2ull << i) - 1);   // candidates after i
        }
        WS_PROF_T(t3);
        WS_PROF_ACC(0, t1 - t0);
        WS_PROF_ACC(1, t2 - t1);
        WS_PROF_ACC(2, t3 - t2);
        WS_PROF_ACC(5, 1);
        if (full) break;
    }
    WS_PROF_ACC(3, steps);
    WS_PROF_FLUSH();
    return kept;
}

// Greedy suppression of one long run s[s0, s0 + len) by all waves, NT
// candidates per round: every wave screens one block of 64 against the boxes
// kept before the round (the bulk of the tests, in parallel), then wave 0
// takes the round's blocks in order, screens each against the boxes kept
// earlier in the round and settles it as resolve_run does.  Kept boxes,
// their areas and positions go to k_box / k_area / k_pos in rank order
// (capacity max_det); kept candidates get bit 0 set in s.  Returns how many
// were kept (uniform).
template <bool STAGED, int NT>
__device__ __forceinline__ int coop_resolve(const DetParams& p, uint64_t* s, const float4* s_box, int s0, int len,
                            float4* k_box, float* k_area, uint16_t* k_pos, uint64_t* s_alive, int* s_kept,
                            bool any_class, int tid) {
#pragma clang fp contract(off)
    constexpr int W = NT / 64;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const double mid = p.iou_mid;
    const bool tie_up = p.iou_tie_up != 0;
    const int end = s0 + len;
    // Uniform LDS addresses: broadcast reads.  Entries past the kept ones
    // hold NaN boxes, which suppress nothing (the screening reads up to
    // seven past the end).
    auto kept = [&](int j, float4& a, float& aa) {
        a = k_box[j];
        aa = k_area[j];
    };
    const float qnan = __uint_as_float(0x7FC00000u);
    for (int j = tid; j < p.max_det + kCoopPad; j += NT) {
        k_box[j] = make_float4(qnan, qnan, qnan, qnan);
        k_area[j] = qnan;
    }
    __syncthreads();
    int K = 0;
    [[maybe_unused]] int steps = 0, round_steps = 0;
    WS_PROF_DECL;
    for (int w0 = s0; w0 < end; w0 += NT) {
        const int K0 = K;
        WS_PROF_T(ta);
        {
            const int e = w0 + wave * 64 + lane;
            const bool valid = e < end;
            float4 box = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) box = box_at<STAGED>(p, s_box, e, s[e], any_class);
            const uint64_t alive =
                screen<8, true>((uint64_t)__ballot(valid), box, box_area(box), 0, K0, kept, mid, tie_up, steps);
            if (lane == 0) s_alive[wave] = alive;
        }
        WS_PROF_T(tb);
        WS_PROF_ACC(1, tb - ta);
        __syncthreads();
        WS_PROF_T(tc);
        WS_PROF_ACC(6, tc - tb);
        if (wave == 0) {
            bool full = false;
            for (int b = 0; b < W && !full; ++b) {
                const int c0 = w0 + b * 64;
                if (c0 >= end) break;
                wave_lds_sync();   // k_box writes of earlier blocks are visible
                WS_PROF_T(t0);
                const int e = c0 + lane;
                const bool valid = e < end;
                const uint64_t key = valid ? s[e] : 0;
                float4 box = make_float4(0.f, 0.f, 0.f, 0.f);
                if (valid) box = box_at<STAGED>(p, s_box, e, key, any_class);
                const float area = box_area(box);
                WS_PROF_WAIT();
                WS_PROF_T(t1);
                uint64_t alive = screen<4, true>(s_alive[b], box, area, K0, K, kept, mid, tie_up, round_steps);
                WS_PROF_T(t2);
                WS_PROF_ACC(0, t1 - t0);
                WS_PROF_ACC(7, t2 - t1);
                WS_PROF_ACC(5, 1);
                uint64_t pending = alive;
                while (pending != 0) {
                    const int i = __ffsll((unsigned long long)pending) - 1;
                    if (lane == i) {
                        k_box[K] = box;
                        k_area[K] = area;
                        k_pos[K] = (uint16_t)e;
                        s[e] = key | 1u;
                    }
                    ++K;
                    WS_PROF_ACC(4, 1);
                    if (K == p.max_det) {
                        full = true;
                        break;
                    }
                    const bool sup = (lane > i) & iou_above(readlane4(box, i), readlanef(area, i), box,
                                                            area, mid, tie_up);
                    alive &= ~(uint64_t)__ballot(sup);
                    pending = alive & ~((2ull << i) - 1);
                }
            }
            if (lane == 0) *s_kept = K;
        }
        WS_PROF_T(td);
        if (wave == 0) WS_PROF_ACC(2, td - tc);
        __syncthreads();
        K = *s_kept;
        if (K >= p.max_det) break;
    }
    WS_PROF_ACC(3, steps);
    WS_PROF_FLUSH();
    return K;
}

// Kept boxes a class run resolves by selection before it switches to
// sorting what is left (selection costs a pass over the run per kept box).
constexpr int kSelectBudget = 8;

// Greedy suppression of one class run s[s0, s0 + len), len <= 64 K, in one
// wave.  The run is held K keys per lane in registers and resolved by
// selection: the largest live key is the next kept box (every candidate of
// the run ranked above it is kept or suppressed by then, which is the greedy
// order), it suppresses the live candidates it overlaps, and so on; dead
// candidates get key 0.  A run that keeps kSelectBudget boxes with
// candidates still alive is finished in rank order instead: the live keys
// are sorted in registers and laid out after the kept ones, the rest of the
// run is cleared, and resolve_run continues from the kept list.  Boxes are
// staged at the run's positions in s_box and by compact position in s_tmp
// (STAGED), or read by slot.  Kept
// candidates get bit 0 set in s.  Returns how many were kept.
template <int K, bool STAGED>
__device__ __forceinline__ int select_run_k(const DetParams& p, uint64_t* s, float4* s_box, const float4* s_tmp,
                            const uint16_t* s_pre, int s0, int len, uint16_t* kept_pos, int lane) {
#pragma clang fp contract(off)
    const double mid = p.iou_mid;
    const bool tie_up = p.iou_tie_up != 0;
    auto staged_box = [&](uint64_t k) {
        const int slot = key_slot(k, false);
        return s_tmp[s_pre[slot >> 6] + (slot & 63)];
    };
    uint64_t key[K];
    float4 box[K];
    float area[K];
#pragma unroll
    for (int r = 0; r < K; ++r) {
        const int e = r * 64 + lane;
        key[r] = e < len ? s[s0 + e] : 0;
        box[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < len) box[r] = STAGED ? s_box[s0 + e] : p.boxes[key_slot(key[r], false)];
        area[r] = box_area(box[r]);
    }
    int kept = 0;
    bool live = false;
    WS_PROF_DECL;
    while (true) {
        // The largest live key: first its bits 52..21 (the run's class bit
        // and the probability; a dead key is 0) by a 32-bit reduction, then,
        // only when several candidates share that probability, the largest
        // full key among them.
        uint32_t hp[K];
#pragma unroll
        for (int r = 0; r < K; ++r) hp[r] = (uint32_t)(key[r] >> 21);
        uint32_t mh = hp[0];
#pragma unroll
        for (int r = 1; r < K; ++r) mh = max(mh, hp[r]);
        mh = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_u32(mh, lane));
        if (mh == 0) break;
        if (kept == kSelectBudget && K > 1) {   // uniform
            live = true;
            break;
        }
        // Its register and lane (keys are distinct).
        int rs = 0, ls = 0, ties = 0;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            const uint64_t b = __ballot(hp[r] == mh);
            ties += __popcll(b);
            if (b) {
                rs = r;
                ls = __ffsll((unsigned long long)b) - 1;
            }
        }
        if (ties > 1) {   // uniform: equal probabilities, the slot decides
            uint64_t m = 0;
#pragma unroll
            for (int r = 0; r < K; ++r) m = umax64(m, hp[r] == mh ? key[r] : 0);
            const uint64_t t = readlane64(wave_max64(m, lane), 0);
#pragma unroll
            for (int r = 0; r < K; ++r) {
                const uint64_t b = __ballot(key[r] == t);
                if (b) {
                    rs = r;
                    ls = __ffsll((unsigned long long)b) - 1;
                }
            }
        }
        float4 kb = make_float4(0.f, 0.f, 0.f, 0.f);
        float ka = 0.0f;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            if (r == rs) {
                kb = readlane4(box[r], ls);
                ka = readlanef(area[r], ls);
                if (lane == ls) {
                    s[s0 + r * 64 + ls] = key[r] | 1u;
                    kept_pos[kept] = (uint16_t)(s0 + r * 64 + ls);
                    key[r] = 0;
                }
            }
        }
        ++kept;
        WS_PROF_ACC(4, 1);
        if (kept == p.max_det) break;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            if (__ballot(key[r] != 0) != 0) {
                if (iou_above(kb, ka, box[r], area[r], mid, tie_up)) key[r] = 0;
            }
        }
    }
    if (live) {   // uniform
        // Kept keys first, then the live ones in rank order, then zeros.
        sort_block<K>(key, true, lane);
        int nlive = 0;
#pragma unroll
        for (int r = 0; r < K; ++r) nlive += __popcll(__ballot(key[r] != 0));
        wave_lds_sync();   // kept_pos written
        const uint64_t kk = lane < kept ? s[kept_pos[lane]] : 0;
        wave_lds_sync();   // kept keys read before the run is rewritten
        if (lane < kept) {
            s[s0 + lane] = kk;
            kept_pos[lane] = (uint16_t)(s0 + lane);
        }
#pragma unroll
        for (int r = 0; r < K; ++r) {
            const int e = r * 64 + lane;
            if (e < nlive) s[s0 + kept + e] = key[r];
        }
        for (int e = kept + nlive + lane; e < len; e += 64) s[s0 + e] = 0;
        wave_lds_sync();
        if (STAGED) {
            for (int e = lane; e < kept + nlive; e += 64) s_box[s0 + e] = staged_box(s[s0 + e]);
            wave_lds_sync();
        }
        kept = resolve_run<STAGED>(p, s, s_box, s0 + kept, nlive, kept_pos, false, lane, kept);
    }
    WS_PROF_FLUSH();
    return kept;
}

// A class run of up to kRunSortMax candidates, by one wave (select_run_k).
template <bool STAGED>
__device__ __forceinline__ int select_run(const DetParams& p, uint64_t* s, float4* s_box, const float4* s_tmp,
                                          const uint16_t* s_pre, int s0, int len, uint16_t* kept_pos,
                                          int lane) {
    if (len == 1) {   // a lone candidate is kept
        if (lane == 0) s[s0] |= 1u;
        return 1;
    }
    if (len <= 64) return select_run_k<1, STAGED>(p, s, s_box, s_tmp, s_pre, s0, len, kept_pos, lane);
    if (len <= 128) return select_run_k<2, STAGED>(p, s, s_box, s_tmp, s_pre, s0, len, kept_pos, lane);
    if (len <= 256) return select_run_k<4, STAGED>(p, s, s_box, s_tmp, s_pre, s0, len, kept_pos, lane);
    return select_run_k<8, STAGED>(p, s, s_box, s_tmp, s_pre, s0, len, kept_pos, lane);
}

// Decode group holding compact position i: the last g with s_pre[g] <= i
// (binary search over s_pre[0 .. groups], s_pre[groups] = n > i).
__device__ __forceinline__ int group_of(const uint16_t* s_pre, int groups, int i) {
    int lo = 0, hi = groups;   // s_pre[lo] <= i < s_pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)s_pre[mid] <= i) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Keys (and, with STAGED, boxes) of every candidate: each thread takes
// compact positions i = tid, tid + NT, ..., finds each one's slot and issues
// the loads of up to four positions before storing any.  A candidate goes
// to its class bucket, cstart[class] + its place in the class (the boxes to
// s_box at the same place), and with STAGED its box also to s_tmp[i].
template <int NT, bool STAGED>
__device__ __forceinline__ void gather(const DetParams& p, const uint64_t* __restrict__ keys, uint64_t* s,
                                       float4* s_box, float4* s_tmp, const uint16_t* s_pre,
                                       const uint16_t* cstart, int groups, int n, bool any_class, int tid) {
    for (int i0 = tid; i0 < n; i0 += 4 * NT) {
        int sl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * NT;
            sl[u] = 0;
            if (i < n) {
                const int g = group_of(s_pre, groups, i);
                sl[u] = g * kDecodeBlock + (i - (int)s_pre[g]);
            }
        }
        uint64_t k[4];
        uint32_t o[4];
        float4 b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            k[u] = keys[sl[u]];
            o[u] = p.offs[sl[u]];
            if (STAGED) b[u] = p.boxes[sl[u]];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * NT;
            if (i < n) {
                const int pos = (int)cstart[any_class ? 0 : key_class(k[u])] + (int)o[u];
                s[pos] = k[u];
                if (STAGED) {
                    s_box[pos] = b[u];
                    s_tmp[i] = b[u];
                }
            }
        }
    }
}

// Up to this many kept boxes are placed by counting, not sorted.
constexpr int kRankByCountMax = 256;

// Bytes of the suppression kernel's shared region after the keys, run
// starts and prefix sums: per-wave kept-position lists, or (at other times)
// the class counters (two 16-bit counters per word) or the kept boxes, areas
// and positions of a run resolved by all waves (the only use in any-class
// mode).
__host__ __device__ constexpr int nms_aux_bytes(int max_det, int nc, int waves, bool any_class) {
    const int lists = any_class ? 0 : waves * max_det * 2;
    const int hist = any_class ? 0 : ((nc + 1) / 2) * 4;
    const int coop = (max_det + kCoopPad) * (16 + 4) + max_det * 2;
    const int m = lists > hist ? (lists > coop ? lists : coop) : (hist > coop ? hist : coop);
    return (m + 15) & ~15;
}

template <int NT>
__global__ __launch_bounds__(NT) void det_nms_kernel(
    const uint32_t* counts, const uint64_t* keys, int32_t groups, int32_t sort_cap, int32_t agnostic,
    int32_t max_det, const DetParams p) {
#pragma clang fp contract(off)
    constexpr int W = NT / 64;
    // Dynamic LDS: keys [sort_cap] | run starts [kRunSlots] | decode prefix
    // sums [kPreSlots] | aux (nms_aux_bytes).  The keys' region past the
    // sort size holds the boxes when they fit.
    extern __shared__ uint64_t s_dyn[];
    uint64_t* s = s_dyn;
    uint16_t* s_run = reinterpret_cast<uint16_t*>(s_dyn + sort_cap);
    uint16_t* s_pre = s_run + kRunSlots;
    uint8_t* aux = reinterpret_cast<uint8_t*>(s_pre + kPreSlots);
    __shared__ uint32_t s_tot[W];
    __shared__ uint64_t s_alive[W];
    __shared__ uint32_t s_coop[kCoopCap];   // long class runs: start | length << 16
    __shared__ int s_n, s_runs, s_total, s_next, s_maxlen, s_kept, s_ncoop;

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool any_class = agnostic != 0;
    [[maybe_unused]] const int mark = 16 * wave;
#ifdef WS_CLOCK_MARKS
    // Marks stay in registers and are written out at the end, so that taking
    // them adds no stores for the barriers to wait on.
    uint64_t mk_[16] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#define NMS_MARK(slot)                                                  \
    do {                                                                \
        __builtin_amdgcn_sched_barrier(0);                              \
        mk_[(slot)] = __builtin_amdgcn_s_memrealtime();                 \
        __builtin_amdgcn_sched_barrier(0);                              \
    } while (0)
#define NMS_MARK_AFTER_LOADS(slot)                       \
    do {                                                 \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); \
        NMS_MARK(slot);                                  \
    } while (0)
#define NMS_MARKS_OUT()                                                              \
    do {                                                                             \
        if (lane == 0)                                                               \
            for (int k_ = 0; k_ < 16; ++k_) g_marks[kNmsMarks + mark + k_] = mk_[k_];  \
    } while (0)
#else
#define NMS_MARK(slot) do {} while (0)
#define NMS_MARK_AFTER_LOADS(slot) do {} while (0)
#define NMS_MARKS_OUT() do {} while (0)
#endif
    NMS_MARK(0);
    if (tid == 0) {
        s_total = 0;
        s_next = W;
        s_maxlen = 0;
        s_ncoop = 0;
    }

    // 0. One round trip for everything the candidate layout needs.  Wave 0
    //    loads every decode workgroup's candidate count (four per lane) and,
    //    up to 256 classes, every class's count (four per lane), then works
    //    out alone the candidates' numbering, the class starts and the runs
    //    (longest first).  With more classes the workgroup reads and scans
    //    the class counts.
    const int nc = any_class ? 1 : p.nc;
    const bool few_classes = nc <= 4 * 64;   // uniform
    uint32_t* hist = reinterpret_cast<uint32_t*>(aux);
    uint16_t* cstart = reinterpret_cast<uint16_t*>(aux);
    // The loads are unconditional, their indices clamped into the arrays (a
    // lane past the end re-reads the last element and drops it), so that all
    // are in flight before the first is used.
    uint32_t gc[4] = {0u, 0u, 0u, 0u}, cc[4] = {0u, 0u, 0u, 0u};
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) gc[j] = counts[min(lane * 4 + j, groups - 1)];
        if (few_classes) {
#pragma unroll
            for (int j = 0; j < 4; ++j) cc[j] = p.cls_counts[min(lane * 4 + j, nc - 1)];
        }
    }
    if (!few_classes) {
        for (int w = tid; w < (nc + 1) / 2; w += NT) {
            const int c0 = 2 * w;
            const uint32_t a = p.cls_counts[c0];
            const uint32_t b = c0 + 1 < nc ? p.cls_counts[c0 + 1] : 0u;
            hist[w] = a | (b << 16);
        }
    }
    // Class starts and run starts: one prefix sum of (count | nonempty << 16)
    // over the classes (counts stay below 2^15, so the low half never
    // carries).  A class with more than kRunSortMax candidates is also listed
    // as a long run.
    auto publish = [&](int c, uint32_t cn, uint32_t run) {
        cstart[c] = (uint16_t)(run & 0xFFFFu);
        if (cn > 0) {
            s_run[run >> 16] = (uint16_t)(run & 0xFFFFu);
            if (cn > (uint32_t)kRunSortMax) s_coop[atomicAdd(&s_ncoop, 1)] = (run & 0xFFFFu) | (cn << 16);
        }
    };
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gc[j] = lane * 4 + j < groups ? gc[j] : 0u;
            cc[j] = lane * 4 + j < nc ? cc[j] : 0u;
        }
        const uint32_t t = gc[0] + gc[1] + gc[2] + gc[3];
        const uint32_t incl = wave_incl_scan(t);
        uint32_t base = incl - t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = lane * 4 + j;
            if (g < groups) s_pre[g] = (uint16_t)base;
            base += gc[j];
        }
        if (lane == 63) {
            s_pre[groups] = (uint16_t)incl;
            s_n = (int)incl;
        }
        if (few_classes) {
            uint32_t loc[4];
            uint32_t sum = 0;
            int maxc = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t cn = cc[e];
                loc[e] = cn | (cn ? 1u << 16 : 0u);
                sum += loc[e];
                maxc = max(maxc, (int)cn);
            }
            const uint32_t cincl = wave_incl_scan(sum);
            uint32_t run = cincl - sum;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = lane * 4 + e;
                if (c < nc) publish(c, loc[e] & 0xFFFFu, run);
                run += loc[e];
            }
            maxc = (int)wave_max_u32((uint32_t)maxc, lane);
            const int nruns = (int)(cincl >> 16);   // lane 63: all runs
            const int total_runs = __builtin_amdgcn_readlane(nruns, 63);
            if (lane == 63) {
                s_runs = total_runs;
                s_maxlen = maxc;
                s_run[total_runs] = (uint16_t)(cincl & 0xFFFFu);   // sentinel: a run ends where the next starts
            }
            // Longest runs first (up to 64 runs): (length, start) sorted
            // descending; a start is below 2^14 and a length at most 2^14,
            // so both fit one 32-bit key.  The lengths go to
            // s_run[kRunLen + r].
            if (!any_class && total_runs > 1 && total_runs <= 64) {
                wave_lds_sync();   // the run starts and the sentinel are written
                const uint32_t start = lane < total_runs ? s_run[lane] : 0u;
                const uint32_t len = lane < total_runs ? (uint32_t)s_run[lane + 1] - start : 0u;
                const uint32_t ord = wave_sort<true>(lane < total_runs ? (len << 16) | start : 0u, lane);
                wave_lds_sync();   // every start was read before any is overwritten
                if (lane < total_runs) {
                    s_run[lane] = (uint16_t)(ord & 0xFFFFu);
                    s_run[kRunLen + lane] = (uint16_t)(ord >> 16);
                }
            }
        }
    }
    __syncthreads();
    const int n = s_n;   // uniform
    NMS_MARK(1);
    if (n == 0) {   // no candidates: every class count is zero already
        if (tid == 0) {
            p.out->count = 0;
            p.out->candidates = 0;
        }
        NMS_MARKS_OUT();
        return;
    }
    // The class counts are read: clear them for the next frame.
    for (int c = tid; c < nc; c += NT) p.cls_counts[c] = 0;

    // 1. More than 256 classes: the workgroup scans the class counts, E per
    //    thread; the class starts overwrite the counters once all are read.
    int runs = 1;
    bool ordered = false;
    bool run_sort = false;
    if (!few_classes) {
        constexpr int E = WS_DET_MAX_CLASSES / NT;
        uint32_t loc[E];
        uint32_t sum = 0;
        int maxc = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = tid * E + e;
            const uint32_t cn = c < nc ? (hist[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu : 0u;
            loc[e] = cn | (cn ? 1u << 16 : 0u);
            sum += loc[e];
            maxc = max(maxc, (int)cn);
        }
        uint32_t tot2;
        uint32_t run = block_excl_scan<NT>(sum, s_tot, tot2, tid);   // all counters are read
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = tid * E + e;
            if (c < nc) publish(c, loc[e] & 0xFFFFu, run);
            run += loc[e];
        }
        if (maxc > 0) atomicMax(&s_maxlen, maxc);
        if (tid == 0) {
            s_runs = (int)(tot2 >> 16);
            s_run[tot2 >> 16] = (uint16_t)n;
        }
        __syncthreads();
    }
    runs = s_runs;
    NMS_MARK(12);

    // 2. Gather: every candidate's key (and box) to its class bucket, the
    //    box also by compact position (for lookups by slot).  Boxes are
    //    staged when the sort space past P has room for them twice.
    int P = 64;
    while (P < n) P <<= 1;
    const bool staged = (int64_t)P + 4 * (int64_t)n <= (int64_t)sort_cap;   // uniform
    float4* s_box = reinterpret_cast<float4*>(s + P);   // P * 8 is a multiple of 512
    float4* s_tmp = s_box + n;
    if (staged) gather<NT, true>(p, keys, s, s_box, s_tmp, s_pre, cstart, groups, n, any_class, tid);
    else gather<NT, false>(p, keys, s, s_box, s_tmp, s_pre, cstart, groups, n, any_class, tid);
    NMS_MARK(11);
    __syncthreads();
    NMS_MARK(2);
    if (!any_class) {
        run_sort = s_maxlen <= kRunSortMax;   // uniform
        ordered = runs > 1 && runs <= 64;
        if (!few_classes && ordered) {
            // Longest runs first, as above, after the workgroup's scan.
            if (wave == 0) {
                const uint32_t start = lane < runs ? s_run[lane] : 0u;
                const uint32_t len = lane < runs ? (uint32_t)s_run[lane + 1] - start : 0u;
                const uint32_t ord = wave_sort<true>(lane < runs ? (len << 16) | start : 0u, lane);
                wave_lds_sync();   // every start was read before any is overwritten
                if (lane < runs) {
                    s_run[lane] = (uint16_t)(ord & 0xFFFFu);
                    s_run[kRunLen + lane] = (uint16_t)(ord >> 16);
                }
            }
            __syncthreads();
        }
    }
    NMS_MARK(3);
    auto run_len = [&](int r) -> int {
        return ordered ? (int)s_run[kRunLen + r] : (int)s_run[r + 1] - (int)s_run[r];
    };
    // Each wave takes run `wave` first, then whichever run is next when it is
    // done, so long runs do not queue behind each other on one wave.
    auto next_run = [&]() -> int {
        int r = 0;
        if (lane == 0) r = atomicAdd(&s_next, 1);
        return __builtin_amdgcn_readfirstlane(r);
    };
    uint16_t* kept_pos = reinterpret_cast<uint16_t*>(aux) + wave * max_det;
    float4* k_box = reinterpret_cast<float4*>(aux);
    float* k_area = reinterpret_cast<float*>(k_box + max_det + kCoopPad);
    uint16_t* k_pos = reinterpret_cast<uint16_t*>(k_area + max_det + kCoopPad);
    int any_kept = 0;
#ifdef WS_CLOCK_MARKS
    int runs_done = 0;
#define WS_COUNT_RUN() ++runs_done
#else
#define WS_COUNT_RUN()
#endif

    if (run_sort) {
        // 3a. Class runs of at most kRunSortMax: one wave holds a run in its
        //     registers and resolves it by selection (no sort).
        NMS_MARK(4);
        for (int r = wave; r < runs; r = next_run()) {
            const int start = s_run[r];
            const int len = run_len(r);
            if (staged) select_run<true>(p, s, s_box, s_tmp, s_pre, start, len, kept_pos, lane);
            else select_run<false>(p, s, s_box, s_tmp, s_pre, start, len, kept_pos, lane);
            WS_COUNT_RUN();
        }
    } else {
        // 3b. One sort of everything (class-major order in class-aware mode,
        //     so the buckets stay where they are), boxes staged in sorted
        //     order, then the long runs by all waves and the rest one wave per
        //     run.
        for (int e = n + tid; e < P; e += NT) s[e] = 0;
        __syncthreads();
        sort_desc<NT>(s, P, tid);
        if (staged) {
            for (int e = tid; e < n; e += NT) {
                const int slot = key_slot(s[e], any_class);
                s_box[e] = s_tmp[s_pre[slot >> 6] + (slot & 63)];
            }
            __syncthreads();
        }
        NMS_MARK(4);
        if (any_class) {
            any_kept = staged
                ? coop_resolve<true, NT>(p, s, s_box, 0, n, k_box, k_area, k_pos, s_alive, &s_kept, true, tid)
                : coop_resolve<false, NT>(p, s, s_box, 0, n, k_box, k_area, k_pos, s_alive, &s_kept, true, tid);
        } else {
            const int ncoop = s_ncoop;
            for (int c = 0; c < ncoop; ++c) {
                const int start = (int)(s_coop[c] & 0xFFFFu);
                const int len = (int)(s_coop[c] >> 16);
                if (staged)
                    coop_resolve<true, NT>(p, s, s_box, start, len, k_box, k_area, k_pos, s_alive, &s_kept, false, tid);
                else
                    coop_resolve<false, NT>(p, s, s_box, start, len, k_box, k_area, k_pos, s_alive, &s_kept, false, tid);
            }
            for (int r = wave; r < runs; r = next_run()) {
                const int len = run_len(r);
                if (len > kRunSortMax) continue;
                if (staged) resolve_run<true>(p, s, s_box, s_run[r], len, kept_pos, false, lane);
                else resolve_run<false>(p, s, s_box, s_run[r], len, kept_pos, false, lane);
                WS_COUNT_RUN();
            }
        }
    }
#undef WS_COUNT_RUN
    NMS_MARK(5);
#ifdef WS_CLOCK_MARKS
    mk_[9] = (uint64_t)runs_done;
#endif
    __syncthreads();
    NMS_MARK(6);

    // 4. Kept boxes in rank order.  Any class: the kept list, in rank order
    //    already.  Otherwise gather the flagged keys of all runs; up to
    //    kRankByCountMax of them are placed by counting (keys are distinct,
    //    so a key's place is the number of kept keys above it), more are
    //    sorted.
    int kept_total;
    if (any_class) {
        kept_total = any_kept;   // uniform: every wave took part
    } else {
        // NT positions at a time: every thread reads its key, then the flagged
        // ones are appended.  A slot is below the number of keys flagged so
        // far, hence below every position still to be read.
        for (int base = 0; base < n; base += NT) {   // uniform
            const int e = base + tid;
            const uint64_t k = e < n ? s[e] : 0;
            __syncthreads();
            if (k & 1u) s[atomicAdd(&s_total, 1)] = to_rank_key(k);
        }
        __syncthreads();
        kept_total = s_total;
        if (kept_total > kRankByCountMax) {   // uniform
            int P2 = 64;
            while (P2 < kept_total) P2 <<= 1;
            for (int e = kept_total + tid; e < P2; e += NT) s[e] = 0;
            __syncthreads();
            sort_desc<NT>(s, P2, tid);
        }
    }
    NMS_MARK(7);

    // 5. The first max_det, mapped to source pixels, to the mapped slot.
    const int count = min(kept_total, max_det);
    auto emit = [&](uint64_t k, const float4 b, int q) {
        ws_det d;
        d.x1 = to_source(b.x, p.left, p.sx, p.src_w);
        d.y1 = to_source(b.y, p.top, p.sy, p.src_h);
        d.x2 = to_source(b.z, p.left, p.sx, p.src_w);
        d.y2 = to_source(b.w, p.top, p.sy, p.src_h);
        d.score = __uint_as_float((uint32_t)(k >> 33));
        d.class_id = (int32_t)((k >> 7) & 0xFFFu);
        p.out->det[q] = d;
    };
    // Box of a rank key: staged by compact position, else by slot (separate
    // loops, so each loads from one address space).
    auto staged_box = [&](uint64_t k) {
        const int slot = key_slot(k, true);
        return s_tmp[s_pre[slot >> 6] + (slot & 63)];
    };
    auto global_box = [&](uint64_t k) { return p.boxes[key_slot(k, true)]; };
    if (any_class) {
        for (int q = tid; q < count; q += NT) emit(s[k_pos[q]] & ~1ull, k_box[q], q);
    } else if (kept_total <= kRankByCountMax) {
        // Eight lanes rank each kept key: lane j of the group counts the keys
        // above it among keys j, j + 8, ... (eight reads in flight), and the
        // eight counts are summed across the group (lane distances 1, 2, 4).
        // A group's lanes are all below `pairs` or all at or above it.
        const int pairs = kept_total * 8;
        for (int base = 0; base < pairs; base += NT) {   // uniform
            const int e = base + tid;
            if (e < pairs) {
                const int t = e >> 3, j = e & 7;
                const uint64_t x = s[t];
                uint32_t r = 0;
                for (int i0 = j; i0 < kept_total; i0 += 64) {
                    uint64_t v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int i = i0 + 8 * u;
                        v[u] = i < kept_total ? s[i] : 0;   // 0 is above no key
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) r += v[u] > x ? 1u : 0u;
                }
                r += xor_lane32<1>(r, lane);
                r += xor_lane32<2>(r, lane);
                r += xor_lane32<4>(r, lane);
                if (j == 0 && (int)r < count) {
                    if (staged) emit(x, staged_box(x), (int)r);
                    else emit(x, global_box(x), (int)r);
                }
            }
        }
    } else if (staged) {
        for (int q = tid; q < count; q += NT) emit(s[q], staged_box(s[q]), q);
    } else {
        for (int q = tid; q < count; q += NT) emit(s[q], global_box(s[q]), q);
    }
    if (tid == 0) {
        p.out->count = count;
        p.out->candidates = n;
    }
    NMS_MARK(8);
    NMS_MARKS_OUT();
#undef NMS_MARK
#undef NMS_MARK_AFTER_LOADS
#undef NMS_MARKS_OUT
}

// Dynamic LDS one workgroup may take: 160 KiB on gfx950, less room for the
// kernels' static LDS (under 1 KiB).
constexpr int kNmsLdsCap = 160 * 1024 - 1024;

constexpr int nms_lds_bytes(int sort_cap, int max_det, int nc, int threads, bool any_class) {
    return sort_cap * (int)sizeof(uint64_t) + (kRunSlots + kPreSlots) * (int)sizeof(uint16_t) +
           nms_aux_bytes(max_det, nc, threads / 64, any_class);
}

static_assert(nms_lds_bytes(WS_DET_MAX_ANCHORS, WS_DET_MAX_DET, WS_DET_MAX_CLASSES, kNmsNarrow, false) <=
                  kNmsLdsCap,
              "the narrow suppression kernel fits every lane within the limits of ws.h");

int nms_threads(int sort_cap, int max_det, int nc, bool any_class) {
    if (nms_lds_bytes(sort_cap, max_det, nc, kNmsWide, any_class) <= kNmsLdsCap) return kNmsWide;
    if (nms_lds_bytes(sort_cap, max_det, nc, kNmsNarrow, any_class) <= kNmsLdsCap) return kNmsNarrow;
    return 0;
}

}  // namespace

int det_nms_lds_bytes(int sort_cap, int max_det, int nc, bool any_class) {
    const int nt = nms_threads(sort_cap, max_det, nc, any_class);
    return nt ? nms_lds_bytes(sort_cap, max_det, nc, nt, any_class) : 0;
}

hipError_t set_detect_attributes() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(det_nms_kernel<kNmsNarrow>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kNmsLdsCap);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(det_nms_kernel<kNmsWide>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kNmsLdsCap);
    return e;
}

hipError_t launch_detect(const DetParams& p, hipStream_t stream) {
    const int nt = nms_threads(p.sort_cap, p.max_det, p.nc, p.agnostic != 0);
    if (nt == 0 || p.groups < 1 || p.groups > kDetMaxGroups ||
        (int64_t)p.groups * kDetDecodeAnchors < (int64_t)p.anchors || p.sort_cap < p.anchors)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(det_decode_kernel, dim3((unsigned)p.groups), dim3(kDecodeThreads), 0, stream,
                       p.head, p.anchors, p.nc, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned lds = (unsigned)nms_lds_bytes(p.sort_cap, p.max_det, p.nc, nt, p.agnostic != 0);
    auto nms = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3(1), dim3(threads), lds, stream, p.counts, p.keys, p.groups,
                           p.sort_cap, p.agnostic, p.max_det, p);
    };
    if (nt == kNmsWide)
        nms(det_nms_kernel<kNmsWide>, kNmsWide);
    else
        nms(det_nms_kernel<kNmsNarrow>, kNmsNarrow);
    return hipGetLastError();
}

}  // namespace ws

#ifdef WS_CLOCK_MARKS
// Instrumented builds only: copy out (or clear) the detection kernels' marks.
extern "C" int ws_debug_detect_marks(uint64_t* host, size_t n, int32_t clear) {
    if (n > (size_t)ws::kMarkSlots) n = ws::kMarkSlots;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess && host && n)
        e = hipMemcpyFromSymbol(host, HIP_SYMBOL(ws::g_marks), n * sizeof(uint64_t), 0,
                                hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(ws::g_marks));
        if (e == hipSuccess) e = hipMemset(p, 0, sizeof(uint64_t) * ws::kMarkSlots);
        if (e == hipSuccess) e = hipDeviceSynchronize();
    }
    return e == hipSuccess ? 0 : -6;
}
#endif
