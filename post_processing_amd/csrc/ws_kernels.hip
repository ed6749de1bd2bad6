// ws_kernels.hip -- the two kernels of the frame pipeline, written for gfx950
// (CDNA4, wave64).
//
// preprocess_kernel: WarpStream TRT article, fused-preprocess passage and its
//   dataflow figure -- one pass from interleaved RGB8 to the planar FP32
//   tensor: centre-aligned bilinear sample, x 1/255, (v - mean) / std, store
//   into the destination channel plane; no intermediate image.  Letterbox
//   placement per the yolo.cu README.
// topk_kernel: the article's Top-K passage -- exact K best of FP32 scores,
//   ties to the lower index, NaN as -inf, only K pairs leave the GPU; the
//   large-label-space advice (hierarchical selection) gives the partial +
//   merge split across workgroups.
#include <hip/hip_runtime.h>

#include "ws_kernels.h"

namespace ws {
namespace {

// ===========================================================================
// Preprocess
//
// One workgroup owns `rows_per_group` consecutive output rows of one frame.
//  1. For each output row it stages the two source rows its vertical taps
//     read (only the byte span the horizontal taps touch) into LDS with
//     16-byte global loads, all issued before any LDS write.
//  2. Each thread owns 4 adjacent output columns of one row: it computes the
//     exact taps, fetches each RGB triple from LDS as one aligned dword pair
//     funnel-shifted into place, interpolates and normalises in FP32, and
//     writes one 16-byte vector per channel plane.
// Taps are exact integers: src = ((2d + 1) S - R) / (2R), clamped at 0;
// i0 = floor, the weight is the remainder times 1/(2R) in FP32.

constexpr int kStageUnroll = 16;   // 16-byte loads in flight per thread
constexpr int kMaxSlots = 128;     // 2 staged rows x at most 64 output rows

struct AxisTap {
    uint32_t i0, i1;
    float w;
};

__device__ __forceinline__ AxisTap exact_tap(int d, int S, int R, float inv_den) {
    int num = (2 * d + 1) * S - R;
    num = num < 0 ? 0 : num;
    const uint32_t den = 2u * (uint32_t)R;
    const uint32_t i0 = (uint32_t)num / den;
    const uint32_t rem = (uint32_t)num - i0 * den;
    AxisTap t;
    t.i0 = i0;
    t.i1 = i0 + 1 < (uint32_t)S ? i0 + 1 : (uint32_t)S - 1;
    t.w = (float)rem * inv_den;
    return t;
}

// Three bytes (R, G, B) starting at LDS byte offset `byte`, in bits 0..23.
__device__ __forceinline__ uint32_t lds_rgb(const uint32_t* lds32, uint32_t byte) {
    const uint32_t w = byte >> 2;
    const uint32_t lo = lds32[w];
    const uint32_t hi = lds32[w + 1];
    return __builtin_amdgcn_alignbyte(hi, lo, byte & 3u);
}

__device__ __forceinline__ float chan(uint32_t rgb, int c) {
    return (float)((rgb >> (8 * c)) & 0xffu);
}

__global__ __launch_bounds__(512) void preprocess_kernel(PreParams p) {
    extern __shared__ uint4 lds_dyn[];
    __shared__ int64_t slot_addr[kMaxSlots];   // unaligned start of a staged row, -1 = none

    uint32_t* lds32 = reinterpret_cast<uint32_t*>(lds_dyn);
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int f = blockIdx.x / p.groups_per_frame;
    const int grp = blockIdx.x - f * p.groups_per_frame;
    const int y_base = grp * p.rows_per_group;
    const int nrows = min(p.rows_per_group, p.dst_h - y_base);
    const int nslots = 2 * nrows;
    const int64_t fbase = (int64_t)f * p.frame_bytes;
    const int64_t row_bytes = 3 * (int64_t)p.src_w;
    const uint32_t slot_bytes = 16u * (uint32_t)p.slot_chunks;

    // 1a. Where each staged row starts.
    for (int s = tid; s < nslots; s += nthr) {
        const int dy = y_base + (s >> 1) - p.top;
        int64_t a = -1;
        if (dy >= 0 && dy < p.reg_h) {
            const AxisTap ty = exact_tap(dy, p.src_h, p.reg_h, p.inv_den_y);
            const uint32_t yy = (s & 1) ? ty.i1 : ty.i0;
            a = fbase + (int64_t)yy * row_bytes + p.span_lo;
        }
        slot_addr[s] = a;
    }
    __syncthreads();

    // 1b. Stage the rows: chunk c of the dense LDS image is 16 bytes of slot
    //     c / slot_chunks, read from that row's 16-byte-aligned start.
    const int nchunks = nslots * p.slot_chunks;
    for (int c0 = 0; c0 < nchunks; c0 += nthr * kStageUnroll) {
        uint4 v[kStageUnroll];
#pragma unroll
        for (int u = 0; u < kStageUnroll; ++u) {
            const int c = c0 + u * nthr + tid;
            v[u] = make_uint4(0u, 0u, 0u, 0u);
            if (c < nchunks) {
                const int s = c / p.slot_chunks;
                const int j = c - s * p.slot_chunks;
                const int64_t a = slot_addr[s];
                if (a >= 0) {
                    const int64_t g = (a & ~(int64_t)15) + 16 * (int64_t)j;
                    if (g + 16 <= p.total_bytes) {
                        v[u] = *reinterpret_cast<const uint4*>(p.src + g);
                    } else if (g < p.total_bytes) {
                        // Last partial chunk of the whole input: byte loads.
                        uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                        for (int b = 0; b < 16; ++b)
                            if (g + b < p.total_bytes)
                                wd[b >> 2] |= (uint32_t)p.src[g + b] << (8 * (b & 3));
                        v[u] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kStageUnroll; ++u) {
            const int c = c0 + u * nthr + tid;
            if (c < nchunks) lds_dyn[c] = v[u];
        }
    }
    __syncthreads();

    // 2. Resample, normalise, store planar.
    const int q = p.quads_per_row;
    const int work = nrows * q;
    const int64_t plane = (int64_t)p.dst_h * p.dst_w;
    float* const frame_out = p.dst + (int64_t)f * 3 * plane;
    for (int wi = tid; wi < work; wi += nthr) {
        const int r = wi / q;
        const int x_first = 4 * (wi - r * q);
        const int y = y_base + r;
        const int dy = y - p.top;
        const bool row_in = dy >= 0 && dy < p.reg_h;
        float wy = 0.0f;
        uint32_t base0 = 0, base1 = 0;
        if (row_in) {
            wy = exact_tap(dy, p.src_h, p.reg_h, p.inv_den_y).w;
            base0 = (uint32_t)(2 * r) * slot_bytes + (uint32_t)(slot_addr[2 * r] & 15);
            base1 = (uint32_t)(2 * r + 1) * slot_bytes + (uint32_t)(slot_addr[2 * r + 1] & 15);
        }
        float out[3][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dx = x_first + i - p.left;
            if (row_in && dx >= 0 && dx < p.reg_w) {
                const AxisTap tx = exact_tap(dx, p.src_w, p.reg_w, p.inv_den_x);
                const uint32_t o0 = 3u * tx.i0 - (uint32_t)p.span_lo;
                const uint32_t o1 = 3u * tx.i1 - (uint32_t)p.span_lo;
                const uint32_t t00 = lds_rgb(lds32, base0 + o0);
                const uint32_t t01 = lds_rgb(lds32, base0 + o1);
                const uint32_t t10 = lds_rgb(lds32, base1 + o0);
                const uint32_t t11 = lds_rgb(lds32, base1 + o1);
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const float p00 = chan(t00, c), p01 = chan(t01, c);
                    const float p10 = chan(t10, c), p11 = chan(t11, c);
                    const float h0 = fmaf(tx.w, p01 - p00, p00);
                    const float h1 = fmaf(tx.w, p11 - p10, p10);
                    const float v = fmaf(wy, h1 - h0, h0);
                    out[c][i] = fmaf(v, p.a[c], p.b[c]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 3; ++c) out[c][i] = p.padv[c];
            }
        }
        float* const row_out = frame_out + (int64_t)y * p.dst_w + x_first;
        if (p.vec4) {
#pragma unroll
            for (int c = 0; c < 3; ++c)
                *reinterpret_cast<float4*>(row_out + c * plane) =
                    make_float4(out[c][0], out[c][1], out[c][2], out[c][3]);
        } else {
#pragma unroll
            for (int c = 0; c < 3; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (x_first + i < p.dst_w) row_out[c * plane + i] = out[c][i];
        }
    }
}

// ===========================================================================
// Top-K
//
// Order key: (value descending, index ascending) as one unsigned 64-bit
// integer, larger = better:  high word = order-preserving image of the FP32
// bits (NaN -> -inf, -0 -> +0 first), low word = ~index.  Integer compares
// keep subnormals unflushed and make every key distinct, so the selection is
// unique and needs no tie logic.  Key 0 is below every real key (sentinel).
//
// Each wave64 keeps a sorted list of its 64 best keys, one per lane (lane 0
// best).  Scores stream past in tiles of 64 (one per lane); a tile is skipped
// unless some lane beats the current K-th best.  A tile with many winners is
// bitonic-sorted across lanes and merged (elementwise max against the list,
// then a bitonic clean-up); a few winners are inserted one at a time.

__device__ __forceinline__ uint64_t order_key(float v, uint32_t idx) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) > 0x7f800000u) b = 0xff800000u;   // NaN -> -inf
    if (b == 0x80000000u) b = 0u;                             // -0 -> +0
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int mask) {
    const int lo = __shfl_xor((int)(uint32_t)v, mask);
    const int hi = __shfl_xor((int)(uint32_t)(v >> 32), mask);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t prev_lane64(uint64_t v) {
    const int lo = __shfl_up((int)(uint32_t)v, 1);
    const int hi = __shfl_up((int)(uint32_t)(v >> 32), 1);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a < b ? b : a; }

// Bitonic sort of one key per lane into ascending lane order.
__device__ __forceinline__ uint64_t wave_sort_asc(uint64_t x, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t y = xor_lane64(x, j);
            const bool up = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            x = (lower == up) ? umin64(x, y) : umax64(x, y);
        }
    }
    return x;
}

// Sort a bitonic sequence (one key per lane) into descending lane order.
__device__ __forceinline__ uint64_t wave_clean_desc(uint64_t x, int lane) {
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
        const uint64_t y = xor_lane64(x, j);
        x = (lane & j) == 0 ? umax64(x, y) : umin64(x, y);
    }
    return x;
}

struct WaveTopK {
    uint64_t best;   // this lane's entry of the wave's sorted list
    uint64_t thr;    // K-th best key so far (wave-uniform)
    int k;
    int lane;

    __device__ __forceinline__ void init(int k_, int lane_) {
        best = 0;
        thr = 0;
        k = k_;
        lane = lane_;
    }

    // Merge a full sorted-descending list held one key per lane.
    __device__ __forceinline__ void merge_sorted_desc_list(uint64_t other_asc) {
        best = wave_clean_desc(umax64(best, other_asc), lane);
        thr = readlane64(best, k - 1);
    }

    // Offer one tile: every lane contributes `key` (0 = nothing).
    __device__ __forceinline__ void offer(uint64_t key) {
        uint64_t m = __ballot(key > thr);
        if (m == 0) return;
        if (__popcll(m) > 4) {
            const uint64_t t = wave_sort_asc(key > thr ? key : 0, lane);
            best = wave_clean_desc(umax64(best, t), lane);
            thr = readlane64(best, k - 1);
            return;
        }
        while (m) {
            const int src = __ffsll((long long)m) - 1;
            m &= m - 1;
            const uint64_t c = readlane64(key, src);
            if (c > thr) {
                const int pos = __popcll(__ballot(best > c));
                const uint64_t shifted = prev_lane64(best);
                best = lane < pos ? best : (lane == pos ? c : shifted);
                thr = readlane64(best, k - 1);
            }
        }
    }
};

// Merge the four waves' lists of one workgroup into wave 0.
__device__ __forceinline__ void block_merge(WaveTopK& st, uint64_t (*s_best)[64], int wave,
                                            int lane) {
    s_best[wave][lane] = st.best;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 1; w < kTopkThreads / 64; ++w) st.merge_sorted_desc_list(s_best[w][63 - lane]);
    }
}

__device__ __forceinline__ void write_result(const TopkParams& p, uint64_t key, int lane) {
    // K <= N guarantees K real keys; the guard only keeps a sentinel in bounds.
    const uint32_t idx = ~(uint32_t)key;
    uint32_t bits = 0xff800000u;
    if ((int64_t)idx < p.n) bits = __float_as_uint(p.scores[idx]);
    if ((bits & 0x7fffffffu) > 0x7f800000u) bits = 0xff800000u;   // NaN reported as -inf
    p.result[lane] = make_uint2(bits, idx);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
    __shared__ uint64_t s_best[kTopkThreads / 64][64];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    WaveTopK st;
    st.init(p.k, lane);

    const int64_t g0 = (int64_t)blockIdx.x * p.chunk;
    const int64_t g1 = min(p.n, g0 + (int64_t)p.chunk);
    const int iters = (int)((g1 - g0 + 1023) / 1024);
    for (int it0 = 0; it0 < iters; it0 += 4) {
        float4 v[4];
        int64_t base[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            base[u] = g0 + (int64_t)(it0 + u) * 1024 + 4 * tid;
            v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (it0 + u < iters) {
                if (base[u] + 4 <= g1) {
                    v[u] = *reinterpret_cast<const float4*>(p.scores + base[u]);
                } else {
                    if (base[u] + 0 < g1) v[u].x = p.scores[base[u] + 0];
                    if (base[u] + 1 < g1) v[u].y = p.scores[base[u] + 1];
                    if (base[u] + 2 < g1) v[u].z = p.scores[base[u] + 2];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (it0 + u >= iters) break;
            const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = base[u] + j;
                st.offer(i < g1 ? order_key(e[j], (uint32_t)i) : 0);
            }
        }
    }
    block_merge(st, s_best, wave, lane);

    if (p.groups == 1) {
        if (wave == 0 && lane < p.k) write_result(p, st.best, lane);
        return;
    }

    // Publish this workgroup's K best; the last workgroup to arrive merges all.
    if (wave == 0 && lane < p.k) p.partials[(int64_t)blockIdx.x * p.k + lane] = st.best;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(p.counter, 1u) == (uint32_t)(p.groups - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    WaveTopK mt;
    mt.init(p.k, lane);
    const int total = p.groups * p.k;
    constexpr int kMergeUnroll = 8;
    for (int i0 = 0; i0 < total; i0 += kTopkThreads * kMergeUnroll) {
        uint64_t key[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int i = i0 + u * kTopkThreads + tid;
            key[u] = i < total ? p.partials[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) mt.offer(key[u]);
    }
    __syncthreads();   // every wave is done reading s_best from the first merge
    block_merge(mt, s_best, wave, lane);
    if (wave == 0) {
        if (lane < p.k) write_result(p, mt.best, lane);
        if (lane == 0) *p.counter = 0u;   // ready for the next launch
    }
}

}  // namespace

hipError_t launch_preprocess(const PreParams& p, int groups, int block, int lds_bytes,
                             hipStream_t stream) {
    hipLaunchKernelGGL(preprocess_kernel, dim3((unsigned)groups), dim3((unsigned)block),
                       (unsigned)lds_bytes, stream, p);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)p.groups), dim3(kTopkThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t set_kernel_attributes() {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(preprocess_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
}

}  // namespace ws
