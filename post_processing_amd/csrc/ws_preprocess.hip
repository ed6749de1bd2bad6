// ws_preprocess.hip -- the fused preprocess kernels of the frame pipeline,
// written for gfx950 (CDNA4, wave64).
//
// WarpStream TRT article, fused-preprocess passage and its dataflow figure:
// one pass from interleaved 8-bit RGB (or BGR, the yolo.cu README's producer
// order) to the planar tensor -- centre-aligned bilinear sample, x 1/255,
// (v - mean) / std, store into the destination channel plane; no
// intermediate image.  Letterbox placement per the yolo.cu README.  The
// tensor is FP32, or FP16 / BF16 (the article's precision-specialised
// preprocessing next step), computed in FP32 and rounded once to nearest
// even.
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "ws_kernels.h"

namespace ws {
namespace {
// ===========================================================================
// Preprocess
//
// Two kernels.  The default, preprocess_gather_kernel (one output column per
// thread), reads each thread's taps straight from global memory.  The staged
// preprocess_kernel<PX> (PX = 2 or 4 columns per thread) works as follows.
// One workgroup owns `rows_per_group` consecutive output rows of one frame.
//  1. For each output row it stages the two source rows its vertical taps
//     read (only the byte span the horizontal taps touch) into LDS with
//     16-byte global loads, all issued before any LDS write.
//  2. Each thread owns PX adjacent output columns of one row: it computes
//     the exact taps, fetches each RGB triple from LDS as one aligned dword
//     pair funnel-shifted into place, interpolates and normalises in FP32,
//     and writes one PX-wide vector per channel plane.
// Taps are exact integers: src = ((2d + 1) S - R) / (2R), clamped at 0;
// i0 = floor, the weight is the remainder times 1/(2R) in FP32.  The floor
// is a multiply by M = floor(2^32 / 2R) + 1 keeping the high word: for
// numerators below 2^29 that exceeds the true quotient by less than 1/8, so
// it is exact or one too large, which the sign of the remainder shows.

constexpr int kStageUnroll = 16;   // 16-byte loads in flight per thread
constexpr int kMaxSlots = 128;     // 2 staged rows x at most 64 output rows

struct AxisTap {
    uint32_t i0, i1;
    float w;
};

__device__ __forceinline__ AxisTap exact_tap(int d, int S, int R, float inv_den, uint32_t magic) {
    int num = (2 * d + 1) * S - R;
    num = num < 0 ? 0 : num;
    const uint32_t den = 2u * (uint32_t)R;
    uint32_t i0 = __umulhi((uint32_t)num, magic);
    uint32_t rem = (uint32_t)num - i0 * den;
    if ((int32_t)rem < 0) {
        --i0;
        rem += den;
    }
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

// Byte `shift / 8` of a pixel's 3-byte group as a float (v_cvt_f32_ubyteN).
__device__ __forceinline__ float chan(uint32_t px, uint32_t shift) {
    return (float)((px >> shift) & 0xffu);
}

// Output element types: FP32, or FP16 / BF16 rounded to nearest even.
template <typename T> struct OutFormat;
template <> struct OutFormat<float> {
    __device__ static float cvt(float x) { return x; }
    __device__ static void store_nt(float* d, float x) { __builtin_nontemporal_store(x, d); }
};
template <> struct OutFormat<__half> {
    __device__ static uint16_t bits(float x) { return __half_as_ushort(__float2half_rn(x)); }
    __device__ static __half cvt(float x) { return __float2half_rn(x); }
    __device__ static uint32_t pack2(const float* v) { return bits(v[0]) | ((uint32_t)bits(v[1]) << 16); }
    __device__ static void store_nt(__half* d, float x) {
        __builtin_nontemporal_store(bits(x), reinterpret_cast<uint16_t*>(d));
    }
};
template <> struct OutFormat<__hip_bfloat16> {
    __device__ static uint16_t bits(float x) { return __bfloat16_as_ushort(__float2bfloat16(x)); }
    __device__ static __hip_bfloat16 cvt(float x) { return __float2bfloat16(x); }
    __device__ static uint32_t pack2(const float* v) { return bits(v[0]) | ((uint32_t)bits(v[1]) << 16); }
    __device__ static void store_nt(__hip_bfloat16* d, float x) {
        __builtin_nontemporal_store(bits(x), reinterpret_cast<uint16_t*>(d));
    }
};

// Two or four output values as one non-temporal store: the tensor is
// written once per frame and not read again by this kernel, so its lines
// need not stay in the caches, which keeps more of them for the frames.
// (64 frames of 1280x720 -> 224x224: 29.0 -> 28.1 us per launch; 1280x720
// letterboxed into 640x640, two columns per thread: 5.07 -> 4.83 us.  One
// column per thread gained nothing, so those stores stay ordinary.)
__device__ __forceinline__ void store_stream(float* dst, const float (&v)[4]) {
    typedef float V __attribute__((ext_vector_type(4)));
    const V x = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(x, reinterpret_cast<V*>(dst));
}
template <typename H>
__device__ __forceinline__ void store_stream(H* dst, const float (&v)[4]) {
    typedef uint32_t V __attribute__((ext_vector_type(2)));
    const V x = {OutFormat<H>::pack2(v), OutFormat<H>::pack2(v + 2)};
    __builtin_nontemporal_store(x, reinterpret_cast<V*>(dst));
}
__device__ __forceinline__ void store_stream(float* dst, const float (&v)[2]) {
    typedef float V __attribute__((ext_vector_type(2)));
    const V x = {v[0], v[1]};
    __builtin_nontemporal_store(x, reinterpret_cast<V*>(dst));
}
template <typename H>
__device__ __forceinline__ void store_stream(H* dst, const float (&v)[2]) {
    __builtin_nontemporal_store(OutFormat<H>::pack2(v), reinterpret_cast<uint32_t*>(dst));
}

template <int PX, typename OutT>
__global__ __launch_bounds__(512) void preprocess_kernel(PreParams p) {
    using Fmt = OutFormat<OutT>;
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
            const AxisTap ty = exact_tap(dy, p.src_h, p.reg_h, p.inv_den_y, p.magic_y);
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
    const int q = p.threads_per_row;
    const int work = nrows * q;
    const int64_t plane = (int64_t)p.dst_h * p.dst_w;
    OutT* const frame_out = reinterpret_cast<OutT*>(p.dst) + (int64_t)f * 3 * plane;
    for (int wi = tid; wi < work; wi += nthr) {
        const int r = wi / q;
        const int x_first = PX * (wi - r * q);
        const int y = y_base + r;
        const int dy = y - p.top;
        const bool row_in = dy >= 0 && dy < p.reg_h;
        float wy = 0.0f;
        uint32_t base0 = 0, base1 = 0;
        if (row_in) {
            wy = exact_tap(dy, p.src_h, p.reg_h, p.inv_den_y, p.magic_y).w;
            base0 = (uint32_t)(2 * r) * slot_bytes + (uint32_t)(slot_addr[2 * r] & 15);
            base1 = (uint32_t)(2 * r + 1) * slot_bytes + (uint32_t)(slot_addr[2 * r + 1] & 15);
        }
        float out[3][PX];
#pragma unroll
        for (int i = 0; i < PX; ++i) {
            const int dx = x_first + i - p.left;
            if (row_in && dx >= 0 && dx < p.reg_w) {
                const AxisTap tx = exact_tap(dx, p.src_w, p.reg_w, p.inv_den_x, p.magic_x);
                const uint32_t o0 = 3u * tx.i0 - (uint32_t)p.span_lo;
                const uint32_t o1 = 3u * tx.i1 - (uint32_t)p.span_lo;
                const uint32_t t00 = lds_rgb(lds32, base0 + o0);
                const uint32_t t01 = lds_rgb(lds32, base0 + o1);
                const uint32_t t10 = lds_rgb(lds32, base1 + o0);
                const uint32_t t11 = lds_rgb(lds32, base1 + o1);
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const uint32_t sh = p.shift[c];   // byte of output channel c
                    const float p00 = chan(t00, sh), p01 = chan(t01, sh);
                    const float p10 = chan(t10, sh), p11 = chan(t11, sh);
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
        OutT* const row_out = frame_out + (int64_t)y * p.dst_w + x_first;
        if (p.vec) {   // dst_w % PX == 0: the PX columns are one aligned vector
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                if constexpr (PX > 1)
                    store_stream(row_out + c * plane, out[c]);
                else
                    row_out[c * plane] = Fmt::cvt(out[c][0]);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 3; ++c)
#pragma unroll
                for (int i = 0; i < PX; ++i)
                    if (x_first + i < p.dst_w) row_out[c * plane + i] = Fmt::cvt(out[c][i]);
        }
    }
}

// The pixel whose first byte is byte e (0..6) of a window.
__device__ __forceinline__ uint32_t window_rgb(const uint32_t (&w)[3], uint32_t e) {
    const uint32_t lo = e < 4 ? w[0] : w[1];
    const uint32_t hi = e < 4 ? w[1] : w[2];
    return __builtin_amdgcn_alignbyte(hi, lo, e & 3u);
}

// A source row's window for one output column: the 4-byte-aligned address at
// or below the column's first tap byte, split into a part common to the
// workgroup (the row's base, rounded down to 4 bytes, and its remainder) and
// the lane's 32-bit offset from that base.
struct RowBase {
    const uint8_t* ptr;   // source row start rounded down to 4 bytes
    uint32_t mis;         // row start - ptr (0..3)
    uint32_t avail;       // bytes of the input from ptr on, capped at 2^32 - 1
};

__device__ __forceinline__ RowBase row_base(const PreParams& p, int64_t row_start) {
    RowBase r;
    const int64_t a = row_start & ~(int64_t)3;
    r.ptr = p.src + a;
    r.mis = (uint32_t)(row_start - a);
    const int64_t rest = p.total_bytes - a;
    r.avail = rest > (int64_t)0xffffffff ? 0xffffffffu : (uint32_t)rest;
    return r;
}

// Three dwords at byte offset `off` (a multiple of 4) from the row base, when
// the caller has checked that they lie inside the input.
// NT: non-temporal loads (a frame streamed through once does not displace
// cached data).
template <bool NT>
__device__ __forceinline__ void load_window_fast(const RowBase& rb, uint32_t off, uint32_t (&w)[3]) {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(rb.ptr + off);
    if constexpr (NT) {
        w[0] = __builtin_nontemporal_load(s);
        w[1] = __builtin_nontemporal_load(s + 1);
        w[2] = __builtin_nontemporal_load(s + 2);
    } else {
        w[0] = s[0];
        w[1] = s[1];
        w[2] = s[2];
    }
}

// Three dwords at byte offset `off` (a multiple of 4) from the row base, or,
// past the end of the input, its bytes below the end and zeros above.
__device__ __forceinline__ void load_window_at(const RowBase& rb, uint32_t off, uint32_t (&w)[3]) {
    if (off + 12u <= rb.avail) {
        const uint32_t* s = reinterpret_cast<const uint32_t*>(rb.ptr + off);
        w[0] = s[0];
        w[1] = s[1];
        w[2] = s[2];
    } else {
        w[0] = w[1] = w[2] = 0u;
        for (uint32_t b = 0; b < 12; ++b)
            if (off + b < rb.avail) w[b >> 2] |= (uint32_t)rb.ptr[off + b] << (8 * (b & 3));
    }
}

// One source-row pair of an output row, as the gather kernel sees it: the
// same for the whole workgroup, so it lives in scalar registers.
struct GatherRow {
    bool inside;          // the output row lies in the resampled region (else pad)
    bool fast;            // every lane's windows end inside the input
    float wy;             // vertical weight
    RowBase b0, b1;       // the two source rows' bases
};

__device__ __forceinline__ GatherRow gather_row(const PreParams& p, int64_t fbase, int y) {
    GatherRow g;
    const int dy = y - p.top;
    g.inside = dy >= 0 && dy < p.reg_h;
    // Pad rows read (and ignore) the region's nearest row, so their loads
    // stay inside the frame.
    const int dyc = dy < 0 ? 0 : (dy >= p.reg_h ? p.reg_h - 1 : dy);
    const AxisTap ty = exact_tap(dyc, p.src_h, p.reg_h, p.inv_den_y, p.magic_y);
    g.wy = ty.w;
    const int64_t row_bytes = 3 * (int64_t)p.src_w;
    g.b0 = row_base(p, fbase + (int64_t)ty.i0 * row_bytes);
    g.b1 = row_base(p, fbase + (int64_t)ty.i1 * row_bytes);
    // The last window of a row starts at most 3 (src_w - 1) + 3 bytes past
    // the row base.
    const uint32_t last = (uint32_t)(3 * (p.src_w - 1) + 3) & ~3u;
    g.fast = last + 12u <= g.b0.avail && last + 12u <= g.b1.avail;
    return g;
}

// Device-resident frames, each thread reading its taps straight from global
// memory, one window per source row, so nothing is staged and no barrier
// precedes the loads.  Same taps and arithmetic as preprocess_kernel<PX>.
// Workgroup (blockIdx.x, blockIdx.y) owns rows_per_group consecutive output
// rows of frame blockIdx.y; a thread owns output columns threadIdx.x,
// + blockDim.x, ... of each of those rows.  What depends on the row alone
// (vertical taps, source and output row addresses) is the same for the whole
// workgroup and is computed on the scalar unit; a lane keeps its column's
// horizontal taps across rows and addresses the frame with 32-bit offsets
// from the row bases.  The channel bytes sit at fixed positions of a pixel
// word (SH0..SH2), so each unpacks with one conversion.  NT selects
// non-temporal frame loads and tensor stores.  PAD_ROWS marks a letterbox
// with pad rows above or below the region: those rows store the pad value
// without loading (a separate instance, since the extra scalar test ahead of
// the loads slowed the plain resize's streaming launch).  (Two or four columns
// per thread, with all their windows requested together, and workgroups that
// walk many rows with the next row's windows requested ahead, both ran
// slower on MI355X: the most short-lived waves streamed best.)
template <typename OutT, int SH0, int SH1, int SH2, bool NT, bool PAD_ROWS>
__global__ __launch_bounds__(1024) void preprocess_gather_kernel(PreParams p) {
    using Fmt = OutFormat<OutT>;
    constexpr uint32_t kShift[3] = {SH0, SH1, SH2};
    const int y_base = (int)blockIdx.x * p.rows_per_group;
    const int nrows = min(p.rows_per_group, p.dst_h - y_base);
    const int64_t fbase = (int64_t)blockIdx.y * p.frame_bytes;
    const int64_t plane = (int64_t)p.dst_h * p.dst_w;
    OutT* const frame_out = reinterpret_cast<OutT*>(p.dst) + (int64_t)blockIdx.y * 3 * plane;
    for (uint32_t x = threadIdx.x; x < (uint32_t)p.dst_w; x += blockDim.x) {
        // Pad columns take the region's nearest column's taps, so every load
        // stays inside the frame.
        const int dx = (int)x - p.left;
        const bool col_in = dx >= 0 && dx < p.reg_w;
        const int dxc = dx < 0 ? 0 : (dx >= p.reg_w ? p.reg_w - 1 : dx);
        const AxisTap tx = exact_tap(dxc, p.src_w, p.reg_w, p.inv_den_x, p.magic_x);
        const uint32_t cx = 3u * tx.i0;                 // first tap byte within a row
        const uint32_t d = 3u * (tx.i1 - tx.i0);        // 0 (edge clamp) or 3
        for (int r = 0; r < nrows; ++r) {
            const int y = y_base + r;
            const GatherRow g = gather_row(p, fbase, y);
            uint32_t w0[3], w1[3];
            if (!PAD_ROWS || g.inside) {
                if (g.fast) {
                    load_window_fast<NT>(g.b0, (g.b0.mis + cx) & ~3u, w0);
                    load_window_fast<NT>(g.b1, (g.b1.mis + cx) & ~3u, w1);
                } else {
                    // The input's last rows: windows near its end read bytewise.
                    load_window_at(g.b0, (g.b0.mis + cx) & ~3u, w0);
                    load_window_at(g.b1, (g.b1.mis + cx) & ~3u, w1);
                }
            }
            float out[3];
            if (g.inside && col_in) {
                const uint32_t o0 = (g.b0.mis + cx) & 3u, o1 = (g.b1.mis + cx) & 3u;
                const uint32_t t00 = window_rgb(w0, o0), t01 = window_rgb(w0, o0 + d);
                const uint32_t t10 = window_rgb(w1, o1), t11 = window_rgb(w1, o1 + d);
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const uint32_t sh = kShift[c];
                    const float p00 = chan(t00, sh), p01 = chan(t01, sh);
                    const float p10 = chan(t10, sh), p11 = chan(t11, sh);
                    const float h0 = fmaf(tx.w, p01 - p00, p00);
                    const float h1 = fmaf(tx.w, p11 - p10, p10);
                    const float v = fmaf(g.wy, h1 - h0, h0);
                    out[c] = fmaf(v, p.a[c], p.b[c]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 3; ++c) out[c] = p.padv[c];
            }
            OutT* const row_out = frame_out + (int64_t)y * p.dst_w;
            if constexpr (NT) {
#pragma unroll
                for (int c = 0; c < 3; ++c) Fmt::store_nt(&row_out[c * plane + x], out[c]);
            } else {
#pragma unroll
                for (int c = 0; c < 3; ++c) row_out[c * plane + x] = Fmt::cvt(out[c]);
            }
        }
    }
}

template <typename OutT, int SH0, int SH1, int SH2>
void launch_gather(const PreParams& p, dim3 g, dim3 b, hipStream_t stream) {
    const bool pad_rows = p.reg_h < p.dst_h;
    if (p.streaming) {
        if (pad_rows)
            hipLaunchKernelGGL((preprocess_gather_kernel<OutT, SH0, SH1, SH2, true, true>), g, b, 0, stream, p);
        else
            hipLaunchKernelGGL((preprocess_gather_kernel<OutT, SH0, SH1, SH2, true, false>), g, b, 0, stream, p);
    } else {
        if (pad_rows)
            hipLaunchKernelGGL((preprocess_gather_kernel<OutT, SH0, SH1, SH2, false, true>), g, b, 0, stream, p);
        else
            hipLaunchKernelGGL((preprocess_gather_kernel<OutT, SH0, SH1, SH2, false, false>), g, b, 0, stream, p);
    }
}

template <typename OutT>
hipError_t launch_preprocess_as(const PreParams& p, dim3 g, dim3 b, unsigned lds,
                                hipStream_t stream) {
    switch (p.pixels_per_thread) {
        case 1: {
            // Frame in the grid's y dimension, row group in x.
            const dim3 gg((unsigned)p.groups_per_frame, g.x / (unsigned)p.groups_per_frame);
            // Channel byte positions of a pixel word: RGB or BGR producers.
            if (p.shift[0] == 0)
                launch_gather<OutT, 0, 8, 16>(p, gg, b, stream);
            else
                launch_gather<OutT, 16, 8, 0>(p, gg, b, stream);
            break;
        }
        case 2: hipLaunchKernelGGL((preprocess_kernel<2, OutT>), g, b, lds, stream, p); break;
        case 4: hipLaunchKernelGGL((preprocess_kernel<4, OutT>), g, b, lds, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename OutT>
hipError_t raise_lds_limit() {
    // Only the staged kernels (two or four columns per thread) take dynamic
    // LDS; the gather kernel that runs one column per thread holds none.
    const void* fns[2] = {reinterpret_cast<const void*>(preprocess_kernel<2, OutT>),
                          reinterpret_cast<const void*>(preprocess_kernel<4, OutT>)};
    for (const void* f : fns) {
        const hipError_t e =
            hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_preprocess(const PreParams& p, int groups, int block, int lds_bytes,
                             hipStream_t stream) {
    const dim3 g((unsigned)groups), b((unsigned)block);
    switch (p.dtype) {
        case WS_DTYPE_F32: return launch_preprocess_as<float>(p, g, b, (unsigned)lds_bytes, stream);
        case WS_DTYPE_F16: return launch_preprocess_as<__half>(p, g, b, (unsigned)lds_bytes, stream);
        case WS_DTYPE_BF16:
            return launch_preprocess_as<__hip_bfloat16>(p, g, b, (unsigned)lds_bytes, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t set_preprocess_attributes() {
    hipError_t e = raise_lds_limit<float>();
    if (e == hipSuccess) e = raise_lds_limit<__half>();
    if (e == hipSuccess) e = raise_lds_limit<__hip_bfloat16>();
    return e;
}

}  // namespace ws
