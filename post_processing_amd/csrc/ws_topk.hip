// ws_topk.hip -- the exact Top-K kernels of the frame pipeline, written for
// gfx950 (CDNA4, wave64).
//
// WarpStream TRT article, Top-K passage: exact K best of FP32 scores, ties to
// the lower index, NaN as -inf, only K pairs leave the GPU; its advice for
// large label spaces (hierarchical selection) gives the partial + merge split
// across workgroups.
#include <hip/hip_runtime.h>

#include "ws_kernels.h"
#include "ws_lanes.h"
#include "ws_marks.h"

namespace ws {
namespace {

#ifdef WS_CLOCK_MARKS
// Phase marks of the Top-K kernels: the partial kernel's wave w of workgroup
// g writes slots (4 g + w) * 8 + phase, the merge kernels' wave w slots
// kMergeMarks + 8 w + phase.
__device__ uint64_t g_marks[kMarkSlots];
#endif
constexpr int kMergeMarks = 1 << 16;

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
// best).  Scores arrive in batches of 1024 or 2048 (16 or 32 per lane).  Only
// scores at or above the running K-th best can matter; in a wave's first
// batch the K-th largest of the 64 lane maxima is also a lower bound (K
// distinct scores of the batch reach it), which prunes the rest.  Survivors
// get exact keys and are compacted through the wave's LDS scratch.  A few are
// inserted one by one; when the list's K best and the survivors fit one key
// per lane they are bitonic-sorted together (over the smallest power-of-two
// block of lanes that holds them); more go in tiles of 64, each sorted
// across lanes and merged into the list (elementwise max against the reversed
// tile, then a bitonic clean-up).  All lane exchanges run on the VALU: DPP
// for lane distances 1, 2, 4, 8 and the permlane swaps for 16 and 32.  Waves of a
// workgroup merge pairwise through LDS.  With several workgroups, each
// publishes its K best and a one-workgroup merge kernel, next in stream
// order, selects the K best of those lists.  Up to 128 lists it folds them
// pairwise with bitonic merges; beyond that it derives a lower bound on the
// K-th best from the lists, keeps only the keys at or above it and selects
// from them.  The kernel boundary orders the two, so no fence or arrival
// counter sits on the path.

// Order-preserving unsigned image of an FP32 value: NaN -> -inf and -0 -> +0
// first; then negative values have all bits flipped, others the sign bit set.
__device__ __forceinline__ uint32_t order_image(float v) {
    uint32_t b = __float_as_uint(v);
    b = (b & 0x7fffffffu) > 0x7f800000u ? 0xff800000u : b;   // NaN -> -inf
    b = b == 0x80000000u ? 0u : b;                            // -0 -> +0
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// The lane number through an empty asm: the lane masks of a network given
// this value are shared within that network only, not hoisted to the
// kernel's start with every other network's.
__device__ __forceinline__ int fresh_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// Sort a bitonic sequence (one key per lane) into descending lane order.
__device__ __forceinline__ uint64_t wave_clean_desc(uint64_t x, int lane) {
    return bitonic_stages<64, 32, true>(x, fresh_lane(lane));
}

constexpr int kInsertMax = 4;                      // fewer survivors: insert one by one

// K-th largest of one 32-bit value per lane, with multiplicity: lane k - 1 of
// the 64 values sorted descending across the wave.  The 21 stages of the
// sorting network are short lane exchanges; selecting the value bit by bit
// from the top instead takes 32 rounds of compare, ballot and count, each
// waiting on the last.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t m, int k, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_sort<true>(m, fresh_lane(lane)), k - 1);
}

// Number of the n keys of v (LDS) greater than x; sixteen loads are issued
// before their compares.
__device__ __forceinline__ int count_greater(const uint64_t* v, int n, uint64_t x) {
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

// Largest of N floats as a pairwise tree (log2 N dependent steps instead of
// N - 1); a NaN never wins over a number, as with a running fmaxf.
template <int N>
__device__ __forceinline__ float tree_max(const float (&f)[N]) {
    float m[N / 2];
#pragma unroll
    for (int j = 0; j < N / 2; ++j) m[j] = fmaxf(f[2 * j], f[2 * j + 1]);
#pragma unroll
    for (int w = N / 4; w >= 1; w /= 2) {
#pragma unroll
        for (int j = 0; j < w; ++j) m[j] = fmaxf(m[2 * j], m[2 * j + 1]);
    }
    return m[0];
}

// E scores per lane per batch (16 or 32): a batch is 64 E scores per wave.
template <int E>
struct WaveTopK {
    static_assert(E == 16 || E == 32, "16 or 32 scores per lane");
    static constexpr int kBatchE = 64 * E;
    static constexpr int kCountBits = E == 16 ? 5 : 6;   // bits of a lane's survivor count
    static constexpr int kStageRow = E + 4;               // floats per lane row of the score stage
    uint64_t best;   // this lane's entry of the wave's sorted list
    uint64_t thr;    // K-th best key so far (wave-uniform)
    int k;
    int lane;
    bool empty;      // nothing merged yet (wave-uniform)
    int mark = -1;   // clock-mark slot of the first batch's phases (marks builds)

    __device__ __forceinline__ void init(int k_, int lane_) {
        best = 0;
        thr = 0;
        k = k_;
        lane = lane_;
        empty = true;
    }

    // Merge a list sorted ascending across lanes (e.g. a reversed list).
    __device__ __forceinline__ void merge_ascending(uint64_t asc) {
        best = wave_clean_desc(umax64(best, asc), lane);
        thr = readlane64(best, k - 1);
    }

    __device__ __forceinline__ void insert(uint64_t c) {
        if (c <= thr) return;
        const int pos = __popcll(__ballot(best > c));
        const uint64_t shifted = prev_lane64(best);
        best = lane < pos ? best : (lane == pos ? c : shifted);
        thr = readlane64(best, k - 1);
    }

    // Merge `cnt` compacted survivors scratch[0..cnt) into the list.
    //  - a few: insert one by one;
    //  - into an empty list, at most 64: sort them;
    //  - list and survivors fit one key per lane: one bitonic sort of both;
    //  - otherwise, 64 at a time: sort ascending, then the elementwise
    //    maximum against the descending list is the top 64 of their union as
    //    a bitonic sequence, which a clean-up network sorts.
    // Lanes at or past k may keep real keys below the K-th best; every
    // consumer reads the list sorted across all 64 lanes, so they never matter.
    __device__ __forceinline__ void merge_survivors(uint64_t* scratch, int cnt) {
        if (cnt <= kInsertMax) {
            const uint64_t cand = lane < cnt ? scratch[lane] : 0;
            for (int i = 0; i < cnt; ++i) insert(readlane64(cand, i));
        } else if (empty && cnt <= 64) {
            // The first keys: sorted, they are the list.
            best = wave_sort_desc_first(lane < cnt ? scratch[lane] : 0, fresh_lane(lane), cnt);
            thr = readlane64(best, k - 1);
        } else if (k + cnt <= 64) {
            const uint64_t x = lane < k ? best : (lane < k + cnt ? scratch[lane - k] : 0);
            best = wave_sort_desc_first(x, fresh_lane(lane), k + cnt);
            thr = readlane64(best, k - 1);
        } else {
            for (int t = 0; t < cnt; t += 64) {
                const uint64_t tile = t + lane < cnt ? scratch[t + lane] : 0;
                best = wave_clean_desc(umax64(best, wave_sort<false>(tile, fresh_lane(lane))), lane);
            }
            thr = readlane64(best, k - 1);
        }
        empty = false;
    }

    // Offer one batch of order keys, E per lane (0 = nothing).
    // `scratch` is this wave's LDS area of kBatchE keys.
    __device__ __forceinline__ void offer(const uint64_t (&key)[E], uint64_t* scratch) {
        uint64_t cut = thr;
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) cnt += __popcll(__ballot(key[j] > cut));
        if (cnt == 0) return;
        if (cnt > 64) {
            // K lanes hold a key whose value image is at least the K-th largest
            // lane maximum t, so every key of the K best has value image >= t.
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < E; ++j) m = max(m, (uint32_t)(key[j] >> 32));
            const uint32_t t = wave_kth_largest(m, k, lane);
            const uint64_t tcut = ((uint64_t)t << 32) - 1;   // key > tcut <=> value image >= t
            if (t != 0 && tcut > cut) {
                cut = tcut;
                cnt = 0;
#pragma unroll
                for (int j = 0; j < E; ++j) cnt += __popcll(__ballot(key[j] > cut));
            }
        }
        int base = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool take = key[j] > cut;
            const uint64_t b = __ballot(take);
            if (take) scratch[base + lanes_below(b)] = key[j];
            base += __popcll(b);
        }
        wave_lds_sync();
        merge_survivors(scratch, cnt);
        wave_lds_sync();
    }

    // Offer one batch of raw scores: f[4u + j] sits at position
    // wb + 4 (lane + 64 u) + j; positions at or past the end hold -inf.
    // Once the cut is a positive value, scores are screened on their raw bits
    // and only survivors get exact order keys; otherwise every score does.
    __device__ __forceinline__ void offer_scores(const float (&f)[E], int32_t wb,
                                                 int32_t g1, uint64_t* scratch, float* fstage) {
        uint32_t cut_ord = (uint32_t)(thr >> 32);          // value image of the K-th best
        if (cut_ord <= 0x80000000u) {
            // No positive cut yet: the K-th largest lane maximum bounds the
            // batch's K best from below.
            const uint32_t t = wave_kth_largest(order_image(tree_max<E>(f)), k, lane);
            cut_ord = max(cut_ord, t);
            if (mark >= 0) WS_MARK(mark + 5);
        }
        if (cut_ord <= 0x80000000u) {   // cut at or below +0: exact keys for all
            uint64_t key[E];
#pragma unroll
            for (int u = 0; u < E / 4; ++u) {
                const int32_t e = wb + 4 * (lane + 64 * u);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint64_t kk = ((uint64_t)order_image(f[4 * u + j]) << 32) |
                                        (uint32_t)~(uint32_t)(e + j);
                    key[4 * u + j] = kk & (0ull - (uint64_t)(e + j < g1));
                }
            }
            offer(key, scratch);
            return;
        }
        // Positive cut t: a score can be among the K best only if x >= t (a
        // NaN compares false and ranks as -inf; pad positions hold -inf).
        // Survivors equal to t are kept too: they are genuine scores, so the
        // merge still returns the exact K best.  Each lane counts its
        // survivors and marks their slots; an exclusive scan of the counts
        // (one ballot per count bit) gives each lane its first slot in
        // `scratch`; each lane then walks its own survivors, reading the
        // values back from its row of `fstage`, and writes their exact keys.
        // Rows are kStageRow = E + 4 floats apart: the 16-byte row stores
        // then cover all banks eight lanes at a time, and the read-back of
        // one float per lane conflicts at most 8 ways (a stride of E floats
        // put every lane on the same banks).
        const float tf = __uint_as_float(cut_ord & 0x7fffffffu);
        int cnt = 0;
        uint32_t marks = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const bool pass = f[j] >= tf;
            cnt += pass ? 1 : 0;
            marks |= pass ? (1u << j) : 0u;
        }
        int off = 0, total = 0;
#pragma unroll
        for (int bit = 0; bit < kCountBits; ++bit) {   // cnt <= E
            const uint64_t b = __ballot((cnt >> bit) & 1);
            off += lanes_below(b) << bit;
            total += __popcll(b) << bit;
        }
        if (total == 0) return;
        float4* row = reinterpret_cast<float4*>(fstage + lane * kStageRow);
#pragma unroll
        for (int u = 0; u < E / 4; ++u)
            row[u] = make_float4(f[4 * u], f[4 * u + 1], f[4 * u + 2], f[4 * u + 3]);
        wave_lds_sync();
        while (marks != 0) {
            const int j = __builtin_ctz(marks);
            marks &= marks - 1;
            const int32_t e = wb + 4 * (lane + 64 * (j >> 2)) + (j & 3);
            const float x = fstage[lane * kStageRow + j];
            scratch[off++] = ((uint64_t)order_image(x) << 32) | (uint32_t)~(uint32_t)e;
        }
        wave_lds_sync();
        if (mark >= 0) WS_MARK(mark + 6);
        merge_survivors(scratch, total);
        wave_lds_sync();
        if (mark >= 0) WS_MARK(mark + 7);
        mark = -1;
    }
};

// Into wave 0: lanes < k of st.best hold the workgroup's k best, descending,
// other lanes 0.  Each wave's k best go to its LDS row; wave 0 folds rows 1
// and 3, read reversed, into rows 0 and 2 side by side (one per half), the
// lower half ending descending and the upper ascending, then the upper half,
// swapped down, into the lower: one LDS round trip.
template <int E>
__device__ __forceinline__ void block_merge(WaveTopK<E>& st, uint64_t (*s_list)[64], int wave,
                                            int waves) {
    if (waves == 1) return;
    const int lane = st.lane, k = st.k;
    if (lane < k) s_list[wave][lane] = st.best;
    __syncthreads();
    if (wave != 0) return;
    const int h = lane & 31, r = 31 - h;
    const int dw = lane < 32 ? 0 : 2, aw = dw + 1;
    const uint64_t d = (dw < waves && h < k) ? s_list[dw][h] : 0;
    const uint64_t a = (aw < waves && r < k) ? s_list[aw][r] : 0;
    const uint64_t x = bitonic_stages<32, 16, true>(umax64(d, a), lane);
    const uint64_t y = bitonic_stages<64, 16, true>(umax64(x, xor_lane64<32>(x, lane)), lane);
    st.best = lane < 32 ? y : 0;
    st.thr = readlane64(st.best, k - 1);
}

// Result slot `slot` from an order key.  The value is the inverse of its
// order image, which is exact except for a zero's sign (both zeros share an
// image), so only a zero is read back from the scores.  NaN was ranked as -inf
// and is reported as -inf.  K <= N guarantees K real keys; the sentinel key 0
// only keeps a malformed call in bounds.
__device__ __forceinline__ void write_result(const TopkParams& p, uint64_t key, int slot) {
    const uint32_t idx = ~(uint32_t)key;
    const uint32_t img = (uint32_t)(key >> 32);
    uint32_t bits = (img & 0x80000000u) ? (img ^ 0x80000000u) : ~img;
    if (key == 0) bits = 0xff800000u;
    else if (img == 0x80000000u && (int64_t)idx < p.n) bits = __float_as_uint(p.scores[idx]);
    p.result[slot] = make_uint2(bits, idx);
}

// One wave's batch: E scores per lane as E / 4 float4 loads, lane-interleaved
// so each load instruction covers 1 KiB of consecutive scores.  Score
// positions fit in 31 bits (the vector length is an int32).
template <int E>
__device__ __forceinline__ void load_batch(const float* __restrict__ scores, int32_t wb, int32_t g1,
                                           int lane, float4 (&v)[E / 4]) {
#pragma unroll
    for (int u = 0; u < E / 4; ++u) {
        const int32_t e = wb + 4 * (lane + 64 * u);
        const float ninf = -__builtin_inff();
        v[u] = make_float4(ninf, ninf, ninf, ninf);
        if (e + 4 <= g1) {
            v[u] = *reinterpret_cast<const float4*>(scores + e);
        } else {
            if (e + 0 < g1) v[u].x = scores[e + 0];
            if (e + 1 < g1) v[u].y = scores[e + 1];
            if (e + 2 < g1) v[u].z = scores[e + 2];
        }
    }
}

constexpr int kTopkWaveSlots = kTopkMaxThreads / 64;

// Dynamic LDS: per wave, 64 E survivor keys, then per wave 64 staged score
// rows of E + 4 floats.
template <int E>
constexpr int topk_lds_bytes() {
    return kTopkWaveSlots * 64 * (E * (int)sizeof(uint64_t) + (E + 4) * (int)sizeof(float));
}

// The Top-K kernels take TopkParams's fields as plain scalar and pointer
// arguments: the library is built with amdgpu-kernarg-preload-count, so they
// arrive in scalar registers at wave launch, where a by-value struct is read
// with scalar loads after the launch (~0.3 us before the scores can be
// requested; Top-K stage 3.27 -> 3.01 us for 1,000 scores, 9.35 -> 9.05 us
// for 672,000).
__device__ __forceinline__ TopkParams topk_params(const float* scores, int64_t n, int32_t k,
                                                  int32_t chunk, int32_t keys_per_lane,
                                                  int32_t groups, int32_t waves,
                                                  uint64_t* partials, uint2* result) {
    TopkParams p;
    p.scores = scores;
    p.n = n;
    p.k = k;
    p.chunk = chunk;
    p.keys_per_lane = keys_per_lane;
    p.groups = groups;
    p.waves = waves;
    p.partials = partials;
    p.result = result;
    return p;
}

template <int E>
__global__ __launch_bounds__(kTopkMaxThreads) void topk_kernel(
    const float* scores, int64_t n, int32_t k, int32_t chunk, int32_t keys_per_lane,
    int32_t groups, int32_t waves_arg, uint64_t* partials, uint2* result) {
    const TopkParams p =
        topk_params(scores, n, k, chunk, keys_per_lane, groups, waves_arg, partials, result);
    constexpr int kBatchE = 64 * E;
    constexpr int kTopkStageKeys = kTopkWaveSlots * kBatchE;   // the scratch area, in keys
    extern __shared__ uint4 lds_dyn[];
    uint64_t* const s_keys = reinterpret_cast<uint64_t*>(lds_dyn);
    float* const s_vals = reinterpret_cast<float*>(s_keys + kTopkStageKeys);
    __shared__ uint64_t s_list[kTopkWaveSlots][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int waves = p.waves;

    WaveTopK<E> st;
    st.init(p.k, lane);
    const int mark = ((int)blockIdx.x * kTopkWaveSlots + wave) * 8;
    (void)mark;
    WS_MARK(mark + 0);

    // 1. This workgroup's chunk, one 64 E-score batch per wave per round; the
    //    next round's scores are loaded while the current batch is offered.
    const int32_t g0 = (int32_t)blockIdx.x * p.chunk;
    const int32_t g1 = (int32_t)min(p.n, (int64_t)g0 + p.chunk);
    const int32_t round = waves * kBatchE;
    float4 v[E / 4];
    load_batch<E>(p.scores, g0 + wave * kBatchE, g1, lane, v);
    WS_MARK_AFTER_LOADS(mark + 1);
#ifdef WS_CLOCK_MARKS
    st.mark = mark;
#endif
    for (int32_t rb = g0; rb < g1; rb += round) {
        const int32_t wb = rb + wave * kBatchE;
        float f[E];
#pragma unroll
        for (int u = 0; u < E / 4; ++u) {
            f[4 * u + 0] = v[u].x;
            f[4 * u + 1] = v[u].y;
            f[4 * u + 2] = v[u].z;
            f[4 * u + 3] = v[u].w;
        }
        if (rb + round < g1) load_batch<E>(p.scores, wb + round, g1, lane, v);
        st.offer_scores(f, wb, g1, s_keys + wave * kBatchE, s_vals + wave * 64 * (E + 4));
    }
    WS_MARK(mark + 2);
    block_merge(st, s_list, wave, waves);
    WS_MARK(mark + 3);

    if (p.groups == 1) {
        if (wave == 0 && lane < p.k) write_result(p, st.best, lane);
        WS_MARK(mark + 4);
        return;
    }

    // 2. Publish this workgroup's K best for the merge kernel, which follows
    //    in stream order.
    if (wave == 0 && lane < p.k) p.partials[(int64_t)blockIdx.x * p.k + lane] = st.best;
    WS_MARK(mark + 4);
}

// Merge of up to kFoldMaxLists workgroup lists by folding.  A register holds
// two lists of up to 32 keys, one per 32-lane half, zero-padded past K.  A
// descending register (both halves sorted descending) and an ascending one
// meet half by half as one descending and one ascending list, so their
// elementwise maximum holds the 32 largest keys of each half's union as a
// bitonic sequence, and a clean-up over distances 16 .. 1 sorts it either
// way.  Keys are distinct (the index is in the low word), so each fold is
// exact.  Each wave loads R registers (list pairs wave, wave + 4, ...), each
// in the order its place in the fold asks for, and folds them; the
// root leaves the lower half descending and the upper ascending, so the
// upper half, swapped down, folds into the lower.  The four waves merge
// through LDS.  Nothing depends on the data: no bound, no survivor count, no
// atomic.  Lists are loaded in address order (a half whose lanes read
// descending addresses took several times as long to arrive), and an
// ascending leaf is reversed in registers.
constexpr int kFoldMaxLists = 128;

// The fold runs level by level: nodes 2q and 2q + 1 of a level fold into node
// q of the next, and an odd level's last node passes through to the next
// level's last.  The pairs of a level are independent, so each clean-up
// distance is issued for all of them before the next: their dependent
// compare-exchange chains interleave instead of running one after another.
// A pair folds a descending node (even index) with an ascending one (odd), so
// a leaf's order is fixed by its index at the first level where it is paired.
constexpr bool fold_node_desc(int i, int n) {
    return n <= 1 ? true
                  : ((n & 1) && i == n - 1 ? fold_node_desc((n + 1) / 2 - 1, (n + 1) / 2)
                                           : (i & 1) == 0);
}

// Bit r set: leaf r of R is loaded descending.
template <int R>
constexpr uint32_t fold_leaf_mask() {
    uint32_t m = 0;
    for (int r = 0; r < R; ++r) m |= fold_node_desc(r, R) ? 1u << r : 0u;
    return m;
}

// Bit q set: node q of a level of NN nodes ends descending.
template <int NN>
constexpr uint32_t fold_desc_mask() {
    uint32_t m = 0;
    for (int q = 0; q < NN; ++q) m |= fold_node_desc(q, NN) ? 1u << q : 0u;
    return m;
}

// Clean-up distances J .. 1 for the first M nodes of a level of NN: each ends
// in the order the next level needs of it, both halves of a register alike.
// Each step is written for all M registers at once (exchanges, then compares
// and picks), so the registers' chains interleave in the issued code.
template <int J, int M, int NN>
__device__ __forceinline__ void fold_stage(uint64_t (&y)[NN], int lane) {
    constexpr uint32_t kDesc = fold_desc_mask<NN>();
    const bool lower = (lane & J) == 0;
    uint64_t o[M];
#pragma unroll
    for (int q = 0; q < M; ++q) o[q] = xor_lane64<J>(y[q], lane);
    bool keep[M];
#pragma unroll
    for (int q = 0; q < M; ++q) keep[q] = (y[q] > o[q]) == (lower == (((kDesc >> q) & 1u) != 0));
#pragma unroll
    for (int q = 0; q < M; ++q) y[q] = keep[q] ? y[q] : o[q];
    if constexpr (J > 1) fold_stage<J / 2, M>(y, lane);
}

// Folds N registers into one whose lower half is descending and upper half
// ascending (the root pairs the last two nodes half by half that way).
template <int N>
__device__ __forceinline__ uint64_t fold_levels(const uint64_t (&x)[N], int lane) {
    if constexpr (N == 1) {
        return x[0];
    } else if constexpr (N == 2) {
        return bitonic_stages<32, 16, true>(umax64(x[0], x[1]), lane);
    } else {
        constexpr int M = N / 2, NN = (N + 1) / 2;
        uint64_t y[NN];
#pragma unroll
        for (int q = 0; q < M; ++q) y[q] = umax64(x[2 * q], x[2 * q + 1]);
        fold_stage<16, M>(y, lane);
        if constexpr (N & 1) y[NN - 1] = x[N - 1];
        return fold_levels<NN>(y, lane);
    }
}

template <int R>
__global__ __launch_bounds__(kTopkMaxThreads) void topk_fold_kernel(
    const float* scores, int64_t n, int32_t k_arg, int32_t chunk, int32_t keys_per_lane,
    int32_t groups, int32_t waves_arg, uint64_t* partials, uint2* result) {
    const TopkParams p = topk_params(scores, n, k_arg, chunk, keys_per_lane, groups, waves_arg,
                                     partials, result);
    __shared__ uint64_t s_list[kTopkWaveSlots][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int k = p.k, G = p.groups;
    const int half = lane >> 5, h = lane & 31;
    const int last = G * k - 1;   // the published keys are partials[0 .. last]
    const int mark = kMergeMarks + 8 * wave;
    (void)mark;
    WS_MARK(mark + 0);
    // Every load is issued, in bounds, before any is used: a lane with no key
    // reads a spare published key (lanes on distinct addresses) and drops it.
    uint64_t x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int list = 2 * (wave + kTopkWaveSlots * r) + half;
        const bool valid = list < G && h < k;
        x[r] = p.partials[valid ? list * k + h : min(lane + 64 * r, last)];
    }
    __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first is used
    WS_MARK_AFTER_LOADS(mark + 1);
    constexpr uint32_t kLeafDesc = fold_leaf_mask<R>();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int list = 2 * (wave + kTopkWaveSlots * r) + half;
        const uint64_t v = list < G && h < k ? x[r] : 0;   // descending in both halves
        if constexpr (R == 1) {
            const uint64_t rev = reverse_half64(v, lane);
            x[r] = half == 0 ? v : rev;
        } else {
            x[r] = ((kLeafDesc >> r) & 1u) ? v : reverse_half64(v, lane);
        }
    }
    uint64_t w = fold_levels<R>(x, lane);
    w = bitonic_stages<64, 16, true>(umax64(w, xor_lane64<32>(w, lane)), lane);
    WS_MARK(mark + 2);
    WaveTopK<16> st;
    st.init(k, lane);
    st.best = w;
    block_merge(st, s_list, wave, kTopkWaveSlots);
    WS_MARK(mark + 3);
    if (wave == 0 && lane < k) write_result(p, st.best, lane);
    WS_MARK(mark + 4);
}

// Merge of more than kFoldMaxLists workgroup lists, by one workgroup of four
// waves, 256 lists per round.  Any K distinct keys bound the K-th
// best from below, so the bound is the larger of the K-th key of any one
// list and the K-th largest of the lists' maxima.  Every key of the K best
// is in its own workgroup's list, so the keys at or above the bound are all
// that can matter; they are compacted into LDS.  Keys are distinct, so a
// survivor's rank is the number of survivors above it, counted against
// broadcast LDS reads; the K that rank below K write their slots directly.
// The bound comes from this launch's lists alone: no state carries over
// between launches.  With more than 256 lists, or more survivors than two per
// thread, each wave merges a quarter of every round's survivors into its
// list instead and the lists are merged across waves.
constexpr int kMergeLists = kTopkMaxThreads;
constexpr int kMergeKeys = 32;                  // keys per thread per round (K <= 32)
constexpr int kRankMax = 2 * kTopkMaxThreads;   // survivors ranked by counting

// Survivors' area [kMergeLists * k] then one junk slot per lane.
int topk_merge_lds_bytes(int k) { return (kMergeLists * k + 64) * (int)sizeof(uint64_t); }

__global__ __launch_bounds__(kTopkMaxThreads) void topk_merge_kernel(TopkParams p) {
    extern __shared__ uint64_t s_surv[];   // [kMergeLists * k + 64]
    __shared__ uint64_t s_list[kTopkWaveSlots][64];
    __shared__ uint64_t s_max[kMergeLists];
    __shared__ uint64_t s_bound[kTopkWaveSlots];
    __shared__ int s_cnt;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int k = p.k, G = p.groups;
    const int junk = kMergeLists * k;
    uint64_t bound = 1;   // real keys are non-zero
    WaveTopK<16> st;
    st.init(k, lane);
    for (int l0 = 0; l0 < G; l0 += kMergeLists) {   // uniform
        const int lists = min(kMergeLists, G - l0);
        const int nkeys = lists * k;
        const uint64_t* part = p.partials + (int64_t)l0 * k;
        // List `tid`'s first and K-th keys, then this round's keys coalesced
        // (registers past `regs` stay unused).  The bound needs only the
        // first two, so it is worked out while the rest are still arriving.
        const uint64_t mx = tid < lists ? part[tid * k] : 0;
        uint64_t kth = tid < lists ? part[tid * k + k - 1] : 0;
        // Two keys per 16-byte load, every load unconditional so the bound
        // can start once the first two arrive.  A lane past the last pair
        // reads an earlier pair (its own index masked below the count, so
        // lanes stay on distinct addresses) and masks the keys to 0.
        const int regs = 2 * ((nkeys + 2 * kTopkMaxThreads - 1) / (2 * kTopkMaxThreads));
        const int last_pair = (nkeys - 1) >> 1;
        const int spread = (int)((0xffffffffu >> __builtin_clz((uint32_t)last_pair + 1u)) >> 1);   // 2^j - 1 <= last_pair
        uint64_t key[kMergeKeys];
#pragma unroll
        for (int m = 0; m < kMergeKeys / 2; ++m) {
            const int q = tid + m * kTopkMaxThreads;
            const ulonglong2 v = reinterpret_cast<const ulonglong2*>(part)[q <= last_pair ? q : (tid & spread)];
            key[2 * m] = 2 * q < nkeys ? v.x : 0;
            key[2 * m + 1] = 2 * q + 1 < nkeys ? v.y : 0;
        }
        __builtin_amdgcn_sched_barrier(0);   // every load issues before the bound's first use
        kth = umax64(kth, xor_lane64<32>(kth, lane));
        kth = umax64(kth, xor_lane64<16>(kth, lane));
        kth = umax64(kth, xor_lane64<8>(kth, lane));
        kth = umax64(kth, xor_lane64<4>(kth, lane));
        kth = umax64(kth, xor_lane64<2>(kth, lane));
        kth = umax64(kth, xor_lane64<1>(kth, lane));
        s_max[tid] = mx;
        if (tid == 0) s_cnt = 0;
        __syncthreads();
        // The K-th largest list maximum: the one with exactly K - 1 above it.
        uint64_t kmax = 0;
        if (tid < lists && lists >= k && count_greater(s_max, lists, mx) == k - 1) kmax = mx;
        const uint64_t b = __ballot(kmax != 0);
        if (b != 0) kmax = readlane64(kmax, __ffsll((unsigned long long)b) - 1);
        if (lane == 0) s_bound[wave] = umax64(umax64(kmax, kth), st.thr);
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kTopkWaveSlots; ++w) bound = umax64(bound, s_bound[w]);
        // Survivors per lane on the VALU, a prefix of those counts across the
        // wave (one ballot per count bit), one LDS atomic per wave, then each
        // lane stores its survivors in order.  A key below the bound goes to
        // the lane's junk slot past the survivors' area, which no one reads.
        int c = 0;
#pragma unroll
        for (int m = 0; m < kMergeKeys; ++m) c += key[m] >= bound ? 1 : 0;   // keys past the round are 0
        int off = 0, tot = 0;
#pragma unroll
        for (int bit = 0; bit < 6; ++bit) {   // c <= 32
            const uint64_t bb = __ballot((c >> bit) & 1);
            off += lanes_below(bb) << bit;
            tot += __popcll(bb) << bit;
        }
        int base = 0;
        if (lane == 0 && tot > 0) base = atomicAdd(&s_cnt, tot);
        off += __builtin_amdgcn_readfirstlane(base);
#pragma unroll
        for (int m = 0; m < kMergeKeys; ++m) {
            if (m < regs) {   // uniform
                const uint64_t x = key[m];
                const bool take = x >= bound;
                s_surv[take ? off : junk + lane] = x;
                off += take ? 1 : 0;
            }
        }
        __syncthreads();
        const int cnt = s_cnt;
        if (G <= kMergeLists && cnt <= kRankMax) {
            for (int i = tid; i < cnt; i += kTopkMaxThreads) {
                const uint64_t x = s_surv[i];
                const int r = count_greater(s_surv, cnt, x);
                if (r < k) write_result(p, x, r);
            }
            return;
        }
        const int lo = wave * cnt / kTopkWaveSlots, hi = (wave + 1) * cnt / kTopkWaveSlots;
        st.merge_survivors(s_surv + lo, hi - lo);
        __syncthreads();   // the survivors' area is rewritten by the next round
    }
    block_merge(st, s_list, wave, kTopkWaveSlots);
    if (wave == 0 && lane < k) write_result(p, st.best, lane);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
    const dim3 g((unsigned)p.groups), b((unsigned)(64 * p.waves));
    if (p.keys_per_lane == 32)
        hipLaunchKernelGGL(topk_kernel<32>, g, b, (unsigned)topk_lds_bytes<32>(), stream, p.scores,
                           p.n, p.k, p.chunk, p.keys_per_lane, p.groups, p.waves, p.partials,
                           p.result);
    else if (p.keys_per_lane == 16)
        hipLaunchKernelGGL(topk_kernel<16>, g, b, (unsigned)topk_lds_bytes<16>(), stream, p.scores,
                           p.n, p.k, p.chunk, p.keys_per_lane, p.groups, p.waves, p.partials,
                           p.result);
    else
        return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.groups == 1) return e;
    const dim3 one(1), block(kTopkMaxThreads);
    if (p.groups <= kFoldMaxLists) {
        // Registers per wave: list pairs over four waves, rounded up to a
        // size the fold is built for.
        const int need = ((p.groups + 1) / 2 + kTopkWaveSlots - 1) / kTopkWaveSlots;
        auto fold = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, one, block, 0, stream, p.scores, p.n, p.k, p.chunk,
                               p.keys_per_lane, p.groups, p.waves, p.partials, p.result);
        };
        if (need <= 1) fold(topk_fold_kernel<1>);
        else if (need <= 2) fold(topk_fold_kernel<2>);
        else if (need <= 4) fold(topk_fold_kernel<4>);
        else if (need <= 8) fold(topk_fold_kernel<8>);
        else if (need <= 12) fold(topk_fold_kernel<12>);
        else fold(topk_fold_kernel<16>);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_merge_kernel, one, block, (unsigned)topk_merge_lds_bytes(p.k), stream,
                       p);
    return hipGetLastError();
}

hipError_t set_kernel_attributes() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel<32>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       topk_lds_bytes<32>());
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_merge_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, topk_merge_lds_bytes(32));
    if (e == hipSuccess) e = set_preprocess_attributes();
    return e;
}

}  // namespace ws

#ifdef WS_CLOCK_MARKS
// Instrumented builds only: copy out (or clear) the Top-K kernels' marks.
extern "C" int ws_debug_topk_marks(uint64_t* host, size_t n, int32_t clear) {
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
