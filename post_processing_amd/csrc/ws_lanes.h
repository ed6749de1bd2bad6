// ws_lanes.h -- cross-lane primitives of a wave64 on CDNA (gfx950), shared
// by the library's kernels.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ws {

// Value held by lane (lane ^ J).  Every source lane is inside the wave, so
// the DPP forms need no "old" operand (bound_ctrl).
template <int J>
__device__ __forceinline__ uint32_t xor_lane32(uint32_t v, int lane) {
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);   // quad_perm 2,3,0,1
    } else if constexpr (J == 4) {
        const uint32_t fwd = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0xF, true);  // row_ror:12 -> lane+4
        const uint32_t bwd = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true);  // row_ror:4  -> lane-4
        return (lane & 4) ? bwd : fwd;
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);  // row_ror:8
    } else if constexpr (J == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? s[0] : s[1];
    } else {
        static_assert(J == 32, "lane distance must be a power of two below 64");
        const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? s[0] : s[1];
    }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int lane) {
    const uint32_t lo = xor_lane32<J>((uint32_t)v, lane);
    const uint32_t hi = xor_lane32<J>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Value held by lane 31 - h of the same 32-lane half (h = lane % 32): DPP
// row_mirror reverses each row of 16 lanes, then the rows of a half swap.
__device__ __forceinline__ uint64_t reverse_half64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, 0x140, 0xF, 0xF, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), 0x140, 0xF, 0xF, true);
    return xor_lane64<16>(((uint64_t)hi << 32) | lo, lane);
}

// Value held by lane - 1 (lane 0 keeps its own): DPP wave_shr:1.
__device__ __forceinline__ uint64_t prev_lane64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v,
                                                              0x138, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32),
                                                              (int)(uint32_t)(v >> 32), 0x138, 0xF,
                                                              0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a < b ? b : a; }

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Orders LDS traffic between lanes of one wave (in-order per wave on CDNA).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One bitonic network stage for block size B at lane distance J.  Lanes in a
// block whose bit B is clear run ascending, the others descending; DESC flips
// the whole network.  B = 64 with J = 32 is the final merge.  One compare per
// stage: a lane keeps its own key when "mine is larger" agrees with the side
// of the pair it must end on.
template <int B, int J, bool DESC, typename T>
__device__ __forceinline__ T bitonic_stage(T x, int lane) {
    T y;
    if constexpr (sizeof(T) == 8) y = xor_lane64<J>(x, lane);
    else y = xor_lane32<J>(x, lane);
    const bool lower = (lane & J) == 0;
    const bool ascending_block = (lane & B) == 0;
    const bool keep_large = (lower != ascending_block) != DESC;
    if constexpr (sizeof(T) == 4) {
        // 32-bit keys: maximum and minimum are single instructions, and the
        // pick between them is a select on a lane mask fixed per stage.
        const T hi = x < y ? y : x;
        const T lo = x < y ? x : y;
        x = keep_large ? hi : lo;
    } else {
        x = ((x > y) == keep_large) ? x : y;
    }
    return x;
}

template <int B, int J, bool DESC, typename T>
__device__ __forceinline__ T bitonic_stages(T x, int lane) {
    x = bitonic_stage<B, J, DESC>(x, lane);
    if constexpr (J > 1) return bitonic_stages<B, J / 2, DESC>(x, lane);
    return x;
}

// Sort one key per lane within each block of S lanes (S a power of two up to
// 64): block 0 ends in DESC order, the next block in the other order, and so
// on.  S = 64 sorts the whole wave.
template <int S, bool DESC, typename T>
__device__ __forceinline__ T sort_lanes(T x, int lane) {
    if constexpr (S > 2) x = sort_lanes<S / 2, DESC>(x, lane);
    return bitonic_stages<S, S / 2, DESC>(x, lane);
}

// Sort one key per lane across the wave.
template <bool DESC, typename T>
__device__ __forceinline__ T wave_sort(T x, int lane) {
    return sort_lanes<64, DESC>(x, lane);
}

// Sort one key per lane across the wave when only lanes below n (n <= 64,
// wave-uniform) hold keys and every other lane holds the smallest key (0 for
// unsigned keys): a sort of the smallest power-of-two block of lanes that
// covers n leaves block 0 sorted and the rest all-smallest, which is the whole
// wave sorted descending.  Fewer stages for few keys: 6 up to 8, 10 up to 16,
// 21 beyond.
template <typename T>
__device__ __forceinline__ T wave_sort_desc_first(T x, int lane, int n) {
    if (n <= 8) return sort_lanes<8, true>(x, lane);
    if (n <= 16) return sort_lanes<16, true>(x, lane);
    return sort_lanes<64, true>(x, lane);
}

// Bitonic network over a block of 64*K keys held K per lane -- key r*64 +
// lane of the block is x[r] -- so pairs at distance 64 or more are two
// registers of one lane and closer pairs one register of two lanes (DPP and
// permlane swaps); the K independent chains keep a wave's VALU busy.

// Stages (B, J), (B, J/2), ..., (B, 1) on one block.  Inside a bitonic block
// of size B a pair orders descending when bit B of its index is clear and
// ascending otherwise; when B exceeds the block that bit is the same for the
// whole block and blk_desc gives it.
template <int K, int B, int J>
__device__ __forceinline__ void cx_stages(uint64_t (&x)[K], bool blk_desc, int lane) {
    constexpr int Q = 64 * K;
    if constexpr (J >= 64) {
        constexpr int R = J / 64;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            if (r & R) continue;
            const bool desc = B < Q ? ((r * 64) & B) == 0 : blk_desc;
            const uint64_t a = x[r], b = x[r + R];
            const bool swap = (a < b) == desc;
            x[r] = swap ? b : a;
            x[r + R] = swap ? a : b;
        }
    } else {
        const bool lower = (lane & J) == 0;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            bool desc;
            if constexpr (B < 64) desc = (lane & B) == 0;
            else desc = B < Q ? ((r * 64) & B) == 0 : blk_desc;
            const uint64_t y = xor_lane64<J>(x[r], lane);
            x[r] = ((x[r] > y) == (lower == desc)) ? x[r] : y;
        }
    }
    if constexpr (J > 1) cx_stages<K, B, J / 2>(x, blk_desc, lane);
}

// Every level of the network inside one block: afterwards the block is sorted
// descending if blk_desc, else ascending.
template <int K, int B = 2>
__device__ __forceinline__ void sort_block(uint64_t (&x)[K], bool blk_desc, int lane) {
    cx_stages<K, B, B / 2>(x, blk_desc, lane);
    if constexpr (B < 64 * K) sort_block<K, 2 * B>(x, blk_desc, lane);
}

}  // namespace ws
