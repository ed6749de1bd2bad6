// ws_marks.h -- clock marks for timing kernel phases.  Internal to the
// library.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ws {

// Clock marks for timing kernel phases, compiled in only when the library is
// built with WS_CLOCK_MARKS (`python -m post_processing_amd.build --marks`
// writes it as libws_marks.so); otherwise every mark is empty and the
// kernels are unchanged.  Lane 0 of a wave stores the GPU's 100 MHz constant
// clock (s_memrealtime, the same for every CU) into the calling source
// file's `g_marks` array, read at that point of the program (scheduling
// barriers keep the compiler from moving it); WS_MARK_AFTER_LOADS first
// waits for the wave's outstanding vector loads.
#ifdef WS_CLOCK_MARKS
constexpr int kMarkSlots = 1 << 17;
#define WS_MARK(slot)                                                          \
    do {                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                     \
        const uint64_t t_ = __builtin_amdgcn_s_memrealtime();                  \
        __builtin_amdgcn_sched_barrier(0);                                     \
        if ((threadIdx.x & 63) == 0 && (slot) < ::ws::kMarkSlots) g_marks[(slot)] = t_; \
    } while (0)
#define WS_MARK_AFTER_LOADS(slot)                      \
    do {                                               \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); \
        WS_MARK(slot);                                 \
    } while (0)
#else
#define WS_MARK(slot) \
    do {              \
    } while (0)
#define WS_MARK_AFTER_LOADS(slot) \
    do {                          \
    } while (0)
#endif

}  // namespace ws
