/*
 * ws_bench.h -- native latency harness around the lane ABI in ws.h.
 *
 * The WarpStream TRT article's benchmark passage times each replay with GPU
 * events recorded just before the graph launch and just after Top-K, and
 * measures throughput across one or more lanes with a host wall clock; the
 * producer's write and the consumer's work are excluded.  These calls run
 * that loop in native code so no interpreter overhead enters the wall clock.
 * They are harness, not part of the per-frame product path.
 */
#ifndef WS_BENCH_H
#define WS_BENCH_H

#include "ws.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch geometry a lane chose at construction (for reports). */
typedef struct ws_lane_plan {
    int32_t pre_groups;       /* preprocess workgroups per launch            */
    int32_t pre_block;        /* preprocess threads per workgroup            */
    int32_t rows_per_group;   /* output rows per preprocess workgroup        */
    int32_t pre_lds_bytes;    /* LDS per preprocess workgroup                */
    int32_t topk_groups;      /* Top-K workgroups (0 = no Top-K stage)       */
    int32_t topk_block;       /* Top-K threads per workgroup                 */
    int32_t topk_chunk;       /* scores per Top-K workgroup                  */
    int32_t graph_nodes;      /* kernel nodes in the captured graph          */
    int32_t pixels_per_thread;/* output pixels per preprocess thread         */
    int32_t det_anchors;      /* detection anchors (0 = no detection stage)  */
    int32_t det_decode_groups;/* decode workgroups (64 anchors each)         */
    int32_t topk_keys_per_lane;/* Top-K scores per lane per batch: 16 or 32  */
    int32_t streaming;         /* 1 = non-temporal frame loads and tensor
                                  stores (WS_CACHE_*)                         */
} ws_lane_plan;

/* Fill *plan for lane.  Returns WS_OK or WS_E_INVALID_ARG (NULL). */
int ws_lane_describe(const ws_lane *lane, ws_lane_plan *plan);

/*
 * Run `replays` x (ws_submit, ws_wait) on one lane from the calling thread.
 *   gpu_ms     optional, `replays` entries: start->done event time per replay.
 *   host_us    optional, `replays` entries: host time from just before
 *              ws_submit to the return of ws_wait, per replay.
 *   submit_us  optional, `replays` entries: host time spent inside ws_submit
 *              (the two event records and the graph launch), per replay; the
 *              rest of host_us is ws_wait.
 *   wall_s     optional: host wall time from before the first submit to after
 *              the last wait.
 * Returns the first non-OK status of any call, else WS_OK.
 */
int ws_bench_replays(ws_lane *lane, int32_t replays, float *gpu_ms, float *host_us,
                     float *submit_us, double *wall_s);

/*
 * Drive `nlanes` lanes concurrently, one host thread per lane, each running
 * `replays` x (ws_submit, ws_wait).  Threads start together after all are
 * ready; wall_s spans from that release to the last thread's finish.
 *   gpu_ms   optional, nlanes * replays entries, lane-major.
 * Returns the first non-OK status seen, else WS_OK.
 */
int ws_bench_lanes(ws_lane **lanes, int32_t nlanes, int32_t replays, float *gpu_ms,
                   double *wall_s);

/* Stages of the per-frame launch sequence, for ws_bench_stage. */
#define WS_STAGE_PREPROCESS 0
#define WS_STAGE_TOPK       1
#define WS_STAGE_DETECT     2   /* decode + NMS: two kernels per launch     */

/*
 * Time one stage's kernel alone: `launches` back-to-back direct launches on
 * the lane's stream between two events, then a synchronisation.  The lane
 * must be READY and stays READY; its buffers receive that stage's output.
 *   ms_per_launch  receives the elapsed event time divided by `launches`.
 * Returns WS_OK, WS_E_STATE (in flight), WS_E_INVALID_ARG (NULL, bad stage,
 * launches < 1, or a Top-K or detection stage the lane does not have) or
 * WS_E_HIP.
 */
int ws_bench_stage(ws_lane *lane, int32_t stage, int32_t launches, double *ms_per_launch);

/*
 * Time one stage's kernels with the caches evicted before each launch.  For
 * each of `launches` runs, a flush kernel on the lane's stream streams over
 * the first `flush_bytes` of the caller's device buffer `flush` (reading it,
 * or writing zeros over it when `flush_write` is 1); then the start event,
 * the stage's kernels and the done event follow in stream order, so the
 * start event fires when the flush ends and the interval holds the stage
 * alone (its dispatch included).  The flush buffer must be larger than the
 * last-level cache for the launch to start cold.
 *   ms  `launches` entries: start->done time of each run, in milliseconds.
 * The lane must be READY and stays READY.  Returns WS_OK, WS_E_STATE,
 * WS_E_INVALID_ARG (NULL, flush not 16-byte aligned, flush_bytes < 16,
 * launches < 1, or a stage the lane does not have) or WS_E_HIP.
 */
int ws_bench_stage_cold(ws_lane *lane, int32_t stage, void *flush, size_t flush_bytes,
                        int32_t flush_write, int32_t launches, float *ms);

/*
 * Time one stage's kernels launched back to back over several lanes in turn:
 * launch i runs the stage of lanes[i % nlanes], every launch on lanes[0]'s
 * stream, between lanes[0]'s two events.  When the lanes' buffers together
 * exceed the last-level cache, each launch finds its own inputs evicted by
 * the other lanes' launches since its last turn, while the launches still
 * follow each other with no host gap.
 *   warmup         untimed launches first, in the same rotation.
 *   ms_per_launch  receives the elapsed event time divided by `launches`.
 * Every lane must be READY (and stays READY) and on one device.  Returns
 * WS_OK, WS_E_STATE, WS_E_INVALID_ARG (NULL, nlanes < 1, launches < 1,
 * warmup < 0, lanes on different devices, or a stage a lane does not have)
 * or WS_E_HIP.
 */
int ws_bench_stage_rotate(ws_lane **lanes, int32_t nlanes, int32_t stage, int32_t warmup,
                          int32_t launches, double *ms_per_launch);

/* Launch forms for ws_bench_launch_cost. */
#define WS_LAUNCH_GRAPH        0   /* events recorded around one graph replay   */
#define WS_LAUNCH_DIRECT       1   /* events around direct kernel launches      */

/*
 * Cost of launching a chain of `nodes` (1..8) kernels that do no work, each
 * 224 workgroups of 256 threads, on a non-blocking stream of `device` created
 * for the call: the per-frame launch overhead with the kernels' own work
 * taken out.  The streams handbook's graph chapter and the WarpStream TRT
 * article's benchmark passage (graph replay against direct launches) are what
 * it measures.  `warmup` untimed rounds, then `replays` timed rounds, each
 * waited for (spinning on the done event, as ws_wait does) before the next:
 *   launch_us  host time of the launch call(s) of each round;
 *   total_us   host time from the first call of the round (the start event
 *              record) to completion observed;
 *   gpu_us     start->done event interval.
 * Each array holds `replays` entries.  hip_error (optional) receives the
 * hipError_t of the call that failed, else 0.  Returns WS_OK,
 * WS_E_INVALID_ARG (NULL, nodes outside 1..8, replays < 1, warmup < 0,
 * unknown form) or WS_E_HIP.
 */
int ws_bench_launch_cost(int32_t device, int32_t nodes, int32_t form, int32_t warmup,
                         int32_t replays, float *launch_us, float *total_us, float *gpu_us,
                         int32_t *hip_error);

#ifdef __cplusplus
}
#endif

#endif /* WS_BENCH_H */
