/*
 * ws.h -- C ABI of the fixed-shape batch-1 frame pipeline for MI355X (gfx950).
 *
 * A lane is one execution rail of the pipeline the WarpStream TRT article
 * describes (its dataflow figure and its "lane" passage): the producer writes
 * an interleaved RGB8 frame into a fixed input slot; a fused kernel resamples
 * it (bilinear resize, or aspect-preserving letterbox as in the yolo.cu
 * README), normalises it with a per-channel mean and standard deviation and
 * writes the FP32 NCHW tensor; an exact Top-K kernel selects the K best
 * entries of a fixed device-resident FP32 score vector and writes only the K
 * score/index pairs into a mapped host result slot.  Both kernels are captured
 * once into one hipGraph per lane and replayed per frame with no host decision
 * point in between.  (In the article a network sits between the two stages;
 * here the score vector is an independent input.)
 *
 * Everything is allocated, resolved and captured in ws_create_lane ("dynamism
 * belongs at startup"); ws_submit and ws_wait allocate nothing and make no
 * host decision on GPU data.
 *
 * Error convention: every call returns int, WS_OK (0) on success and a
 * negative WS_E_* code otherwise.  Nothing throws across this boundary.  The
 * last HIP error seen by a lane is kept and can be read with
 * ws_lane_hip_error().
 *
 * Threading: at most one host thread may use a lane at a time.  Different
 * lanes are independent and may be driven from different threads.
 *
 * HIP runtime: the library links libamdhip64.so.7.  A process must hold one
 * HIP runtime: when the same process uses a framework that ships its own
 * (PyTorch wheels do), load that framework first, so this library binds to
 * the copy already loaded; loading it afterwards maps a second HIP and HSA
 * runtime, and device calls then fail (typically WS_E_NO_DEVICE).
 */
#ifndef WS_H
#define WS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- optional detection stage --------------------------------------------
 * Decode + greedy NMS of a YOLO-style detection head, as in the yolo.cu
 * README (its end-to-end pipeline passage: DFL decode and NMS inside the one
 * graph; the GPU-resident NMS highlight: greedy suppression over the live
 * candidates in score order, only the final boxes cross to pinned memory;
 * the embedding example: up to 300 boxes in source-image coordinates).
 *
 * Head layout, float32 [4 * WS_DET_REG_MAX + nc][A], channel-major:
 *   channels 16*s .. 16*s+15  logits of the distance distribution of box
 *                             side s (0 left, 1 top, 2 right, 3 bottom), in
 *                             cells of the anchor's grid;
 *   channels 64 .. 64+nc-1    class probabilities (already through the
 *                             head's sigmoid).
 * Anchors: the cells of the stride-8, -16 and -32 grids over the dst_w x
 * dst_h network input, grid by grid, row-major within a grid, each at its
 * cell centre.  A = sum over s of (dst_w/s) * (dst_h/s).
 *
 * Per frame:
 *   1. each anchor's best class is the first maximum of its probabilities
 *      (NaN never wins); the anchor is a candidate when that probability
 *      > det_conf;
 *   2. a candidate's distances are softmax expectations of bin index, and
 *      its box is (cx - l, cy - t, cx + r, cy + b) * stride;
 *   3. candidates are taken by probability descending, then anchor
 *      ascending; each is kept unless an already kept box of the same class
 *      (any class when det_agnostic) has IoU > det_iou with it; at most
 *      det_max_det are kept;
 *   4. kept boxes are mapped back through the letterbox (or plain resize)
 *      to source pixels and clipped to the frame.
 * All of it runs in binary32 with a fixed operation order and no fused
 * multiply-add, with the exponential computed by Cody and Waite's reduction
 * plus a degree-7 Taylor polynomial, so the result is reproducible bit for
 * bit.  Box logits must be finite.
 */
#define WS_DET_REG_MAX      16     /* DFL bins per box side                  */
#define WS_DET_MAX_DET      1024   /* upper bound of det_max_det             */
#define WS_DET_MAX_ANCHORS  16384  /* upper bound of A                       */
#define WS_DET_MAX_CLASSES  4096

/* One kept box: source-frame pixels (x right, y down), its class
 * probability and class.  24 bytes. */
typedef struct ws_det {
    float   x1, y1, x2, y2;
    float   score;
    int32_t class_id;
} ws_det;

/* Detection result slot (mapped host memory, written by the GPU in-graph):
 * `count` kept boxes in keep order (score descending), and the number of
 * candidates that passed det_conf. */
typedef struct ws_det_result {
    int32_t count;
    int32_t candidates;
    ws_det  det[WS_DET_MAX_DET];
} ws_det_result;

/* ---- status codes ---------------------------------------------------- */
#define WS_OK              0
#define WS_E_INVALID_ARG  (-1)  /* NULL pointer, size or value out of range  */
#define WS_E_STATE        (-2)  /* submit while in flight, wait with nothing */
#define WS_E_NO_MAP_HOST  (-3)  /* device cannot map pinned host memory      */
#define WS_E_OOM          (-4)  /* a device or pinned allocation failed      */
#define WS_E_CAPTURE      (-5)  /* graph capture / instantiation failed      */
#define WS_E_HIP          (-6)  /* any other HIP runtime error               */
#define WS_E_NO_DEVICE    (-7)  /* no such HIP device                        */

/* ---- enumerations ------------------------------------------------------ */
#define WS_RESIZE_BILINEAR   0  /* stretch the frame onto the whole tensor   */
#define WS_RESIZE_LETTERBOX  1  /* keep aspect, centre, pad the rest         */

#define WS_INPUT_MAPPED_HOST 0  /* producer writes pinned host memory the GPU
                                   reads over the bus (zero-copy slot)        */
#define WS_INPUT_DEVICE      1  /* frame already resides in device memory    */
#define WS_INPUT_COPY        2  /* producer writes pinned host memory; each
                                   replay first copies the whole frame into a
                                   fixed device buffer (a DMA memcpy node of
                                   the graph), then preprocess reads HBM     */

#define WS_DTYPE_F32   0        /* tensor element: IEEE single               */
#define WS_DTYPE_F16   1        /* IEEE half, rounded to nearest even        */
#define WS_DTYPE_BF16  2        /* bfloat16, rounded to nearest even         */

#define WS_CHANNELS_RGB 0       /* producer bytes per pixel: R, G, B         */
#define WS_CHANNELS_BGR 1       /* producer bytes per pixel: B, G, R         */

#define WS_WAIT_SPIN   0        /* ws_wait polls the completion event        */
#define WS_WAIT_BLOCK  1        /* ws_wait blocks in the runtime             */

#define WS_CACHE_AUTO   0       /* WS_CACHE_STREAM for device-resident batches
                                   of WS_STREAM_MIN_BATCH frames or more,
                                   WS_CACHE_KEEP otherwise                   */
#define WS_CACHE_KEEP   1       /* frame loads and tensor stores allocate in
                                   the caches                                */
#define WS_CACHE_STREAM 2       /* frame loads and tensor stores are
                                   non-temporal: a batch streamed through
                                   once does not displace other data         */
#define WS_STREAM_MIN_BATCH 8

/* Limits checked by ws_create_lane. */
#define WS_MAX_K       32
#define WS_MAX_BATCH   64
#define WS_MAX_SIDE    16384
#define WS_MAX_SCORES  (1 << 30)

/* One selected entry: the score (original bits; NaN reported as -inf) and its
 * position in the score vector.  8 bytes, array of structs, rank order. */
typedef struct ws_topk_entry {
    float   score;
    int32_t index;
} ws_topk_entry;

/* Lane construction parameters.  All fields are read once, by ws_create_lane.
 * Zero-initialise the struct and set what you need. */
typedef struct ws_lane_config {
    int32_t device;        /* HIP device ordinal                              */
    int32_t batch;         /* frames per submit, 1..WS_MAX_BATCH              */
    int32_t src_w, src_h;  /* producer frame width and height, 1..WS_MAX_SIDE */
    int32_t dst_w, dst_h;  /* tensor width and height, 1..WS_MAX_SIDE         */
    int32_t resize_mode;   /* WS_RESIZE_*                                     */
    int32_t input_mode;    /* WS_INPUT_*                                      */
    double  pad_value;     /* letterbox fill in byte units, 0..255            */
    double  mean[3];       /* per output channel R, G, B, unit range          */
    double  std[3];        /* per RGB channel, unit range, > 0                */
    int32_t num_scores;    /* N, 0..WS_MAX_SCORES; 0 = no Top-K stage        */
    int32_t k;             /* 1..min(WS_MAX_K, N) when N > 0                  */
    int32_t use_graph;     /* 1 = replay the captured graph (the product);
                              0 = launch the same kernels directly (for the
                              graph vs direct-launch comparison only)        */
    int32_t wait_mode;     /* WS_WAIT_*                                       */
    /* Optional borrowed device buffers (NULL = the lane allocates its own).
     * Each must be 16-byte aligned, large enough for its layout below,
     * outlive the lane and never move: their addresses are baked into the
     * graph. */
    const uint8_t *input_dev;  /* WS_INPUT_DEVICE only                         */
    const float   *scores_dev;
    void          *tensor_dev;   /* element type per tensor_dtype              */
    /* Tuning knobs (0 = automatic choice); they change speed, never results. */
    int32_t rows_per_group;    /* preprocess: output rows per workgroup        */
    int32_t topk_chunk;        /* Top-K: scores per workgroup (multiple of 1024) */
    int32_t pixels_per_thread; /* preprocess: output columns per thread: 1
                                  (the automatic choice: each thread reads its
                                  taps straight from the frame), or 2 or 4
                                  (source rows staged through LDS first)       */
    /* Formats (0 = FP32 tensor from RGB bytes). */
    int32_t tensor_dtype;      /* WS_DTYPE_*                                    */
    int32_t channel_order;     /* WS_CHANNELS_*; the tensor planes are always
                                  R, G, B                                       */
    int32_t autotune;          /* 1 = time candidate launch geometries on the
                                  lane's buffers at create and keep the fastest
                                  (knobs above then only seed the search)       */
    /* Detection stage (see above); det_classes = 0 leaves it out. */
    int32_t det_classes;       /* nc, 0..WS_DET_MAX_CLASSES; needs dst_w and
                                  dst_h multiples of 32 and A <= 16384          */
    int32_t det_max_det;       /* 1..WS_DET_MAX_DET                             */
    float   det_conf;          /* candidate threshold, 0 <= det_conf < 1        */
    float   det_iou;           /* suppression threshold, 0 <= det_iou <= 1      */
    int32_t det_agnostic;      /* 1 = boxes of any class suppress each other    */
    int32_t det_reserved;      /* must be 0                                     */
    const float *det_head_dev; /* borrowed head, or NULL: the lane owns one,
                                  zero-filled at create                         */
    /* How the preprocess kernel reads device-resident frames and writes the
     * tensor (a tuning knob: it changes speed, never results). */
    int32_t cache_policy;      /* WS_CACHE_*                                    */
    int32_t reserved;          /* must be 0                                     */
} ws_lane_config;

/* Stable views of a lane's buffers, valid from ws_create_lane to ws_destroy.
 *   input   uint8  [batch][src_h][src_w][3]   interleaved RGB, rows packed
 *   tensor  [batch][3][dst_h][dst_w]          planar R, G, B; FP32, FP16
 *                                             or BF16 per tensor_dtype
 *   scores  float  [num_scores]
 *   result  ws_topk_entry [k]                 mapped host memory, rank order
 */
typedef struct ws_lane_view {
    uint8_t             *input_host;   /* producer's slot (mapped / copy mode), else NULL */
    const uint8_t       *input_dev;    /* address the preprocess kernel reads      */
    void                *tensor_dev;
    float               *scores_dev;   /* NULL when num_scores == 0                */
    const ws_topk_entry *result_host;  /* NULL when num_scores == 0                */
    size_t               input_bytes;
    size_t               tensor_bytes;
    float               *det_head_dev;     /* NULL without a detection stage   */
    const ws_det_result *det_result_host;  /* NULL without a detection stage   */
} ws_lane_view;

typedef struct ws_lane ws_lane;

/*
 * ws_create_lane -- validate cfg, then allocate and bind everything the lane
 * will ever use: input slot (hipHostMalloc mapped, coherent; for the copy mode
 * pinned host memory plus a device copy) or device input,
 * tensor, scores, mapped result slot, Top-K scratch, one non-blocking
 * stream and two timing events, and fixes the launch geometry.  Runs the kernels
 * once outside capture (warm-up), captures them into one graph, instantiates
 * and uploads it, and replays it once.  Source: the article's lane and
 * initialisation passages (allocate once, bind once, capture once; map-host
 * enabled before use, failing loudly when the device cannot map).
 *
 *   cfg   read only; not retained.
 *   out   receives the lane handle (owned by the caller until ws_destroy).
 *   view  optional (may be NULL); receives the stable buffer views.
 * Returns WS_OK, WS_E_INVALID_ARG, WS_E_NO_DEVICE, WS_E_NO_MAP_HOST,
 * WS_E_OOM, WS_E_CAPTURE or WS_E_HIP.  On failure nothing is leaked and *out
 * is set to NULL.
 */
int ws_create_lane(const ws_lane_config *cfg, ws_lane **out, ws_lane_view *view);

/*
 * ws_submit -- READY -> IN_FLIGHT: record the start event, replay the lane's
 * graph (preprocess, then Top-K, then detection decode and NMS, in stream
 * order, each stage present when configured), record the done event.
 * No allocation, no synchronisation, no host branch on GPU data.  The input
 * slot, scores and detection head must hold the frame's data before this
 * call and must not
 * be modified until ws_wait returns.  Source: the article's submit passage.
 * Returns WS_E_STATE if the lane is already in flight (a lane cannot be
 * reused while busy; there is no queue), WS_E_INVALID_ARG for NULL, WS_E_HIP
 * if a launch fails (the lane stays READY).
 *
 * Host cost: with the HIP runtime's default interrupt-driven completion
 * signals, the graph launch inside this call takes ~20-25 us of host time on
 * ROCm 7 (most of a single frame's replay); with polled signals
 * (HSA_ENABLE_INTERRUPT=0 in the environment before the process starts the
 * HIP runtime) it takes ~3-4 us, at the price of host threads that poll
 * instead of sleeping when they wait on the GPU.  The library does not set
 * it: the setting is process-wide.
 */
int ws_submit(ws_lane *lane);

/*
 * ws_wait -- IN_FLIGHT -> READY: wait for the done event (spinning or
 * blocking per cfg.wait_mode).  If gpu_ms is not NULL it receives the GPU
 * time between the start and done events in milliseconds.  Afterwards the
 * result slot and the tensor hold this frame's output until the next
 * ws_submit.  Returns WS_E_STATE if nothing is in flight, WS_E_HIP on a
 * runtime error.
 */
int ws_wait(ws_lane *lane, float *gpu_ms);

/*
 * ws_destroy -- release everything the lane owns (borrowed buffers are left
 * alone).  Valid in any state: an in-flight lane is waited for first, so no
 * memory the GPU may still touch is freed.  NULL is accepted (no-op).
 */
int ws_destroy(ws_lane *lane);

/*
 * ws_run_noalloc -- for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Enqueues
 * one frame of the launch sequence ws_submit replays -- preprocess, then
 * Top-K when num_scores > 0 -- as direct launches on `stream`, reading and
 * writing only the caller's buffers, and allocates nothing.
 *   cfg     as for ws_create_lane, with input_mode WS_INPUT_DEVICE and the
 *           borrowed device buffers input_dev, tensor_dev and (when
 *           num_scores > 0) scores_dev set; det_classes and autotune 0;
 *           use_graph and wait_mode are ignored.  cfg->device must be the
 *           calling thread's current device.  Read only; not retained.
 *   result  device-visible memory (device or mapped host, 8-byte aligned)
 *           for k ws_topk_entry in rank order; NULL when num_scores == 0.
 *   stream  a hipStream_t of that device, or NULL for its null stream.
 * When the scores span several Top-K workgroups, their partial lists live in
 * a scratch array of the library: WS_NOALLOC_SCRATCH_BYTES on each device
 * the call runs on, held until the process ends.  A plan that needs more
 * (workgroups x k x 8 bytes) is rejected.  Every call on one device shares
 * that array and the last call's contents stay in it: calls that may
 * overlap on one device (other streams, other threads) race, so the caller
 * serialises them.  The first call on a device also looks up the array's
 * address and sets the kernels' LDS limits.  The call returns once the
 * launches are enqueued; the tensor and result are complete when the
 * stream's work before the next event on it has finished.
 * Returns WS_OK, WS_E_INVALID_ARG (a field out of range or unsupported, a
 * missing buffer, a plan beyond the scratch limit, a device that is not
 * current), WS_E_NO_DEVICE or WS_E_HIP (a launch failed).
 */
#define WS_NOALLOC_SCRATCH_BYTES (1u << 20)
int ws_run_noalloc(const ws_lane_config *cfg, ws_topk_entry *result, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *ws_status_str(int status);

/* Last hipError_t value the lane saw (0 if none); 0 for NULL. */
int ws_lane_hip_error(const ws_lane *lane);

#ifdef __cplusplus
}
#endif

#endif /* WS_H */
