/*
 * bkv.h -- C ABI of the bounded-KV block attention library (libbkv.so), MI355X / gfx950.
 *
 * What it computes.  Streaming block-causal attention for autoregressive
 * video-DiT avatar generation over a cache of constant size:
 *
 *   PR-Sink (LiveAnimate page, section 方法, the three PR-Sink bullets; section
 *   关键发现, constant memory and per-block latency): block m's queries attend
 *   to a static sink (the first generated block, kept for good), dynamic sink
 *   blocks retrieved by pose similarity (same page, section 局限), a rolling
 *   window of the last three blocks, and block m itself (full attention inside
 *   the block).
 *
 *   ConvKV (Soul App开源实时数字人生成框架SoulX-LiveAct详解 page, section 技术内核,
 *   ConvKV Memory bullet): the last blocks keep exact KV; older frames are
 *   compressed along time by a 1D conv (stride = kernel, 5:1) into a fixed
 *   memory, and RoPE positions restart from 0 over [memory, window, current].
 *
 * One stream of blocks per handle.  Per block: bkv_retrieve (opens block m,
 * runs the pose top-k), then bkv_attend for every (sampling step, layer), then
 * bkv_commit (appends block m, evicts, compresses).  The sampling steps of a
 * block all read the same context; a block's K/V enter the cache as written by
 * its last bkv_attend per layer (LiveAnimate page, section 方法: three steps).
 *
 * Memory.  The path never allocates device memory (the measurement aid
 * bkv_probe_mfma allocates a 4-byte sink per call).  The caller provides one
 * device workspace of bkv_workspace_size() bytes at create time; the cache,
 * pose bank, RoPE tables, selection and scratch are carved from it, so cache
 * bytes are constant over the stream by construction.  Q/K/V/out, the pose and
 * the conv weights are caller-owned device buffers, read or written only
 * during the call's stream work.  The handle holds a little host state.
 *
 * Streams.  Every device operation is enqueued on the caller's stream; no
 * call synchronizes except those documented as synchronizing.  The calls on
 * one handle share its workspace (cache slots, the selection, split slots, q
 * scratch): they must run on one stream, or the caller must order them
 * across streams (events), as a later call reads what an earlier one wrote.
 * A handle is not thread-safe; use one handle per host thread.
 *
 * Errors.  Every call returns bkv_status and never throws.  BKV_ERR_ARG and
 * BKV_ERR_STATE leave the handle unchanged.  BKV_ERR_DEVICE (a failed launch
 * or runtime call) puts the handle in an error state in which everything but
 * bkv_reset/bkv_destroy/bkv_stats returns BKV_ERR_STATE.  bkv_last_error()
 * returns a message for the last non-OK status of the calling thread.
 */
#ifndef BKV_H_
#define BKV_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bkv_cache_s* bkv_cache; /* opaque handle: one per stream of blocks */

typedef enum {
  BKV_OK = 0,
  BKV_ERR_ARG = 1,         /* null pointer, bad size/shape/dtype, layer out of range, bad config */
  BKV_ERR_STATE = 2,       /* call out of order (see each call), or handle in error state */
  BKV_ERR_WORKSPACE = 3,   /* workspace too small or misaligned (256-byte alignment needed) */
  BKV_ERR_DEVICE = 4,      /* HIP launch or runtime error */
  BKV_ERR_UNSUPPORTED = 5  /* valid request the library does not implement */
} bkv_status;

typedef enum { BKV_PR_SINK = 0, BKV_CONVKV = 1 } bkv_mode;
/* BKV_BF16_FP8K: bf16 Q/K/V/out and V cache, with an FP8 key cache (head_dim
   128).  The SoulX-LiveAct page (sections 关键信息速览 and 上手实践) runs
   attention in FP8 without fixing a scheme; this library reads it as: K
   after RoPE is held as OCP E4M3 (bias 7, largest finite 448, round to
   nearest even) with one power-of-two scale 2^e per (head, 64-token tile of
   a context segment, counted from the segment's first token), e the
   smallest integer with max|K~| * 2^-e <= 448 (0 for an all-zero tile),
   clamped to [-120, 120]; Q after RoPE, times softmax_scale * log2(e), is
   quantised the same way with one scale per (token, head); the logits Q K^T
   are formed from these E4M3 values on the scaled FP8 matrix instruction
   (each product is exact; the matrix core's sum of them is not, measured
   within 3.2e-5 of sum |q_i k_i|); softmax and P V are as for BKV_BF16.  PR-Sink with absolute
   positions stores the E4M3 K in the slots (cache bytes per token and head:
   128 (K) + 256 (V) + 4/64).  ConvKV and context-relative PR-Sink keep raw
   bf16 K in the slots (the conv and the per-block rotation read it) and
   quantise the rotated context, segment by segment (memory frames, blocks),
   as they gather it.
   BKV_BF16_FP8KV: the FP8 KV cache (the same page's 上手实践 notes offer an
   "FP8 KV cache"): K as for BKV_BF16_FP8K, and V held as E4M3 too, with the
   same tile rule (one power-of-two scale per head and 64-token tile of a
   segment, over all channels); the softmax numerator P is held as E4M3 with
   that rule applied to each query row (one power-of-two scale per row, its
   largest P mapped into (224, 448]) and P V runs on the scaled FP8 matrix
   instruction; the softmax denominator sums the unrounded P.  The library
   moves its running max by whole numbers only, starting each row's largest
   P in (4, 8], so its P codes are the row's own: E4M3 rounds alike at every
   power of two, and the lower scale changes only values in its subnormal
   range, 2^9 below the row's largest P.  A P whose exact value lies within
   the logit's summation error of a rounding boundary between two codes may
   take either code.  Cache bytes per token and head: 128 (K) +
   128 (V) + 8/64 (exponents); ConvKV slots also keep the raw bf16 V the conv
   reads. */
typedef enum { BKV_F32 = 0, BKV_BF16 = 1, BKV_BF16_FP8K = 2, BKV_BF16_FP8KV = 3 } bkv_dtype;

/* Temporal RoPE positions (bkv_config.rope_positions).
   BKV_POS_DEFAULT: PR-Sink absolute (frame f of block b at
     reference_frames + b*frames_per_block + f; K rotated once, at append);
     ConvKV context-relative (SoulX-LiveAct page, section 技术内核: memory
     frames at 0..M-1, then the window blocks and the current block at
     consecutive frames).
   BKV_POS_CONTEXT: PR-Sink context-relative: the open block's context blocks
     (static, retrieved, window, current) sit at consecutive frames in
     stream-id order after the reference frames, the gaps between them
     removed, and their K is re-rotated at those positions every block (the
     ConvKV page's position reset applied to PR-Sink).  ConvKV: as
     BKV_POS_DEFAULT.
   BKV_POS_ABSOLUTE: PR-Sink: as BKV_POS_DEFAULT.  ConvKV: only the memory's
     positions restart (memory frame j at t = j); the window and current
     blocks keep their absolute frame indices b*frames_per_block + f (the
     literal alternative reading of the same passage). */
typedef enum { BKV_POS_DEFAULT = 0, BKV_POS_CONTEXT = 1, BKV_POS_ABSOLUTE = 2 } bkv_positions;

/* PR-Sink bank replacement (bkv_config.bank_policy).  The LiveAnimate page
   (section 关键发现) keeps a fixed number of blocks without saying which
   leave.  BKV_BANK_FIFO: the bank holds the last bank_blocks blocks that left
   the window.  BKV_BANK_POSE: a block leaving the window into a full bank
   displaces the member whose pose has the largest cosine with its own
   (fp64, ranked as retrieval ranks: exact ties displace the lower stream id;
   a zero pose, and a pose holding Inf or NaN, scores 0), and joins the bank;
   needs pose_dim >= 1 and bank_blocks >= 1.  The ranking runs on the device,
   which holds the bank's membership; the displaced member's id comes back to
   the host asynchronously (its slot is reused once it has), so no call
   waits for the device except a bkv_retrieve that finds the host more than
   two blocks ahead of it (the workspace holds two spare slots for this). */
typedef enum { BKV_BANK_FIFO = 0, BKV_BANK_POSE = 1 } bkv_bank_policy;

typedef enum {
  BKV_SEG_STATIC = 0,   /* static sink block */
  BKV_SEG_DYNAMIC = 1,  /* pose-retrieved bank block */
  BKV_SEG_WINDOW = 2,   /* rolling-window block */
  BKV_SEG_CURRENT = 3,  /* the open block */
  BKV_SEG_MEMORY = 4,   /* ConvKV compressed memory frame */
  BKV_SEG_REFERENCE = 5 /* PR-Sink reference frames (reference_frames > 0), id -1 */
} bkv_segment_kind;

/* Cache configuration.  Set struct_size = sizeof(bkv_config) (ABI guard). */
typedef struct {
  uint32_t struct_size;
  int32_t mode;             /* bkv_mode */
  int32_t dtype;            /* bkv_dtype of Q/K/V/out and of the cache */
  int32_t layers;           /* >= 1; each layer has its own cache */
  int32_t heads;            /* >= 1 */
  int32_t head_dim;         /* 64 or 128 (bf16 and FP8-key paths: 128) */
  int32_t frames_per_block; /* latent frames per block, >= 1 */
  int32_t grid_h, grid_w;   /* latent grid; tokens per block T = frames*grid_h*grid_w */
  int32_t window_blocks;    /* rolling window length, 1..8 (3 on the pages) */
  int32_t static_blocks;    /* PR-Sink: 0 or 1 (block 0 is the sink); ConvKV: 0 */
  int32_t dynamic_k;        /* PR-Sink: blocks retrieved per block, 0..8; ConvKV: 0 */
  int32_t bank_blocks;      /* PR-Sink: bank of evicted blocks, 0..256 (FIFO or pose-aware,
                               bank_policy); ConvKV: 0 */
  int32_t pose_dim;         /* PR-Sink with dynamic_k > 0: 1..1024 fp32 values per pose */
  int32_t rope_t, rope_h, rope_w; /* RoPE channel split [t|h|w]; all 0 = none, else each
                                     even and summing to head_dim */
  double rope_theta;        /* RoPE base, > 0 (10000) */
  int32_t conv_kernel;      /* ConvKV: taps (5); must equal conv_stride */
  int32_t conv_stride;      /* ConvKV: stride (5) */
  int32_t memory_frames;    /* ConvKV: compressed frames kept, 1..4 */
  float softmax_scale;      /* 0 -> 1/sqrt(head_dim) */
  int32_t reference_frames; /* PR-Sink: reference latent frames R kept as a permanent first
                               context segment, 0..8 (0 = none); ConvKV: 0.  See
                               bkv_set_reference. */
  int32_t rope_positions;   /* bkv_positions: temporal RoPE positions of the context (0 = the
                               mode's own reading) */
  int32_t bank_policy;      /* PR-Sink: bkv_bank_policy (0 = FIFO); ConvKV: 0 */
} bkv_config;

/* One context segment as the open block sees it (host view). */
typedef struct {
  int32_t kind;    /* bkv_segment_kind */
  int32_t id;      /* block stream id; memory: memory-frame index */
  int32_t tokens;  /* keys contributed */
  int32_t t0;      /* RoPE temporal position of the segment's first frame, as rope_positions
                      sets it (the reference segment: 0) */
} bkv_segment;

typedef struct {
  int64_t block;           /* id of the open block, or of the next block if none is open */
  int32_t open;            /* 1 between bkv_retrieve and bkv_commit */
  int32_t n_segments;      /* segments of the open block's context (0 if closed) */
  int64_t n_keys;          /* keys of the open block's context (0 if closed) */
  int64_t last_evicted;    /* id that left the window at the last commit, -1 if none */
  int32_t bank_count;      /* PR-Sink: blocks in the bank */
  int32_t memory_count;    /* ConvKV: memory frames present */
  size_t workspace_bytes;  /* bytes of workspace in use (constant for the handle's life) */
  int64_t split_attends;   /* bf16 attends since create/reset whose attention cut its last,
                              unfilled round of units (heads x 256-query tiles; > 15% of 256
                              workgroup slots idle) into key parts: a second attention launch,
                              and a third that merges the parts when a unit has more than one */
} bkv_stats_t;

/* Workspace bytes needed for cfg.  Pure host call.
   Errors: BKV_ERR_ARG for a null pointer or an invalid config. */
bkv_status bkv_workspace_size(const bkv_config* cfg, size_t* bytes);

/* Create a handle on the current HIP device over a caller-owned device
   workspace (>= bkv_workspace_size bytes, 256-byte aligned; the caller frees it
   after bkv_destroy).  Clears the workspace and builds the RoPE tables in it
   on `stream`.
   The new handle is at block 0 with no block open.
   Errors: BKV_ERR_ARG (config), BKV_ERR_WORKSPACE, BKV_ERR_DEVICE. */
bkv_status bkv_create(const bkv_config* cfg, void* workspace, size_t bytes, hipStream_t stream,
                      bkv_cache* out);

/* Destroy the handle (host state only).  The caller must make sure work
   enqueued on the handle's streams has finished before freeing the workspace. */
bkv_status bkv_destroy(bkv_cache h);

/* Back to block 0, empty cache, error state cleared.  No (de)allocation; conv
   weights and reference frames already set are kept. */
bkv_status bkv_reset(bkv_cache h);

/* ConvKV: set layer's depthwise conv weights from device buffers wk, wv, each
   fp32 [heads][head_dim][conv_kernel] (tap 0 multiplies the oldest frame).
   Copied into the workspace on `stream`; the caller's buffers may be reused
   once that copy ran.  Errors: BKV_ERR_UNSUPPORTED on a PR-Sink handle. */
bkv_status bkv_set_conv_weights(bkv_cache h, int32_t layer, const float* wk, const float* wv,
                                hipStream_t stream);

/* PR-Sink with reference_frames R > 0: set layer's reference frames.  The
   LiveAnimate page (section 方法) conditions every block on the reference
   image, and the Live Avatar page (abstract) recalibrates appearance from a
   cached reference image; this library reads that as R latent frames of
   grid_h x grid_w tokens that every block attends to, first in its context,
   at temporal RoPE positions 0..R-1 (token (f*grid_h + y)*grid_w + x at
   (f, y, x)), while frame f of generated block b moves to R + b*frames_per_block
   + f.  k, v: device, dtype, contiguous [R*grid_h*grid_w][heads][head_dim];
   K is rotated and stored (E4M3 with per-64-token tile scales for
   BKV_BF16_FP8K, as for blocks) and V stored on `stream`; the caller's
   buffers may be reused once that work ran.  Call it for every layer before
   the first bkv_retrieve; it may be called again (no block open) to replace
   the reference.  bkv_reset keeps it.
   Errors: BKV_ERR_UNSUPPORTED if reference_frames is 0; BKV_ERR_STATE while a
   block is open; BKV_ERR_ARG (layer, null pointer, k aliasing v). */
bkv_status bkv_set_reference(bkv_cache h, int32_t layer, const void* k, const void* v, hipStream_t stream);

/* Open the next block m (pose retrieval; LiveAnimate page, section 方法, Dynamic
   Sink bullet).  With BKV_BANK_POSE it first takes in the bank members that
   earlier commits displaced, waiting on `stream` only if it needs a slot
   whose displacement has not come back yet.  With reference_frames > 0, BKV_ERR_STATE until the reference
   of every layer is set.  pose: device fp32 [pose_dim], the block's pose embedding; it is
   stored with the block for later retrieval.  Selects the top-min(dynamic_k,
   bank_count) bank blocks by cosine similarity to `pose` (fp64 arithmetic;
   exact ties to the lower stream id; a zero-norm pose, and a pose holding a
   non-finite value (Inf, NaN), scores 0) on the device: the host is not
   synchronized.  ConvKV: pose may be NULL.
   Errors: BKV_ERR_STATE if a block is already open; BKV_ERR_ARG if pose is NULL
   where needed. */
bkv_status bkv_retrieve(bkv_cache h, const float* pose, hipStream_t stream);

/* Attention of the open block at `layer` for one sampling step.  q, k, v, out:
   device, dtype, contiguous [T][heads][head_dim] token-major (token index
   (f*grid_h + y)*grid_w + x).  Rotates K (3D RoPE at the block's positions) and
   stores K, V as the open block's entry of `layer` (a later call for the same
   layer in the same block overwrites it), then writes
       out[i] = sum_j softmax_j(scale * q~_i . k~_j) v_j
   over every key j of the context (q~, k~ rotated), accumulating in fp32.
   out must not alias q, k or v.
   Errors: BKV_ERR_STATE if no block is open; BKV_ERR_ARG (layer, null). */
bkv_status bkv_attend(bkv_cache h, int32_t layer, const void* q, const void* k, const void* v,
                      void* out, hipStream_t stream);

/* For callers that cannot allocate device memory or must not touch more of it
   than they pass (code under HIP graph capture, tight serving loops): the
   same as bkv_attend, except that the split attention launch keeps its part
   states (fp32 O, m, l of each key part of a cut unit; needed when heads x
   256-query units leave the last round of 256 workgroups more than 15%
   idle) in a file-scope device array of the library instead of the
   workspace's split slots.  That array holds 256 slots of 132 KiB (33 MiB)
   on each device the library runs on, until the process ends; its address
   is looked up once per device, at the first call there.  It allocates
   nothing and needs no clearing (a call reads only part states it wrote).
   Every call of this entry point on one device shares the array: calls that
   overlap on one device (other streams, other handles) race, so order them.
   Errors: as bkv_attend; BKV_ERR_DEVICE if the array's address cannot be
   found. */
bkv_status bkv_attend_static_scratch(bkv_cache h, int32_t layer, const void* q, const void* k, const void* v,
                                     void* out, hipStream_t stream);

/* Fused QKV projection + attention of the open block at `layer` for one sampling
   step (the operator fusion of the LiveAnimate page, section 方法, and the
   fused-QKV build of the SoulX-LiveAct page, section 上手实践; neither writes the
   operation out, the plain reading is taken).  x: device bf16 [T][model_dim] hidden
   states of the block (token order as in bkv_attend); w: device bf16
   [3*heads*head_dim][model_dim] projection weights, rows ordered q heads, k heads,
   v heads (a head's head_dim rows together: the nn.Linear layout); b: device bf16
   [3*heads*head_dim] bias or NULL.  Computes [q | k | v] = x w^T + b with fp32
   accumulation (q, k, v rounded to bf16 as they are stored) and then does what
   bkv_attend does with them: K rotated and stored with V as the block's entry of
   `layer`, attention written to out [T][heads][head_dim] bf16.  q goes through a
   workspace scratch; k and v never leave the cache.  model_dim: a positive multiple
   of 32; x and w each below 2 GiB.
   With BKV_BF16_FP8K the rotated k is quantised to E4M3 in the projection's
   epilogue (one tile scale per head and 64 tokens, as the append does).
   Errors: as bkv_attend; BKV_ERR_UNSUPPORTED for BKV_F32. */
bkv_status bkv_attend_qkv(bkv_cache h, int32_t layer, const void* x, const void* w, const void* b,
                          int32_t model_dim, void* out, hipStream_t stream);

/* Close the open block: it joins the window; the oldest window block leaves
   (PR-Sink: into the bank, the oldest bank block dropped when full -- or,
   with BKV_BANK_POSE, the member most similar by pose, found on `stream`
   without waiting for it; ConvKV: its raw frames feed the conv memory,
   rebuilt here on `stream` once conv_kernel frames were evicted).  Does not
   synchronize.  Errors: BKV_ERR_STATE if no block is open or some layer was
   not attended in this block. */
bkv_status bkv_commit(bkv_cache h, hipStream_t stream);

/* Stream ids retrieved for the open block, in rank order (cosine descending,
   id ascending).  Synchronizes `stream`.  ids: host, capacity cap; *n = count.
   Errors: BKV_ERR_STATE if no block is open; BKV_ERR_ARG if cap < count. */
bkv_status bkv_selection(bkv_cache h, int32_t* ids, int32_t cap, int32_t* n, hipStream_t stream);

/* Context of the open block in attention order: static, dynamic (rank order),
   window (oldest first), current; ConvKV: memory, window, current.  segs: host,
   capacity cap.  Synchronizes `stream` when the context has dynamic segments. */
bkv_status bkv_context(bkv_cache h, bkv_segment* segs, int32_t cap, int32_t* n, hipStream_t stream);

/* Counters of the handle (host only). */
bkv_status bkv_stats(bkv_cache h, bkv_stats_t* out);

/* Inspection: copy context segment `seg` of the open block at `layer` as
   attention reads it -- K rotated, V as stored -- into device k_out, v_out
   [tokens][heads][head_dim] in the cache dtype (BKV_BF16_FP8K(V): bf16, K (and V) as
   its dequantised E4M3 value code * 2^e, which bf16 holds exactly).  For the current segment this
   needs an earlier bkv_attend of `layer` in this block.
   Errors: BKV_ERR_STATE (no open block / current block not yet written). */
bkv_status bkv_export_segment(bkv_cache h, int32_t layer, int32_t seg, void* k_out, void* v_out,
                              hipStream_t stream);

/* Per-kernel device time, measured with HIP events recorded on the caller's
   stream immediately before and after each kernel the handle launches. */
typedef struct {
  char kernel[24];         /* "retrieve", "append", "attention", "gather", "conv", "export", "qkv",
                              "replace" (pose-bank ranking), "vquant" (FP8 V of the ConvKV memory) */
  int64_t launches;
  double total_ms;         /* sum of per-launch event intervals */
  double max_ms;
} bkv_kernel_time;

/* Start recording per-launch kernel times for up to max_launches launches
   (later launches are not timed).  Creates 2*max_launches HIP events (host
   call, no device memory from the workspace).  Errors: BKV_ERR_STATE if a
   recording is already running; BKV_ERR_ARG if max_launches < 1. */
bkv_status bkv_profile_start(bkv_cache h, int32_t max_launches);

/* Stop recording: waits for the recorded events, sums the intervals per
   kernel into out[0..*n) (capacity cap) and releases the events.
   Errors: BKV_ERR_STATE if no recording is running; BKV_ERR_ARG if cap is too small. */
bkv_status bkv_profile_stop(bkv_cache h, bkv_kernel_time* out, int32_t cap, int32_t* n);

/* Measurement aid, not a step of the path: the sustained rate of the bf16
   matrix instruction the attention and projection kernels use
   (v_mfma_f32_32x32x16_bf16), for normalising their throughput to what the
   device sustains under its power limit rather than its nominal clock.
   Launches `workgroups` workgroups of 8 waves (2 per SIMD, as the attention
   kernel runs), each wave issuing `iters` rounds of 8 independent MFMAs on
   register operands holding full-mantissa pseudo-random values (the matrix
   core's power, and so the sustained clock, depends on the data), between
   two events on `stream`, and waits for them.
   *tflops = workgroups * 8 * iters * 8 * 32768 flop / elapsed time.
   Uses the current device; allocates 4 bytes of device memory per call (the
   kernel's result sink) and frees it.  Errors: BKV_ERR_ARG for workgroups or
   iters < 1 or a null tflops; BKV_ERR_DEVICE. */
bkv_status bkv_probe_mfma(int32_t workgroups, int32_t iters, double* tflops, hipStream_t stream);

/* Human-readable name of a status; message of the calling thread's last error. */
const char* bkv_status_str(bkv_status s);
const char* bkv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BKV_H_ */
