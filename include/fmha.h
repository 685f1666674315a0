/*
 * fmha.h -- C ABI of the MI355X (gfx950) attention forward library.
 *
 * Exact scaled-dot-product attention forward with per-row log-sum-exp:
 *
 *   O[i,h,:] = sum_j softmax_j(scale * q[i,h,:] . k[j,h_kv,:] + mask) v[j,h_kv,:]
 *   LSE[h,i] = ln sum_{j allowed} exp(scale * q[i,h,:] . k[j,h_kv,:])
 *
 * with split-KV (each split writes a partial (O_s, lse_s) into a workspace and
 * an LSE-weighted combine merges them) and packed variable-length batches.
 *
 * Where the operation is defined (web pages on split-KV flash attention):
 *  - "Adds variable sequence lengths to the Hopper CuTe DSL FMHA example"
 *    (CUTLASS), section Interface: cumulative int32 sequence lengths
 *    [0, s0, s0+s1, ...] for Q and K independently, None (here NULL) for a
 *    fixed-length side, variable-length tensors packed along the sequence
 *    dimension with batch size 1, and a max_seqlen_q bound; section
 *    Implementation: the grid covers the longest query sequence, tiles past a
 *    sequence's end or with an empty key sequence are skipped so rows of a
 *    query sequence with no keys are not written, tails are masked, rows of
 *    a tail tile past the sequence are not stored, the default softmax scale
 *    is 1/sqrt(head_dim) and an unsupported configuration is refused up front
 *    instead of dropping rows; section Tests: bottom-right causal for
 *    different q/k lengths, sliding window (128, 0), GQA 8:8 / 8:2 / 8:1.
 *  - "[FlyDSL] Enable FP8 FMHA split-K for short cached-prefix queries"
 *    (aiter), description and review: explicit num_kv_splits or an automatic
 *    split choice, a per-call fp32 split workspace, FP8 e4m3 inputs with
 *    per-tensor scales, return_lse, the split combine timed together with the
 *    attention, graph replay, and an invalid combination refused with an
 *    error (ValueError in Python).
 *  - "[Cute,Fwd,Sm100] Support q_stage=1 for inference" (flash-attention),
 *    description and benchmark table: split KV over a sweep of split counts
 *    for single-token decode.
 *
 * Conventions for every call:
 *  - Ownership: every pointer is caller-owned device memory (cu_seqlens
 *    included).  The library allocates nothing and keeps no pointer after a
 *    call returns.
 *  - Asynchrony: the launching calls only enqueue work on `stream` (a
 *    hipStream_t; NULL = the null stream).  They never synchronise and never
 *    read device memory from the host, so they can be captured in a HIP graph.
 *  - Errors: every check runs on the host before any launch.  On any non-zero
 *    return nothing has been enqueued and no output byte has been written.
 *  - Layout: the last (head-dim) dimension of q, k, v and out is contiguous;
 *    all other strides are in elements.  Token t of a fixed-length side of
 *    batch b is at b*stride_batch + t*stride_tok; token t of sequence b of a
 *    variable-length side is at (cu_seqlens[b] + t)*stride_tok.  Base
 *    pointers of q, k, v, out must be 16-byte aligned and every stride of
 *    theirs, in bytes, a multiple of 16.
 *  - Device data that cannot be checked: cu_seqlens must be non-decreasing,
 *    start at 0, end at total_q / total_k, and no sequence may exceed
 *    max_seqlen_q / max_seqlen_k.  Violations are undefined behaviour.
 *  - Rows not written: every row of a query sequence whose key sequence is
 *    empty is left untouched (O and LSE).  A row whose allowed key set is
 *    empty for any other reason (causal with more queries than keys, a narrow
 *    window) is written as O = 0, LSE = -inf.
 */
#ifndef FMHA_H_
#define FMHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  FP8 is OCP e4m3fn (bias 7, max 448, no infinities). */
typedef enum fmha_dtype {
  FMHA_DTYPE_F32 = 0,
  FMHA_DTYPE_F16 = 1,
  FMHA_DTYPE_BF16 = 2,
  FMHA_DTYPE_FP8_E4M3 = 3
} fmha_dtype;

/* Return codes (Python maps every non-zero code to ValueError). */
typedef enum fmha_status {
  FMHA_OK = 0,
  FMHA_ERR_INVALID_ARG = 1, /* null/mismatched argument, Hq % Hkv != 0, bad window,
                               bad scale, bad split count, misaligned pointer/stride */
  FMHA_ERR_UNSUPPORTED = 2, /* no compiled kernel for (dtype, head dims, out dtype), or
                               token strides a kernel cannot address (prefill kernels:
                               key block x token stride must stay below 2^31 bytes) */
  FMHA_ERR_WORKSPACE = 3,   /* split workspace missing or too small */
  FMHA_ERR_HIP = 4          /* a HIP launch or device query failed */
} fmha_status;

/* Largest explicit split count accepted. */
#define FMHA_MAX_SPLITS 256

/*
 * Arguments of one forward call.  Zero-initialise, then fill in.
 *
 *  q, k, v      : inputs, element type in_dtype.
 *                 q [B, Sq, Hq, Dqk] or packed [total_q, Hq, Dqk];
 *                 k [B, Sk, Hkv, Dqk] or packed [total_k, Hkv, Dqk];
 *                 v [B, Sk, Hkv, Dv]  or packed [total_k, Hkv, Dv].
 *  out          : output, element type out_dtype, [B, Sq, Hq, Dv] or packed
 *                 [total_q, Hq, Dv].
 *  lse          : fp32 natural-log LSE, or NULL to skip it (return_lse=False).
 *                 Row (b, h, i) is at b*lse_stride_batch + h*lse_stride_head + i
 *                 for fixed-length Q and at h*lse_stride_head + cu_seqlens_q[b] + i
 *                 for variable-length Q.
 *  cu_seqlens_q / cu_seqlens_k : int32 [batch+1] on the device, or NULL for a
 *                 fixed-length side (then seqlen_q / seqlen_k apply).
 *  batch        : number of sequences B (>= 0).
 *  seqlen_q/k   : fixed lengths (ignored for a variable-length side).
 *  max_seqlen_q/k : host-known upper bounds of the variable-length side
 *                 (ignored for a fixed side, where they equal seqlen_q/k).
 *  total_q/k    : packed token counts of a variable-length side (ignored for
 *                 a fixed side, where they are batch*seqlen).
 *  num_heads_q/kv : Hq, Hkv with Hq % Hkv == 0; query head h reads kv head
 *                 h / (Hq / Hkv).
 *  head_dim_qk/v: Dqk, Dv.
 *  *_stride_*   : strides in elements (batch strides only used by a
 *                 fixed-length side).
 *  in_dtype     : element type of q, k, v.
 *  out_dtype    : in_dtype for f32/f16/bf16 inputs; BF16 for FP8 inputs.
 *  q/k/v_descale: device fp32 scalars for FP8 inputs (real = stored * descale);
 *                 NULL means 1.  Ignored for other dtypes.
 *  softmax_scale: > 0, or 0 for the default 1/sqrt(Dqk).  Negative or
 *                 non-finite values are rejected.
 *  causal       : bottom-right aligned: key j is allowed for query i iff
 *                 j <= i + sk - sq.
 *  window_left/right : sliding window around the same diagonal, inclusive:
 *                 i + sk - sq - left <= j <= i + sk - sq + right; -1 means
 *                 unbounded.  With causal, right is clamped to 0.
 *  num_kv_splits: 0 = automatic, 1 = no split, n in [2, 256] = explicit.
 *                 Split s of sequence b covers keys [s*chunk, (s+1)*chunk) of
 *                 that sequence, chunk = ceil(max_seqlen_k / n) rounded up to
 *                 the kernel's key block; sequence b uses ceil(sk_b / chunk)
 *                 splits.
 *  workspace    : device scratch for split partials and the tile table of the
 *                 length-aware order (fmha_fwd_workspace_size bytes, 256-byte
 *                 aligned); may be NULL when no split is used (a plan that
 *                 would sort its tiles then keeps the grouped order).
 *                 Its counter block (fmha_fwd_plan.counter_offset, counter_bytes)
 *                 must be zero before the first fmha_fwd that uses it; every
 *                 call leaves it zero (allocate the workspace zeroed once and
 *                 reuse it).  A call that finds it non-zero writes NaN rows or
 *                 waits a bounded time, and never hangs.
 *  num_cus      : compute units used by the automatic split choice
 *                 (0 = 256, the MI355X count).
 *  combine_mode : 0 = split partials combined by a second launch (default);
 *                 1 = combined inside the attention launch by the split
 *                 workgroups themselves when the plan allows it (see
 *                 fmha_fwd_plan.combine_in_kernel), else by a second launch.
 *                 Measured on MI355X for the fp8 short-prefix shape, the
 *                 second launch is 6-9 % faster: both move the fp32 partials
 *                 through memory once, and the in-kernel form adds the wait
 *                 for a tile's slowest split.  The plan takes this form only
 *                 when its grid fits the device's compute units, assuming the
 *                 launch has them to itself: a split workgroup kept from
 *                 starting for longer than the bounded wait (about a quarter
 *                 of a second; e.g. behind a long kernel on another stream)
 *                 makes its tile's rows NaN instead of hanging.
 *  persistent   : 1 = when the plan sorts its tiles on the device (tile order 4,
 *                 f16/bf16), launch one round of workgroups that take tiles
 *                 from the table until none is left, instead of one workgroup
 *                 per tile; 0 = one workgroup per tile (default).  Measured on
 *                 MI355X the default is faster (by 44 % on 128 causal
 *                 sequences at head dim 128).
 */
typedef struct fmha_fwd_args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t batch;
  int32_t seqlen_q;
  int32_t seqlen_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t total_q;
  int32_t total_k;
  int32_t num_heads_q;
  int32_t num_heads_kv;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int64_t q_stride_batch, q_stride_tok, q_stride_head;
  int64_t k_stride_batch, k_stride_tok, k_stride_head;
  int64_t v_stride_batch, v_stride_tok, v_stride_head;
  int64_t o_stride_batch, o_stride_tok, o_stride_head;
  int64_t lse_stride_batch, lse_stride_head;
  int32_t in_dtype;
  int32_t out_dtype;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  float softmax_scale;
  int32_t causal;
  int32_t window_left;
  int32_t window_right;
  int32_t num_kv_splits;
  void* workspace;
  size_t workspace_bytes;
  int32_t num_cus;
  int32_t combine_mode;
  int32_t persistent;
} fmha_fwd_args;

/*
 * What a call resolves to (filled by fmha_fwd_check).  Split partials live in
 * the workspace as fp32 o_part [num_splits, total_q, Hq, Dv] at
 * o_part_offset and fp32 lse_part [num_splits, Hq, total_q] at
 * lse_part_offset, where total_q counts fixed-length Q as batch*seqlen_q.
 */
typedef struct fmha_fwd_plan {
  float softmax_scale;  /* resolved: 0 -> 1/sqrt(head_dim_qk) */
  int32_t window_left;  /* resolved, -1 = unbounded */
  int32_t window_right; /* resolved, causal folded in (0) */
  int32_t num_splits;   /* resolved split count, 1 = no split */
  int32_t split_chunk;  /* keys per split */
  int32_t rows_per_tile;
  int32_t num_q_tiles;
  int32_t key_block;    /* keys one workgroup loads per iteration */
  int32_t kernel_id;    /* internal kernel instance (informational) */
  int64_t grid_main;    /* workgroups of the attention launch */
  int64_t grid_combine; /* workgroups of the combine launch (0 if none) */
  size_t workspace_bytes;
  size_t o_part_offset;
  size_t lse_part_offset;
  size_t counter_offset; /* split plans: arrival counters, one 128-byte line per (sequence,
                            kv head, query tile), counter_bytes in all */
  size_t counter_bytes;
  int32_t combine_in_kernel; /* 1: fmha_fwd combines the split partials inside the
                            attention launch (no second launch): combine_mode 1,
                            multi-row kernels whose whole grid fits one workgroup
                            per compute unit (num_cus, checked against the device
                            at launch), at most 64 splits.  The counter block must
                            then be zero when the call starts; every call leaves
                            it zero. */
  size_t sched_offset;  /* tile_order 4: the tile table in the workspace */
  int32_t sched_items;  /* tile_order 4: grid positions the table maps */
  int32_t persistent;   /* tile_order 4: 1 = a persistent grid (grid_main workgroups)
                           takes the table's positions */
  int32_t tile_order;   /* 0: tiles grouped by (sequence, kv head); 1: all tiles
                           longest first (32-row-tile prefill kernels, one split,
                           causal or a right-only window, batch <= 64); 2: decode
                           splits, full ones first, then the partial ones longest
                           first (decode kernel, more than one split, batch <= 64);
                           3: the kv heads of one (sequence, split) together
                           (multi-row kernels, one query tile, several splits);
                           4: (sequence, kv head) groups dealt to XCDs longest
                           first by a schedule kernel on the device, each
                           group's tiles together (32-row-tile prefill, one
                           split, a causal or window mask, 65..1024 sequences or
                           a left window; needs the workspace, else order 0) */
} fmha_fwd_plan;

/*
 * Validate `args` for an fmha_fwd call and resolve defaults, split count and
 * workspace size.  Defined by "Adds variable sequence lengths to the Hopper
 * CuTe DSL FMHA example", section Implementation (the default softmax scale
 * 1/sqrt(head_dim) for scale 0, pinned by a host test for non-square shapes;
 * an unsupported configuration refused up front) and "[FlyDSL] Enable FP8
 * FMHA split-K ...", review (an invalid split combination raises).
 * Host only: makes no HIP call and reads no device memory, so
 * it runs without a GPU.  `plan` may be NULL.  The workspace pointer/size are
 * checked only when a split is used.  With args->out == NULL the arguments are
 * checked for fmha_fwd_splitkv_partials instead.  Returns FMHA_OK or an error
 * code.
 */
int fmha_fwd_check(const fmha_fwd_args* args, fmha_fwd_plan* plan);

/* Resolved split count for `args` (host only; automatic when num_kv_splits == 0).
 * The split choice of "[FlyDSL] Enable FP8 FMHA split-K ...", description
 * (explicit num_kv_splits or the automatic heuristic), whose effect the split
 * sweep of "[Cute,Fwd,Sm100] Support q_stage=1 for inference", section
 * Benchmarks, shows.  A shape query: data pointers are not checked and may be
 * NULL.  Returns FMHA_OK or the error code fmha_fwd_check would give. */
int fmha_num_splits(const fmha_fwd_args* args, int32_t* splits_out);

/* Workspace bytes `args` needs (host only; 0 when no split is used): the
 * per-call fp32 split workspace of "[FlyDSL] Enable FP8 FMHA split-K ...",
 * review, laid out as in fmha_fwd_plan.  A shape query: data pointers are not
 * checked and may be NULL.  Returns FMHA_OK or an error code. */
int fmha_fwd_workspace_size(const fmha_fwd_args* args, size_t* bytes_out);

/*
 * Enqueue the forward pass on `stream`: one attention launch, plus the split
 * combine when more than one split is used.  Writes out (and lse if given).
 * The operation of "Adds variable sequence lengths to the Hopper CuTe DSL FMHA
 * example", sections Interface and Implementation (packed variable-length or
 * fixed sides, rows of a query sequence without keys left unwritten), with the
 * split-K of "[FlyDSL] Enable FP8 FMHA split-K ...", description and
 * measurement (attention and split combine in one call, return_lse).
 * Reads q, k, v, cu_seqlens and descales; writes only out and lse (and the
 * workspace).  On an error nothing is enqueued (see the conventions above).
 */
int fmha_fwd(const fmha_fwd_args* args, void* stream);

/*
 * fmha_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches, with the split partials in a scratch array the library holds
 * in device memory (one per GPU it runs on, FMHA_NO_ALLOC_SCRATCH_BYTES each,
 * kept until the process ends) instead of args->workspace, which is ignored.
 * Makes no allocation.  The caller still passes q, k, v, out, lse.
 * combine_mode is taken as 0: the split combine always runs as the second
 * launch (the in-launch form needs a zeroed counter block, which the shared
 * scratch cannot promise).
 * Returns FMHA_ERR_WORKSPACE (nothing enqueued) when the resolved plan needs
 * a larger workspace than the scratch (fmha_fwd_workspace_size tells), and
 * FMHA_ERR_HIP if the scratch address cannot be looked up; otherwise as
 * fmha_fwd.  Every call on one GPU shares that GPU's scratch and leaves its
 * partials there: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 */
#define FMHA_NO_ALLOC_SCRATCH_BYTES (32u << 20)
int fmha_fwd_no_alloc(const fmha_fwd_args* args, void* stream);

/*
 * Enqueue only the attention launch of a split forward (split KV as in
 * "[Cute,Fwd,Sm100] Support q_stage=1 for inference", description: each split
 * of the key range is its own unit of work): writes the fp32
 * partials (O_s normalised within split s, lse_s natural log; (0, -inf) for a
 * split with no allowed key) into the workspace at the plan's offsets, for
 * every split s < ceil(sk_b / chunk) of every sequence b with keys.  Requires
 * a resolved split count > 1 (else FMHA_ERR_INVALID_ARG).  `out`/`lse` are
 * not touched and may be NULL.  fmha_fwd is this call followed by fmha_splitkv_combine.
 */
int fmha_fwd_splitkv_partials(const fmha_fwd_args* args, void* stream);

/*
 * Arguments of the split combine.
 *  o_part   : fp32 [num_splits, total_q, Hq, Dv] partial outputs.
 *  lse_part : fp32 [num_splits, Hq, total_q] partial natural-log LSEs.
 *  Row i of sequence b (query token t = its packed index, or b*seqlen_q + i
 *  for fixed-length Q) combines splits s < ceil(sk_b / split_chunk):
 *    L = max_s lse_s; if L = -inf: O = 0, LSE = -inf;
 *    else LSE = L + ln sum_s exp(lse_s - L), O = sum_s exp(lse_s - LSE) O_s.
 *  Rows of sequences with sk_b == 0 are not written.  out / lse addressing
 *  and dtypes as in fmha_fwd_args (lse may be NULL).
 */
typedef struct fmha_combine_args {
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t batch;
  int32_t seqlen_q;
  int32_t seqlen_k;
  int32_t max_seqlen_q;
  int32_t total_q;
  int32_t num_heads_q;
  int32_t head_dim_v;
  int32_t num_splits;
  int32_t split_chunk;
  int64_t o_stride_batch, o_stride_tok, o_stride_head;
  int64_t lse_stride_batch, lse_stride_head;
  int32_t out_dtype;
} fmha_combine_args;

/* Enqueue the LSE-weighted combine of split partials on `stream`: the split
 * combine that "[FlyDSL] Enable FP8 FMHA split-K ...", measurement and author
 * reply, times together with the attention.  Reads o_part, lse_part and
 * cu_seqlens; writes out and lse.  Returns FMHA_ERR_INVALID_ARG (nothing
 * enqueued) for a bad argument, FMHA_ERR_HIP if the launch fails. */
int fmha_splitkv_combine(const fmha_combine_args* args, void* stream);

/* Human-readable name of a status code (static string; the message Python
 * puts in its ValueError, as "[FlyDSL] Enable FP8 FMHA split-K ...", review,
 * has invalid calls raise). */
const char* fmha_status_str(int status);

/*
 * Check a cumulative sequence-length array on the device against the
 * contract above ("Adds variable sequence lengths to the Hopper CuTe DSL FMHA
 * example", section Interface): cu_seqlens[0] == 0, non-decreasing,
 * cu_seqlens[batch] == total, and no sequence longer than max_seqlen.  Enqueues one single-workgroup kernel on `stream` that reads
 * cu_seqlens[0..batch] (caller-owned device memory, batch + 1 int32) and
 * writes one int32 to `result` (caller-owned device memory): 0 if the array
 * meets the contract, else 1 + the smallest index b at which it fails (b == 0:
 * a non-zero first entry; b in 1..batch: a decrease or a sequence longer than
 * max_seqlen ending at b; b == batch also: a last entry other than total).
 * A debug aid for arrays that come from elsewhere: the forward calls never
 * read cu_seqlens on the host.  Returns FMHA_ERR_INVALID_ARG (nothing
 * enqueued) for a NULL pointer or a negative batch, total or max_seqlen,
 * FMHA_ERR_HIP if the launch fails.
 */
int fmha_check_seqlens(const int32_t* cu_seqlens, int32_t batch, int32_t total, int32_t max_seqlen,
                       int32_t* result, void* stream);

/* Compute units of the current HIP device (a HIP query; FMHA_ERR_HIP on
 * failure): the device size the automatic split choice of "[FlyDSL] Enable
 * FP8 FMHA split-K ...", description, is sized against. */
int fmha_device_num_cus(int32_t* num_cus_out);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H_ */
