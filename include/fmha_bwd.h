/*
 * fmha_bwd.h -- C ABI of the MI355X (gfx950) fused multi-head attention backward.
 *
 * Computes dQ, dK, dV (and optionally dbias) of softmax attention
 * O = softmax(scale * Q K^T + bias + mask) V, with optional dropout on the probabilities, from
 * Q, K, V, the forward output O, its gradient dO and the forward log-sum-exp.  Three device
 * stages run on the caller's stream:
 *   1. D = rowsum(dO * O) into the workspace                                   (HBM bound)
 *   2. the main kernel: per (segment, K/V head, run of key tiles) it recomputes
 *      P = exp(S - LSE), accumulates dV += P^T dO and dK += dS^T Q in registers and emits the
 *      tiles' contribution dS K to the dQ accumulator (fp32 splits, fp32 atomics or bf16
 *      atomics)                                                                  (MFMA bound)
 *   3. dQ = bf16(scale * sum over splits of the accumulator), and dbias       (HBM bound)
 * fmha_fwd_run computes O and LSE with the same arguments.
 *
 * The workspace protocol follows "[CK_TILE] FMHA BWD Use Persistent Kernels in Deterministic
 * Mode" (aiter PR 2216), commit messages: the launcher reports a workspace size, the caller
 * allocates it, a prepare call initialises it, then the run call uses it.  As there, only the
 * atomic accumulation needs a zeroed accumulator; group mode without sequence offsets is
 * rejected; a workspace that is too small is an error, never a silent truncation.
 * Deterministic mode writes one fp32 dQ partial per key tile into an nsplits-deep workspace
 * and reduces it in a fixed order (the split/convert scheme of that page's Motivation).
 *
 * One pure host function (the plan) derives every size, offset and launch shape from the
 * arguments; fmha_bwd_workspace_size, fmha_bwd_prepare_workspace and fmha_bwd_run all call
 * it, so the sizing pass and the run pass cannot disagree -- the failure class described in
 * "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path (gfx950)", Root cause.
 *
 * Conventions
 *   - bf16 tensors (q, k, v, o, dout, dq, dk, dv) have the head dimension contiguous and
 *     element strides {batch, sequence, head}.  Batch mode (BSHD): element (b, s, h, c) is at
 *     b*stride[0] + s*stride[1] + h*stride[2] + c.  Group mode (THD, ragged): stride[0] is
 *     ignored and token t (a physical row given by the seqstart offsets) is at
 *     t*stride[1] + h*stride[2] + c.
 *   - lse is fp32, natural logarithm, as written by the forward: batch mode
 *     lse[b*lse_stride[0] + h*lse_stride[1] + s]; group mode lse[h*lse_stride[1] + t].
 *     A row with no allowed key carries -inf.
 *   - Grouped-query attention: query head h uses K/V head h / (Hq / Hkv).
 *   - Masks (numbering mirrors the mask-type table in the review of
 *     "Update AITER subcommit and refactor internal AITER/CK FA API usage", TransformerEngine
 *     PR 446): with Lq, Lk the lengths of a segment, key j is allowed for query i iff
 *     j < Lk and
 *       FMHA_MASK_NONE                 always
 *       FMHA_MASK_CAUSAL_TOP_LEFT      j <= i
 *       FMHA_MASK_CAUSAL_BOTTOM_RIGHT  j <= i + (Lk - Lq)
 *       FMHA_MASK_WINDOW               (left < 0 or j >= i + Lk - Lq - left) and
 *                                      (right < 0 or j <= i + Lk - Lq + right)
 *     window_left/window_right must be -1 for the first three types.
 *   - Rows with no allowed key get dQ = 0 and contribute nothing to dK and dV.
 *
 * Ownership: the caller owns every tensor and the workspace; the library allocates no device
 * memory and keeps no state between calls (fmha_bwd_run_noalloc's static scratch aside).  Host seqstart arrays are read during the call
 * only.  Device pointers must stay valid until the stream work completes.  One workspace must
 * not serve two runs in flight at the same time, and fmha_bwd_prepare_workspace must precede
 * every fmha_bwd_run (it writes the workspace header, and in the atomic modes it zeroes the
 * accumulator each time).
 *
 * ABI history (fields are only ever appended): 2 padded THD slots, 3 dq_acc_dtype, 4 bias and
 * dbias, 5 dropout, 6 plan_info.reduce_read_bytes, 7 plan_info.kv_parts and the dK/dV
 * partials region, 8 the layout overrides (tune_*) and plan_info.kernel.
 *
 * Errors: every function returns FMHA_OK or a negative fmha_status and never aborts.  Set
 * FMHA_BWD_LOG=1 in the environment to have the reason printed to stderr.
 */
#ifndef FMHA_BWD_H
#define FMHA_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMHA_BWD_ABI_VERSION 8u

#if defined(__GNUC__)
#define FMHA_BWD_API __attribute__((visibility("default")))
#else
#define FMHA_BWD_API
#endif

enum fmha_mask_type {
  FMHA_MASK_NONE = 0,
  FMHA_MASK_CAUSAL_TOP_LEFT = 1,
  FMHA_MASK_CAUSAL_BOTTOM_RIGHT = 2,
  FMHA_MASK_WINDOW = 3
};

/* dQ accumulation type of the non-deterministic mode (fmha_bwd_args.dq_acc_dtype). */
enum fmha_dq_acc_dtype {
  FMHA_DQ_ACC_FP32 = 0, /* fp32 accumulator, fp32 atomic adds (deterministic = 0) or fp32
                           split partials (deterministic = 1) */
  FMHA_DQ_ACC_BF16 = 1  /* deterministic = 0 only: packed bf16 atomic adds into a bf16
                           accumulator with one padded slot per segment, the "atomic16"
                           accumulation of "[ROCm] Fix THD/ragged dQ backward on the bf16
                           dq_shuffle path (gfx950)" (Root cause, Fix).  About half the
                           atomic traffic of fp32; every add rounds the running sum to bf16,
                           so dQ is less accurate than in the fp32 modes */
};

enum fmha_status {
  FMHA_OK = 0,
  FMHA_ERR_INVALID_ARG = -1,          /* bad shape, pointer, stride, mask or seqstart */
  FMHA_ERR_UNSUPPORTED = -2,          /* valid but not built: head dims, alignment */
  FMHA_ERR_WORKSPACE_TOO_SMALL = -3,  /* workspace_bytes below fmha_bwd_workspace_size */
  FMHA_ERR_PLAN_MISMATCH = -4,        /* FMHA_BWD_DEBUG=1 only: the workspace was prepared for
                                         other arguments (plan fingerprint in its header) */
  FMHA_ERR_HIP = -5                   /* a HIP runtime call or kernel launch failed */
};

typedef struct fmha_bwd_args {
  uint32_t struct_size;  /* sizeof(fmha_bwd_args), checked against the library's */
  uint32_t abi_version;  /* FMHA_BWD_ABI_VERSION */
  int32_t B;             /* batch size (batch mode) or number of segments (group mode) */
  int32_t Hq, Hkv;       /* query heads, K/V heads; Hq % Hkv == 0 */
  int32_t Sq, Sk;        /* sequence lengths (batch mode) or maximum segment lengths (group) */
  int32_t d_qk, d_v;     /* head dims; supported pairs: (64,64), (128,128), (192,128) */
  float scale;           /* softmax scale, > 0, usually 1/sqrt(d_qk) */
  int32_t mask_type;     /* enum fmha_mask_type */
  int32_t window_left;   /* FMHA_MASK_WINDOW only; -1 = unbounded */
  int32_t window_right;  /* FMHA_MASK_WINDOW only; -1 = unbounded */
  int32_t deterministic; /* 1: fp32 partials per run of key tiles + ordered reduction,
                            bit-reproducible; 0: atomic accumulation of dQ (fp32, or bf16
                            with dq_acc_dtype) */
  /* Group (THD) mode iff seqstart_q_host != NULL.  Then all four arrays are required and hold
     the same B+1 non-decreasing physical token offsets (host copies for planning, device
     copies for the kernels); segment b covers tokens [seqstart[b], seqstart[b+1]). */
  const int32_t* seqstart_q_host;
  const int32_t* seqstart_k_host;
  const int32_t* seqstart_q_dev;
  const int32_t* seqstart_k_dev;
  const void* q;     /* bf16 [.., Sq|T_q, Hq, d_qk] */
  const void* k;     /* bf16 [.., Sk|T_k, Hkv, d_qk] */
  const void* v;     /* bf16 [.., Sk|T_k, Hkv, d_v] */
  const void* o;     /* bf16 [.., Sq|T_q, Hq, d_v] forward output */
  const void* dout;  /* bf16 [.., Sq|T_q, Hq, d_v] gradient of o */
  const float* lse;  /* fp32 forward log-sum-exp, see conventions */
  void* dq;          /* bf16 [.., Sq|T_q, Hq, d_qk], every segment row overwritten */
  void* dk;          /* bf16 [.., Sk|T_k, Hkv, d_qk], every segment row overwritten */
  void* dv;          /* bf16 [.., Sk|T_k, Hkv, d_v], every segment row overwritten */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], do_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  int64_t lse_stride[2]; /* {batch, head}; the sequence stride is 1 */
  /* Padded THD (group mode, optional; the cu_seqlens_padded arrays next to cu_seqlens in
     "Update AITER subcommit and refactor internal AITER/CK FA API usage", review): the tensors
     hold segment b in a slot of physical rows [padded[b], padded[b+1]) that may be longer than
     its length seqstart[b+1] - seqstart[b].  Its rows are the first ones of the slot; the rest
     of the slot is never read, and dq/dk/dv rows there are left as they are.  lse is indexed
     by physical row.  For q and for k independently: both the host and the device array
     (B+1 non-decreasing offsets with padded[b] + length_b <= padded[b+1]), or neither (the
     slots are then the segments themselves). */
  const int32_t* seqstart_q_padded_host;
  const int32_t* seqstart_k_padded_host;
  const int32_t* seqstart_q_padded_dev;
  const int32_t* seqstart_k_padded_dev;
  int32_t dq_acc_dtype;  /* enum fmha_dq_acc_dtype; FMHA_DQ_ACC_BF16 needs deterministic = 0 */
  int32_t reserved;      /* must be 0 */
  /* Additive attention bias, batch mode only ("Update AITER subcommit and refactor internal
     AITER/CK FA API usage", review threads on the bias and dbias strides).  The logits are
     scale * q k^T + bias[b', h', i, j], b' = b if bias_b == B else 0, h' = h if bias_h == Hq
     else 0 (the shapes 11SS, 1HSS, B1SS, BHSS), before the mask and the softmax;
     fmha_fwd_run adds it as well, so its lse includes it.  Group mode with a bias is
     FMHA_ERR_UNSUPPORTED. */
  const void* bias;        /* bf16 [bias_b][bias_h][Sq][Sk], strides bias_stride (row stride
                              >= Sk); NULL = none */
  void* dbias;             /* bf16 gradient of bias, same shape, strides dbias_stride: the
                              full [B][Hq][Sq][Sk] gradient (fp32 in the workspace) summed over
                              the broadcast dimensions in ascending batch, then head order;
                              every element is overwritten.  NULL = not computed (needs bias) */
  int64_t bias_stride[3];  /* {batch, head, row} element strides; the column stride is 1; the
                              batch stride is unused when bias_b == 1, the head stride when
                              bias_h == 1 */
  int64_t dbias_stride[3];
  int32_t bias_b;          /* 1 or B (ignored without bias) */
  int32_t bias_h;          /* 1 or Hq */
  /* Dropout on the attention probabilities, driven by a Philox seed and offset as in "Update
     AITER subcommit and refactor internal AITER/CK FA API usage" (backward entry point).
     The generator is Philox4x32-10 (Salmon et al., SC 2011).  Element (b, h, i, j) (segment
     or batch b, query head h, positions i, j inside the segment) reads byte (j mod 4) of
     output word (i mod 4) for key (seed low 32 bits, seed high 32 bits) and counter
     (j / 4, i / 4, b * Hq + h, offset low 32 bits).  It is kept iff that byte is below
     k = round((1 - p_drop) * 256), and a kept probability is scaled by 256 / k.  Dropout
     applies to P in O = P V (fmha_fwd_run) and in the backward's dV and dP; lse is that of
     the softmax without dropout.  p_drop = 0 (k = 256) is no dropout. */
  float p_drop;            /* in [0, 1); k must come out >= 1 */
  int32_t reserved2;       /* must be 0 */
  uint64_t philox_seed;
  uint64_t philox_offset;  /* only its low 32 bits are used */
  /* Layout overrides for tests and tuning; 0 = the plan's own choice.  They are arguments
     like the others: the plan reads nothing but this struct and the host seqstart arrays, so
     the sizing, prepare and run calls of one argument struct always agree, and the plan's
     fingerprint covers the layout they select.  A value the chosen kernel cannot use is
     FMHA_ERR_INVALID_ARG. */
  int32_t tune_kernel;          /* FMHA_KERNEL_* below */
  int32_t tune_tile_m;          /* query rows per block of the four-wave kernel: 32 or 64 at
                                   d_qk = 128, 64 or 128 at d_qk = 64 */
  int32_t tune_tiles_per_item;  /* deterministic mode: key tiles per work item, 1, 2, 4 or 8 */
  int32_t tune_kv_parts;        /* work groups sharing one work item's steps, 1 .. 8 */
} fmha_bwd_args;

/* Main-kernel layouts (fmha_bwd_args.tune_kernel, fmha_bwd_plan_info.kernel). */
enum fmha_kernel {
  FMHA_KERNEL_AUTO = 0,  /* the plan's choice: FMHA_KERNEL_WIDE where it applies */
  FMHA_KERNEL_FOUR_WAVE = 1, /* 256 threads, 128-key tiles, 32-128-row query blocks; every
                                head dim, bias and dropout */
  FMHA_KERNEL_WIDE = 2   /* 512 threads (two waves per SIMD), 256-key tiles, 32-row query
                            blocks; d_qk = d_v = 128 or 64 without a bias (dropout is
                            allowed) */
};

/* Workspace bytes that prepare/run need for these arguments.  Host only: no GPU call, no
   allocation, no synchronisation; device pointers are not dereferenced. */
FMHA_BWD_API int fmha_bwd_workspace_size(const fmha_bwd_args* args, size_t* bytes);

/* Initialise the workspace on `stream` (a hipStream_t; NULL = the default stream): write its
   header (a magic value and a fingerprint of the plan: every size, offset and split count and
   the host seqstart arrays), and in the atomic modes (fp32 and bf16) zero the dQ
   accumulator; deterministic mode needs no other initialisation (every partial the reduction
   reads is written by the run).  Asynchronous; no memset nodes (graph capture safe).  Must
   precede every fmha_bwd_run. */
FMHA_BWD_API int fmha_bwd_prepare_workspace(const fmha_bwd_args* args, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Enqueue the three stages on `stream`.  Asynchronous; returns after the launches.  With
   FMHA_BWD_DEBUG=1 in the environment it first synchronizes `stream`, reads the workspace
   header back and returns FMHA_ERR_PLAN_MISMATCH if prepare ran for other arguments (the
   sizing/run disagreement of "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path
   (gfx950)", Root cause); without it the header is not read. */
FMHA_BWD_API int fmha_bwd_run(const fmha_bwd_args* args, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Forward pass with the same argument struct: reads q, k, v (and the masks, seqstart and
   padded-slot arrays, scale) and writes o = softmax(scale * q k^T + mask) v (bf16, layout of
   dout in the backward, strides o_stride) and lse (fp32 natural-log log-sum-exp, the layout
   the backward reads; -inf for a row with no allowed key, whose o row is 0).  dout, dq, dk and
   dv are not used.  No workspace; asynchronous on `stream`.  The forward computation is the
   one the backward differentiates (the plain definition, fp32 softmax statistics, bf16 P in
   the P.V product). */
FMHA_BWD_API int fmha_fwd_run(const fmha_bwd_args* args, void* stream);

/* Static string naming a status code. */
FMHA_BWD_API const char* fmha_bwd_status_string(int status);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
   loops, harnesses that forbid hipMalloc): fmha_bwd_prepare_workspace followed by fmha_bwd_run
   on `stream`, with a workspace the library owns instead of a caller's -- a static device
   array of FMHA_BWD_NOALLOC_MAX_BYTES bytes, one per GPU, held until the process ends (its
   address is looked up on the first call on each device).  Calls no allocating routine.
   Arguments whose fmha_bwd_workspace_size exceeds the maximum return
   FMHA_ERR_WORKSPACE_TOO_SMALL before any device work.  Every call on one GPU shares that
   GPU's array, which keeps the last call's contents (prepare re-initialises what must start
   at zero): calls that overlap on one GPU (other streams, other threads) race and must be
   serialised by the caller.  Results equal those of prepare + run with a caller workspace. */
#define FMHA_BWD_NOALLOC_MAX_BYTES (256u << 20)
FMHA_BWD_API int fmha_bwd_run_noalloc(const fmha_bwd_args* args, void* stream);

/* ---- test and measurement hooks -------------------------------------------------------- */

/* What the plan decided for these arguments (host only, like fmha_bwd_workspace_size). */
typedef struct fmha_bwd_plan_info {
  int32_t group_mode;      /* 1 for THD */
  int32_t tile_m;          /* query rows per block in the main kernel */
  int32_t tile_n;          /* keys per tile (one work item) */
  int32_t n_kv_tiles;      /* key tiles of the longest segment */
  int32_t n_q_blocks;      /* query blocks of the longest segment */
  int32_t nsplits;         /* depth of the dQ accumulator: ceil(n_kv_tiles / tiles_per_item),
                              or 1 in atomic mode */
  int32_t needs_zero;      /* prepare zeroes the accumulator */
  int32_t tiles_per_item;  /* key tiles per main-kernel work item (deterministic split) */
  int64_t rows_q;          /* T_q: B*Sq (batch), seqstart_q[B] (group) or the padded q
                              offsets' last entry (padded group) */
  int64_t d_offset;        /* byte offset of D = rowsum(dO*O), fp32 [Hq][rows_q]; bytes 0..255
                              of the workspace hold its header (magic, plan fingerprint) */
  int64_t dq_acc_offset;   /* byte offset of the fp32 accumulator [nsplits][Hq][acc_rows][d_qk] */
  int64_t dq_acc_bytes;
  int64_t workspace_bytes; /* == fmha_bwd_workspace_size */
  int64_t pairs;           /* allowed (query, key) pairs summed over heads and segments */
  double flops;            /* 2*(3*d_qk + 2*d_v) * pairs: the five contractions */
  int64_t acc_rows;        /* accumulator rows per head and split, or per segment and head in
                              bf16 mode (see below) */
  int32_t dq_acc_elem_bytes; /* 4 (fp32 accumulator) or 2 (bf16) */
  int32_t kv_parts;        /* work groups that share one work item's steps (query heads x
                              blocks); > 1 when there are too few K/V heads and tiles to fill
                              the GPU, or for long causal segments in deterministic mode: each
                              part stores fp32 dK/dV partials that the reduce stage sums in
                              ascending part order (see below) */
  int64_t dbias_acc_offset;  /* byte offset of the fp32 full-shape dS [B][Hq][Sq][Sk] (dbias) */
  int64_t dbias_acc_bytes;   /* 0 without dbias, or when dbias is full-shape (written directly) */
  int64_t reduce_read_bytes; /* bytes of the dQ accumulator the reduce stage reads (the
                                splits that touch each query block, or the atomic modes'
                                segment rows): for achieved-bandwidth figures */
  int64_t dkv_acc_offset;    /* byte offset of the fp32 dK, dV partials [kv_parts][Hkv][rows_k]
                                [d_qk + d_v] (only when kv_parts > 1) */
  int64_t dkv_acc_bytes;
  int32_t kernel;            /* enum fmha_kernel: the main-kernel layout the run launches */
  int32_t ordered_groups;    /* > 0: the main kernel's work groups take their work items in
                                descending order of their steps (a list of this many entries
                                that the run's D stage writes at the end of the workspace);
                                0: grid order */
} fmha_bwd_plan_info;
/* Accumulator layout.  Atomic mode: one split, rows_q rows, row-major ([row][d_qk]), row of
   a query = its D/LSE row.  Deterministic mode: split s holds the sum of the partials of key
   tiles s*T .. s*T+T-1 (T = tiles_per_item, added in ascending tile order);
   acc_rows = rows_q + B*tile_m and query block i of segment b (rows b_0 + i*tile_m ..) is
   the tile_m*d_qk values starting at row a_b + i*tile_m, a_b = (first D row of segment b) +
   b*tile_m, so blocks of different segments never share rows.  Inside a block the values
   are grouped in 32x32 tiles, tile t = (r/32)*(d_qk/32) + c/32 at offset 1024*t, and tile
   element (r, c) (r, c < 32) at 256*(r/8) + 4*(c + 32*((r/4)%2)) + r%4: the result layout of
   a 32x32 matrix-core product (lane c + 32*((r/4)%2), register 4*(r/8) + r%4) stored as four
   1 KB chunks, chunk u holding registers 4u .. 4u+3 of every lane in lane order, so that
   one 16-byte-per-lane access covers a contiguous kilobyte.  bf16 mode (dq_acc_dtype =
   FMHA_DQ_ACC_BF16): bf16 [B][Hq][acc_rows][d_qk], acc_rows = the longest segment's query
   count rounded up to a multiple of tile_m, and query i of segment b in block i/tile_m of
   slot (b, h): the slot is indexed by the logical position, so neither the physical
   (padded) layout of the tensors nor other segments' rows can move it.  Each block of
   tile_m*d_qk values is in matrix-core tile order: tile t = (r/32)*(d_qk/32) + c/32 at
   1024*t, and in it element pair w (elements 2w, 2w+1; w = 64*k + l, k < 8, l < 64) holds
   row 8*(q/4) + 4*(l/32) + q%4 (q = k + 8*(l%2)) of the tile, columns 2*((l%32)/2) and the
   next, so that each packed atomic of the main kernel covers 256 contiguous bytes.  The unscaled sum dS K is accumulated
   there; the reduction multiplies by scale and rounds to bf16 into dq.
   dK/dV partials (kv_parts > 1): fp32 [kv_parts][Hkv][rows_k][d_qk + d_v], rows_k = B*Sk in
   batch mode (key j of batch entry b at row b*Sk + j), else the last entry of the padded or
   plain key offsets (key j of segment b at row start_b + j); each row holds the unscaled dK
   sum, then the dV sum, of the part's steps.  The reduce stage writes dK = bf16(scale * sum)
   and dV = bf16(sum) over the parts; with kv_parts > 1 dK and dV are therefore written by the
   reduce stage, not the main one. */

FMHA_BWD_API int fmha_bwd_plan_query(const fmha_bwd_args* args, fmha_bwd_plan_info* info);

/* Run a subset of the stages of fmha_bwd_run (bit mask of fmha_bwd_stage), for unit tests
   of one kernel and per-kernel timing.  Same contract as fmha_bwd_run. */
enum fmha_bwd_stage { FMHA_STAGE_DOT = 1, FMHA_STAGE_MAIN = 2, FMHA_STAGE_REDUCE = 4 };
FMHA_BWD_API int fmha_bwd_run_stages(const fmha_bwd_args* args, void* workspace, size_t workspace_bytes,
                        int stages, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_BWD_H */
