// plan.cpp -- argument validation and workspace layout (host only).
//
// Workspace layout (byte offsets 256-aligned):
//   header  2 x uint64 (magic, plan fingerprint) written by prepare; 256 bytes
//   D       fp32 [Hq][rows_q]                     rowsum(dO * O) from the first stage
//   L       fp32 [Hq][rows_q]                     LSE * log2(e), also from the first stage
//   dq_acc  fp32 [nsplits][Hq][acc_rows][d_qk]    dQ partials (deterministic: split s = key
//                                                 tiles s*T..s*T+T-1 of the segment, T =
//                                                 tiles_per_item, blocks of tile_m rows
//                                                 in matrix-core tile order, tile_m rows of
//                                                 padding per segment; atomic: one split,
//                                                 row-major, acc_rows = rows_q)
//   dbias_acc fp32 [B][Hq][Sq][Sk]              full-shape dS when dbias is requested
//   dkv_acc fp32 [kv_parts][Hkv][rows_k][d_qk + d_v]  dK, dV partials when kv_parts > 1
//           or bf16 [B][Hq][acc_rows][d_qk]       bf16 atomic mode: one slot of
//                                                 acc_rows = the longest lq rounded up to
//                                                 tile_m rows per (segment, head), indexed
//                                                 by the logical query position, each block
//                                                 of tile_m rows in matrix-core tile order
// One layout serves batch and group mode: row = b*Sq + i in batch mode and seqstart_q[b] + i
// in group mode (the physical token), so a ragged segment never aliases another one's rows --
// unlike the layout mix-up in "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path
// (gfx950)", Root cause, where ragged segments after the first landed on slot 0.
#include "plan.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tiling.h"

namespace fmha {
namespace {

int fail(int status, char* err, size_t len, const char* msg) {
  if (err && len) {
    snprintf(err, len, "%s", msg);
  }
  return status;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kHeaderBytes = 256;

// FNV-1a, 64 bit, over the bytes of each value in turn.
struct Fnv {
  uint64_t h = 0xcbf29ce484222325ull;
  void add(const void* p, size_t n) {
    const unsigned char* c = (const unsigned char*)p;
    for (size_t i = 0; i < n; ++i) {
      h ^= c[i];
      h *= 0x100000001b3ull;
    }
  }
  template <class T> void v(T x) { add(&x, sizeof x); }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels move 8 bf16 (16 bytes) per lane access along the head dimension, and address
// rows inside one tile with 32-bit offsets (sequence stride < 2^24 elements).
bool strides_ok(const int64_t s[3], bool group) {
  for (int i = group ? 1 : 0; i < 3; ++i) {
    if (s[i] < 0 || (s[i] & 7) != 0) return false;
  }
  return s[1] < (int64_t(1) << 24);
}

}  // namespace

int make_plan(const fmha_bwd_args* a, Plan* p, char* err, size_t el, bool forward) {
  if (!a || !p) return fail(FMHA_ERR_INVALID_ARG, err, el, "null argument");
  if (a->struct_size != sizeof(fmha_bwd_args))
    return fail(FMHA_ERR_INVALID_ARG, err, el, "struct_size does not match this library");
  if (a->abi_version != FMHA_BWD_ABI_VERSION)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "abi_version does not match this library");
  memset(p, 0, sizeof(*p));
  const bool group = a->seqstart_q_host != nullptr;
  p->group_mode = group;
  if (a->B < 0 || a->Sq < 0 || a->Sk < 0)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "B, Sq and Sk must be non-negative");
  if (a->Hq <= 0 || a->Hkv <= 0 || a->Hq % a->Hkv != 0)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "Hq and Hkv must be positive with Hq % Hkv == 0");
  const bool dims_ok = (a->d_qk == 64 && a->d_v == 64) || (a->d_qk == 128 && a->d_v == 128) ||
                       (a->d_qk == 192 && a->d_v == 128);
  if (!dims_ok)
    return fail(FMHA_ERR_UNSUPPORTED, err, el,
                "head dims (d_qk, d_v) must be (64,64), (128,128) or (192,128)");
  if (!isfinite(a->scale)) return fail(FMHA_ERR_INVALID_ARG, err, el, "scale is not finite");
  if (!(a->scale > 0.f)) return fail(FMHA_ERR_UNSUPPORTED, err, el, "scale must be positive");
  if (a->mask_type < FMHA_MASK_NONE || a->mask_type > FMHA_MASK_WINDOW)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "unknown mask_type");
  if (a->mask_type != FMHA_MASK_WINDOW && (a->window_left != -1 || a->window_right != -1))
    return fail(FMHA_ERR_INVALID_ARG, err, el,
                "window_left/window_right must be -1 unless mask_type is FMHA_MASK_WINDOW");
  if (a->window_left < -1 || a->window_right < -1)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "window bounds must be >= -1");
  if (a->deterministic != 0 && a->deterministic != 1)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "deterministic must be 0 or 1");
  if (a->dq_acc_dtype != FMHA_DQ_ACC_FP32 && a->dq_acc_dtype != FMHA_DQ_ACC_BF16)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "unknown dq_acc_dtype");
  if (a->dq_acc_dtype == FMHA_DQ_ACC_BF16 && a->deterministic)
    return fail(FMHA_ERR_INVALID_ARG, err, el,
                "the bf16 dQ accumulator is for atomic (deterministic = 0) mode only");
  if (a->reserved != 0) return fail(FMHA_ERR_INVALID_ARG, err, el, "reserved must be 0");
  if (a->dbias && !a->bias)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "dbias needs a bias");
  if (!(a->p_drop >= 0.f && a->p_drop < 1.f))
    return fail(FMHA_ERR_INVALID_ARG, err, el, "p_drop must be in [0, 1)");
  if (a->reserved2 != 0) return fail(FMHA_ERR_INVALID_ARG, err, el, "reserved2 must be 0");
  p->drop_k = (int)floor((1.0 - (double)a->p_drop) * 256.0 + 0.5);
  if (p->drop_k < 1)
    return fail(FMHA_ERR_UNSUPPORTED, err, el, "p_drop too close to 1 (keep threshold rounds to 0)");

  p->B = a->B;
  p->Hq = a->Hq;
  p->Hkv = a->Hkv;
  p->group_size = a->Hq / a->Hkv;
  p->Sq = a->Sq;
  p->Sk = a->Sk;
  p->d_qk = a->d_qk;
  p->d_v = a->d_v;
  // Layout overrides (arguments like the others: nothing here reads the environment, so one
  // argument struct always yields one plan)
  if (a->tune_kernel < FMHA_KERNEL_AUTO || a->tune_kernel > FMHA_KERNEL_WIDE)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "unknown tune_kernel");
  if (a->tune_tiles_per_item != 0 && a->tune_tiles_per_item != 1 && a->tune_tiles_per_item != 2 &&
      a->tune_tiles_per_item != 4 && a->tune_tiles_per_item != 8)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "tune_tiles_per_item must be 0, 1, 2, 4 or 8");
  if (a->tune_kv_parts < 0 || a->tune_kv_parts > 8)
    return fail(FMHA_ERR_INVALID_ARG, err, el, "tune_kv_parts must be in 0 .. 8");
  const bool with_bias = a->bias != nullptr;
  // The wide kernel (eight waves, 256-key tiles) serves d_qk = d_v = 128 or 64 without a
  // bias (with or without dropout).  It addresses 256-row key tiles, and a query head's Q and dO rows of a whole
  // segment, with 32-bit byte offsets: sequence strides below 2^22 elements, and Sq rows (plus
  // a block) times the Q and dO sequence strides below 2^30 elements.
  const bool wide_ok = ((a->d_qk == 128 && a->d_v == 128) || (a->d_qk == 64 && a->d_v == 64)) &&
                       !with_bias &&
                       a->q_stride[1] < (int64_t(1) << 22) && a->k_stride[1] < (int64_t(1) << 22) &&
                       a->v_stride[1] < (int64_t(1) << 22) && a->do_stride[1] < (int64_t(1) << 22) &&
                       ((int64_t)a->Sq + 32) * a->q_stride[1] < (int64_t(1) << 30) &&
                       ((int64_t)a->Sq + 32) * a->do_stride[1] < (int64_t(1) << 30);
  if (a->tune_kernel == FMHA_KERNEL_WIDE && !wide_ok)
    return fail(FMHA_ERR_INVALID_ARG, err, el,
                "tune_kernel = FMHA_KERNEL_WIDE needs d_qk = d_v = 128 or 64, no bias, "
                "sequence strides below 2^22 and (Sq + 32) times the q and dout sequence strides "
                "below 2^30");
  p->kernel = (a->tune_kernel == FMHA_KERNEL_FOUR_WAVE || !wide_ok) ? FMHA_KERNEL_FOUR_WAVE
                                                                    : FMHA_KERNEL_WIDE;
  if (p->kernel == FMHA_KERNEL_WIDE) {
    p->tile_m = 32;
    p->tile_n = 256;
    if (a->tune_tile_m != 0 && a->tune_tile_m != 32)
      return fail(FMHA_ERR_INVALID_ARG, err, el, "the wide kernel's query blocks have 32 rows");
  } else {
    // query rows per block (register and LDS budget): 64 for d_qk = 128, 32 for d_qk = 192,
    // and for d_qk = 64 128 rows (its smaller accumulators leave room for four 32-row
    // tiles, which halves the per-step overheads per FLOP) except with fp32 dQ atomics,
    // which were faster with 64-row blocks
    const bool fp32_atomics = a->deterministic == 0 && a->dq_acc_dtype == FMHA_DQ_ACC_FP32;
    p->tile_m = a->d_qk == 192 ? 32 : (a->d_qk == 64 && !fp32_atomics ? 128 : 64);
    // with a bias, blocks are half as tall (32 rows at d_qk = 128, 64 at d_qk = 64): the bias
    // registers of the taller blocks do not fit beside the rest of the main kernel's
    // registers (dropout alone does fit).  At d_qk = 128, 64-row blocks stay when the kernel
    // can stage the bias in 16-byte chunks (rows 16-byte aligned, Sk a multiple of 8; the
    // same test as the kernel's), which needs no bias registers across the step.
    const int64_t bstr = (a->bias_b == 1 ? 0 : a->bias_stride[0]) | (a->bias_h == 1 ? 0 : a->bias_stride[1]) |
                         a->bias_stride[2];
    const bool staged = ((uintptr_t)a->bias & 15u) == 0 && (bstr & 7) == 0 && (a->Sk & 7) == 0;
    if (with_bias && a->d_qk == 128) p->tile_m = staged ? 64 : 32;
    if (with_bias && a->d_qk == 64) p->tile_m = 64;
    if (a->tune_tile_m != 0) {
      const int v = a->tune_tile_m;
      const bool ok = (a->d_qk == 128 && (v == 32 || (v == 64 && (!with_bias || staged)))) ||
                      (a->d_qk == 64 && ((v == 64) || (v == 128 && !with_bias))) ||
                      (a->d_qk == 192 && v == 32);
      if (!ok) return fail(FMHA_ERR_INVALID_ARG, err, el, "tune_tile_m is not a block height of this kernel");
      p->tile_m = v;
    }
    p->tile_n = 128;
  }
  p->deterministic = a->deterministic == 1;
  p->dq_bf16 = a->dq_acc_dtype == FMHA_DQ_ACC_BF16;

  int64_t max_lq = a->Sq, max_lk = a->Sk;
  if (group) {
    if (!a->seqstart_k_host || !a->seqstart_q_dev || !a->seqstart_k_dev)
      return fail(FMHA_ERR_INVALID_ARG, err, el,
                  "group mode needs host and device seqstart arrays for both q and k");
    const int32_t* sq = a->seqstart_q_host;
    const int32_t* sk = a->seqstart_k_host;
    const int32_t* pq = a->seqstart_q_padded_host;
    const int32_t* pk = a->seqstart_k_padded_host;
    if ((pq == nullptr) != (a->seqstart_q_padded_dev == nullptr) ||
        (pk == nullptr) != (a->seqstart_k_padded_dev == nullptr))
      return fail(FMHA_ERR_INVALID_ARG, err, el,
                  "padded seqstart arrays come in host/device pairs");
    if (sq[0] < 0 || sk[0] < 0 || (pq && pq[0] < 0) || (pk && pk[0] < 0))
      return fail(FMHA_ERR_INVALID_ARG, err, el, "seqstart offsets must be non-negative");
    max_lq = 0;
    max_lk = 0;
    for (int b = 0; b < a->B; ++b) {
      const int64_t lq = (int64_t)sq[b + 1] - sq[b];
      const int64_t lk = (int64_t)sk[b + 1] - sk[b];
      if (lq < 0 || lk < 0)
        return fail(FMHA_ERR_INVALID_ARG, err, el, "seqstart offsets must be non-decreasing");
      if (lq > a->Sq || lk > a->Sk)
        return fail(FMHA_ERR_INVALID_ARG, err, el,
                    "a segment is longer than Sq/Sk (the maximum segment lengths)");
      if (lq > max_lq) max_lq = lq;
      if (lk > max_lk) max_lk = lk;
      if ((pq && (int64_t)pq[b] + lq > pq[b + 1]) || (pk && (int64_t)pk[b] + lk > pk[b + 1]))
        return fail(FMHA_ERR_INVALID_ARG, err, el,
                    "a segment does not fit its padded slot (padded[b] + length > padded[b+1])");
    }
    p->rows_q = a->B > 0 ? (pq ? pq[a->B] : sq[a->B]) : 0;
    p->rows_k = a->B > 0 ? (pk ? pk[a->B] : sk[a->B]) : 0;
  } else {
    if (a->seqstart_k_host || a->seqstart_q_dev || a->seqstart_k_dev)
      return fail(FMHA_ERR_INVALID_ARG, err, el,
                  "seqstart arrays must be all null (batch mode) or all set (group mode)");
    if (a->seqstart_q_padded_host || a->seqstart_k_padded_host || a->seqstart_q_padded_dev ||
        a->seqstart_k_padded_dev)
      return fail(FMHA_ERR_INVALID_ARG, err, el, "padded seqstart arrays need group mode");
    p->rows_q = (int64_t)a->B * a->Sq;
    p->rows_k = (int64_t)a->B * a->Sk;
  }

  // pointers and strides (only when there is data to touch)
  const bool any_q = p->rows_q > 0;
  const bool any_k = group ? (a->B > 0 && a->seqstart_k_host[a->B] > 0) : ((int64_t)a->B * a->Sk > 0);
  if (any_q) {
    if (!a->q || !a->o || !a->lse || (!forward && (!a->dout || !a->dq)))
      return fail(FMHA_ERR_INVALID_ARG, err, el,
                  forward ? "q, o and lse must be set" : "q, o, dout, dq and lse must be set");
    if (!aligned16(a->q) || !aligned16(a->o) ||
        (!forward && (!aligned16(a->dout) || !aligned16(a->dq))))
      return fail(FMHA_ERR_UNSUPPORTED, err, el, "bf16 tensors must be 16-byte aligned");
    if (((uintptr_t)a->lse & 3u) != 0)
      return fail(FMHA_ERR_INVALID_ARG, err, el, "lse must be 4-byte aligned");
    if (!strides_ok(a->q_stride, group) || !strides_ok(a->o_stride, group) ||
        (!forward && (!strides_ok(a->do_stride, group) || !strides_ok(a->dq_stride, group))))
      return fail(FMHA_ERR_UNSUPPORTED, err, el,
                  "q/o/dout/dq strides must be non-negative multiples of 8 elements (sequence stride < 2^24)");
    if ((!group && a->lse_stride[0] < 0) || a->lse_stride[1] < 0)
      return fail(FMHA_ERR_INVALID_ARG, err, el, "lse strides must be non-negative");
  }
  if (any_k) {
    if (!a->k || !a->v || (!forward && (!a->dk || !a->dv)))
      return fail(FMHA_ERR_INVALID_ARG, err, el,
                  forward ? "k and v must be set" : "k, v, dk and dv must be set");
    if (!aligned16(a->k) || !aligned16(a->v) ||
        (!forward && (!aligned16(a->dk) || !aligned16(a->dv))))
      return fail(FMHA_ERR_UNSUPPORTED, err, el, "bf16 tensors must be 16-byte aligned");
    if (!strides_ok(a->k_stride, group) || !strides_ok(a->v_stride, group) ||
        (!forward && (!strides_ok(a->dk_stride, group) || !strides_ok(a->dv_stride, group))))
      return fail(FMHA_ERR_UNSUPPORTED, err, el,
                  "k/v/dk/dv strides must be non-negative multiples of 8 elements (sequence stride < 2^24)");
  }

  // additive bias (batch mode only)
  p->has_bias = a->bias != nullptr;
  p->has_dbias = !forward && a->dbias != nullptr;
  p->bias_b = p->has_bias ? a->bias_b : 0;
  p->bias_h = p->has_bias ? a->bias_h : 0;
  p->bias_plane_bytes = 0;
  if (p->has_bias) {
    if (group) return fail(FMHA_ERR_UNSUPPORTED, err, el, "a bias needs batch mode");
    if ((a->bias_b != 1 && a->bias_b != a->B) || (a->bias_h != 1 && a->bias_h != a->Hq))
      return fail(FMHA_ERR_INVALID_ARG, err, el, "bias_b must be 1 or B and bias_h 1 or Hq");
    const int64_t* bs = a->bias_stride;
    if (((uintptr_t)a->bias & 1u) != 0 || bs[0] < 0 || bs[1] < 0 || bs[2] < a->Sk)
      return fail(FMHA_ERR_UNSUPPORTED, err, el,
                  "bias must be 2-byte aligned with non-negative strides and row stride >= Sk");
    // row offsets inside a plane, including one block of rows past the end, stay below 2^31
    if (((int64_t)a->Sq + 256) * bs[2] + a->Sk >= (int64_t(1) << 30))
      return fail(FMHA_ERR_UNSUPPORTED, err, el, "bias plane too large ((Sq + 256) * row stride >= 2^30)");
    p->bias_plane_bytes = (a->Sq > 0 && a->Sk > 0) ? (uint32_t)((((int64_t)a->Sq - 1) * bs[2] + a->Sk) * 2) : 0u;
    if (p->has_dbias) {
      const int64_t* ds = a->dbias_stride;
      if (((uintptr_t)a->dbias & 1u) != 0 || ds[0] < 0 || ds[1] < 0 || ds[2] < a->Sk)
        return fail(FMHA_ERR_UNSUPPORTED, err, el,
                    "dbias must be 2-byte aligned with non-negative strides and row stride >= Sk");
      if (((int64_t)a->Sq + 256) * a->Sk >= (int64_t(1) << 30) ||
          ((int64_t)a->Sq + 256) * ds[2] + a->Sk >= (int64_t(1) << 30))
        return fail(FMHA_ERR_UNSUPPORTED, err, el, "dbias plane too large ((Sq + 256) * row stride >= 2^30)");
    }
  }

  p->n_kv_tiles = (int)((max_lk + p->tile_n - 1) / p->tile_n);
  p->n_q_blocks = (int)((max_lq + p->tile_m - 1) / p->tile_m);
  // Deterministic mode: one work item walks tiles_per_item consecutive key tiles and adds
  // their dQ contributions into one split, so the reduction reads 1/tiles_per_item of the
  // per-tile partials.  The largest of 4 and 2 that still leaves two work items per compute
  // unit of an MI355X (256 CUs) is used, so that the heaviest causal items do not set the
  // makespan; without a mask, or with a window bounded on both sides, every tile carries
  // about the same work and one item per compute unit suffices.
  p->tiles_per_item = 1;
  if (p->deterministic) {
    const int64_t heads = (int64_t)p->Hkv * p->B;
    const bool even_work = a->mask_type == FMHA_MASK_NONE ||
                           (a->mask_type == FMHA_MASK_WINDOW && a->window_left >= 0 && a->window_right >= 0);
    const int64_t min_items = even_work ? 256 : 2 * 256;
    for (int t : {4, 2}) {
      if ((int64_t)((p->n_kv_tiles + t - 1) / t) * heads >= min_items) {
        p->tiles_per_item = t;
        break;
      }
    }
  }
  // Long causal segments (8192 keys or more) whose 4-tile items (counted in 128-key tiles)
  // number between one and two per CU: 4 tiles per item, split into parts that make about
  // 1024 work groups of the four-wave layout or 512 of the wide one (one per CU at a time,
  // two rounds).  The parts balance the heavy causal items, and the dK/dV partials they add
  // are small next to the work of such long rows, while the dQ reduction reads 1/4 of what
  // one-tile items leave.
  p->kv_parts = 1;
  bool long_rule = false;
  if (p->deterministic && max_lk >= 8192) {
    const int64_t heads = (int64_t)p->Hkv * p->B;
    const bool even_work = a->mask_type == FMHA_MASK_NONE ||
                           (a->mask_type == FMHA_MASK_WINDOW && a->window_left >= 0 && a->window_right >= 0);
    const int64_t tiles128 = (max_lk + 127) / 128;
    const int64_t items4_128 = (tiles128 + 3) / 4 * heads;
    if (!even_work && items4_128 >= 256 && items4_128 < 512) {
      p->tiles_per_item = 4;
      const int64_t items4 = (int64_t)((p->n_kv_tiles + 3) / 4) * heads;
      const int64_t target = p->kernel == FMHA_KERNEL_WIDE ? 512 : 1024;
      const int64_t parts = (target + items4 - 1) / items4;
      p->kv_parts = (int)(parts > 4 ? 4 : parts);
      long_rule = true;
    }
  }
  // Wide layout, uneven items: the (segment, K/V head, key tile) items' steps (query heads x
  // query blocks) are counted from the mask and the segment lengths.  When the heaviest item
  // has more than 1.6 times the steps each CU would get with a perfect split, and the items
  // are long enough (64 steps or more on average) for the fp32 dK/dV partials to be cheap
  // next to their work, two parts halve the heaviest item.  Measured on MI355X: 8192 ragged
  // tokens of the Llama-3-8B head shape gain 12-15%, while 2x16x2048 causal (36 steps per
  // item) loses 10%, its partials costing more than the balance gains.
  // (Batches of more than 4096 segment tiles fill the GPU anyway and skip the count.)
  const int nseg = group ? a->B : (a->B > 0 ? 1 : 0);
  if (p->kernel == FMHA_KERNEL_WIDE && !long_rule && !forward && (int64_t)nseg * p->n_kv_tiles <= 4096) {
    int64_t total = 0, heaviest = 0, nonempty = 0;
    for (int b = 0; b < nseg; ++b) {
      const int64_t lq = group ? (int64_t)a->seqstart_q_host[b + 1] - a->seqstart_q_host[b] : a->Sq;
      const int64_t lk = group ? (int64_t)a->seqstart_k_host[b + 1] - a->seqstart_k_host[b] : a->Sk;
      const int64_t reps = group ? p->Hkv : (int64_t)p->Hkv * a->B;
      const MaskGeom g = mask_geom(a->mask_type, a->window_left, a->window_right, lq, lk);
      for (int j = 0; (int64_t)j * p->tile_n < lk; ++j) {
        int64_t lo, hi;
        qblocks_for_tile(g, lq, lk, j, p->tile_m, p->tile_n, &lo, &hi);
        if (hi < lo) continue;
        const int64_t steps = (hi - lo + 1) * p->group_size;
        total += steps * reps;
        nonempty += reps;
        if (steps > heaviest) heaviest = steps;
      }
    }
    if (nonempty > 0 && heaviest * 256 * 5 > total * 8 && total >= 64 * nonempty) p->kv_parts = 2;
  }
  // Too few (K/V head, key tile) items to give every CU one: split each item's steps (query
  // heads x query blocks) over kv_parts work groups that add fp32 dK/dV partials, summed in
  // ascending part order afterwards, aiming at 512 work groups.  A part owns the same (query
  // head, query block) pairs on every tile of its item, so deterministic items keep the
  // largest of 4 and 2 tiles for which 8 parts still reach that count.
  {
    const int64_t heads = (int64_t)p->Hkv * p->B;
    const int64_t items_now = (int64_t)((p->n_kv_tiles + p->tiles_per_item - 1) / p->tiles_per_item) * heads;
    if (items_now > 0 && items_now < 256) {
      p->tiles_per_item = 1;
      if (p->deterministic) {
        for (int t : {4, 2}) {
          if ((int64_t)((p->n_kv_tiles + t - 1) / t) * heads * 8 >= 512) {
            p->tiles_per_item = t;
            break;
          }
        }
      }
      const int64_t items = (int64_t)((p->n_kv_tiles + p->tiles_per_item - 1) / p->tiles_per_item) * heads;
      const int64_t parts = (512 + items - 1) / items;
      p->kv_parts = (int)(parts < 1 ? 1 : (parts > 8 ? 8 : parts));
    }
  }
  // the overrides, each replacing its own choice
  if (a->tune_tiles_per_item != 0 && p->deterministic) p->tiles_per_item = a->tune_tiles_per_item;
  if (a->tune_kv_parts != 0) p->kv_parts = a->tune_kv_parts;
  // bf16 accumulation rounds the running sum once per key tile: past 64 additions per dQ
  // element its error estimate (relative rms u*sqrt(n/6), u = 2^-8) leaves the cosine bar
  if (p->dq_bf16 && p->n_kv_tiles > 64)
    return fail(FMHA_ERR_UNSUPPORTED, err, el,
                "the bf16 dQ accumulator is limited to 64 key tiles per segment (accuracy); use fp32");
  const int n_items = (p->n_kv_tiles + p->tiles_per_item - 1) / p->tiles_per_item;
  p->nsplits = p->deterministic ? (n_items > 0 ? n_items : 1) : 1;
  p->needs_zero = !p->deterministic;
  p->max_rows_q = p->rows_q;

  p->acc_pad = p->deterministic ? p->tile_m : 0;
  p->acc_rows = p->rows_q + (int64_t)p->B * p->acc_pad;
  if (p->dq_bf16) p->acc_rows = align_up(max_lq, p->tile_m);  // one slot per (segment, head)
  p->head_stride = p->acc_rows * p->d_qk;
  p->split_stride = (int64_t)p->Hq * p->head_stride;
  p->d_offset = kHeaderBytes;
  p->d_bytes = (int64_t)p->Hq * p->rows_q * 4;
  p->lse2_offset = align_up(p->d_offset + p->d_bytes, 256);
  p->dq_acc_offset = align_up(p->lse2_offset + p->d_bytes, 256);
  p->dq_acc_bytes = p->dq_bf16 ? (int64_t)p->B * p->split_stride * 2
                               : (int64_t)p->nsplits * p->split_stride * 4;
  // A full-shape dbias (no broadcast dimension) is dS itself: the main kernel writes it as
  // bf16, and the reduce stage only fills the pairs it skipped with zeros.  Broadcast shapes
  // sum the full-shape dS, kept in fp32 in the workspace.
  p->dbias_direct = p->has_dbias && p->bias_b == p->B && p->bias_h == p->Hq;
  p->dbias_plane_bytes = (p->has_dbias && a->Sq > 0 && a->Sk > 0)
                             ? (uint32_t)((((int64_t)a->Sq - 1) * a->dbias_stride[2] + a->Sk) * 2) : 0u;
  p->dbias_acc_offset = align_up(p->dq_acc_offset + p->dq_acc_bytes, 256);
  p->dbias_acc_bytes = p->has_dbias && !p->dbias_direct ? (int64_t)p->B * p->Hq * p->Sq * p->Sk * 4 : 0;
  p->dkv_acc_offset = align_up(p->dbias_acc_offset + p->dbias_acc_bytes, 256);
  p->dkv_acc_bytes = p->kv_parts > 1 && !forward
                         ? (int64_t)p->kv_parts * p->Hkv * p->rows_k * (p->d_qk + p->d_v) * 4 : 0;
  // Ragged batches in the wide layout: the main kernel's work groups take their items longest
  // first (a list one extra work group of the D stage builds), instead of in grid order, where the short
  // segments' items and the empty ones of the grid's rectangle interleave with the long ones.
  // A greedy longest-first list schedule of the 8192-token packings' work groups on 256 CUs
  // ends about 12% earlier than the grid order.  Up to 2048 work groups (the list is ranked by
  // one work group); larger grids fill the GPU in any order.
  p->order_n = 0;
  p->order_offset = align_up(p->dkv_acc_offset + p->dkv_acc_bytes, 256);
  if (group && !forward && p->kernel == FMHA_KERNEL_WIDE) {
    const int64_t wgs = (int64_t)((p->n_kv_tiles + p->tiles_per_item - 1) / p->tiles_per_item) *
                        p->kv_parts * p->Hkv * p->B;
    if (wgs > 1 && wgs <= 2048) p->order_n = (int)wgs;
  }
  p->workspace_bytes = align_up(p->order_offset + (int64_t)p->order_n * 4, 256);
  // what a run reads from the workspace depends on exactly these (and the segment offsets)
  Fnv f;
  for (int64_t x : {(int64_t)p->B, (int64_t)p->Hq, (int64_t)p->Hkv, (int64_t)p->Sq, (int64_t)p->Sk,
                    (int64_t)p->d_qk, (int64_t)p->d_v, (int64_t)p->tile_m, (int64_t)p->tile_n,
                    (int64_t)p->tiles_per_item, (int64_t)p->nsplits, (int64_t)p->deterministic,
                    (int64_t)p->dq_bf16, (int64_t)p->group_mode, p->rows_q, p->acc_rows,
                    (int64_t)p->acc_pad, p->d_offset, p->lse2_offset, p->dq_acc_offset,
                    p->dq_acc_bytes, p->dbias_acc_offset, p->dbias_acc_bytes, p->workspace_bytes,
                    (int64_t)p->kv_parts, p->dkv_acc_offset, p->dkv_acc_bytes,
                    (int64_t)a->mask_type, (int64_t)a->window_left, (int64_t)a->window_right,
                    (int64_t)p->kernel, (int64_t)p->order_n, p->order_offset})
    f.v(x);
  if (group && a->B > 0) {
    f.add(a->seqstart_q_host, sizeof(int32_t) * (a->B + 1));
    f.add(a->seqstart_k_host, sizeof(int32_t) * (a->B + 1));
    if (a->seqstart_q_padded_host) f.add(a->seqstart_q_padded_host, sizeof(int32_t) * (a->B + 1));
    if (a->seqstart_k_padded_host) f.add(a->seqstart_k_padded_host, sizeof(int32_t) * (a->B + 1));
  }
  p->fingerprint = f.h;
  if (p->workspace_bytes == 0) p->workspace_bytes = 256;
  return FMHA_OK;
}

int64_t count_pairs(const fmha_bwd_args* a) {
  const bool group = a->seqstart_q_host != nullptr;
  int64_t pairs = 0;
  for (int b = 0; b < (group ? a->B : (a->B > 0 ? 1 : 0)); ++b) {
    const int64_t lq = group ? (int64_t)a->seqstart_q_host[b + 1] - a->seqstart_q_host[b] : a->Sq;
    const int64_t lk = group ? (int64_t)a->seqstart_k_host[b + 1] - a->seqstart_k_host[b] : a->Sk;
    const MaskGeom g = mask_geom(a->mask_type, a->window_left, a->window_right, lq, lk);
    int64_t seg = 0;
    for (int64_t i = 0; i < lq; ++i) seg += keys_of_row(g, i, lk);
    pairs += group ? seg : seg * a->B;
  }
  return pairs * a->Hq;
}

int64_t reduce_read_bytes(const fmha_bwd_args* a, const Plan& p) {
  const bool group = a->seqstart_q_host != nullptr;
  int64_t total = 0;
  for (int b = 0; b < a->B; ++b) {
    const int64_t lq = group ? (int64_t)a->seqstart_q_host[b + 1] - a->seqstart_q_host[b] : a->Sq;
    const int64_t lk = group ? (int64_t)a->seqstart_k_host[b + 1] - a->seqstart_k_host[b] : a->Sk;
    if (!p.deterministic) {  // one row-major split: the segment's rows
      total += lq * p.d_qk * (p.dq_bf16 ? 2 : 4);
      continue;
    }
    // per query block: the splits whose key tiles touch it (as k_dq_reduce finds them)
    const MaskGeom g = mask_geom(a->mask_type, a->window_left, a->window_right, lq, lk);
    const int64_t nblk = (lq + p.tile_m - 1) / p.tile_m;
    const int ntiles = (int)((lk + p.tile_n - 1) / p.tile_n);
    for (int64_t qb = 0; qb < nblk; ++qb) {
      int jlo = -1, jhi = -1;
      for (int j = 0; j < ntiles; ++j) {
        int64_t lo, hi;
        qblocks_for_tile(g, lq, lk, j, p.tile_m, p.tile_n, &lo, &hi);
        if (qb >= lo && qb <= hi) {
          if (jlo < 0) jlo = j;
          jhi = j;
        }
      }
      if (jlo >= 0)
        total += (int64_t)(jhi / p.tiles_per_item - jlo / p.tiles_per_item + 1) * p.tile_m * p.d_qk * 4;
    }
  }
  return total * a->Hq;
}

}  // namespace fmha
