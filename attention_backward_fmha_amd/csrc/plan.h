// plan.h -- the single host-side derivation of every size, offset and launch shape.
//
// fmha_bwd_workspace_size, fmha_bwd_prepare_workspace and fmha_bwd_run all call make_plan on
// the same arguments; nothing else computes a workspace quantity.  Host only (no HIP calls),
// so it runs and is tested on machines without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fmha_bwd.h"

namespace fmha {

struct Plan {
  bool group_mode;
  int B, Hq, Hkv, group_size;
  int Sq, Sk;            // batch: lengths; group: maximum segment lengths
  int d_qk, d_v;
  int kernel;            // enum fmha_kernel: FMHA_KERNEL_FOUR_WAVE or FMHA_KERNEL_WIDE
  int tile_m, tile_n;    // query rows per block, keys per tile
  int n_kv_tiles;        // key tiles of the longest segment
  int tiles_per_item;    // key tiles per main-kernel work item; deterministic split = item
  int n_q_blocks;        // query blocks of the longest segment (grid extent)
  int nsplits;           // accumulator depth
  bool needs_zero;       // prepare zeroes the accumulator (atomic mode)
  bool deterministic;
  bool dq_bf16;          // bf16 accumulator, packed bf16 atomic adds (non-deterministic only)
  int64_t rows_q;        // accumulator / D rows: B*Sq or seqstart_q[B]
  int64_t d_offset, d_bytes;
  int64_t lse2_offset;   // LSE * log2(e), same shape as D
  int64_t dq_acc_offset, dq_acc_bytes;
  int64_t acc_rows;      // accumulator rows per head: rows_q (atomic), rows_q + B*tile_m
                         // (deterministic); bf16: per (segment, head), pad16(longest lq)
  int acc_pad;           // rows of padding per segment: 0 (atomic) or tile_m
  int64_t split_stride;  // elements between consecutive splits: Hq*acc_rows*d_qk (bf16:
                         // between consecutive segments' slots)
  int64_t head_stride;   // elements between heads inside a split: acc_rows*d_qk
  int64_t workspace_bytes;
  int64_t max_rows_q;    // for the D stage grid: rows_q
  bool has_bias, has_dbias;
  int bias_b, bias_h;
  uint32_t bias_plane_bytes;  // bytes of one (batch, head) bias plane the kernels may read
  int64_t dbias_acc_offset, dbias_acc_bytes;  // fp32 [B][Hq][Sq][Sk] full-shape dS
  int drop_k;            // dropout keep threshold on a random byte (256 = no dropout)
  uint64_t fingerprint;  // FNV-1a of every layout quantity and the host seqstart arrays
  int kv_parts;          // work groups per key tile sharing its steps (fp32 dK/dV partials)
  int64_t rows_k;        // K rows: B*Sk, seqstart_k[B] or the padded k offsets' last entry
  int64_t dkv_acc_offset, dkv_acc_bytes;  // fp32 [kv_parts][Hkv][rows_k][d_qk + d_v]
  bool dbias_direct;     // full-shape (BHSS) dbias: the main kernel writes it directly
  uint32_t dbias_plane_bytes;
  int order_n;           // > 0: main-kernel work groups in a cost order of this many entries
  int64_t order_offset;  // int32 [order_n] written by the D stage's first work group
};

// Validates `a` and fills `p`.  Returns FMHA_OK or a negative status; on failure `err`
// (if not null) receives a message.
// forward = true checks the arguments of fmha_fwd_run instead: q, k, v in; o, lse out;
// dout, dq, dk, dv unused.
int make_plan(const fmha_bwd_args* a, Plan* p, char* err, size_t err_len, bool forward = false);

// Allowed (query, key) pairs over all heads and segments (FLOP accounting).
int64_t count_pairs(const fmha_bwd_args* a);

// Bytes of the dQ accumulator that the reduce stage reads (bandwidth accounting).
int64_t reduce_read_bytes(const fmha_bwd_args* a, const Plan& p);

}  // namespace fmha
