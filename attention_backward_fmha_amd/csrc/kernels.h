// kernels.h -- parameters and launchers of the device stages (implemented in kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace fmha {

// Everything a kernel needs, passed by value as the kernel argument.
struct KParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* o_out;  // forward outputs (the same tensors as o and lse)
  float* lse_out;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dsum;    // workspace: D = rowsum(dO * O), [Hq][rows_q]
  float* lse2;    // workspace: LSE * log2(e), [Hq][rows_q]
  float* dq_acc;  // workspace: fp32 dQ partials, [nsplits][Hq][acc_rows][d_qk]
  const int32_t* seqstart_q;  // device offsets, null in batch mode (segment lengths)
  const int32_t* seqstart_k;
  const int32_t* slot_q;      // device offsets of the padded slots (first physical row), or
  const int32_t* slot_k;      // null: the slots are the segments
  int64_t q_s[3], k_s[3], v_s[3], o_s[3], do_s[3], dq_s[3], dk_s[3], dv_s[3];
  int64_t lse_s[2];
  int64_t split_stride;  // elements
  int64_t head_stride;   // elements
  int64_t rows_q;
  int acc_pad;           // accumulator rows of padding per segment (0 or tile_m)
  int B, Hq, Hkv, group_size, Sq, Sk;
  int mask_type, window_left, window_right;
  int deterministic;
  int dq_bf16;           // dq_acc is bf16 [B][Hq][head_stride/d_qk][d_qk] (split_stride = per segment)
  int n_kv_tiles, n_q_blocks;
  int tiles_per_item;    // key tiles per main-kernel work item (deterministic mode: one split each)
  float scale;
  float scale_log2;  // scale * log2(e)
  int tile_m;        // query rows per main-kernel block
  int tile_n;        // keys per main-kernel tile
  // additive bias (batch mode): plane (b, h) at bias + b*bias_s[0] + h*bias_s[1] (strides of
  // broadcast dimensions are 0), row stride bias_s[2]
  const uint16_t* bias;
  int64_t bias_s[3];
  uint32_t bias_plane_bytes;
  int bias_b, bias_h;
  float* dbias_acc;  // workspace: full-shape dS, fp32 [B][Hq][Sq][Sk]; null without dbias
  uint16_t* dbias;   // output, [bias_b][bias_h][Sq][Sk] with strides dbias_s
  int64_t dbias_s[3];
  int dbias_direct;    // BHSS dbias: bf16 dS straight into dbias (plane bytes below)
  uint32_t dbias_plane_bytes;
  int kv_parts;        // work groups per key tile (>1: fp32 dK/dV partials in dkv_acc)
  float* dkv_acc;      // workspace: fp32 [kv_parts][Hkv][rows_k][d_qk + d_v]
  int64_t rows_k;
  int drop_k;          // dropout: keep iff the element's random byte < drop_k (256 = off)
  float drop_scale;    // 256 / drop_k
  unsigned seed_lo, seed_hi, offset_lo;  // Philox key and the counter's offset word
  int32_t* order;      // workspace: the wide kernel's work groups in cost order, or null
  int order_n;
};

hipError_t launch_dot(const Plan& plan, const KParams& kp, hipStream_t stream);
hipError_t launch_fwd(const Plan& plan, const KParams& kp, hipStream_t stream);
hipError_t launch_main(const Plan& plan, const KParams& kp, hipStream_t stream);
hipError_t launch_main_wide(const Plan& plan, const KParams& kp, dim3 grid, hipStream_t stream);
hipError_t launch_reduce(const Plan& plan, const KParams& kp, hipStream_t stream);
hipError_t launch_dbias(const Plan& plan, const KParams& kp, hipStream_t stream);
hipError_t launch_dkv_reduce(const Plan& plan, const KParams& kp, hipStream_t stream);
// Zeroes count floats at ptr and writes the workspace header (as launch_header) in one launch.
hipError_t launch_zero_header(float* ptr, int64_t count, uint64_t* ws, uint64_t magic, uint64_t fingerprint,
                              hipStream_t stream);
// Workspace header: magic value and plan fingerprint at ws[0], ws[1] (one vector store each).
hipError_t launch_header(uint64_t* ws, uint64_t magic, uint64_t fingerprint, hipStream_t stream);
constexpr uint64_t kWorkspaceMagic = 0x31445742414d4846ull;  // bytes "FHMABWD1"

}  // namespace fmha
