// api.cpp -- the extern "C" entry points declared in include/fmha_bwd.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fmha_bwd.h"
#include "kernels.h"
#include "plan.h"

namespace {

bool log_enabled() {
  const char* e = getenv("FMHA_BWD_LOG");
  return e && e[0] == '1';
}

bool debug_enabled() {
  const char* e = getenv("FMHA_BWD_DEBUG");
  return e && e[0] == '1';
}

int report(int status, const char* where, const char* msg) {
  if (status != FMHA_OK && log_enabled()) fprintf(stderr, "[fmha_bwd] %s: %s\n", where, msg);
  return status;
}

int plan_or_fail(const fmha_bwd_args* a, fmha::Plan* p, const char* where, bool forward = false) {
  char err[256] = {0};
  const int st = fmha::make_plan(a, p, err, sizeof err, forward);
  return report(st, where, err);
}

void log_plan(const fmha::Plan& p, const char* where) {
  if (!log_enabled()) return;
  fprintf(stderr,
          "[fmha_bwd] %s: mode=%s dq_acc=%s B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=(%d,%d) tile=(%d,%d) "
          "kv_tiles=%d q_blocks=%d nsplits=%d T=%d parts=%d kernel=%d zero=%d ws=%lld (D@%lld acc@%lld+%lld)\n",
          where, p.group_mode ? "group" : "batch",
          p.deterministic ? "split-fp32" : (p.dq_bf16 ? "atomic-bf16" : "atomic-fp32"), p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.d_qk, p.d_v,
          p.tile_m, p.tile_n, p.n_kv_tiles, p.n_q_blocks, p.nsplits, p.tiles_per_item, p.kv_parts,
          p.kernel, (int)p.needs_zero,
          (long long)p.workspace_bytes, (long long)p.d_offset, (long long)p.dq_acc_offset,
          (long long)p.dq_acc_bytes);
}

fmha::KParams make_params(const fmha_bwd_args* a, const fmha::Plan& p, void* ws) {
  fmha::KParams k;
  memset(&k, 0, sizeof k);
  k.q = (const uint16_t*)a->q;
  k.k = (const uint16_t*)a->k;
  k.v = (const uint16_t*)a->v;
  k.o = (const uint16_t*)a->o;
  k.dout = (const uint16_t*)a->dout;
  k.lse = a->lse;
  k.o_out = (uint16_t*)a->o;
  k.lse_out = (float*)a->lse;
  k.dq = (uint16_t*)a->dq;
  k.dk = (uint16_t*)a->dk;
  k.dv = (uint16_t*)a->dv;
  if (ws != nullptr) {
    k.dsum = (float*)((char*)ws + p.d_offset);
    k.lse2 = (float*)((char*)ws + p.lse2_offset);
    k.dq_acc = (float*)((char*)ws + p.dq_acc_offset);
  }
  k.seqstart_q = p.group_mode ? a->seqstart_q_dev : nullptr;
  k.seqstart_k = p.group_mode ? a->seqstart_k_dev : nullptr;
  k.slot_q = p.group_mode ? a->seqstart_q_padded_dev : nullptr;
  k.slot_k = p.group_mode ? a->seqstart_k_padded_dev : nullptr;
  for (int i = 0; i < 3; ++i) {
    k.q_s[i] = a->q_stride[i];
    k.k_s[i] = a->k_stride[i];
    k.v_s[i] = a->v_stride[i];
    k.o_s[i] = a->o_stride[i];
    k.do_s[i] = a->do_stride[i];
    k.dq_s[i] = a->dq_stride[i];
    k.dk_s[i] = a->dk_stride[i];
    k.dv_s[i] = a->dv_stride[i];
  }
  k.lse_s[0] = a->lse_stride[0];
  k.lse_s[1] = a->lse_stride[1];
  k.split_stride = p.split_stride;
  k.head_stride = p.head_stride;
  k.rows_q = p.rows_q;
  k.acc_pad = p.acc_pad;
  k.B = p.B;
  k.Hq = p.Hq;
  k.Hkv = p.Hkv;
  k.group_size = p.group_size;
  k.Sq = p.Sq;
  k.Sk = p.Sk;
  k.mask_type = a->mask_type;
  k.window_left = a->window_left;
  k.window_right = a->window_right;
  k.deterministic = p.deterministic ? 1 : 0;
  k.dq_bf16 = p.dq_bf16 ? 1 : 0;
  k.n_kv_tiles = p.n_kv_tiles;
  k.tiles_per_item = p.tiles_per_item;
  k.n_q_blocks = p.n_q_blocks;
  k.scale = a->scale;
  k.scale_log2 = a->scale * 1.4426950408889634f;
  k.tile_m = p.tile_m;
  k.tile_n = p.tile_n;
  if (p.has_bias) {
    k.bias = (const uint16_t*)a->bias;
    k.bias_s[0] = p.bias_b == 1 ? 0 : a->bias_stride[0];
    k.bias_s[1] = p.bias_h == 1 ? 0 : a->bias_stride[1];
    k.bias_s[2] = a->bias_stride[2];
    k.bias_plane_bytes = p.bias_plane_bytes;
    k.bias_b = p.bias_b;
    k.bias_h = p.bias_h;
  }
  k.kv_parts = p.kv_parts;
  k.rows_k = p.rows_k;
  if (ws != nullptr && p.dkv_acc_bytes > 0) k.dkv_acc = (float*)((char*)ws + p.dkv_acc_offset);
  k.drop_k = p.drop_k;
  k.drop_scale = 256.0f / (float)p.drop_k;
  k.seed_lo = (unsigned)(a->philox_seed & 0xFFFFFFFFu);
  k.seed_hi = (unsigned)(a->philox_seed >> 32);
  k.offset_lo = (unsigned)(a->philox_offset & 0xFFFFFFFFu);
  if (p.has_dbias) {
    // the fp32 full-shape dS region exists only for a broadcast dbias; with a direct (BHSS)
    // dbias the pointer stays null, so nothing can address a region the workspace lacks
    if (ws != nullptr && p.dbias_acc_bytes > 0) k.dbias_acc = (float*)((char*)ws + p.dbias_acc_offset);
    k.dbias = (uint16_t*)a->dbias;
    k.dbias_direct = p.dbias_direct ? 1 : 0;
    k.dbias_plane_bytes = p.dbias_plane_bytes;
    for (int i = 0; i < 3; ++i) k.dbias_s[i] = a->dbias_stride[i];
  }
  k.order_n = p.order_n;
  k.order = (ws != nullptr && p.order_n > 0) ? (int32_t*)((char*)ws + p.order_offset) : nullptr;
  return k;
}

int check_ws(const fmha::Plan& p, void* ws, size_t bytes, const char* where) {
  if ((size_t)p.workspace_bytes > bytes)
    return report(FMHA_ERR_WORKSPACE_TOO_SMALL, where, "workspace smaller than fmha_bwd_workspace_size");
  if (!ws) return report(FMHA_ERR_INVALID_ARG, where, "null workspace");
  if (((uintptr_t)ws & 255u) != 0)
    return report(FMHA_ERR_INVALID_ARG, where, "workspace must be 256-byte aligned");
  return FMHA_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return FMHA_OK;
  return report(FMHA_ERR_HIP, where, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int fmha_bwd_workspace_size(const fmha_bwd_args* args, size_t* bytes) {
  if (!bytes) return report(FMHA_ERR_INVALID_ARG, "workspace_size", "null bytes pointer");
  fmha::Plan p;
  const int st = plan_or_fail(args, &p, "workspace_size");
  if (st != FMHA_OK) return st;
  *bytes = (size_t)p.workspace_bytes;
  return FMHA_OK;
}

int fmha_bwd_prepare_workspace(const fmha_bwd_args* args, void* ws, size_t bytes, void* stream) {
  fmha::Plan p;
  int st = plan_or_fail(args, &p, "prepare_workspace");
  if (st != FMHA_OK) return st;
  st = check_ws(p, ws, bytes, "prepare_workspace");
  if (st != FMHA_OK) return st;
  log_plan(p, "prepare_workspace");
  if (p.needs_zero)
    return hip_status(fmha::launch_zero_header((float*)((char*)ws + p.dq_acc_offset), p.dq_acc_bytes / 4,
                                               (uint64_t*)ws, fmha::kWorkspaceMagic, p.fingerprint,
                                               (hipStream_t)stream),
                      "prepare_workspace");
  return hip_status(fmha::launch_header((uint64_t*)ws, fmha::kWorkspaceMagic, p.fingerprint, (hipStream_t)stream),
                    "prepare_workspace");
}

int fmha_bwd_run_stages(const fmha_bwd_args* args, void* ws, size_t bytes, int stages, void* stream) {
  fmha::Plan p;
  int st = plan_or_fail(args, &p, "run");
  if (st != FMHA_OK) return st;
  st = check_ws(p, ws, bytes, "run");
  if (st != FMHA_OK) return st;
  if (stages & ~(FMHA_STAGE_DOT | FMHA_STAGE_MAIN | FMHA_STAGE_REDUCE))
    return report(FMHA_ERR_INVALID_ARG, "run", "unknown stage bits");
  log_plan(p, "run");
  const fmha::KParams kp = make_params(args, p, ws);
  hipStream_t s = (hipStream_t)stream;
  if (debug_enabled()) {  // the workspace must have been prepared for these very arguments
    uint64_t hdr[2] = {0, 0};
    st = hip_status(hipStreamSynchronize(s), "run: debug header check");
    if (st != FMHA_OK) return st;
    st = hip_status(hipMemcpy(hdr, ws, sizeof hdr, hipMemcpyDeviceToHost), "run: debug header check");
    if (st != FMHA_OK) return st;
    if (hdr[0] != fmha::kWorkspaceMagic || hdr[1] != p.fingerprint)
      return report(FMHA_ERR_PLAN_MISMATCH, "run",
                    "the workspace was not prepared for these arguments (header fingerprint differs)");
  }
  if (stages & FMHA_STAGE_DOT) {
    st = hip_status(fmha::launch_dot(p, kp, s), "run: dot stage");
    if (st != FMHA_OK) return st;
  }
  if (stages & FMHA_STAGE_MAIN) {
    st = hip_status(fmha::launch_main(p, kp, s), "run: main stage");
    if (st != FMHA_OK) return st;
  }
  if (stages & FMHA_STAGE_REDUCE) {
    st = hip_status(fmha::launch_reduce(p, kp, s), "run: reduce stage");
    if (st != FMHA_OK) return st;
    if (p.has_dbias) {
      st = hip_status(fmha::launch_dbias(p, kp, s), "run: dbias reduce");
      if (st != FMHA_OK) return st;
    }
    if (p.kv_parts > 1) {
      st = hip_status(fmha::launch_dkv_reduce(p, kp, s), "run: dK/dV reduce");
      if (st != FMHA_OK) return st;
    }
  }
  return FMHA_OK;
}

int fmha_bwd_run(const fmha_bwd_args* args, void* ws, size_t bytes, void* stream) {
  return fmha_bwd_run_stages(args, ws, bytes, FMHA_STAGE_DOT | FMHA_STAGE_MAIN | FMHA_STAGE_REDUCE,
                             stream);
}

int fmha_fwd_run(const fmha_bwd_args* args, void* stream) {
  fmha::Plan p;
  int st = plan_or_fail(args, &p, "fwd", true);
  if (st != FMHA_OK) return st;
  log_plan(p, "fwd");
  const fmha::KParams kp = make_params(args, p, nullptr);
  return hip_status(fmha::launch_fwd(p, kp, (hipStream_t)stream), "fwd");
}

const char* fmha_bwd_status_string(int status) {
  switch (status) {
    case FMHA_OK: return "FMHA_OK";
    case FMHA_ERR_INVALID_ARG: return "FMHA_ERR_INVALID_ARG";
    case FMHA_ERR_UNSUPPORTED: return "FMHA_ERR_UNSUPPORTED";
    case FMHA_ERR_WORKSPACE_TOO_SMALL: return "FMHA_ERR_WORKSPACE_TOO_SMALL";
    case FMHA_ERR_HIP: return "FMHA_ERR_HIP";
    case FMHA_ERR_PLAN_MISMATCH: return "FMHA_ERR_PLAN_MISMATCH";
    default: return "unknown fmha_bwd status";
  }
}

int fmha_bwd_plan_query(const fmha_bwd_args* args, fmha_bwd_plan_info* info) {
  if (!info) return report(FMHA_ERR_INVALID_ARG, "plan_query", "null info pointer");
  fmha::Plan p;
  const int st = plan_or_fail(args, &p, "plan_query");
  if (st != FMHA_OK) return st;
  memset(info, 0, sizeof *info);
  info->group_mode = p.group_mode ? 1 : 0;
  info->tile_m = p.tile_m;
  info->tile_n = p.tile_n;
  info->n_kv_tiles = p.n_kv_tiles;
  info->tiles_per_item = p.tiles_per_item;
  info->n_q_blocks = p.n_q_blocks;
  info->nsplits = p.nsplits;
  info->needs_zero = p.needs_zero ? 1 : 0;
  info->rows_q = p.rows_q;
  info->acc_rows = p.acc_rows;
  info->dq_acc_elem_bytes = p.dq_bf16 ? 2 : 4;
  info->kv_parts = p.kv_parts;
  info->dkv_acc_offset = p.dkv_acc_offset;
  info->dkv_acc_bytes = p.dkv_acc_bytes;
  info->dbias_acc_offset = p.dbias_acc_offset;
  info->dbias_acc_bytes = p.dbias_acc_bytes;
  info->d_offset = p.d_offset;
  info->dq_acc_offset = p.dq_acc_offset;
  info->dq_acc_bytes = p.dq_acc_bytes;
  info->workspace_bytes = p.workspace_bytes;
  info->pairs = fmha::count_pairs(args);
  info->flops = 2.0 * (3.0 * p.d_qk + 2.0 * p.d_v) * (double)info->pairs;
  info->reduce_read_bytes = fmha::reduce_read_bytes(args, p);
  info->kernel = p.kernel;
  info->ordered_groups = p.order_n;
  return FMHA_OK;
}

}  // extern "C"
